"""Float64 emulation of split-KV attention with a log-sum-exp merge.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The split-KV verify kernel of "The Fast Gemma Challenge: our verified-SOTA
recipe, in full" (manifest ``SPLITKV_VERIFY``; "Published files" row
``splitkv_verify_patch.py``) divides one query set's KV range into pieces that
are scored independently and then combined.  The pages show no formula; the
standard combination used here is exact in real arithmetic:

  per piece s:  m_s = max_j s_j,  l_s = sum_j exp(s_j - m_s),
                O_s = sum_j exp(s_j - m_s) v_j / l_s,  lse_s = m_s + ln l_s
  merged:       M = max_s lse_s,  w_s = exp(lse_s - M),
                out = sum_s w_s O_s / sum_s w_s

A piece with no key inside the query's window contributes lse_s = -inf and
weight 0.  tests/test_oracle.py checks this against ``attend`` for every split
count, which pins the merge formula the GPU path implements independently.
"""
import numpy as np

from .attend import window_bounds, _gather
from .formats import decode


def attend_split_merge(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale,
                       num_splits, q_format="float", kv_format="float",
                       k_scale=None, v_scale=None):
    block_table = np.asarray(block_table, dtype=np.int64)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    qf = decode(q, q_format)
    B, nq, H, D = qf.shape
    _, Hkv, bs, _ = k_cache.shape
    G = H // Hkv
    lo, hi = window_bounds(ctx_len, n_q, window)
    out = np.empty((B, n_q, H, D))
    for b in range(B):
        # The pieces partition the union of the step's windows.
        u_lo, u_hi = int(lo[b, 0]), int(hi[b, n_q - 1])
        edges = np.linspace(u_lo, u_hi + 1, num_splits + 1).round().astype(np.int64)
        for i in range(n_q):
            for h in range(H):
                g = h // G
                lses, Os = [], []
                for s in range(num_splits):
                    pos = np.arange(max(edges[s], lo[b, i]), min(edges[s + 1], hi[b, i] + 1))
                    if pos.size == 0:
                        lses.append(-np.inf)
                        Os.append(np.zeros(D))
                        continue
                    kj = decode(_gather(k_cache, block_table[b], pos, bs), kv_format)[:, g, :]
                    vj = decode(_gather(v_cache, block_table[b], pos, bs), kv_format)[:, g, :]
                    if k_scale is not None:
                        kj = kj * float(k_scale[g])
                    if v_scale is not None:
                        vj = vj * float(v_scale[g])
                    sc = scale * (kj @ qf[b, i, h])
                    m = sc.max()
                    e = np.exp(sc - m)
                    l = e.sum()
                    Os.append((e @ vj) / l)
                    lses.append(m + np.log(l))
                lses = np.array(lses)
                M = lses.max()
                w = np.exp(lses - M)
                out[b, i, h] = (w[:, None] * np.array(Os)).sum(axis=0) / w.sum()
    return out
