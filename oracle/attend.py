"""Plain-definition oracle: sliding-window verify attention, float64, CPU.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Semantics (from "The Fast Gemma Challenge: our verified-SOTA recipe, in full",
manifest and "What each piece does, and why"):

* One verify step scores ``n_q`` new positions of a sequence: the target token
  plus the MTP drafts (manifest ``SPECULATIVE_CONFIG``: 7 drafts, so n_q = 8;
  ``SPLITKV_VERIFY_MAX_Q``: n_q <= 64).  Plain decode is n_q = 1.
* ``ctx_len[b]`` counts every valid KV position of sequence b *including* the
  n_q new ones, so the first new query sits at p = ctx_len[b] - n_q and query i
  at t = p + i.  (This is the reading under which ``MAX_MODEL_LEN=4096`` keeps
  positions <= 4095.)
* Query i attends to the most recent ``window`` positions up to and including
  its own: keys j with t - window < j <= t (the sliding-window bullet of "What
  each piece does, and why"; the window is per query, so draft i's window starts
  i positions after the target's, and drafts are causal among themselves).
* Grouped-query heads: query head h reads KV head h // (H // Hkv).
* Paged cache: position j of sequence b lives in physical block
  block_table[b, j // bs] at in-block offset j % bs; the cache is laid out
  [num_blocks, Hkv, bs, D].
* out[b, i, h] = sum_j softmax_j(scale * q . k_j) v_j, with no logit cap, bias or
  sink (the pages name none), q and k taken as given (any positional encoding is
  already applied by the caller).
"""
import numpy as np

from .formats import decode


def window_bounds(ctx_len, n_q, window):
    """lo[b, i], hi[b, i]: first and last key position query i of sequence b sees."""
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    p = ctx_len - n_q                                  # position of the target token
    t = p[:, None] + np.arange(n_q, dtype=np.int64)[None, :]
    lo = np.maximum(0, t - window + 1)
    return lo, t


def _gather(cache, block_table_row, positions, bs):
    """Rows of one sequence's logical cache at ``positions``: [n, Hkv, D]."""
    phys = block_table_row[positions // bs]
    off = positions % bs
    return cache[phys, :, off, :]


def _check_shapes(q, k_cache, v_cache, block_table, ctx_len, n_q, window):
    B, nq, H, D = q.shape
    nb, Hkv, bs, Dk = k_cache.shape
    if nq != n_q:
        raise ValueError("q.shape[1] must equal n_q")
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("k_cache / v_cache / q shapes disagree")
    if H % Hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if window < 1:
        raise ValueError("window must be >= 1")
    if block_table.shape[0] != B or len(ctx_len) != B:
        raise ValueError("block_table / ctx_len must have one row per sequence")
    for b in range(B):
        c = int(ctx_len[b])
        if c < n_q or c > block_table.shape[1] * bs:
            raise ValueError(f"ctx_len[{b}]={c} outside [n_q, max_blocks*bs]")
    return B, H, D, Hkv, bs


def attend(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale,
           q_format="float", kv_format="float", k_scale=None, v_scale=None,
           return_weights=False):
    """Exact sliding-window attention for every (sequence, query, head).

    q:            [B, n_q, H, D]  (float array, or uint16 bf16 bits with q_format="bf16")
    k_cache/v_cache: [num_blocks, Hkv, bs, D]  (float, bf16 bits, or e4m3 codes)
    block_table:  [B, max_blocks_per_seq] int
    ctx_len:      [B] int, counts the n_q new positions
    k_scale/v_scale: [Hkv] float scales, multiplied into decoded e4m3 values
    Returns out float64 [B, n_q, H, D]; with return_weights also a float64
    [B, n_q, H, max(ctx_len)] array of softmax weights (0 outside the window).
    """
    block_table = np.asarray(block_table, dtype=np.int64)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    qf = decode(q, q_format)
    B, H, D, Hkv, bs = _check_shapes(qf, k_cache, v_cache, block_table, ctx_len, n_q, window)
    G = H // Hkv
    ks = None if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    vs = None if v_scale is None else np.asarray(v_scale, dtype=np.float64)

    out = np.empty((B, n_q, H, D), dtype=np.float64)
    weights = np.zeros((B, n_q, H, int(ctx_len.max())), dtype=np.float64) if return_weights else None
    lo, hi = window_bounds(ctx_len, n_q, window)
    for b in range(B):
        for i in range(n_q):
            pos = np.arange(lo[b, i], hi[b, i] + 1, dtype=np.int64)
            kj = decode(_gather(k_cache, block_table[b], pos, bs), kv_format)   # [n, Hkv, D]
            vj = decode(_gather(v_cache, block_table[b], pos, bs), kv_format)
            if ks is not None:
                kj = kj * ks[None, :, None]
            if vs is not None:
                vj = vj * vs[None, :, None]
            for h in range(H):
                g = h // G
                s = scale * (kj[:, g, :] @ qf[b, i, h])     # [n]
                e = np.exp(s - s.max())
                w = e / e.sum()
                out[b, i, h] = w @ vj[:, g, :]
                if return_weights:
                    weights[b, i, h, pos] = w
    if return_weights:
        return out, weights
    return out


def attend_bruteforce(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale,
                      q_format="float", kv_format="float", k_scale=None, v_scale=None):
    """Same result by a different route, for tiny inputs only.

    Rebuilds each sequence's whole logical K/V ([ctx, Hkv, D]) position by
    position, builds a dense [n_q, ctx] boolean mask entry by entry from the
    window rule, sets masked scores to -inf and takes the softmax over every
    position.
    """
    block_table = np.asarray(block_table, dtype=np.int64)
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    qf = decode(q, q_format)
    B, H, D, Hkv, bs = _check_shapes(qf, k_cache, v_cache, block_table, ctx_len, n_q, window)
    G = H // Hkv
    out = np.empty((B, n_q, H, D), dtype=np.float64)
    for b in range(B):
        ctx = int(ctx_len[b])
        p = ctx - n_q
        Kf = np.empty((ctx, Hkv, D))
        Vf = np.empty((ctx, Hkv, D))
        for pos in range(ctx):
            blk = int(block_table[b, pos // bs])
            for g in range(Hkv):
                Kf[pos, g] = decode(k_cache[blk, g, pos % bs], kv_format)
                Vf[pos, g] = decode(v_cache[blk, g, pos % bs], kv_format)
                if k_scale is not None:
                    Kf[pos, g] *= float(k_scale[g])
                if v_scale is not None:
                    Vf[pos, g] *= float(v_scale[g])
        mask = np.zeros((n_q, ctx), dtype=bool)
        for i in range(n_q):
            for j in range(ctx):
                mask[i, j] = (j <= p + i) and (j > p + i - window)
        for h in range(H):
            g = h // G
            S = scale * (qf[b, :, h, :] @ Kf[:, g, :].T)   # [n_q, ctx]
            S = np.where(mask, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P = P / P.sum(axis=1, keepdims=True)
            out[b, :, h, :] = P @ Vf[:, g, :]
    return out
