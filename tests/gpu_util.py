"""Helpers shared by the GPU parity tests: device upload of a synthetic
workload, one library call, and the tolerance check against the oracle."""
import functools
import sys

import numpy as np
import torch

import oracle
import speculative_verify_kv_amd as sw
import synth

DEV = "cuda:0"

# Tolerances (numerics of the library: exact bf16/e4m3 inputs, fp32 accumulation,
# softmax weights carried as two bf16 terms, output rounded once):
#   bf16 output: elementwise |got - ref| <= ATOL + 1e-2 * |ref|  (bf16 rounding alone
#                is 2^-9 |ref|, so a literal 2e-3 max-abs cannot hold for |ref| >= 1);
#   f32 output:  max |got - ref| <= ATOL and max over rows of
#                ||got - ref||_inf / ||ref||_inf <= 1e-2;
# with ATOL = 2e-3 for bf16 / fp32 KV and 2e-2 for e4m3 KV.
RTOL = 1e-2


def atol_for(kv_dtype):
    return 2e-2 if kv_dtype == synth.workloads.E4M3 else 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _u16_to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def upload(w):
    """Device tensors of a synth.Workload."""
    t = {}
    t["q"] = _u16_to_bf16(w.q) if w.q_dtype == "bf16" else torch.from_numpy(w.q).to(DEV)
    if w.kv_dtype == "bf16":
        t["k"], t["v"] = _u16_to_bf16(w.k_cache), _u16_to_bf16(w.v_cache)
    else:
        t["k"], t["v"] = torch.from_numpy(w.k_cache).to(DEV), torch.from_numpy(w.v_cache).to(DEV)
    t["bt"] = torch.from_numpy(w.block_table).to(DEV)
    t["ctx"] = torch.from_numpy(w.ctx_len).to(DEV)
    if w.k_scale is not None:
        t["ks"] = torch.from_numpy(w.k_scale).to(DEV)
        t["vs"] = torch.from_numpy(w.v_scale).to(DEV)
    else:
        t["ks"] = t["vs"] = None
    return t


def run(w, t=None, out_f32=False, num_splits=0, variant=0, max_ctx=None, prefill=False, merge=0, workspace=None,
        rows_per_chunk=0, col_splits=0):
    """One swattn_verify (or swattn_prefill) call; returns (float64 numpy output, plan)."""
    t = upload(w) if t is None else t
    mc = int(w.ctx_len.max()) if max_ctx is None else max_ctx
    out, plan = sw.verify(t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale,
                          max_ctx_len=mc, out_dtype=sw.SWATTN_F32 if out_f32 else None,
                          k_scale=t["ks"], v_scale=t["vs"], num_splits=num_splits, variant=variant,
                          prefill=prefill, merge=merge, workspace=workspace, rows_per_chunk=rows_per_chunk,
                          col_splits=col_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), plan


def reference(w):
    return oracle.attend(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_len, w.n_q, w.window,
                         w.scale, q_format=w.q_format, kv_format=w.kv_format,
                         k_scale=w.k_scale, v_scale=w.v_scale)


@functools.lru_cache(maxsize=None)
def named(key):
    w = synth.named_workload(key)
    return w, reference(w)


def errors(got, ref):
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = diff / np.maximum(np.abs(ref), 1e-30)
    max_rel = float(rel.max()) if rel.size else 0.0
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    rows_err = diff.reshape(-1, ref.shape[-1]).max(axis=1)
    row_rel = float((rows_err / np.maximum(rows_ref, 1e-30)).max()) if rows_ref.size else 0.0
    return max_abs, max_rel, row_rel


def check(got, ref, kv_dtype, out_f32, label=""):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    atol = atol_for(kv_dtype)
    max_abs, max_rel, row_rel = errors(got, ref)
    log(f"  {label}: max_abs={max_abs:.3e} max_rel={max_rel:.3e} row_rel={row_rel:.3e}")
    if out_f32:
        assert max_abs <= atol, f"{label}: max_abs {max_abs} > {atol}"
        assert row_rel <= RTOL, f"{label}: row-normwise rel {row_rel} > {RTOL}"
    else:
        bad = np.abs(got - ref) > atol + RTOL * np.abs(ref)
        assert not bad.any(), f"{label}: {int(bad.sum())} elements outside {atol} + {RTOL}|ref|"
