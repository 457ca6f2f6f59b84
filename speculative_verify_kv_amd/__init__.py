"""Python binding of libswattn (sliding-window verify attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libswattn.so``.  The functions mirror the C ABI in
``include/swattn.h`` one for one (``swattn_plan``, ``swattn_workspace_bytes``,
``swattn_workspace_init``, ``swattn_verify``, ``swattn_prefill_plan``, ``swattn_prefill``,
``swattn_append_kv``, ``swattn_append_verify``, ``swattn_greedy_accept_workspace``,
``swattn_greedy_accept``, ``swattn_check_inputs``, ``swattn_status_str``,
``swattn_abi_version``, ``swattn_verify_noalloc``, ``swattn_window_gather``,
``swattn_stream_read``);
``verify`` and ``prefill`` are conveniences that fill the descriptor from torch
tensors and run on torch's current HIP stream.  There is no CPU
fallback: if the library is missing, loading fails with an error.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswattn.so")

SWATTN_F32, SWATTN_BF16, SWATTN_FP8_E4M3 = 0, 1, 2
SWATTN_VARIANT_AUTO, SWATTN_VARIANT_VALU, SWATTN_VARIANT_MFMA = 0, 1, 2
SWATTN_MERGE_AUTO, SWATTN_MERGE_KERNEL, SWATTN_MERGE_FUSED = 0, 1, 2
SWATTN_WORKSPACE_COUNTER_BYTES = 4096
SWATTN_MAX_NQ = 64
SWATTN_MAX_PREFILL_NQ = 512

STATUS = {
    0: "SWATTN_OK", -1: "SWATTN_ERR_NULL", -2: "SWATTN_ERR_SHAPE", -3: "SWATTN_ERR_NQ",
    -4: "SWATTN_ERR_WINDOW", -5: "SWATTN_ERR_DTYPE", -6: "SWATTN_ERR_ALIGN",
    -7: "SWATTN_ERR_WORKSPACE", -8: "SWATTN_ERR_CTX", -9: "SWATTN_ERR_BLOCK",
    -10: "SWATTN_ERR_HIP", -11: "SWATTN_ERR_ARG", -12: "SWATTN_ERR_SCRATCH",
}
SWATTN_STATIC_SCRATCH_BYTES = 16 << 20

# Symbols declared in include/swattn.h.
EXPORTED = ("swattn_plan", "swattn_workspace_bytes", "swattn_workspace_init", "swattn_verify", "swattn_prefill_plan",
            "swattn_prefill", "swattn_append_kv", "swattn_append_verify", "swattn_greedy_accept_workspace",
            "swattn_greedy_accept", "swattn_check_inputs", "swattn_status_str", "swattn_abi_version",
            "swattn_verify_noalloc", "swattn_window_gather", "swattn_stream_read")


class SwattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name}: {swattn_status_str(status)}")


class swattn_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("num_splits", ctypes.c_int32), ("variant", ctypes.c_int32), ("merge", ctypes.c_int32),
        ("rows_per_chunk", ctypes.c_int32), ("col_splits", ctypes.c_int32),
    ]


class swattn_plan_t(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("rows_per_chunk", ctypes.c_int32), ("row_chunks", ctypes.c_int32),
        ("grid", ctypes.c_int32), ("merge_grid", ctypes.c_int32), ("fused_merge", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t), ("col_splits", ctypes.c_int32), ("tile_keys", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
ABI_VERSION = 3          # SWATTN_ABI_VERSION these ctypes mirrors follow


def lib():
    """Load libswattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m speculative_verify_kv_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        L.swattn_abi_version.restype = ctypes.c_int32
        if L.swattn_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.swattn_abi_version()}, the binding expects "
                              f"{ABI_VERSION}: rebuild it with `python -m speculative_verify_kv_amd._build`")
        P = ctypes.POINTER
        L.swattn_plan.argtypes = [P(swattn_desc_t), ctypes.c_int32, ctypes.c_int32, P(swattn_plan_t)]
        L.swattn_plan.restype = ctypes.c_int
        L.swattn_workspace_bytes.argtypes = [P(swattn_desc_t), ctypes.c_int32, ctypes.c_int32,
                                             P(ctypes.c_size_t)]
        L.swattn_workspace_bytes.restype = ctypes.c_int
        L.swattn_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.swattn_workspace_init.restype = ctypes.c_int
        L.swattn_verify.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
        L.swattn_verify.restype = ctypes.c_int
        L.swattn_verify_noalloc.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        L.swattn_verify_noalloc.restype = ctypes.c_int
        L.swattn_window_gather.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.swattn_window_gather.restype = ctypes.c_int
        L.swattn_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.swattn_stream_read.restype = ctypes.c_int
        L.swattn_prefill_plan.argtypes = L.swattn_plan.argtypes
        L.swattn_prefill_plan.restype = ctypes.c_int
        L.swattn_prefill.argtypes = L.swattn_verify.argtypes
        L.swattn_prefill.restype = ctypes.c_int
        L.swattn_append_kv.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.swattn_append_kv.restype = ctypes.c_int
        L.swattn_append_verify.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.swattn_append_verify.restype = ctypes.c_int
        L.swattn_greedy_accept_workspace.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                     P(ctypes.c_size_t)]
        L.swattn_greedy_accept_workspace.restype = ctypes.c_int
        L.swattn_greedy_accept.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.swattn_greedy_accept.restype = ctypes.c_int
        L.swattn_check_inputs.argtypes = [P(swattn_desc_t), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        L.swattn_check_inputs.restype = ctypes.c_int
        L.swattn_status_str.argtypes = [ctypes.c_int]
        L.swattn_status_str.restype = ctypes.c_char_p
        L.swattn_abi_version.argtypes = []
        L.swattn_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _ptr(x):
    """Device pointer of a torch tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def swattn_status_str(status):
    return lib().swattn_status_str(int(status)).decode()


def swattn_abi_version():
    return int(lib().swattn_abi_version())


def swattn_plan(desc, n_q, window, check=True):
    plan = swattn_plan_t()
    st = lib().swattn_plan(ctypes.byref(desc), int(n_q), int(window), ctypes.byref(plan))
    if check and st != 0:
        raise SwattnError(st, "swattn_plan")
    return plan if check else (st, plan)


def swattn_prefill_plan(desc, n_q, window, check=True):
    plan = swattn_plan_t()
    st = lib().swattn_prefill_plan(ctypes.byref(desc), int(n_q), int(window), ctypes.byref(plan))
    if check and st != 0:
        raise SwattnError(st, "swattn_prefill_plan")
    return plan if check else (st, plan)


def swattn_workspace_init(workspace, nbytes, stream=None):
    st = lib().swattn_workspace_init(_ptr(workspace), int(nbytes), _ptr(stream))
    if st != 0:
        raise SwattnError(st, "swattn_workspace_init")


def swattn_workspace_bytes(desc, n_q, window):
    n = ctypes.c_size_t(0)
    st = lib().swattn_workspace_bytes(ctypes.byref(desc), int(n_q), int(window), ctypes.byref(n))
    if st != 0:
        raise SwattnError(st, "swattn_workspace_bytes")
    return int(n.value)


def swattn_verify(desc, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out,
                  workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().swattn_verify(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                             _ptr(block_table), _ptr(ctx_len), int(n_q), int(window),
                             float(scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
                             _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_verify")
    return st


def swattn_verify_noalloc(desc, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out, stream=None,
                          check=True):
    st = lib().swattn_verify_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(ctx_len), int(n_q), int(window), float(scale),
                                     _ptr(out), _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_verify_noalloc")
    return st


def swattn_window_gather(desc, q, k_cache, v_cache, block_table, ctx_len, n_q, window, parts, out, stream=None,
                         check=True):
    st = lib().swattn_window_gather(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                    _ptr(ctx_len), int(n_q), int(window), int(parts), _ptr(out), _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_window_gather")
    return st


def swattn_stream_read(src, nbytes, grid, xor_out, stream=None, check=True):
    st = lib().swattn_stream_read(_ptr(src), int(nbytes), int(grid), _ptr(xor_out), _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_stream_read")
    return st


def swattn_prefill(desc, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out,
                   workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().swattn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _ptr(ctx_len), int(n_q), int(window),
                              float(scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
                              _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_prefill")
    return st


def swattn_append_kv(desc, k_new, v_new, new_dtype, block_table, ctx_len, n_new, k_cache, v_cache,
                     stream=None, check=True):
    st = lib().swattn_append_kv(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), int(new_dtype),
                                _ptr(block_table), _ptr(ctx_len), int(n_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_append_kv")
    return st


def swattn_append_verify(desc, q, k_new, v_new, new_dtype, k_cache, v_cache, block_table, ctx_len, n_q, window,
                         scale, out, workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().swattn_append_verify(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), int(new_dtype),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_len), int(n_q),
                                    int(window), float(scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
                                    _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_append_verify")
    return st


def swattn_greedy_accept_workspace(batch, n_q, vocab):
    n = ctypes.c_size_t(0)
    st = lib().swattn_greedy_accept_workspace(int(batch), int(n_q), int(vocab), ctypes.byref(n))
    if st != 0:
        raise SwattnError(st, "swattn_greedy_accept_workspace")
    return int(n.value)


def swattn_greedy_accept(logits, logits_dtype, batch, n_q, vocab, draft_ids, target_ids, accepted, next_token,
                         workspace, workspace_bytes, stream=None, check=True):
    st = lib().swattn_greedy_accept(_ptr(logits), int(logits_dtype), int(batch), int(n_q), int(vocab),
                                    _ptr(draft_ids), _ptr(target_ids), _ptr(accepted), _ptr(next_token),
                                    _ptr(workspace), int(workspace_bytes), _ptr(stream))
    if check and st != 0:
        raise SwattnError(st, "swattn_greedy_accept")
    return st


def greedy_accept(logits, draft_ids, stream=None):
    """Run swattn_greedy_accept on torch device tensors (logits [B, n_q, vocab] float32
    or bfloat16, draft_ids [B, n_q - 1] int32); returns (target_ids, accepted, next_token)."""
    import torch
    B, n_q, vocab = logits.shape
    code = SWATTN_BF16 if logits.dtype == torch.bfloat16 else SWATTN_F32
    tgt = torch.empty((B, n_q), dtype=torch.int32, device=logits.device)
    acc = torch.empty((B,), dtype=torch.int32, device=logits.device)
    nxt = torch.empty((B,), dtype=torch.int32, device=logits.device)
    nbytes = swattn_greedy_accept_workspace(B, n_q, vocab)
    ws = torch.empty(max(nbytes, 8) // 8, dtype=torch.int64, device=logits.device)
    if stream is None:
        stream = torch.cuda.current_stream(logits.device).cuda_stream
    swattn_greedy_accept(logits, code, B, n_q, vocab, draft_ids if n_q > 1 else None, tgt, acc, nxt, ws,
                         ws.numel() * 8, stream)
    return tgt, acc, nxt


def swattn_check_inputs(desc, block_table, ctx_len, n_q, window, stream=None):
    return int(lib().swattn_check_inputs(ctypes.byref(desc), _ptr(block_table), _ptr(ctx_len),
                                         int(n_q), int(window), _ptr(stream)))


# ---------------------------------------------------------------------------
# torch convenience layer (marshalling only)
# ---------------------------------------------------------------------------
def _dtype_code(t):
    import torch
    m = {torch.float32: SWATTN_F32, torch.bfloat16: SWATTN_BF16,
         torch.uint8: SWATTN_FP8_E4M3, torch.float8_e4m3fn: SWATTN_FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def make_desc(q, k_cache, block_table, max_ctx_len, out_dtype=None, k_scale=None, v_scale=None,
              num_splits=0, variant=SWATTN_VARIANT_AUTO, merge=SWATTN_MERGE_AUTO, rows_per_chunk=0, col_splits=0):
    """Descriptor for q [B, n_q, H, D], k_cache [num_blocks, Hkv, bs, D],
    block_table [B, max_blocks]; out_dtype defaults to q's dtype."""
    B, _, H, D = q.shape
    nb, Hkv, bs, _ = k_cache.shape
    d = swattn_desc_t()
    d.batch, d.num_heads, d.num_kv_heads, d.head_dim = B, H, Hkv, D
    d.block_size, d.max_blocks_per_seq, d.num_blocks = bs, block_table.shape[1], nb
    d.max_ctx_len = int(max_ctx_len)
    d.q_dtype = _dtype_code(q)
    d.kv_dtype = _dtype_code(k_cache)
    d.out_dtype = d.q_dtype if out_dtype is None else out_dtype
    d.k_scale = _ptr(k_scale)
    d.v_scale = _ptr(v_scale)
    d.num_splits = int(num_splits)
    d.variant = int(variant)
    d.merge = int(merge)
    d.rows_per_chunk = int(rows_per_chunk)
    d.col_splits = int(col_splits)
    return d


def verify(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, max_ctx_len,
           out=None, out_dtype=None, k_scale=None, v_scale=None, num_splits=0,
           variant=SWATTN_VARIANT_AUTO, workspace=None, stream=None, prefill=False,
           merge=SWATTN_MERGE_AUTO, rows_per_chunk=0, col_splits=0):
    """Run swattn_verify (or swattn_prefill) on torch device tensors; returns (out, plan).

    Allocates ``out`` and a zero-filled workspace with torch when they are not given
    (a caller under graph capture passes both)."""
    import torch
    desc = make_desc(q, k_cache, block_table, max_ctx_len, out_dtype, k_scale, v_scale,
                     num_splits, variant, merge, rows_per_chunk, col_splits)
    plan = (swattn_prefill_plan if prefill else swattn_plan)(desc, n_q, window)
    if out is None:
        tdt = torch.float32 if desc.out_dtype == SWATTN_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=tdt, device=q.device)
    if workspace is None and plan.workspace_bytes > 0:
        workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    (swattn_prefill if prefill else swattn_verify)(desc, q, k_cache, v_cache, block_table, ctx_len, n_q,
                                                   window, scale, out, workspace, ws_bytes, stream)
    return out, plan


def prefill(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, max_ctx_len, **kw):
    """Run swattn_prefill (n_q up to SWATTN_MAX_PREFILL_NQ); arguments as ``verify``."""
    return verify(q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, max_ctx_len,
                  prefill=True, **kw)
