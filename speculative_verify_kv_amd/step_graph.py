"""One decode step of a model's attention layers, captured as HIP graphs.

A model runs its layers one after another.  Per layer, the step's n_q new K/V rows
go into that layer's paged cache and the layer's verify attention runs.  After the
last layer, the target's logits decide how many drafts are accepted.  The step is
captured once per buffer slot and the graphs are replayed round-robin.  This is the
decode loop of "The Fast Gemma Challenge: our verified-SOTA recipe, in full"
(manifest ONEGRAPH, LOOPGRAPH_REQUIRE_CAPTURE=1, LOOPGRAPH_PINGPONG_SLOTS=3,
LOOPGRAPH_WARMUP_CALLS=20; "What each piece does, and why": one graph per step
takes the per-kernel launch overhead away).

Three forms issue the same step:

* ``fused``: per layer, one ``swattn_append_verify`` call;
* ``separate``: per layer, ``swattn_append_kv`` then ``swattn_verify``;
* ``stacked``: one ``swattn_append_kv`` and one ``swattn_verify`` over all layers
  at once (the layers stacked along the batch axis).

Each form ends with one ``swattn_greedy_accept`` call.  This module only
sequences library calls and captures them; every step runs in libswattn's kernels.
"""
import torch

from . import (SWATTN_BF16, SWATTN_F32, swattn_append_kv, swattn_append_verify, swattn_desc_t,
               swattn_greedy_accept, swattn_greedy_accept_workspace, swattn_plan, swattn_verify)

FORMS = ("fused", "separate", "stacked")


def _desc(batch, H, k_cache, max_blocks, max_ctx_len, num_splits, out_dtype):
    nb, Hkv, bs, D = k_cache.shape
    d = swattn_desc_t()
    d.batch, d.num_heads, d.num_kv_heads, d.head_dim = batch, H, Hkv, D
    d.block_size, d.max_blocks_per_seq, d.num_blocks = bs, max_blocks, nb
    d.max_ctx_len = int(max_ctx_len)
    d.q_dtype, d.kv_dtype, d.out_dtype = SWATTN_BF16, SWATTN_BF16, out_dtype
    d.k_scale = d.v_scale = None
    d.num_splits = int(num_splits)
    d.variant = d.merge = 0
    return d


class LayerStep:
    """The step of L layers whose bfloat16 caches share one pool: layer l's blocks are
    listed in ``block_table[l]`` and its context length is ``ctx_len[l]`` (counting the
    step's n_q new positions).

    ``issue(inputs, outputs, stream)`` enqueues one step, with ``inputs`` a dict of
    q [L, n_q, H, D], kn / vn [L, n_q, Hkv, D] (bfloat16), logits [1, n_q, vocab]
    (bfloat16) and drafts [1, n_q - 1] (int32), and ``outputs`` one made by
    ``new_outputs()``.  ``capture(inputs, outputs)`` returns the step as a
    torch.cuda.CUDAGraph."""

    def __init__(self, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, num_heads, vocab,
                 form="fused", num_splits=0, max_ctx_len=4096, out_dtype=SWATTN_BF16):
        if form not in FORMS:
            raise ValueError(f"form must be one of {FORMS}")
        self.k, self.v, self.bt, self.ctx = k_cache, v_cache, block_table, ctx_len
        self.L = int(block_table.shape[0])
        self.n_q, self.window, self.scale, self.H, self.vocab = int(n_q), int(window), float(scale), num_heads, vocab
        self.form, self.out_dtype = form, out_dtype
        dev = k_cache.device
        mb = int(block_table.shape[1])
        self.desc_layer = _desc(1, num_heads, k_cache, mb, max_ctx_len, num_splits, out_dtype)
        self.desc_all = _desc(self.L, num_heads, k_cache, mb, max_ctx_len, num_splits, out_dtype)
        self.plan_layer = swattn_plan(self.desc_layer, n_q, window)
        self.plan_all = swattn_plan(self.desc_all, n_q, window)
        # the per-layer calls run one after another on the stream: one workspace serves them all
        ws_bytes = self.plan_all.workspace_bytes if form == "stacked" else self.plan_layer.workspace_bytes
        self.ws_bytes = ws_bytes
        self.ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.ws_acc = torch.empty(swattn_greedy_accept_workspace(1, n_q, vocab) // 8 + 1, dtype=torch.int64,
                                  device=dev)

    def new_outputs(self):
        dev = self.k.device
        D = self.k.shape[3]
        tdt = torch.float32 if self.out_dtype == SWATTN_F32 else torch.bfloat16
        return dict(out=torch.empty((self.L, self.n_q, self.H, D), dtype=tdt, device=dev),
                    tgt=torch.empty((1, self.n_q), dtype=torch.int32, device=dev),
                    acc=torch.empty((1,), dtype=torch.int32, device=dev),
                    nxt=torch.empty((1,), dtype=torch.int32, device=dev))

    def issue(self, inputs, outputs, stream):
        n, W, sc = self.n_q, self.window, self.scale
        q, kn, vn, out = inputs["q"], inputs["kn"], inputs["vn"], outputs["out"]
        if self.form == "fused":
            for l in range(self.L):
                swattn_append_verify(self.desc_layer, q[l:l + 1], kn[l:l + 1], vn[l:l + 1], SWATTN_BF16, self.k,
                                     self.v, self.bt[l:l + 1], self.ctx[l:l + 1], n, W, sc, out[l:l + 1], self.ws,
                                     self.ws_bytes, stream)
        elif self.form == "separate":
            for l in range(self.L):
                swattn_append_kv(self.desc_layer, kn[l:l + 1], vn[l:l + 1], SWATTN_BF16, self.bt[l:l + 1],
                                 self.ctx[l:l + 1], n, self.k, self.v, stream)
                swattn_verify(self.desc_layer, q[l:l + 1], self.k, self.v, self.bt[l:l + 1], self.ctx[l:l + 1], n, W,
                              sc, out[l:l + 1], self.ws, self.ws_bytes, stream)
        else:
            swattn_append_kv(self.desc_all, kn, vn, SWATTN_BF16, self.bt, self.ctx, n, self.k, self.v, stream)
            swattn_verify(self.desc_all, q, self.k, self.v, self.bt, self.ctx, n, W, sc, out, self.ws, self.ws_bytes,
                          stream)
        swattn_greedy_accept(inputs["logits"], SWATTN_BF16, 1, n, self.vocab, inputs["drafts"], outputs["tgt"],
                             outputs["acc"], outputs["nxt"], self.ws_acc, self.ws_acc.numel() * 8, stream)

    def capture(self, inputs, outputs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.issue(inputs, outputs, torch.cuda.current_stream(self.k.device).cuda_stream)
        return g
