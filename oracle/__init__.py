"""Float64 CPU oracle for sliding-window verify attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library under
``speculative_verify_kv_amd/`` and its Python binding) imports, links or calls
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant with the GPU path.

What it computes follows "The Fast Gemma Challenge: our verified-SOTA recipe,
in full" (dev.to, VIDRAFT): the manifest's ``SLIDING_WINDOW=188`` /
``FA_SLIDING=1`` and the "What each piece does, and why" section (attention is
restricted to the most recent W tokens because decode is bound by KV-cache
bandwidth), the manifest's ``SPECULATIVE_CONFIG`` (MTP with 7 draft tokens, so a
verify step scores 1 + 7 positions) and ``SPLITKV_VERIFY_MAX_Q=64`` (at most 64
verify queries), and ``MAX_MODEL_LEN=4096``.

Pins (tests/test_oracle*.py, CPU): brute force over an explicitly built dense
mask, torch's float64 scaled_dot_product_attention for the full-causal case,
window = 1 returning the query's own V row bit for bit, softmax-weight
normalisation, block-table permutation invariance, GQA == MHA on repeated K/V,
closed forms (K = 0 gives a moving average, two-key sigmoid, constant V),
hand-derived fixtures under tests/golden/, and every e4m3 / bf16 code against
torch's own conversions; for the KV append (kv_append.py), E4M3 and bfloat16
rounding against torch's casts and hand-derived cases, and the write pattern
against a dense per-position reference; for the greedy acceptance (accept.py),
hand-built acceptance patterns and the argmax against a sorting definition.
No function here is "parity unpinned".
"""
from .formats import decode_e4m3, decode_bf16, e4m3_value_table
from .attend import attend, attend_bruteforce, window_bounds
from .splitmerge import attend_split_merge
from .kv_append import append_kv, quantize_e4m3, f32_to_bf16_rne
from .accept import greedy_accept, row_argmax

__all__ = [
    "decode_e4m3",
    "decode_bf16",
    "e4m3_value_table",
    "attend",
    "attend_bruteforce",
    "window_bounds",
    "attend_split_merge",
    "append_kv",
    "quantize_e4m3",
    "f32_to_bf16_rne",
    "greedy_accept",
    "row_argmax",
]
