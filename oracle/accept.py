"""Greedy speculative-verify acceptance (test infrastructure only; see the package
docstring for who may use it).

What it computes.  Generation is greedy ("The Fast Gemma Challenge: our
verified-SOTA recipe, in full", manifest OVERRIDE_GENERATION_CONFIG: temperature
0, top_p 1, top_k 0), so the target model's token after each input is the argmax
of its logits, and a verify step of n_q inputs [x0, d1, ..., d(n_q-1)] (the last
accepted token and the drafter's guesses, manifest SPECULATIVE_CONFIG) keeps the
drafts up to the first one the target disagrees with; the argmax is fused into
this step rather than sampled (manifest FUSED_SPARSE_ARGMAX).

For sequence b with logits L[b][i][v] (i < n_q, v < vocab) and drafts
draft[b][j] (j < n_q - 1, draft[b][j] is the guess for the token after input j):

    target[b][i] = argmax_v L[b][i][v]        (lowest index among equal maxima; a NaN
                                               counts as larger than every number, so
                                               the first NaN wins; -0 equals +0)
    accepted[b]  = the largest a <= n_q - 1 with draft[b][j] == target[b][j] for all j < a
    next[b]      = target[b][accepted[b]]     (the token the target adds after the
                                               accepted drafts)

Pinned in tests/test_accept_oracle.py: hand-built acceptance patterns (all, none,
a mismatch in the middle, n_q = 1), ties, NaN and signed-zero rows, and the argmax
against an independent definition by stable sorting, on random inputs.
"""
import numpy as np


def row_argmax(logits):
    """[..., vocab] float array -> int64 [...] argmax with the rules above."""
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=-1)          # numpy: first maximal index, a NaN is maximal, -0 == +0


def greedy_accept(logits, draft_ids):
    """logits [B][n_q][vocab] (float), draft_ids [B][n_q - 1] (int) ->
    (target [B][n_q] int64, accepted [B] int64, next_token [B] int64)."""
    logits = np.asarray(logits)
    B, n_q, _ = logits.shape
    draft_ids = np.asarray(draft_ids).reshape(B, max(n_q - 1, 0))
    target = row_argmax(logits)
    accepted = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = 0
        while a < n_q - 1 and int(draft_ids[b, a]) == int(target[b, a]):
            a += 1
        accepted[b] = a
        nxt[b] = target[b, a]
    return target.astype(np.int64), accepted, nxt
