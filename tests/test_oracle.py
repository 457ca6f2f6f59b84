"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: an independent dense
mask construction, torch's scaled_dot_product_attention, closed forms, exact
invariances and hand-derived fixtures.  ``test_pins_catch_planted_mistakes``
plants plausible bugs in a copy of the oracle and checks that a pin fails.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attend, attend_bruteforce, attend_split_merge, window_bounds
import importlib

oracle_attend = importlib.import_module("oracle.attend")


def paged_inputs(rng, B, H, Hkv, D, n_q, ctx, bs, shuffle=True, extra_blocks=0):
    """Random float64 q and a random paged cache; every stored value is finite
    random data, including positions outside any window."""
    ctx = np.broadcast_to(np.asarray(ctx), (B,)).astype(np.int64)
    nblk = [(int(c) + bs - 1) // bs for c in ctx]
    maxb = max(nblk)
    pool = sum(nblk) + extra_blocks
    perm = rng.permutation(pool) if shuffle else np.arange(pool)
    table = np.zeros((B, maxb), dtype=np.int64)
    s = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[s:s + nblk[b]]
        s += nblk[b]
    q = rng.standard_normal((B, n_q, H, D))
    k = rng.standard_normal((pool, Hkv, bs, D))
    v = rng.standard_normal((pool, Hkv, bs, D))
    return q, k, v, table, ctx


def logical(cache, table, ctx, bs):
    """Contiguous [B][ctx][Hkv][D] view of a paged cache (independent gather)."""
    out = []
    for b, c in enumerate(ctx):
        rows = [cache[table[b][pos // bs], :, pos % bs, :] for pos in range(int(c))]
        out.append(np.stack(rows))
    return out


# --------------------------------------------------------------------------
# brute force over an explicitly built dense mask
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n_q,window,bs", list(itertools.product(
    [1, 2, 5, 8], [1, 2, 3, 7, 16, 40], [1, 3, 16, 40])))
def test_matches_bruteforce(n_q, window, bs):
    rng = np.random.default_rng(1000 * n_q + 10 * window + bs)
    B, H, Hkv, D = 2, 4, 2, 8
    ctx = [max(n_q, 23), 40]
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, ctx, bs)
    scale = 0.37
    a = attend(q, k, v, table, ctx, n_q, window, scale)
    b = attend_bruteforce(q, k, v, table, ctx, n_q, window, scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# window >= context: full bottom-right causal attention (library routine)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n_q,ctx,G", [(1, 30, 1), (8, 30, 4), (8, 8, 2), (5, 64, 8)])
def test_full_window_equals_sdpa(n_q, ctx, G):
    rng = np.random.default_rng(7 + n_q + ctx + G)
    B, Hkv, D, bs = 2, 2, 16, 16
    H = Hkv * G
    q, k, v, table, ctxs = paged_inputs(rng, B, H, Hkv, D, n_q, ctx, bs)
    scale = 1.0 / np.sqrt(D)
    ours = attend(q, k, v, table, ctxs, n_q, window=ctx + 5, scale=scale)
    K, V = logical(k, table, ctxs, bs), logical(v, table, ctxs, bs)
    for b in range(B):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)                      # [H, n_q, D]
        kt = torch.from_numpy(K[b]).permute(1, 0, 2).repeat_interleave(G, 0)  # [H, ctx, D]
        vt = torch.from_numpy(V[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        mask = torch.ones(n_q, ctx, dtype=torch.bool).tril(diagonal=ctx - n_q)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(ours[b], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# window = 1: the query's own V row, bit for bit
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [1, 16, 300])
def test_window_one_is_own_value_row(bs):
    rng = np.random.default_rng(bs)
    B, H, Hkv, D, n_q = 3, 8, 2, 32, 8
    ctx = [8, 45, 300]
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, ctx, bs)
    out = attend(q, k, v, table, ctx, n_q, window=1, scale=0.5)
    for b in range(B):
        for i in range(n_q):
            pos = int(ctx[b]) - n_q + i
            for h in range(H):
                g = h // (H // Hkv)
                row = v[table[b][pos // bs], g, pos % bs, :]
                assert np.array_equal(out[b, i, h], row)


# --------------------------------------------------------------------------
# normalisation and the zero pattern of the weights
# --------------------------------------------------------------------------
def test_weights_normalised_and_zero_outside_window():
    rng = np.random.default_rng(3)
    B, H, Hkv, D, n_q, window, bs = 2, 4, 1, 16, 8, 11, 4
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [30, 19], bs)
    out, w = attend(q, k, v, table, ctx, n_q, window, 0.3, return_weights=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    for b in range(B):
        p = int(ctx[b]) - n_q
        for i in range(n_q):
            t = p + i
            inside = np.zeros(w.shape[-1], dtype=bool)
            inside[max(0, t - window + 1):t + 1] = True
            assert (w[b, i][:, ~inside] == 0.0).all()
            assert (w[b, i][:, inside] > 0.0).all()
    # the weights reproduce the output
    K = logical(k, table, ctx, bs)
    V = logical(v, table, ctx, bs)
    for b in range(B):
        c = int(ctx[b])
        for h in range(H):
            ref = w[b, :, h, :c] @ V[b][:, h // (H // Hkv), :]
            np.testing.assert_allclose(out[b, :, h], ref, rtol=0, atol=1e-13)


def test_window_bounds_reading():
    lo, hi = window_bounds([10, 300], n_q=3, window=4)
    assert lo.tolist() == [[4, 5, 6], [294, 295, 296]]
    assert hi.tolist() == [[7, 8, 9], [297, 298, 299]]
    lo, hi = window_bounds([3], n_q=3, window=188)
    assert lo.tolist() == [[0, 0, 0]] and hi.tolist() == [[0, 1, 2]]


# --------------------------------------------------------------------------
# paging: any block-table permutation gives the contiguous result bit for bit
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [1, 16, 300])
def test_paged_equals_contiguous(bs):
    rng = np.random.default_rng(11 + bs)
    B, H, Hkv, D, n_q, window = 2, 4, 2, 16, 8, 37
    ctx = np.array([300, 123])
    q = rng.standard_normal((B, n_q, H, D))
    kc = rng.standard_normal((B, 300, Hkv, D))                # contiguous logical data
    vc = rng.standard_normal((B, 300, Hkv, D))
    # contiguous layout: one block per sequence, block size = 300
    k_cont = kc.transpose(0, 2, 1, 3).copy()                  # [B, Hkv, 300, D]
    v_cont = vc.transpose(0, 2, 1, 3).copy()
    ref = attend(q, k_cont, v_cont, np.arange(B)[:, None], ctx, n_q, window, 0.25)
    nblk = (300 + bs - 1) // bs
    pool = B * nblk
    for trial in range(3):
        perm = rng.permutation(pool)
        table = perm.reshape(B, nblk)
        kp = np.full((pool, Hkv, bs, D), np.nan)
        vp = np.full((pool, Hkv, bs, D), np.nan)
        for b in range(B):
            for pos in range(300):
                kp[table[b, pos // bs], :, pos % bs] = kc[b, pos]
                vp[table[b, pos // bs], :, pos % bs] = vc[b, pos]
        got = attend(q, kp, vp, table, ctx, n_q, window, 0.25)
        assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# GQA == MHA on repeated K/V
# --------------------------------------------------------------------------
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_equals_mha_on_repeated_kv(G):
    rng = np.random.default_rng(G)
    B, Hkv, D, n_q, window, bs = 2, 2, 16, 8, 20, 16
    H = Hkv * G
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [64, 41], bs)
    gqa = attend(q, k, v, table, ctx, n_q, window, 0.2)
    k_mha = np.repeat(k, G, axis=1)          # head h of the expanded cache = kv head h // G
    v_mha = np.repeat(v, G, axis=1)
    mha = attend(q, k_mha, v_mha, table, ctx, n_q, window, 0.2)
    assert np.array_equal(gqa, mha)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def test_zero_keys_give_moving_average():
    rng = np.random.default_rng(5)
    B, H, Hkv, D, n_q, window, bs = 2, 4, 2, 8, 8, 13, 16
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [50, 20], bs)
    k[:] = 0.0
    out = attend(q, k, v, table, ctx, n_q, window, 1.7)
    V = logical(v, table, ctx, bs)
    for b in range(B):
        c = int(ctx[b])
        csum = np.concatenate([np.zeros((1, Hkv, D)), np.cumsum(V[b], axis=0)])
        for i in range(n_q):
            t = c - n_q + i
            lo = max(0, t - window + 1)
            mean = (csum[t + 1] - csum[lo]) / (t + 1 - lo)
            for h in range(H):
                np.testing.assert_allclose(out[b, i, h], mean[h // (H // Hkv)], rtol=0, atol=1e-12)


def test_constant_values_give_that_value():
    rng = np.random.default_rng(6)
    B, H, Hkv, D, n_q, window, bs = 2, 4, 2, 8, 8, 9, 4
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [50, 20], bs)
    vec = rng.standard_normal((Hkv, D))
    v[:] = vec[None, :, None, :]
    out = attend(q, k, v, table, ctx, n_q, window, 3.0)
    for h in range(H):
        np.testing.assert_allclose(out[:, :, h], np.broadcast_to(vec[h // 2], out[:, :, h].shape),
                                   rtol=1e-14, atol=1e-14)


def test_two_keys_sigmoid():
    rng = np.random.default_rng(8)
    D = 16
    for _ in range(20):
        q = rng.standard_normal((1, 1, 1, D)) * 3
        k = rng.standard_normal((1, 1, 2, D))
        v = rng.standard_normal((1, 1, 2, D))
        scale = rng.uniform(0.1, 2.0)
        out = attend(q, k, v, np.zeros((1, 1), np.int64), [2], 1, 2, scale)
        s0 = scale * np.dot(q[0, 0, 0], k[0, 0, 0])
        s1 = scale * np.dot(q[0, 0, 0], k[0, 0, 1])
        sig = lambda x: 1.0 / (1.0 + np.exp(-x))
        ref = sig(s0 - s1) * v[0, 0, 0] + sig(s1 - s0) * v[0, 0, 1]
        np.testing.assert_allclose(out[0, 0, 0], ref, rtol=0, atol=1e-13)


def test_golden_two_key_fixture(golden_dir):
    with open(os.path.join(golden_dir, "two_key_closed_form.json")) as f:
        g = json.load(f)
    k = np.array(g["k"])[None, None]             # [1 block, 1 head, 2 positions, D]
    v = np.array(g["v"])[None, None]
    for case in g["cases"]:
        n_q = case["n_q"]
        q = np.broadcast_to(np.array(g["q"]), (1, n_q, 1, 2))
        out = attend(q, k, v, np.zeros((1, 1), np.int64), [2], n_q, case["window"], g["scale"])
        np.testing.assert_allclose(out[0, :, 0, :], np.array(case["expected"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# e4m3 storage: decode-then-scale equals attention on the decoded values
# --------------------------------------------------------------------------
def test_e4m3_storage_equals_decoded_values():
    rng = np.random.default_rng(9)
    B, H, Hkv, D, n_q, window, bs = 2, 4, 2, 16, 8, 21, 16
    q, _, _, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [64, 40], bs)
    pool = int(table.max()) + 1
    kc = rng.integers(0, 256, size=(pool, Hkv, bs, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(pool, Hkv, bs, D)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C              # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x41
    ks = np.array([0.01, 0.03])
    vs = np.array([0.2, 0.05])
    got = attend(q, kc, vc, table, ctx, n_q, window, 0.125, kv_format="e4m3", k_scale=ks, v_scale=vs)
    kt = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * ks[None, :, None, None]
    vt = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * vs[None, :, None, None]
    ref = attend(q, kt, vt, table, ctx, n_q, window, 0.125)
    assert np.array_equal(got, ref)


def test_bf16_q_storage_equals_decoded_values():
    rng = np.random.default_rng(10)
    B, H, Hkv, D, n_q, window, bs = 1, 2, 1, 8, 3, 5, 4
    _, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [12], bs)
    qf = torch.randn(B, n_q, H, D, dtype=torch.float32, generator=torch.Generator().manual_seed(0))
    qb = qf.to(torch.bfloat16)
    bits = qb.view(torch.int16).numpy().view(np.uint16)
    got = attend(bits, k, v, table, ctx, n_q, window, 0.5, q_format="bf16")
    ref = attend(qb.to(torch.float64).numpy(), k, v, table, ctx, n_q, window, 0.5)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# split-KV + log-sum-exp merge identity
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 5, 13])
def test_split_merge_identity(S):
    rng = np.random.default_rng(20 + S)
    B, H, Hkv, D, n_q, window, bs = 2, 4, 2, 16, 8, 30, 16
    q, k, v, table, ctx = paged_inputs(rng, B, H, Hkv, D, n_q, [90, 37], bs)
    q = q * 4.0                                   # sharp softmax stresses the merge
    ref = attend(q, k, v, table, ctx, n_q, window, 0.5)
    got = attend_split_merge(q, k, v, table, ctx, n_q, window, 0.5, num_splits=S)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# the pins above catch plausible mistakes (planted in the oracle, on the CPU)
# --------------------------------------------------------------------------
def _planted_window_off_by_one(ctx_len, n_q, window):
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    t = (ctx_len - n_q)[:, None] + np.arange(n_q)[None, :]
    return np.maximum(0, t - window), t                  # keeps one key too many


def _planted_shared_window(ctx_len, n_q, window):
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    t = (ctx_len - n_q)[:, None] + np.arange(n_q)[None, :]
    lo = np.maximum(0, t[:, :1] - window + 1)            # every draft uses the target's window start
    return np.broadcast_to(lo, t.shape), t


def _planted_no_causal(ctx_len, n_q, window):
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    t = (ctx_len - n_q)[:, None] + np.arange(n_q)[None, :]
    return np.maximum(0, t - window + 1), np.broadcast_to(t[:, -1:], t.shape)


@pytest.mark.parametrize("planted", [_planted_window_off_by_one, _planted_shared_window,
                                     _planted_no_causal])
def test_pins_catch_planted_mistakes(monkeypatch, planted):
    monkeypatch.setattr(oracle_attend, "window_bounds", planted)
    rng = np.random.default_rng(99)
    q, k, v, table, ctx = paged_inputs(rng, 1, 2, 1, 8, 4, [20], 4)
    a = oracle_attend.attend(q, k, v, table, ctx, 4, 5, 0.5)
    b = attend_bruteforce(q, k, v, table, ctx, 4, 5, 0.5)
    assert not np.allclose(a, b, atol=1e-6)


def test_pin_catches_transposed_gqa_mapping(monkeypatch):
    # A plausible mistake: kv head h % Hkv instead of h // (H // Hkv).
    rng = np.random.default_rng(5)
    H, Hkv, G = 4, 2, 2
    q, k, v, table, ctx = paged_inputs(rng, 1, H, Hkv, 8, 2, [16], 16)
    k_mha = np.repeat(k, G, axis=1)
    v_mha = np.repeat(v, G, axis=1)
    ref = attend(q, k_mha, v_mha, table, ctx, 2, 6, 0.3)
    wrong_k = k[:, [h % Hkv for h in range(H)]]
    wrong_v = v[:, [h % Hkv for h in range(H)]]
    bad = attend(q, wrong_k, wrong_v, table, ctx, 2, 6, 0.3)
    assert not np.allclose(bad, ref)
    assert np.array_equal(attend(q, k, v, table, ctx, 2, 6, 0.3), ref)
