"""GPU parity of swattn_greedy_accept (through the C ABI) against oracle.accept.

Integer outputs, compared exactly: the argmax ids of every position, the number
of accepted drafts and the next token, on random logits with planted ties, NaNs,
signed zeros and infinities, float32 and bfloat16, vocab sizes on both sides of
the 16-byte load path and of the argmax chunk size.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_kv_amd as sw
import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()


def make_case(B, n_q, vocab, seed, bf16, specials=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, n_q, vocab)).astype(np.float32)
    x[:, :, rng.integers(0, vocab, 3)] = np.round(x[:, :, rng.integers(0, vocab, 3)], 0)
    if vocab >= 4:
        # a planted tie for the maximum in every other row
        for b in range(B):
            for i in range(0, n_q, 2):
                j1, j2 = sorted(rng.choice(vocab, 2, replace=False))
                x[b, i, j1] = x[b, i, j2] = x[b, i].max() + 1.0
    if specials and vocab >= 8:
        x[0, 0, :] = -0.0
        x[0, 0, 5] = 0.0                      # -0 == +0: index 0 wins
        if n_q > 1:
            x[0, 1, 3] = np.nan
            x[0, 1, 6] = np.nan               # first NaN wins
        if n_q > 2:
            x[0, 2, :] = -np.inf              # all equal: index 0
        if n_q > 3:
            x[0, 3, 7] = np.inf
        if n_q > 7:
            # inf and -inf without a NaN (their sum is NaN: the scan's NaN probe fires and
            # finds none): the first +inf wins
            x[0, 4, 2] = -np.inf
            x[0, 4, 4] = np.inf
            x[0, 4, vocab - 1] = np.inf
            # a single NaN in an otherwise -inf row, at the last index
            x[0, 5, :] = -np.inf
            x[0, 5, vocab - 1] = np.nan
            # the largest value a positive denormal, the larger of two coming later
            x[0, 6, :] = -1.0
            x[0, 6, 1] = 1e-40
            x[0, 6, min(vocab - 1, 5000)] = 2e-40
            # an early +inf, then a NaN far later (another thread, for long rows): NaN wins
            x[0, 7, 0] = np.inf
            x[0, 7, min(vocab - 1, 4099)] = np.nan
    if bf16:
        bits = oracle.f32_to_bf16_rne(x)
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        dev = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        vals = x
        dev = torch.from_numpy(x).to(DEV)
    target = oracle.row_argmax(vals)
    drafts = target[:, :n_q - 1].copy().astype(np.int32)
    cut = rng.integers(0, n_q, B)
    for b in range(B):
        if cut[b] < n_q - 1:
            drafts[b, cut[b]] = (drafts[b, cut[b]] + 1) % max(vocab, 2)
            if vocab == 1:
                drafts[b, cut[b]] = 1                          # an id the 1-entry vocab cannot produce
    return vals, dev, drafts


def check(vals, dev, drafts):
    B, n_q, vocab = vals.shape
    d = torch.from_numpy(np.ascontiguousarray(drafts)).to(DEV) if n_q > 1 else None
    t, a, nx = sw.greedy_accept(dev, d)
    torch.cuda.synchronize()
    et, ea, en = oracle.greedy_accept(vals, drafts)
    assert np.array_equal(t.cpu().numpy(), et), "target ids differ"
    assert np.array_equal(a.cpu().numpy(), ea), "accepted counts differ"
    assert np.array_equal(nx.cpu().numpy(), en), "next tokens differ"


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("vocab", [1, 7, 8, 1000, 8192, 8193, 50001, 262144])
def test_accept_matches_oracle(vocab, bf16):
    gu.log(f"[accept] vocab {vocab} bf16 {bf16}")
    vals, dev, drafts = make_case(5, 8, vocab, seed=vocab, bf16=bf16, specials=True)
    check(vals, dev, drafts)


@pytest.mark.parametrize("n_q", [1, 2, 64])
def test_accept_positions(n_q):
    vals, dev, drafts = make_case(3, n_q, 3000, seed=n_q, bf16=True)
    check(vals, dev, drafts)


def test_accept_unaligned_rows_and_many_sequences():
    # an odd vocab makes every row start unaligned: the element-wise load path
    vals, dev, drafts = make_case(64, 8, 2049, seed=9, bf16=False, specials=True)
    check(vals, dev, drafts)


def test_accept_host_errors():
    x = torch.zeros((1, 8, 16), dtype=torch.float32, device=DEV)
    o = torch.zeros(64, dtype=torch.int32, device=DEV)
    ws = torch.zeros(64, dtype=torch.int64, device=DEV)
    st = sw.swattn_greedy_accept(x, sw.SWATTN_F32, 1, 65, 16, o, o, o, o, ws, 512, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_NQ"
    st = sw.swattn_greedy_accept(x, sw.SWATTN_FP8_E4M3, 1, 8, 16, o, o, o, o, ws, 512, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_DTYPE"
    st = sw.swattn_greedy_accept(x, sw.SWATTN_F32, 1, 8, 16, o, o, o, o, ws, 4, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_WORKSPACE"
    st = sw.swattn_greedy_accept(x, sw.SWATTN_F32, 1, 8, 16, None, o, o, o, ws, 512, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_NULL"
