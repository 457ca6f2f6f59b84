"""CPU pins of oracle.accept: greedy acceptance and the argmax rules."""
import numpy as np

from oracle import accept as ac


def argmax_by_sorting(x):
    """Independent definition: sort (value descending, index ascending), take the
    first; NaN ranks above every number."""
    out = []
    for row in np.asarray(x, dtype=np.float64).reshape(-1, x.shape[-1]):
        nan = np.isnan(row)
        if nan.any():
            out.append(int(np.flatnonzero(nan)[0]))
            continue
        key = np.where(row == 0.0, 0.0, row)                    # -0 ranks with +0
        order = np.lexsort((np.arange(len(row)), -key))         # last key is primary
        out.append(int(order[0]))
    return np.array(out).reshape(x.shape[:-1])


def test_argmax_matches_sorting_definition():
    rng = np.random.default_rng(0)
    for vocab in (1, 2, 7, 64, 1000):
        x = rng.standard_normal((3, 5, vocab))
        x[..., ::3] = np.round(x[..., ::3], 1)                  # plenty of ties
        assert np.array_equal(ac.row_argmax(x), argmax_by_sorting(x))
        xi = rng.integers(-3, 4, (4, 6, vocab)).astype(np.float64)   # integer values: many equal maxima
        assert np.array_equal(ac.row_argmax(xi), argmax_by_sorting(xi))


def test_ties_nan_and_signed_zero():
    x = np.array([[[1.0, 3.0, 3.0, -1.0],            # tie -> lowest index 1
                   [-0.0, 0.0, -1.0, -2.0],          # -0 == +0 -> index 0
                   [1.0, np.nan, 5.0, np.nan],       # first NaN -> 1
                   [-np.inf, -np.inf, -np.inf, -np.inf]]])   # all equal -> 0
    assert list(ac.row_argmax(x)[0]) == [1, 0, 1, 0]


def test_acceptance_patterns():
    vocab, n_q = 10, 8
    target = np.array([[3, 1, 4, 1, 5, 9, 2, 6],
                       [3, 1, 4, 1, 5, 9, 2, 6],
                       [3, 1, 4, 1, 5, 9, 2, 6],
                       [7, 7, 7, 7, 7, 7, 7, 7]])
    logits = np.full((4, n_q, vocab), -1.0)
    for b in range(4):
        for i in range(n_q):
            logits[b, i, target[b, i]] = 2.0
    drafts = np.array([[3, 1, 4, 1, 5, 9, 2],          # every draft matches -> 7 accepted, bonus 6
                       [3, 1, 4, 0, 5, 9, 2],          # mismatch at j = 3 -> 3 accepted, bonus target[3] = 1
                       [0, 1, 4, 1, 5, 9, 2],          # first draft wrong -> 0 accepted, bonus 3
                       [7, 7, 7, 7, 7, 7, 8]])         # last draft wrong -> 6 accepted, bonus 7
    t, a, nxt = ac.greedy_accept(logits, drafts)
    assert np.array_equal(t, target)
    assert list(a) == [7, 3, 0, 6]
    assert list(nxt) == [6, 1, 3, 7]
    # later matches after a mismatch do not count
    assert a[1] == 3 and drafts[1, 4] == target[1, 4]


def test_single_position():
    logits = np.array([[[0.5, 2.5, 1.0]]])
    t, a, nxt = ac.greedy_accept(logits, np.zeros((1, 0), np.int64))
    assert t[0, 0] == 1 and a[0] == 0 and nxt[0] == 1


def test_random_against_direct_rule():
    rng = np.random.default_rng(1)
    B, n_q, vocab = 50, 8, 300
    logits = rng.standard_normal((B, n_q, vocab)).astype(np.float32)
    target = argmax_by_sorting(logits)
    drafts = target[:, :n_q - 1].copy()
    cut = rng.integers(0, n_q, B)                            # first wrong draft (n_q - 1: none)
    for b in range(B):
        if cut[b] < n_q - 1:
            drafts[b, cut[b]] = (drafts[b, cut[b]] + 1 + rng.integers(0, vocab - 1)) % vocab
    t, a, nxt = ac.greedy_accept(logits, drafts)
    assert np.array_equal(t, target)
    assert np.array_equal(a, np.minimum(cut, n_q - 1))
    assert np.array_equal(nxt, target[np.arange(B), a])
