"""Pins of the oracle's nearest-neighbour search (CPU): the top-k against a
brute-force selection written as plain loops (ties by key index), and the
recall@1@k bookkeeping against hand-made lists."""
import numpy as np
import pytest

from oracle import tq_oracle as O


def _keys(cd, x):
    r = O.quantize_prod(cd, x)
    return dict(idx=r["idx"], signs=r["signs"], norms=r["norms"], rnorms=r["rnorms"])


@pytest.mark.parametrize("k", [1, 5, 12])
def test_topk_equals_a_loop_selection_with_index_tie_break(k):
    d, n = 24, 40
    rng = np.random.default_rng(k)
    x = rng.standard_normal((n, d))
    x[7] = x[3]   # exact duplicates: equal scores, ordered by index
    x[30] = x[3]
    cd = O.make_codec(d, 3, O.PROD, 2)
    keys = _keys(cd, x)
    q = rng.standard_normal((4, d))
    sc, idx = O.topk_plain(cd, q, keys, k)
    full = O.logits_plain(cd, q, keys)
    for i in range(q.shape[0]):
        items = [(full[i, t], t) for t in range(n)]
        chosen = []
        for _ in range(k):  # repeatedly take the best remaining
            best = None
            for s_, t in items:
                if t in chosen:
                    continue
                if best is None or s_ > best[0] or (s_ == best[0] and t < best[1]):
                    best = (s_, t)
            chosen.append(best[1])
        assert list(idx[i]) == chosen
        assert np.array_equal(sc[i], full[i, chosen])
    # the duplicates of key 3 come out in index order wherever they rank
    for i in range(q.shape[0]):
        pos = [list(idx[i]).index(t) for t in (3, 7, 30) if t in idx[i]]
        assert pos == sorted(pos)


def test_recall_bookkeeping():
    top1 = np.array([4, 9, 2, 7])
    lists = np.array([[4, 1, 2], [0, 9, 3], [5, 6, 8], [7, 7, 7]])
    r = O.recall_at(top1, lists, [1, 2, 3])
    assert r == {1: 0.5, 2: 0.75, 3: 0.75}


def test_recall_is_monotone_and_complete():
    d, n = 32, 200
    rng = np.random.default_rng(1)
    x = rng.standard_normal((n, d))
    q = rng.standard_normal((30, d))
    cd = O.make_codec(d, 2, O.PROD, 5)
    _, idx = O.topk_plain(cd, q, _keys(cd, x), n)
    true = np.argmax(q @ x.T, axis=1)
    r = O.recall_at(true, idx, range(1, n + 1))
    vals = [r[k] for k in range(1, n + 1)]
    assert all(a <= b for a, b in zip(vals, vals[1:]))
    assert vals[-1] == 1.0


def test_high_resolution_codes_recover_the_exact_top1():
    """With 8-bit mse codes the estimate is within ~1e-3 of the inner
    product, so well-separated exact top-1s are recovered at k = 1."""
    d, n = 64, 300
    rng = np.random.default_rng(2)
    x = rng.standard_normal((n, d))
    q = x[rng.choice(n, 25, replace=False)] + 0.05 * rng.standard_normal((25, d))
    cd = O.make_codec(d, 8, O.MSE, 3)
    idx8, nu, _ = O.quantize_mse(cd, x)
    _, top = O.topk_plain(cd, q, dict(idx=idx8, norms=nu), 1)
    true = np.argmax(q @ x.T, axis=1)
    assert O.recall_at(true, top, [1])[1] == 1.0
