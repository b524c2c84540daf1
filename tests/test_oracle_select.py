"""Pins of the oracle's budget and selector (CPU only)."""

import itertools

import numpy as np
import pytest

import oracle
from s3r_inputs.configs import SWEEP_S


def test_tiny_config_budget():
    # 5% of 512 positions with a 16-position newest window: 26 positions, 16 of them newest.
    assert oracle.budget(512, 1, 20, 16) == 26
    idx = oracle.select(np.random.default_rng(0).random(512).astype(np.float32), 512, 1, 20, 16)
    assert len(idx) == 26
    assert list(idx[-16:]) == list(range(496, 512))


@pytest.mark.parametrize("s", list(SWEEP_S) + [(1, 1), (0, 1), (3, 7)])
def test_budget_is_exact_ceiling(s):
    s_num, s_den = s
    W = 64
    L = np.arange(0, 40001, dtype=np.int64)
    n = np.array([oracle.budget(int(x), s_num, s_den, W) for x in L])
    frac_ok = (n * s_den >= s_num * L)  # n >= s*L exactly
    assert frac_ok.all()
    floor = np.minimum(W, L)
    tight = (n == floor) | ((n - 1) * s_den < s_num * L)  # n-1 < s*L unless the window sets n
    assert tight.all()
    assert (n <= L).all()
    assert (np.diff(n) >= 0).all() and (np.diff(n) <= 1).all()


def test_float_fraction_would_be_off():
    # Why the budget is an integer ratio: 0.05 held as float32 and widened gives ceil(0.05*20) = 2.
    assert int(np.ceil(np.float64(np.float32(0.05)) * 20)) == 2
    assert oracle.budget(20, 1, 20, 0) == 1


def _dominance_ok(scores, L, s_num, s_den, W):
    idx = oracle.select(scores, L, s_num, s_den, W)
    n = oracle.budget(L, s_num, s_den, W)
    newest = min(W, L)
    assert len(idx) == n
    assert (np.diff(idx) > 0).all()
    assert set(range(L - newest, L)) <= set(idx.tolist())
    kept = [j for j in idx.tolist() if j < L - newest]
    dropped = [j for j in range(L - newest) if j not in set(kept)]

    def before(a, b):  # a ranks before b
        sa, sb = float(scores[a]), float(scores[b])
        return sa > sb or (sa == sb and a < b)

    return all(before(a, b) for a in kept for b in dropped)


def test_select_dominance_bruteforce():
    rng = np.random.default_rng(1)
    pool = np.array([0.0, -0.0, 0.25, 0.25, 1.0, np.inf, 3.5, 1e-30], dtype=np.float32)
    for trial in range(300):
        L = int(rng.integers(1, 40))
        W = int(rng.integers(0, 8))
        s_num, s_den = [(1, 2), (1, 3), (2, 5), (1, 20), (1, 1)][trial % 5]
        if trial % 2:
            sc = pool[rng.integers(0, len(pool), size=L)]
        else:
            sc = rng.random(L).astype(np.float32)
        assert _dominance_ok(sc, L, s_num, s_den, W)


def test_select_matches_lexsort():
    rng = np.random.default_rng(2)
    for trial in range(50):
        L = int(rng.integers(100, 3000))
        sc = rng.integers(0, 20, size=L).astype(np.float32) / 4  # many ties
        W = 64
        n = oracle.budget(L, 1, 20, W)
        newest = min(W, L)
        cand = np.arange(L - newest)
        order = np.lexsort((cand, -sc[:L - newest].astype(np.float64)))
        ref = np.sort(np.concatenate([order[:n - newest], np.arange(L - newest, L)]))
        assert np.array_equal(oracle.select(sc, L, 1, 20, W), ref)


def test_select_hand_cases():
    # ties go to the lower position
    sc = np.array([0.5, 0.9, 0.9, 0.1, 0.0, 0.0], dtype=np.float32)
    assert oracle.select(sc, 6, 1, 2, 2).tolist() == [1, 4, 5]
    # -0.0 equals +0.0: the lower position wins
    sc = np.array([0.0, -0.0, -0.0, 0.0, 0.0], dtype=np.float32)
    sc[0] = -0.0
    sc[1] = 0.0
    assert oracle.select(sc, 5, 2, 5, 1).tolist() == [0, 4]
    # +inf ranks highest
    sc = np.array([1.0, np.inf, 2.0, 0.0], dtype=np.float32)
    assert oracle.select(sc, 4, 1, 2, 1).tolist() == [1, 3]
    # s = 1 keeps everything
    assert oracle.select(np.zeros(7, np.float32), 7, 1, 1, 2).tolist() == list(range(7))
    # L below the window keeps everything
    assert oracle.select(np.zeros(3, np.float32), 3, 1, 20, 16).tolist() == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.select(np.array([np.nan, 1, 2, 3], np.float32), 4, 1, 2, 0)


def test_select_invariant_below_threshold():
    # changing scores of dropped candidates without crossing the threshold keeps the set
    rng = np.random.default_rng(3)
    sc = rng.random(500).astype(np.float32)
    idx = oracle.select(sc, 500, 1, 10, 16)
    kept_old = [j for j in idx.tolist() if j < 484]
    thr = sc[kept_old].min()
    sc2 = sc.copy()
    drop = np.array([j for j in range(484) if j not in set(kept_old)])
    sc2[drop] = sc[drop] * np.float32(0.5)
    assert np.array_equal(oracle.select(sc2, 500, 1, 10, 16), idx)
    assert (sc2[drop] < thr).all()


def test_pairs_exhaustive_small():
    # every score pattern over a 3-value alphabet on L=6: dominance holds
    for pat in itertools.product([0.0, 0.5, 1.0], repeat=6):
        sc = np.array(pat, dtype=np.float32)
        for W in (0, 1, 3):
            assert _dominance_ok(sc, 6, 1, 2, W)
