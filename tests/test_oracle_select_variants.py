"""Pins of the selection variants: whole pages, and one kept set per sequence
from all KV heads (CPU only)."""

import numpy as np
import pytest

import oracle
from oracle import select_variants as SV


def _int_scores(rng, Hkv, L, hi=50):
    # integer values: every float32 sum below 2^24 is exact
    return rng.integers(0, hi, size=(Hkv, L)).astype(np.float32)


def _brute_pages(key_int, L, s_num, s_den, window, unit=16):
    """Full pages older than the window ranked by exact int64 sums with Python's sort."""
    w = min(window, L)
    first = (L - w) // unit  # page holding the oldest window position
    window_pos = list(range(first * unit, L))
    n = oracle.budget(L, s_num, s_den, window)
    need = max(0, n - len(window_pos))
    n_top = min(first, (need + unit - 1) // unit)
    sums = [int(sum(int(key_int[j]) for j in range(p * unit, (p + 1) * unit))) for p in range(first)]
    kept = sorted(sorted(range(first), key=lambda p: (-sums[p], p))[:n_top])
    return [j for p in kept for j in range(p * unit, (p + 1) * unit)] + window_pos


def test_one_head_positions_is_plain_selection():
    rng = np.random.default_rng(0)
    sc = rng.random((1, 900)).astype(np.float32)
    for L in (1, 17, 64, 500, 900):
        got = oracle.select_grouped(sc, L, 1, 20, 64, 1, False)[0]
        assert np.array_equal(got, oracle.select(sc[0], L, 1, 20, 64))
        got = oracle.select_grouped(sc, L, 1, 20, 64, 1, True)[0]
        assert np.array_equal(got, oracle.select(sc[0], L, 1, 20, 64))


def test_all_heads_equals_selection_on_exact_sums():
    rng = np.random.default_rng(1)
    for L in (70, 333, 1000):
        sc = _int_scores(rng, 8, L)
        exact = sc.astype(np.int64).sum(axis=0).astype(np.float32)
        ref = oracle.select(exact, L, 1, 10, 16)
        got = oracle.select_grouped(sc, L, 1, 10, 16, 1, True)
        assert len(got) == 8 and all(np.array_equal(g, ref) for g in got)


@pytest.mark.parametrize("all_heads", [False, True])
def test_pages_equal_brute_force_on_exact_sums(all_heads):
    rng = np.random.default_rng(2)
    for L in (1, 15, 16, 17, 200, 777, 2049):
        for (sn, sd, W) in ((1, 20, 64), (1, 5, 1), (1, 2, 30), (1, 1, 16), (1, 20, 0)):
            sc = _int_scores(rng, 3, L, hi=6)  # many equal page sums: ties to the lower page
            got = oracle.select_grouped(sc, L, sn, sd, W, 16, all_heads)
            for h in range(3):
                key = sc.astype(np.int64).sum(axis=0) if all_heads else sc[h].astype(np.int64)
                assert got[h].tolist() == _brute_pages(key, L, sn, sd, W), (L, sn, sd, W, h)


def test_page_selection_shape():
    rng = np.random.default_rng(3)
    for L in (5, 16, 100, 1000, 24576, 24583):
        sc = rng.random((2, L)).astype(np.float32)
        for (sn, sd, W) in ((1, 20, 64), (1, 50, 64), (1, 5, 8), (1, 1, 64), (1, 20, 0)):
            sel = oracle.select_grouped(sc, L, sn, sd, W, 16, False)
            n = oracle.grouped_count(L, sn, sd, W, 16)
            for s in sel:
                assert len(s) == n and np.all(np.diff(s) > 0)
                # covers the newest window positions and at least the position budget
                assert set(range(L - min(W, L), L)) <= set(s.tolist())
                assert n >= oracle.budget(L, sn, sd, W) or n == L
                # older than the window: whole pages only
                first = (L - min(W, L)) // 16
                older = s[s < first * 16]
                assert len(older) % 16 == 0 and np.all(older.reshape(-1, 16) - older.reshape(-1, 16)[:, :1]
                                                          == np.arange(16))
                assert np.all(older.reshape(-1, 16)[:, 0] % 16 == 0) if len(older) else True
            if (sn, sd) == (1, 1):
                assert all(np.array_equal(s, np.arange(L)) for s in sel)


def test_page_sum_slot_order_is_float32_sequential():
    key = np.array([1e8, 1.0, -1e8, 1.0] + [0.0] * 12, dtype=np.float32)
    # sequential float32: ((1e8 + 1) - 1e8) + 1 = 1 (the first 1 is absorbed), not 2
    assert SV.page_sum(key, 16)[0] == np.float32(1.0)


def test_page_plan_at_the_24k_workload():
    # 24576 positions, s = 1/20 (1229 positions), window 64: 4 window pages plus 73 pages
    assert SV.page_plan(24576, 1, 20, 64) == (1532, 64, 73)
    assert oracle.grouped_count(24576, 1, 20, 64, 16) == 64 + 73 * 16


@pytest.mark.parametrize("all_heads", [False, True])
def test_selection_from_given_page_scores_on_exact_sums(all_heads):
    # page scores that are the exact (integer) sums of integer position scores select what the
    # whole-page rule selects from the position scores, and what brute force selects
    rng = np.random.default_rng(5)
    for L in (1, 16, 17, 250, 1500):
        for (sn, sd, W) in ((1, 20, 64), (1, 5, 1), (1, 2, 30), (1, 20, 0)):
            sc = _int_scores(rng, 3, L + 7, hi=6)
            npg = -(-(L + 7) // 16)
            pages = np.stack([[sc[h, 16 * p:16 * p + 16].astype(np.int64).sum() for p in range(npg)]
                              for h in range(3)]).astype(np.float32)
            got = oracle.select_by_page_scores(pages, L, sn, sd, W, all_heads)
            ref = oracle.select_grouped(sc, L, sn, sd, W, 16, all_heads)
            for h in range(3):
                key = sc.astype(np.int64).sum(axis=0) if all_heads else sc[h].astype(np.int64)
                assert got[h].tolist() == ref[h].tolist() == _brute_pages(key, L, sn, sd, W), (L, sn, sd, W, h)


def test_selection_from_page_scores_ignores_pages_past_the_candidates():
    # only the full pages older than the window are candidates: the window's pages and the pages
    # of the block past L (which the verification scored) never change the choice
    rng = np.random.default_rng(6)
    L = 1000
    pages = rng.random((2, 70)).astype(np.float32)
    ref = oracle.select_by_page_scores(pages, L, 1, 20, 64, False)
    f = (L - 64) // 16
    pages[:, f:] = 1e30
    got = oracle.select_by_page_scores(pages, L, 1, 20, 64, False)
    assert all(np.array_equal(a, b) for a, b in zip(ref, got))
