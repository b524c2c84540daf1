"""Pins of the oracle's exact speculative sampling (CPU only)."""

import json
import os

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(V, k, seed, noise=0.7, std=1.5):
    rng = np.random.default_rng(seed)
    zt = (std * rng.standard_normal((k + 1, V))).astype(np.float32)
    zd = (zt[:k] + noise * rng.standard_normal((k, V))).astype(np.float32)
    return zt, zd


def breakpoints(f, lo=0.0, hi=1.0, tol=1e-15):
    """Measure of each value of a piecewise-constant, monotone-in-pieces f on [lo, hi).

    Splits [lo, hi) recursively until both ends agree (f is monotone in u
    for the functions used here, so equal ends mean no change inside).
    """
    out = {}

    def rec(a, fa, b, fb):
        if fa == fb:
            out[fa] = out.get(fa, 0.0) + (b - a)
            return
        if b - a < tol:
            out[fa] = out.get(fa, 0.0) + (b - a) / 2
            out[fb] = out.get(fb, 0.0) + (b - a) / 2
            return
        m = 0.5 * (a + b)
        fm = f(m)
        rec(a, fa, m, fm)
        rec(m, fm, b, fb)

    top = np.nextafter(hi, lo)
    rec(lo, f(lo), top, f(top))
    return out


def test_softmax_matches_torch():
    zt, _ = _rows(37, 2, 0)
    for T in (1.0, 0.7, 2.5):
        ref = torch.softmax(torch.tensor(zt, dtype=torch.float64) / np.float64(np.float32(T)), dim=-1).numpy()
        for i in range(3):
            np.testing.assert_allclose(S.softmax_t(zt[i], np.float32(T)), ref[i], rtol=1e-14, atol=1e-300)


def test_invcdf_matches_searchsorted():
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[rng.integers(0, V)] = 1.0
        for u in list(rng.random(5)) + [0.0]:
            c = np.cumsum(w)
            ref = int(np.searchsorted(c, u * c[-1], side="right"))
            assert S.invcdf(w, u) == ref
    # no index passes the strict test only through rounding: the last positive weight is used
    assert S.invcdf(np.array([0.0, 1.0, 0.0]), np.nextafter(1.0, 0.0)) == 1


def test_identical_distributions_accept_everything():
    for seed in range(20):
        zt, _ = _rows(64, 6, seed)
        rng = np.random.default_rng(seed)
        d = rng.integers(0, 64, size=6)
        u = rng.random(7).astype(np.float32)
        tokens, n_out, acc = oracle.spec_sample(zt, zt[:6].copy(), d, u, np.float32(1.0))
        assert n_out == 7 and (acc == 1).all()
        assert list(tokens[:6]) == list(d)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_output_law_is_target_exactly(seed):
    """Integrate over u exactly: P(first output = y) equals p_0(y)."""
    V = 6
    zt, zd = _rows(V, 1, seed)
    T = np.float32(1.0)
    p = S.softmax_t(zt[0], T)
    q = S.softmax_t(zd[0], T)
    law = np.zeros(V)
    alpha = 0.0
    for x in range(V):
        acc = breakpoints(lambda u0: int(oracle.spec_sample(zt, zd, [x], [u0, 0.5], T)[2][0]))
        a = acc.get(1, 0.0)
        alpha += q[x] * a
        law[x] += q[x] * a
        if a < 1.0:
            u0 = 1.0 - 1e-15  # a rejecting u0 for this x
            res = breakpoints(lambda u1: int(oracle.spec_sample(zt, zd, [x], [u0, u1], T)[0][0]))
            for y, m in res.items():
                law[y] += q[x] * (1.0 - a) * m
    np.testing.assert_allclose(law, p, atol=1e-12)
    # acceptance probability is sum_x min(p, q)
    assert abs(alpha - np.minimum(p, q).sum()) < 1e-12


def test_bonus_law_is_last_target_row():
    V = 7
    zt, _ = _rows(V, 1, 9)
    zd = zt[:1].copy()  # identical rows: always accepted, the bonus follows p_1
    T = np.float32(1.3)
    law = breakpoints(lambda u1: int(oracle.spec_sample(zt, zd, [3], [0.99, u1], T)[0][1]))
    p1 = S.softmax_t(zt[1], T)
    got = np.array([law.get(y, 0.0) for y in range(V)])
    np.testing.assert_allclose(got, p1, atol=1e-12)


def _chi2_run(decide, V=16, k=3, n=1_000_000, seed=11):
    zt, zd = _rows(V, k, seed, noise=1.0)
    T = np.float32(1.0)
    P = [S.softmax_t(zt[i], T) for i in range(k + 1)]
    Q = [S.softmax_t(zd[i], T) for i in range(k)]
    rng = np.random.default_rng(seed + 100)
    cq = [np.cumsum(q) for q in Q]
    draws = np.stack([np.minimum(np.searchsorted(c, rng.random(n) * c[-1], side="right"), V - 1) for c in cq], axis=1)
    us = rng.random((n, k + 1))
    counts = np.zeros((k + 1, V))
    for t in range(n):
        tokens, n_out, _ = decide(P, Q, draws[t], us[t])
        for i in range(n_out):
            counts[i, tokens[i]] += 1
    pvals = []
    for i in range(k + 1):
        tot = counts[i].sum()
        pvals.append(stats.chisquare(counts[i], P[i] * tot).pvalue)
    return pvals


def test_chi_square_output_law():
    pvals = _chi2_run(S.spec_decide)
    assert min(pvals) > 1e-3, pvals


def test_chi_square_negative_control():
    # planted mistake in a copy of the oracle: the correction is drawn from p instead of the residual
    src = open(S.__file__).read()
    bad = src.replace("r = np.maximum(np.asarray(p_rows[i], dtype=np.float64) - np.asarray(q_rows[i], dtype=np.float64), 0.0)",
                      "r = np.asarray(p_rows[i], dtype=np.float64)")
    assert bad != src
    ns = {"__name__": "mutated_sampling"}
    exec(compile(bad, "mutated_sampling", "exec"), ns)
    pvals = _chi2_run(ns["spec_decide"], n=100_000)
    assert min(pvals) < 1e-6, pvals


def test_golden_first_mismatch():
    g = json.load(open(os.path.join(GOLDEN, "first_mismatch_k5.json")))
    k = g["k"]
    V = 8
    # target and draft agree on tokens 0..2 and disagree sharply on token 3
    zt = np.zeros((k + 1, V), np.float32)
    zd = np.zeros((k, V), np.float32)
    d = np.array([1, 2, 3, 4, 5])
    for i in range(k):
        zt[i, d[i]] = 5.0
        zd[i, d[i]] = 5.0
    zt[3, d[3]] = -5.0  # the target finds the 4th draft unlikely
    u = np.array([0.5] * (k + 1), np.float32)
    tokens, n_out, acc = oracle.spec_sample(zt, zd, d, u, np.float32(1.0))
    assert list(acc) == g["accept_pattern"]
    assert int((acc == 1).sum()) == g["n_accepted"]
    assert n_out == g["n_out"] == g["n_accepted"] + g["n_corrected"]
    assert list(tokens[:3]) == list(d[:3]) and tokens[3] != d[3] and (tokens[n_out:] == -1).all()


def test_golden_full_acceptance():
    g = json.load(open(os.path.join(GOLDEN, "full_acceptance_k6.json")))
    k = g["k"]
    zt, _ = _rows(20, k, 3)
    d = np.arange(k)
    tokens, n_out, acc = oracle.spec_sample(zt, zt[:k].copy(), d, np.full(k + 1, 0.3, np.float32), np.float32(1.0))
    assert list(acc) == g["accept_pattern"] and n_out == g["n_out"]


def test_budget_golden():
    g = json.load(open(os.path.join(GOLDEN, "budget_tiny.json")))
    assert oracle.budget(g["L"], g["s_num"], g["s_den"], g["window"]) == g["n_sel"]
    idx = oracle.select(np.random.default_rng(0).random(g["L"]).astype(np.float32), g["L"], g["s_num"], g["s_den"], g["window"])
    assert int((idx >= g["L"] - g["window"]).sum()) == g["n_newest"]


def test_greedy_temperature_zero():
    zt, zd = _rows(30, 4, 5)
    best = [int(np.argmax(zt[i])) for i in range(5)]
    d = np.array([best[0], best[1], (best[2] + 1) % 30, best[3]])
    tokens, n_out, acc = oracle.spec_sample(zt, zd, d, np.zeros(5, np.float32), np.float32(0.0))
    assert n_out == 3 and list(acc) == [1, 1, 0, -1] and list(tokens[:3]) == best[:3]
    tokens, n_out, acc = oracle.spec_sample(zt, zd, np.array(best[:4]), np.zeros(5, np.float32), np.float32(0.0))
    assert n_out == 5 and tokens[4] == best[4]


def test_expected_tokens_per_round():
    """E[n_out] = sum_i prod_{m<i} alpha_m, integrated exactly over u for k = 2."""
    V = 5
    zt, zd = _rows(V, 2, 21)
    T = np.float32(1.0)
    P = [S.softmax_t(zt[i], T) for i in range(3)]
    Q = [S.softmax_t(zd[i], T) for i in range(2)]
    alphas = [np.minimum(P[i], Q[i]).sum() for i in range(2)]
    exp_n = 1 + alphas[0] + alphas[0] * alphas[1]
    # exact integration: n_out depends on (d0, u0, d1, u1); u2 does not change n_out
    tot = 0.0
    for x0 in range(V):
        a0 = breakpoints(lambda u0: int(oracle.spec_sample(zt, zd, [x0, 0], [u0, 0.0, 0.5], T)[2][0])).get(1, 0.0)
        for x1 in range(V):
            # u0 = 0 always accepts position 0, so position 1 is reached
            a1 = breakpoints(lambda u1: int(oracle.spec_sample(zt, zd, [x0, x1], [0.0, u1, 0.5], T)[2][1])).get(1, 0.0)
            tot += Q[0][x0] * Q[1][x1] * (1 + a0 + a0 * a1)
    assert abs(tot - exp_n) < 1e-12


# ----------------------------------------------------------------- decision margins

def test_margins_hand_built_rows():
    # exact binary fractions: every margin below is exact
    p0 = np.array([0.5, 0.25, 0.125, 0.125])
    q0 = np.array([0.25, 0.5, 0.125, 0.125])
    p1 = np.full(4, 0.25)
    d = [1]
    # accepted (0.25 * 0.5 < 0.25): ratio margin 0.125 / 0.5; bonus t = 0.5 lies on a CDF boundary
    assert S.decide_margins([p0, p1], [q0], d, [0.25, 0.5]) == (0.25, 0.0)
    # bonus t = 0.375: 0.125 from both ends of token 1's interval [0.25, 0.5)
    assert S.decide_margins([p0, p1], [q0], d, [0.25, 0.375]) == (0.25, 0.125)
    # rejected (0.75 * 0.5 >= 0.25): the residual keeps token 0 alone (weight 0.25), t = 0.375 * 0.25
    assert S.decide_margins([p0, p1], [q0], d, [0.75, 0.375]) == (0.25, 0.375)
    # greedy has no margin: it compares the float32 logits themselves
    assert S.spec_margins(np.zeros((2, 4), np.float32), np.zeros((1, 4), np.float32), d, [0.5, 0.5], 0.0) is None


def _flip_checks(p_rows, q_rows, d, u, S=S):
    """The margins are distances to a flip: a change just below each leaves the decision,
    a change just above it (towards the flip) changes it."""
    rm, dm = S.decide_margins(p_rows, q_rows, d, u)
    _, n_out, acc = S.spec_decide(p_rows, q_rows, d, u)
    k = len(d)
    reached = range(n_out if n_out <= k else k)
    # the draft test closest to a flip
    rel = [abs(float(u[i]) * q_rows[i][d[i]] - p_rows[i][d[i]]) / max(p_rows[i][d[i]], q_rows[i][d[i]]) for i in reached]
    i = int(np.argmin(rel))
    x = int(d[i])
    scale = max(p_rows[i][x], q_rows[i][x])
    towards = -1.0 if acc[i] == 1 else 1.0  # lower p to reject, raise p to accept
    for f, flips in ((0.99, False), (1.01, True)):
        pr = [r.copy() for r in p_rows]
        pr[i][x] = p_rows[i][x] + towards * f * rm * scale
        _, _, a2 = S.spec_decide(pr, q_rows, d, u)
        assert (a2[i] != acc[i]) == flips, (f, i)
    # the final draw: u_k moved by just under the draw margin keeps the token; moved by just over
    # it, towards one end or the other, changes it
    tok = S.spec_decide(p_rows, q_rows, d, u)[0][n_out - 1]
    for sgn in (-1.0, 1.0):
        u2 = np.array(u, dtype=np.float64)
        u2[k] = u[k] + sgn * 0.99 * dm
        if 0.0 <= u2[k] < 1.0:
            assert S.spec_decide(p_rows, q_rows, d, u2)[0][n_out - 1] == tok
    changed = False
    for sgn in (-1.0, 1.0):
        u2 = np.array(u, dtype=np.float64)
        u2[k] = u[k] + sgn * 1.01 * dm
        if 0.0 <= u2[k] < 1.0:
            changed |= S.spec_decide(p_rows, q_rows, d, u2)[0][n_out - 1] != tok
    return changed


@pytest.mark.parametrize("seed", range(6))
def test_margins_are_distances_to_a_flip(seed):
    rng = np.random.default_rng(100 + seed)
    k, V = 3, 12
    changed = 0
    for _ in range(150):
        zt, zd = _rows(V, k, int(rng.integers(1 << 30)), noise=1.0)
        p_rows = [S.softmax_t(zt[i], 1.0) for i in range(k + 1)]
        q_rows = [S.softmax_t(zd[i], 1.0) for i in range(k)]
        d = [int(rng.choice(V, p=q_rows[i])) for i in range(k)]
        u = rng.random(k + 1)
        changed += _flip_checks(p_rows, q_rows, d, u)
    assert changed >= 120  # the nearer end is inside [0, 1) in most cases (not below token 0 or above the last)
