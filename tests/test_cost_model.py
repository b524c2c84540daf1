"""Pins of the round cost model against the numbers the pages print (CPU only)."""

import json
import os

import numpy as np

from self_sparse_speculative_amd import cost_model as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_table7_totals_and_break_even():
    g = json.load(open(os.path.join(GOLDEN, "table7_round_costs_k6.json")))
    k = g["k"]
    for row in g["rows"]:
        t_dense, t_draft, t_verify = cm.from_table_row(row["ar"], row["draft"], row["verify"], k)
        # the printed total is the round: 6 draft steps plus the verification
        assert abs(cm.round_cost(k, t_draft, t_verify) - row["total"]) < 0.006, row
        a = cm.break_even_acceptance(t_dense, k, t_draft, t_verify)
        if row["alpha_be"] == ">100%":
            assert a > 1.0, row
        else:
            assert round(100 * a, 1) == row["alpha_be"], (row, 100 * a)
        # at break-even a round is exactly as fast as dense decoding
        assert abs(cm.speedup(cm.break_even_tokens(t_dense, k, t_draft, t_verify), t_dense, k, t_draft, t_verify)
                   - 1.0) < 1e-12


def test_explainer_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "explainer_round_cost.json")))
    k = g["k"]
    assert abs(cm.round_cost(k, g["sparse"], g["verify"]) - g["round_units"]) < 1e-12
    assert abs(cm.break_even_tokens(g["dense"], k, g["sparse"], g["verify"]) - g["round_units"]) < 1e-12
    for s in g["speedups"]:
        got = cm.speedup(s["tokens"], g["dense"], k, g["sparse"], g["verify"])
        assert round(got, s["decimals"]) == s["speedup"], (s, got)
    # the measured break-even near 3.8 tokens per round is the B=32, 16K row of Table 7
    t7 = json.load(open(os.path.join(GOLDEN, "table7_round_costs_k6.json")))
    row = [r for r in t7["rows"] if r["B"] == g["measured_row"]["B"] and r["S"] == g["measured_row"]["S"]][0]
    t = cm.from_table_row(row["ar"], row["draft"], row["verify"], k)
    assert round(cm.break_even_tokens(*t[:1], k, *t[1:]), 1) == g["measured_break_even_tokens"]


def test_expected_tokens_closed_form_and_limits():
    k = 6
    for a in (0.0, 0.3, 0.8, 0.88, 0.999):
        assert abs(cm.expected_tokens(a, k) - (1 - a ** (k + 1)) / (1 - a)) < 1e-12
    assert cm.expected_tokens(1.0, k) == k + 1  # full acceptance: the bonus token too
    assert cm.expected_tokens(0.0, k) == 1.0   # first draft rejected: the correction only
    # reference points: 3.95 tokens at alpha 0.8 and 4.93 at 0.88 (k = 6)
    assert round(cm.expected_tokens(0.8, k), 2) == 3.95 and round(cm.expected_tokens(0.88, k), 2) == 4.93


def test_expected_tokens_matches_simulated_rounds():
    rng = np.random.default_rng(4)
    k, a, n = 6, 0.7, 200_000
    acc = rng.random((n, k)) < a
    first_reject = np.where(acc.all(axis=1), k, acc.argmin(axis=1))
    tokens = first_reject + 1
    assert abs(tokens.mean() - cm.expected_tokens(a, k)) < 4 * tokens.std() / np.sqrt(n)


def test_position_profile_reduces_to_constant_acceptance():
    for a in (0.5, 0.9):
        for k in range(0, 9):
            assert abs(cm.expected_tokens_by_position([a] * 8, k) - cm.expected_tokens(a, k)) < 1e-12


def test_choose_draft_length_is_the_brute_force_argmax():
    rng = np.random.default_rng(5)
    for _ in range(200):
        kmax = int(rng.integers(1, 12))
        alpha = np.sort(rng.random(kmax))[::-1]  # declining along the draft
        t_dense, t_draft = 1.0, float(rng.uniform(0.05, 0.5))
        tv = {k: float(rng.uniform(0.8, 2.0)) + 0.05 * k for k in range(1, kmax + 1)}
        k, gains = cm.choose_draft_length(alpha, t_dense, t_draft, tv, kmax)
        # brute force with exact per-round enumeration of the accepted prefix
        best, best_k = -1.0, None
        for kk in range(1, kmax + 1):
            p_prefix = [np.prod(alpha[:i]) * (1 - (alpha[i] if i < kk else 0.0)) for i in range(kk + 1)]
            tokens = sum((i + 1) * p for i, p in enumerate(p_prefix))
            g = tokens * t_dense / (kk * t_draft + tv[kk])
            if g > best + 1e-12:
                best, best_k = g, kk
        assert k == best_k and abs(gains[k] - best) < 1e-9


def test_degrading_late_positions_shorten_the_horizon():
    t_dense, t_draft = 2.2, 0.12
    tv = {k: 2.9 + 0.1 * k for k in range(1, 9)}
    flat, _ = cm.choose_draft_length([0.9] * 8, t_dense, t_draft, tv, 8)
    steep, _ = cm.choose_draft_length([0.96, 0.9, 0.8, 0.6, 0.4, 0.25, 0.15, 0.1], t_dense, t_draft, tv, 8)
    assert steep < flat


def test_acceptance_tracker_counts():
    tr = cm.AcceptanceTracker(4, decay=0.5)
    acc = np.array([[1, 1, 0, -1], [1, 0, -1, -1], [0, -1, -1, -1], [1, 1, 1, 1]], dtype=np.int8)
    est = tr.update(acc)
    assert est[:4] == [3 / 4, 2 / 3, 1 / 2, 1 / 1]
    est = tr.update(np.array([[0, -1, -1, -1]], dtype=np.int8))
    assert est[0] == 0.5 * 0.75 and est[1:] == [2 / 3, 1 / 2, 1.0]  # unreached positions keep their estimate


def test_calibrated_speedup_limits():
    k = 6
    # a draft that reads the whole cache (rho = 1) and keeps every draft costs exactly the k + 1
    # dense steps it replaces
    assert abs(cm.calibrated_speedup(1.0, 1.0, k) - 1.0) < 1e-15
    # full acceptance outputs k + 1 tokens: the numerator
    assert abs(cm.calibrated_speedup(1.0, 0.05, k) * (k * 0.05 + 1.0) - (k + 1)) < 1e-12
    # nothing accepted: one token for the round's cost
    assert abs(cm.calibrated_speedup(0.0, 0.05, k, 0.2) - 1.0 / (k * 0.05 + 1.2)) < 1e-15
    # the correction only lengthens (c > 0) or shortens the round
    assert cm.calibrated_speedup(0.8, 0.05, k, 0.3) < cm.calibrated_speedup(0.8, 0.05, k, 0.0)
    # the explainer's round in the same terms: 6 steps at 0.35 of a dense step and a verification
    # of 1.4 dense steps are rho = 0.35 and c = 0.4; 5.5 tokens per round give 1.57x
    assert round(cm.calibrated_speedup(4.5 / 6, 0.35, 6, 0.4), 2) == 1.57


def test_constant_correction_fit_recovers_a_planted_constant():
    rng = np.random.default_rng(0)
    pts = []
    for _ in range(24):
        a, rho, k = rng.uniform(0.3, 0.95), rng.uniform(0.01, 0.3), int(rng.integers(2, 9))
        pts.append((a, rho, k, cm.calibrated_speedup(a, rho, k, 0.37)))
    c = cm.fit_constant_correction(pts[:12])
    assert abs(c - 0.37) < 1e-12
    assert cm.mape(pts[12:], c) < 1e-10
    assert cm.mape(pts[12:], 0.0) > 5.0  # the uncorrected model is off
    # the fit minimises the squared error of the modelled round cost: a brute-force scan agrees
    noisy = [(a, rho, k, sp * (1 + 0.02 * rng.standard_normal())) for a, rho, k, sp in pts]
    c_fit = cm.fit_constant_correction(noisy)
    cost = lambda c: sum(((1 + a * k) / sp - (k * rho + 1 + c)) ** 2 for a, rho, k, sp in noisy)
    grid = np.linspace(c_fit - 0.05, c_fit + 0.05, 2001)
    assert abs(grid[int(np.argmin([cost(g) for g in grid]))] - c_fit) <= 0.05 / 1000


def test_acceptance_curve_through_the_pages_points():
    # the listing's abstract: 80.4 % acceptance at s = 0.05, 96.7 % at s = 0.50
    f = cm.acceptance_curve([(0.05, 0.804), (0.50, 0.967)])
    assert abs(f(0.05) - 0.804) < 1e-12 and abs(f(0.50) - 0.967) < 1e-12
    assert abs(f(np.sqrt(0.05 * 0.5)) - (0.804 + 0.967) / 2) < 1e-12  # linear in log s
    assert f(0.02) < f(0.05) < f(0.1) < f(0.2) < f(0.5) and f(10.0) == 1.0


def test_budget_choice_is_the_brute_force_argmax():
    rng = np.random.default_rng(3)
    for _ in range(50):
        k = int(rng.integers(2, 9))
        budgets = sorted(rng.uniform(0.01, 0.5, size=5))
        t_dense = 2.0
        t_round = {s: t_dense * (1.2 + k * s * rng.uniform(0.8, 1.2)) for s in budgets}
        a0, a1 = rng.uniform(0.5, 0.85), rng.uniform(0.86, 0.99)
        f = cm.acceptance_curve([(0.05, a0), (0.5, a1)])
        best, gains = cm.choose_budget(f, t_round, t_dense, k)
        brute = max(budgets, key=lambda s: (sum(f(s) ** i for i in range(k + 1)) * t_dense / t_round[s], -s))
        assert best == brute
        assert all(abs(gains[s] - cm.speedup(cm.expected_tokens(f(s), k), t_dense, k, 0.0, t_round[s])) < 1e-12
                   for s in budgets)
