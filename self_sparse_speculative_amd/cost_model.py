"""Round cost model: when does a draft-and-verify round beat dense decoding?

[listing] "S^3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative
Decoding", appendix Table 7 and its caption: a round costs k sparse draft
steps plus one dense verification; the dense reference runs k + 1 dense
steps (as many tokens as a fully accepted round); alpha_BE is the acceptance
a round needs to break even when the stages run one after another.
[explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
mean?", the worked example in "Where it earns its keep": with the dense step
as the unit, a round wins only if it outputs more tokens than it costs units.

Readings (the pages give the table and the example, not the formulas):
* a round that outputs tau tokens replaces tau dense steps, so its speedup is
  tau * T_dense / (k * T_draft + T_verify);
* the break-even output is (k * T_draft + T_verify) / T_dense tokens per round;
* alpha_BE is the fraction of the k drafts that must be accepted for that
  output under the plain count "accepted drafts + 1": (tokens_BE - 1) / k
  (this reproduces every printed alpha_BE of Table 7);
* with an acceptance probability alpha at every position, a round outputs
  1 + alpha + ... + alpha^k tokens on average (the first rejection ends it).

Adaptive draft length ([digest], the section on per-position acceptance:
acceptance falls along the draft positions, more so for the last ones and
as training proceeds, and the authors propose shortening the draft horizon
when late positions degrade, as future work). Reading adopted: estimate the
acceptance of each draft position given that the earlier ones were
accepted, from the decisions of recent rounds, and pick the k that maximises
the speedup above; a round of k drafts then outputs on average
sum_{i=0..k} prod_{m<i} alpha_m tokens.

Calibrated speedup ([digest], the section on the limits of the speedup
claim; [listing], Figures 12 and 13 captions, Eq. 24 there, which the pages
do not print): the speedup is modelled from the accepted-prefix fraction a
(the share of the k drafts a round keeps on average, so a round outputs
1 + a k tokens) and the effective draft KV-read fraction rho (the positions a
draft step reads over the positions a dense step reads), with one constant
correction fitted to profiled rounds. Reading adopted, in dense-step units:
a round costs k rho for its draft steps plus one verification worth one
dense step, plus the constant c that absorbs everything else (the
verification's extra rows, selection, sampling, launch gaps):
  speedup(a, rho; c) = (1 + a k) / (k rho + 1 + c),
c = 0 being the uncorrected model. c is fitted by least squares on the
calibration points' measured round costs (1 + a k) / speedup - (k rho + 1),
and the model is judged by its mean absolute percentage error on held-out
points, as the digest reports it (84.61 % -> 0.80 % for Qwen3-1.7B, 63.03 %
-> 0.68 % for Qwen3-8B on the pages' hardware).

Adaptive budget ([news], Perspective: adaptive sparse budgets named as a next
step; [listing], Abstract and Figure 6: acceptance rises with the budget,
80.4 % at s = 0.05 and 96.7 % at s = 0.50, while the speedup falls from
1.370x to 1.058x): choose_budget picks, among budgets with measured round
times, the one whose modelled speedup is largest, given an acceptance-
versus-budget curve supplied by the caller (synthetic logits make acceptance
independent of the budget, so the curve is an input, not a measurement).

Host arithmetic on measured or printed times only; nothing here runs on the
device.
"""

import math


def round_cost(k: int, t_draft_step: float, t_verify: float) -> float:
    """Time of one round: k sparse draft steps and one verification."""
    return k * t_draft_step + t_verify


def break_even_tokens(t_dense_step: float, k: int, t_draft_step: float, t_verify: float) -> float:
    """Tokens a round must output to cost no more per token than dense decoding."""
    return round_cost(k, t_draft_step, t_verify) / t_dense_step


def break_even_acceptance(t_dense_step: float, k: int, t_draft_step: float, t_verify: float) -> float:
    """alpha_BE: accepted fraction of the k drafts at break-even (> 1: unreachable)."""
    return (break_even_tokens(t_dense_step, k, t_draft_step, t_verify) - 1.0) / k


def speedup(tokens_per_round: float, t_dense_step: float, k: int, t_draft_step: float, t_verify: float) -> float:
    """Time of tokens_per_round dense steps over the time of one round."""
    return tokens_per_round * t_dense_step / round_cost(k, t_draft_step, t_verify)


def expected_tokens(alpha: float, k: int) -> float:
    """Mean output of a round when each draft is accepted with probability alpha."""
    return sum(alpha ** i for i in range(k + 1))


def from_table_row(ar_total: float, draft_total: float, verify: float, k: int):
    """Per-step times from a row given as (k+1) dense steps, k draft steps and one verification."""
    return ar_total / (k + 1), draft_total / k, verify


def expected_tokens_by_position(alpha_pos, k: int) -> float:
    """Mean output of a round of k drafts when draft m+1 is accepted with probability alpha_pos[m]
    given that drafts 1..m were."""
    total, run = 1.0, 1.0
    for m in range(k):
        run *= float(alpha_pos[m])
        total += run
    return total


def choose_draft_length(alpha_pos, t_dense_step: float, t_draft_step: float, t_verify_of_k, k_max: int,
                        k_min: int = 1):
    """The k in [k_min, k_max] with the largest speedup (ties to the shorter horizon).

    t_verify_of_k: verification time for a block of k + 1 rows (a callable or a mapping).
    Returns (k, {k: speedup})."""
    tv = t_verify_of_k if callable(t_verify_of_k) else (lambda k: t_verify_of_k[k])
    gains = {k: speedup(expected_tokens_by_position(alpha_pos, k), t_dense_step, k, t_draft_step, tv(k))
             for k in range(k_min, k_max + 1)}
    best = max(gains, key=lambda k: (gains[k], -k))
    return best, gains


class AcceptanceTracker:
    """Per-position acceptance from the decisions of recent rounds.

    update() takes the accepted array of a round ([B][k], 1 accepted, 0 the first reject,
    -1 not reached). The estimate of position m is accepted / reached over that round,
    blended into an exponential moving average (weight `decay` on the past)."""

    def __init__(self, k_max: int, decay: float = 0.8, prior: float = 1.0):
        self.k_max, self.decay = int(k_max), float(decay)
        self.alpha = [float(prior)] * self.k_max
        self.seen = [False] * self.k_max

    def update(self, accepted):
        import numpy as np
        a = np.asarray(accepted)
        for m in range(min(a.shape[1], self.k_max)):
            col = a[:, m]
            reached = int((col >= 0).sum())
            if reached == 0:
                continue
            rate = float((col == 1).sum()) / reached
            self.alpha[m] = rate if not self.seen[m] else self.decay * self.alpha[m] + (1 - self.decay) * rate
            self.seen[m] = True
        return list(self.alpha)


def calibrated_speedup(a: float, rho: float, k: int, c: float = 0.0) -> float:
    """Speedup of a round over dense decoding from the accepted-prefix fraction a, the draft
    KV-read fraction rho and the constant correction c (dense-step units)."""
    return (1.0 + a * k) / (k * rho + 1.0 + c)


def fit_constant_correction(points, k_of=None) -> float:
    """Least-squares c over calibration points (a, rho, k, measured speedup): the mean of
    (1 + a k) / speedup - (k rho + 1), which minimises the squared error of the modelled
    round cost."""
    res = [(1.0 + a * k) / sp - (k * rho + 1.0) for a, rho, k, sp in points]
    return sum(res) / len(res)


def mape(points, c: float) -> float:
    """Mean absolute percentage error (%) of calibrated_speedup against measured speedups."""
    errs = [abs(calibrated_speedup(a, rho, k, c) - sp) / sp for a, rho, k, sp in points]
    return 100.0 * sum(errs) / len(errs)


def acceptance_curve(points):
    """Acceptance as a function of the budget s, through (s, alpha) points: linear in log s
    between neighbouring points, the end segments extended, clamped to [0, 1]."""
    pts = sorted((float(s_), float(a_)) for s_, a_ in points)
    if len(pts) < 2:
        raise ValueError("two points at least")

    def alpha(s_: float) -> float:
        x = math.log(float(s_))
        i = 0
        while i < len(pts) - 2 and x > math.log(pts[i + 1][0]):
            i += 1
        (s0, a0), (s1, a1) = pts[i], pts[i + 1]
        t = (x - math.log(s0)) / (math.log(s1) - math.log(s0))
        return min(1.0, max(0.0, a0 + t * (a1 - a0)))

    return alpha


def choose_budget(alpha_of_s, t_round_of_s, t_dense_step: float, k: int):
    """The budget with the largest modelled speedup (ties to the smaller budget).

    alpha_of_s: per-draft acceptance at budget s (callable); t_round_of_s: measured round time
    at each candidate budget (mapping s -> time, same unit as t_dense_step). A round at budget s
    outputs expected_tokens(alpha(s), k) tokens on average. Returns (s, {s: speedup})."""
    gains = {s_: expected_tokens(alpha_of_s(s_), k) * t_dense_step / t for s_, t in t_round_of_s.items()}
    best = max(gains, key=lambda s_: (gains[s_], -s_))
    return best, gains
