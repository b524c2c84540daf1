"""Exact speculative sampling with caller-supplied uniforms.

[explainer], Jargon, "Exact speculative sampling": the accept-or-resample
rule that makes draft-then-verify produce exactly the target model's token
distribution. [explainer], mechanism paragraph and the draft/verify
illustration: drafted tokens that the full model would also produce stay,
the earliest disagreement is swapped for a token drawn by the full model,
and what the draft proposed after it is dropped (the illustration counts
three kept drafts and one correction as four tokens). [news], Interpretation:
exact speculative sampling either accepts candidates or draws from the
residual distribution. [listing], Table 7 caption: a fully accepted round
outputs as many tokens as k + 1 autoregressive steps (the bonus token).

Rule (for each sequence, temperature T > 0):
  p_i = softmax(zt_i / T), i = 0..k;   q_i = softmax(zd_i / T), i = 0..k-1;
  for i = 0..k-1 with x = d_i: accept iff p_i(x) >= q_i(x) or u_i q_i(x) < p_i(x)
  (acceptance probability min(1, p/q));
  first reject at i*: draw y from the residual max(0, p_i* - q_i*), output
  d_0..d_{i*-1}, y, n_out = i* + 1;
  all accepted: draw the bonus y from p_k, n_out = k + 1.

Readings where the pages are silent:
* draws use the inverse CDF in token-index order with a strict ">":
  y = min{y : sum_{y' <= y} w(y') > u * sum(w)}; if rounding leaves no such
  y, the last y with w(y) > 0;
* u_0..u_{k-1} drive the ratio tests; u_k is the single draw for the
  residual or the bonus;
* if the residual is all zero (p == q to the last bit) the draw falls back
  to p;
* T = 0 is greedy: accept iff d_i is the first argmax of zt_i; the
  correction and the bonus are that argmax;
* all of it in float64 from the float32 logits.

Decision margins (decide_margins, spec_margins): how far the given
uniforms sit from a flip of the outcome, so that a bit-exact comparison
with a float64 GPU implementation has a stated distance from a flip. The
ratio margin is the smallest |u_i q_i(x) - p_i(x)| / max(p_i(x), q_i(x)) over
the draft tests the round reaches (a relative change of p or q below it
cannot change an accept into a reject or back); the draw margin is the
distance of t = u_k Z from the nearer end of the CDF interval that holds it,
divided by Z (a change of u_k, or of the cumulative weights relative to Z,
below it cannot change the drawn token).

Pins: p == q accepts every draft; the output law equals p exactly,
integrated over u by locating the breakpoints of the accept test and of
the inverse CDF (bisection through these functions); a chi-square test on
a 16-token vocabulary with a negative control that resamples from p
instead of the residual; invcdf equals numpy.searchsorted(cumsum, t,
side="right"); the first-mismatch and full-acceptance token counts of the
pages' examples (tests/golden); the margins equal the distance to the flip
that bisection over the uniform finds through spec_decide and invcdf, and
hand-built rows with exactly known margins (0 on a CDF boundary).
"""

import numpy as np


def softmax_t(z: np.ndarray, T: float) -> np.ndarray:
    """softmax(z / T) in float64 (T > 0)."""
    x = np.asarray(z, dtype=np.float64) / float(T)
    e = np.exp(x - x.max())
    return e / e.sum()


def invcdf(w: np.ndarray, u: float) -> int:
    """Inverse-CDF draw from non-negative weights w with uniform u in [0, 1)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    t = float(u) * c[-1]
    hit = np.nonzero(c > t)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def spec_decide(p_rows, q_rows, d, u):
    """Decisions from probability rows. Returns (tokens, n_out, accepted).

    p_rows: k+1 target rows; q_rows: k draft rows; d: k draft tokens;
    u: k+1 uniforms. accepted[i] is 1, 0 (the first reject) or -1 (not
    reached).
    """
    k = len(d)
    tokens = np.full(k + 1, -1, dtype=np.int64)
    accepted = np.full(k, -1, dtype=np.int64)
    for i in range(k):
        x = int(d[i])
        p, q = float(p_rows[i][x]), float(q_rows[i][x])
        if p >= q or float(u[i]) * q < p:
            accepted[i] = 1
            tokens[i] = x
            continue
        accepted[i] = 0
        r = np.maximum(np.asarray(p_rows[i], dtype=np.float64) - np.asarray(q_rows[i], dtype=np.float64), 0.0)
        if not r.sum() > 0.0:
            r = np.asarray(p_rows[i], dtype=np.float64)
        tokens[i] = invcdf(r, u[k])
        return tokens, i + 1, accepted
    tokens[k] = invcdf(p_rows[k], u[k])
    return tokens, k + 1, accepted


def _greedy(zt, d):
    k = len(d)
    tokens = np.full(k + 1, -1, dtype=np.int64)
    accepted = np.full(k, -1, dtype=np.int64)
    for i in range(k):
        best = int(np.argmax(np.asarray(zt[i], dtype=np.float64)))
        if int(d[i]) == best:
            accepted[i] = 1
            tokens[i] = best
        else:
            accepted[i] = 0
            tokens[i] = best
            return tokens, i + 1, accepted
    tokens[k] = int(np.argmax(np.asarray(zt[k], dtype=np.float64)))
    return tokens, k + 1, accepted


def spec_sample(zt, zd, d, u, T: float):
    """One sequence: zt [k+1][V], zd [k][V] float32 logits, d [k], u [k+1]."""
    if float(T) == 0.0:
        return _greedy(zt, d)
    k = len(d)
    p_rows = [softmax_t(zt[i], T) for i in range(k + 1)]
    q_rows = [softmax_t(zd[i], T) for i in range(k)]
    return spec_decide(p_rows, q_rows, d, u)


def _draw_margin(w, u: float) -> float:
    """Distance of u * Z from the nearer end of the CDF interval holding it, over Z."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    Z = c[-1]
    t = float(u) * Z
    y = invcdf(w, u)
    if not c[y] > t:  # the no-crossing fallback sits on the boundary itself
        return 0.0
    lo = c[y - 1] if y > 0 else 0.0
    return float(min(t - lo, c[y] - t) / Z)


def decide_margins(p_rows, q_rows, d, u):
    """(ratio margin, draw margin) of the decisions spec_decide takes on these rows."""
    k = len(d)
    ratio = float("inf")
    for i in range(k):
        x = int(d[i])
        p, q = float(p_rows[i][x]), float(q_rows[i][x])
        ratio = min(ratio, abs(float(u[i]) * q - p) / max(p, q))
        if float(u[i]) * q < p or p >= q:  # accepted: spec_decide's test
            continue
        r = np.maximum(np.asarray(p_rows[i], dtype=np.float64) - np.asarray(q_rows[i], dtype=np.float64), 0.0)
        if not r.sum() > 0.0:
            r = np.asarray(p_rows[i], dtype=np.float64)
        return ratio, _draw_margin(r, u[k])
    return ratio, _draw_margin(p_rows[k], u[k])


def spec_margins(zt, zd, d, u, T: float):
    """Margins of one sequence's round (as spec_sample decides it); None at T = 0, where
    every decision compares the float32 logits themselves."""
    if float(T) == 0.0:
        return None
    k = len(d)
    p_rows = [softmax_t(zt[i], T) for i in range(k + 1)]
    q_rows = [softmax_t(zd[i], T) for i in range(k)]
    return decide_margins(p_rows, q_rows, d, u)
