"""KV selector: newest window plus the top-scoring older positions.

[explainer], mechanism paragraph: the positions the drafter reads are the
most recent ones together with those the previous verification pass gave
the most attention weight, chosen again at every round. [news],
Interpretation: the draft attends to a small subset of the cached entries,
picked by attention score.

Readings where the pages are silent or disagree:
* granularity is single positions (one page says "pages"; the others say
  positions / KV entries);
* selection is per KV head of one layer, on scores already summed over the
  query heads of the GQA group (the score definition is in attention.verify);
* order: score descending, ties to the lower position; -0.0 equals +0.0;
  +inf ranks highest; NaN is a caller error;
* the output is the ascending list of kept positions.

Pins: every kept candidate precedes every dropped candidate in the order
(brute force over all pairs on small inputs); equality with numpy's
lexsort on random and tie-heavy rows; hand-built tie, signed-zero and inf
cases; s = 1 keeps all positions; the window is always kept.
"""

import math

import numpy as np

from .budget import budget


def select(scores_row, L: int, s_num: int, s_den: int, window: int) -> np.ndarray:
    """Ascending kept positions of one (sequence, KV head).

    scores_row: float32 scores indexed by position (at least L entries).
    """
    L = int(L)
    n = budget(L, s_num, s_den, window)
    newest = min(window, L)
    n_top = n - newest
    vals = [float(scores_row[j]) for j in range(L - newest)]
    if any(math.isnan(v) for v in vals):
        raise ValueError("NaN score")
    # Python compares -0.0 == 0.0, so the key treats them as equal.
    order = sorted(range(L - newest), key=lambda j: (-vals[j], j))
    kept = sorted(order[:n_top]) + list(range(L - newest, L))
    return np.asarray(kept, dtype=np.int64)
