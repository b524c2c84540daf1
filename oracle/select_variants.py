"""Selection variants: whole pages instead of single positions, and one kept
set per sequence from the scores of all its KV heads.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[explainer], mechanism paragraph: the kept set is described as whole pages,
the recent ones plus those the previous verification weighted most, chosen
again each round. [news], Perspective: adapting the budget and the choice of
context is named as further work.

Readings (the pages name the variants, not their rules):
* all heads: the score of position j for the sequence is the float32 sum of
  the KV heads' scores at j, heads in ascending order; the kept set serves
  every KV head;
* pages (unit 16): page p holds positions [16p, 16p + 16). The newest
  min(window, L) positions are kept as whole pages: from the page f holding
  the oldest of them, f = floor((L - min(window, L)) / 16), every position
  of [16f, L) is kept (wc positions). The candidates are the full pages
  0 .. f-1; a page's score is the float32 sum of its 16 positions' scores in
  slot order. With n = budget(L, s, window) positions, the
  min(f, ceil(max(0, n - wc) / 16)) top candidate pages are kept (score
  descending, ties to the lower page): wc + 16 x that many positions, the
  same for every KV head, at least n unless the whole cache is kept. The
  output is ascending;
* the sums are float32 accumulated in the stated order, since the kernel
  takes its integer decisions on the same sums.

select_by_page_scores takes the page keys as given (the verification's page
scores) instead of forming them from position scores.

Pins: with integer-valued scores (exact sums) the head sum equals an int64
sum and the page choice equals a brute-force sort of int64 page sums; one
KV head at unit 1 is the plain selection; the kept set is whole pages plus
the window, ascending, covers the newest window positions, has the stated
size and at least the position budget; s = 1 keeps all.
"""

import math

import numpy as np

from .budget import budget
from .select import select


def head_sum(scores_rows, L: int) -> np.ndarray:
    """float32 [L]: sum over the KV heads (ascending) of each position's score."""
    acc = np.zeros(int(L), dtype=np.float32)
    for h in range(len(scores_rows)):
        acc = (acc + np.asarray(scores_rows[h][:L], dtype=np.float32)).astype(np.float32)
    return acc


def page_sum(key, L: int, unit: int = 16) -> np.ndarray:
    """float32 [ceil(L / unit)]: each page's sum of its positions' keys, slot order."""
    L = int(L)
    npg = -(-L // unit)
    acc = np.zeros(npg, dtype=np.float32)
    key = np.asarray(key[:L], dtype=np.float32)
    for t in range(unit):
        pages = np.arange(npg)
        pos = pages * unit + t
        ok = pos < L
        acc[ok] = (acc[ok] + key[pos[ok]]).astype(np.float32)
    return acc


def page_plan(L: int, s_num: int, s_den: int, window: int, unit: int = 16):
    """(first window page f, window positions wc, candidate pages kept) for a context of L."""
    L = int(L)
    w = min(int(window), L)
    f = (L - w) // unit
    wc = L - f * unit
    n = budget(L, s_num, s_den, window)
    n_top = min(f, -(-max(0, n - wc) // unit))
    return f, wc, n_top


def select_pages(key, L: int, s_num: int, s_den: int, window: int, unit: int = 16) -> np.ndarray:
    """Ascending kept positions when the older part of the cache is kept in whole pages (one key row)."""
    L = int(L)
    f, _, _ = page_plan(L, s_num, s_den, window, unit)
    return _keep_pages(page_sum(key, f * unit, unit), L, s_num, s_den, window, unit)


def select_by_page_scores(page_rows, L: int, s_num: int, s_den: int, window: int, all_heads: bool,
                          unit: int = 16):
    """Kept positions of every KV head from scores given per page (page p covers positions
    [unit p, unit p + unit)), by the whole-page rule above; with all_heads the page keys are the
    float32 sum of the KV heads' page scores (ascending heads) and one set serves every head."""
    L = int(L)
    Hkv = len(page_rows)
    f, _, _ = page_plan(L, s_num, s_den, window, unit)
    for h in range(Hkv):
        if any(math.isnan(float(v)) for v in np.asarray(page_rows[h][:f])):
            raise ValueError("NaN score")
    keys = [head_sum(page_rows, f)] if all_heads else [np.asarray(page_rows[h][:f], np.float32) for h in range(Hkv)]
    sel = [_keep_pages(k_, L, s_num, s_den, window, unit) for k_ in keys]
    return [sel[0]] * Hkv if all_heads else sel


def _keep_pages(sums, L: int, s_num: int, s_den: int, window: int, unit: int) -> np.ndarray:
    """The whole-page rule on the f candidate pages' keys `sums`: the n_top largest (ties to the
    lower page) plus the window pages, as ascending positions."""
    f, wc, n_top = page_plan(L, s_num, s_den, window, unit)
    vals = [float(v) for v in np.asarray(sums, dtype=np.float32)[:f]]
    order = sorted(range(f), key=lambda p: (-vals[p], p))
    kept = sorted(order[:n_top])
    pos = [j for p in kept for j in range(p * unit, (p + 1) * unit)] + list(range(f * unit, L))
    return np.asarray(pos, dtype=np.int64)


def select_grouped(scores_rows, L: int, s_num: int, s_den: int, window: int, unit: int, all_heads: bool):
    """Kept positions of every KV head of one sequence: a list of Hkv ascending arrays."""
    if unit not in (1, 16):
        raise ValueError("unit must be 1 (positions) or 16 (pages)")
    Hkv = len(scores_rows)
    for h in range(Hkv):
        if any(math.isnan(float(v)) for v in np.asarray(scores_rows[h][:L])):
            raise ValueError("NaN score")
    keys = [head_sum(scores_rows, L)] if all_heads else [np.asarray(scores_rows[h][:L], np.float32)
                                                          for h in range(Hkv)]
    if unit == 1:
        sel = [select(k_, L, s_num, s_den, window) for k_ in keys]
    else:
        sel = [select_pages(k_, L, s_num, s_den, window, unit) for k_ in keys]
    return [sel[0]] * Hkv if all_heads else sel


def grouped_count(L: int, s_num: int, s_den: int, window: int, unit: int) -> int:
    """Number of kept positions of every KV head."""
    if unit == 1:
        return budget(L, s_num, s_den, window)
    _, wc, n_top = page_plan(L, s_num, s_den, window, unit)
    return wc + unit * n_top
