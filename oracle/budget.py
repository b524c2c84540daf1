"""Selection budget: how many KV positions a draft step may read.

[explainer], Jargon, "Sparse attention budget": the budget is a fraction s
of the cached positions (s = 0.05 by default), made of the newest positions
plus the ones the verifier attended to most.

Readings where the pages are silent:
* the fraction is the exact ratio s_num/s_den, and the count is the ceiling
  of s*L (the pages give no rounding; the ceiling keeps at least the stated
  fraction);
* the newest window W counts inside the budget, and the budget never drops
  below the window (or below L when L < W);
* the budget never exceeds L.

Pins: n-1 < s*L <= n checked with exact rationals over a grid of L and s;
monotone in L; window floor; s = 1 keeps everything; tiny-config value
(L = 512, s = 0.05, W = 16) is 26 with 16 newest.
"""


def budget(L: int, s_num: int, s_den: int, window: int) -> int:
    """Number of positions kept for a context of L committed positions."""
    if L < 0 or s_den <= 0 or s_num < 0 or s_num > s_den or window < 0:
        raise ValueError("invalid budget arguments")
    newest = min(window, L)
    frac = -((-s_num * L) // s_den)  # ceil(s_num * L / s_den), exact integers
    return min(L, max(newest, frac))
