"""Writing new K/V rows into the paged cache (the multi-round driver).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[news], Interpretation: verification recomputes the proposed block against
the complete historical KV cache, so the block's K/V rows replace whatever
the draft steps wrote at those positions. [explainer], mechanism paragraph:
each draft step reads this round's own positions besides the kept ones, so
a draft token's K/V row is in the cache before the step that reads it.

Layout (reading, the same as the attention functions): position j of
sequence b lives at slot j % page of physical page block_table[b][j // page],
all KV heads of the position side by side ([pages][Hkv][page][D]).

kv_append writes rows t = 0..n-1 of one sequence at positions pos + t, one
position at a time, every KV head. Nothing else in the cache changes.

Pins: every written position read back through an independent gather of the
layout's definition; every slot not written keeps its old bytes; writes
into pages shared by several block tables are seen through each of them;
appending a sequence's rows one at a time equals appending them at once.
"""

import numpy as np


def kv_append(k_pages: np.ndarray, v_pages: np.ndarray, bt_row, pos: int, k_rows: np.ndarray,
              v_rows: np.ndarray) -> None:
    """Write k_rows[t], v_rows[t] ([n][Hkv][D], the cache's dtype) at positions pos + t, in place."""
    P = k_pages.shape[2]
    bt_row = np.asarray(bt_row)
    n = k_rows.shape[0]
    for t in range(n):
        j = int(pos) + t
        page = int(bt_row[j // P])
        k_pages[page, :, j % P, :] = k_rows[t]
        v_pages[page, :, j % P, :] = v_rows[t]
