"""Round accounting: the state the next round starts from.

[explainer], Jargon, "Block efficiency (tau)": the mean number of tokens
one draft-and-verify round outputs; the illustration counts accepted
drafts plus the one corrected token. [listing], Table 7 caption: a fully
accepted round outputs k + 1 tokens.

After a round the pending token and the accepted drafts are committed to
the cache and the last output token becomes the new pending token, so the
next round starts from L + n_out committed positions (reading; the pages
do not give positions).

commit() is that step for one sequence as the next round needs it: the new
committed length L' = L + n_out, the new pending token (the last token the
round output: the correction, or the bonus after a fully accepted round),
the lengths the next round's draft steps attend up to (L' + j, j = 1..k) and
the next verification's cache length (L' + k + 1). Positions at and beyond
L' hold rows of rejected drafts; nothing reads them before the next round
writes them again (the rollback is implicit).

Pins: the expected n_out over the uniforms equals
sum_{i=0..k} prod_{m<i} alpha_m with alpha_m = sum_x min(p_m, q_m),
integrated exactly on tiny vocabularies; commit after identical draft and
target rows advances by k + 1 with the bonus token pending, after a first
mismatch at draft i by i + 1 with the correction pending (the golden
fixtures of the sampling tests).
"""

import numpy as np


def commit(L: int, n_out: int, tokens, k: int):
    """(L', pending token, [L' + j for j = 1..k], L' + k + 1) after a round that output n_out tokens."""
    n_out = int(n_out)
    assert 1 <= n_out <= k + 1
    L1 = int(L) + n_out
    pending = int(np.asarray(tokens)[n_out - 1])
    return L1, pending, [L1 + j for j in range(1, k + 1)], L1 + k + 1
