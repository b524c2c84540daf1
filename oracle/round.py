"""Round accounting: verified tokens and the next committed lengths.

[explainer], Jargon, "Block efficiency (tau)": the mean number of tokens
one draft-and-verify round outputs; the illustration counts accepted
drafts plus the one corrected token. [listing], Table 7 caption: a fully
accepted round outputs k + 1 tokens.

After a round the pending token and the accepted drafts are committed to
the cache and the last output token becomes the new pending token, so the
next round starts from L + n_out committed positions (reading; the pages
do not give positions).

Pins: the expected n_out over the uniforms equals
sum_{i=0..k} prod_{m<i} alpha_m with alpha_m = sum_x min(p_m, q_m),
integrated exactly on tiny vocabularies.
"""

import numpy as np


def verified_tokens(n_out) -> int:
    return int(np.asarray(n_out, dtype=np.int64).sum())


def next_lengths(L, n_out) -> np.ndarray:
    return np.asarray(L, dtype=np.int64) + np.asarray(n_out, dtype=np.int64)
