"""Plain fp64 CPU oracle of the S3R attention-and-sampling step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package. The
product path (the HIP library and its Python binding) never calls it, and
the two share no code: the only module both sides use is ``s3r_inputs``,
which draws random inputs and holds none of the method's arithmetic.

Every function is the plain definition of what one step computes, in
float64, one sequence at a time: no online softmax, no split over the
context, no fused passes. Inputs arrive as float32 or bfloat16 values and
are widened exactly.

Sources (the web pages about the method), cited by title and section:

* [news] "Long-context RL training stops waiting on autoregressive rollouts:
  sparse self-drafting plus full-attention verification lifts throughput
  1.39x" (ai4snews), sections Interpretation and Perspective;
* [listing] "S^3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative
  Decoding" (thelatestinai paper page): Abstract, Table 1, appendix
  Tables 4-7 and their captions;
* [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
  mean?" (learnaivisually): Jargon list, the mechanism paragraphs, the
  draft/verify illustration and "Where it earns its keep";
* [digest] the wispaper research digest (in Chinese), sections on sparse
  drafting with dense verification and on per-position acceptance.

Pins (the tests that tie each function to something other than itself)
are listed in each module's docstring. Every function here is pinned; no
function is "parity unpinned".
"""

from .budget import budget  # noqa: F401
from .select import select  # noqa: F401
from .attention import attend, gather, sparse_decode, verify, dense_decode, page_scores  # noqa: F401
from .sampling import softmax_t, invcdf, spec_decide, spec_sample, decide_margins, spec_margins  # noqa: F401
from .round import commit  # noqa: F401
from .cache import kv_append  # noqa: F401
from .select_variants import grouped_count, select_grouped, select_by_page_scores  # noqa: F401
