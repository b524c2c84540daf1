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

Host arithmetic on measured or printed times only; nothing here runs on the
device.
"""


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
