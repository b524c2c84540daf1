"""KV-aware AIMD admission of rollout requests (host-side).

[explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
mean?", Jargon "AIMD scheduler": admit one more request while GPU KV memory
has room, halve the limit under pressure; and the paragraph on the one
remaining cost: verification needs the whole KV cache, so sparse drafting
does not shrink memory. [digest] (section on dense verification needing the
complete cache): GPU KV utilisation measures resident pressure, the restore
backlog records the unmet demand of paused requests; low utilisation raises
the concurrency limit additively, high utilisation or a large backlog backs
it off multiplicatively; paused requests keep their tokens and proposal
state and finish under the same frozen rollout snapshot. [news],
Interpretation: a permanently low limit avoids thrashing but gives up
batching when memory is free.

Readings (the pages give the rule, not its constants):
* the limit caps the requests in flight (admitted and not finished, resident
  or paused); it moves once per control step: +1 when utilisation is below
  `low`, x 0.5 (floored, not below `min_limit`) when utilisation is above
  `high` or the restore backlog exceeds `backlog_limit` pages, unchanged in
  between;
* residency is separate from the limit: when the resident requests' pages
  outgrow the GPU the most recently admitted ones are paused (their pages
  leave the GPU); paused requests resume, oldest pause first, as soon as
  their pages fit, before any new request is admitted; a new request is
  admitted only while the requests in flight are below the limit;
* a paused request object is kept as it is: the scheduler never touches its
  state (tokens, pending token, proposal state).

Host code only: the device work of a round is the library's calls; this
decides which requests take part in the next round.
"""

from collections import deque
from dataclasses import dataclass, field


@dataclass
class Request:
    rid: int
    pages: int = 0            # KV pages the request holds (or needs back when paused)
    state: dict = field(default_factory=dict)  # tokens, pending token, proposal state: never touched here


class AIMDAdmission:
    def __init__(self, max_limit: int, min_limit: int = 1, initial_limit: int = None, low: float = 0.75,
                 high: float = 0.90, backlog_limit: int = None, increase: int = 1, decrease: float = 0.5,
                 adaptive: bool = True):
        if not (0.0 <= low <= high <= 1.0) or min_limit < 1 or max_limit < min_limit:
            raise ValueError("invalid AIMD parameters")
        self.max_limit, self.min_limit = int(max_limit), int(min_limit)
        self.limit = int(initial_limit if initial_limit is not None else min_limit)
        self.low, self.high = float(low), float(high)
        self.backlog_limit = None if backlog_limit is None else int(backlog_limit)  # None: no backlog trigger
        self.increase, self.decrease = int(increase), float(decrease)
        self.adaptive = bool(adaptive)  # False: a fixed limit (the comparison policy)
        self.waiting = deque()   # never admitted
        self.active = []          # resident, admission order
        self.paused = deque()     # in flight, pages off the GPU, pause order (oldest first)

    def in_flight(self) -> int:
        return len(self.active) + len(self.paused)

    def backlog(self) -> int:
        return sum(r.pages for r in self.paused)

    def control(self, utilisation: float, backlog_pages: int) -> int:
        """One AIMD step on the measured GPU KV utilisation (0..1) and restore backlog (pages)."""
        if not self.adaptive:
            return self.limit
        if utilisation > self.high or (self.backlog_limit is not None and backlog_pages > self.backlog_limit):
            self.limit = max(self.min_limit, int(self.limit * self.decrease))
        elif utilisation < self.low:
            self.limit = min(self.max_limit, self.limit + self.increase)
        return self.limit

    def submit(self, req: Request):
        self.waiting.append(req)

    def schedule(self, capacity_pages: int):
        """Fit the resident set into capacity_pages (pause the newest), resume paused requests that
        fit (oldest first), then admit new requests while in flight < limit.
        Returns (paused_now, resumed_now, admitted_now)."""
        paused_now, resumed_now, admitted_now = [], [], []
        used = sum(r.pages for r in self.active)
        while used > capacity_pages and len(self.active) > 1:
            r = self.active.pop()
            used -= r.pages
            self.paused.append(r)
            paused_now.append(r)
        while self.paused and used + self.paused[0].pages <= capacity_pages:
            r = self.paused.popleft()
            used += r.pages
            self.active.append(r)
            resumed_now.append(r)
        if not self.paused:
            while self.in_flight() < self.limit and self.waiting and used + self.waiting[0].pages <= capacity_pages:
                r = self.waiting.popleft()
                used += r.pages
                self.active.append(r)
                admitted_now.append(r)
        return paused_now, resumed_now, admitted_now

    def finish(self, req: Request):
        self.active.remove(req)


def simulate(lengths, tokens_per_round, capacity_pages: int, limit: int, adaptive: bool = True, page: int = 16,
             aimd_kwargs=None, max_rounds: int = 1000000):
    """Rollout of requests with the given response lengths on a GPU holding capacity_pages KV pages.

    Every resident request grows by tokens_per_round(rid, round) tokens a round until it reaches its
    length. adaptive: AIMD limit starting at 1 and capped at `limit`, steered each round by the
    utilisation and the backlog; otherwise a fixed limit of `limit` requests in flight. Pages moved =
    pages of every pause plus every resume. Returns {"rounds", "tokens", "pages_moved",
    "pages_moved_per_1k_tokens", "mean_resident"}."""
    reqs = [Request(i) for i in range(len(lengths))]
    done = [0] * len(reqs)
    kw = {"backlog_limit": capacity_pages // 8}
    kw.update(aimd_kwargs or {})
    sch = AIMDAdmission(max_limit=limit, initial_limit=(None if adaptive else limit), adaptive=adaptive, **kw)
    for r in reqs:
        sch.submit(r)
    moved = tokens = resident_sum = rnd = 0
    while rnd < max_rounds and (sch.waiting or sch.active or sch.paused):
        used = sum(r.pages for r in sch.active)
        sch.control(used / capacity_pages, sch.backlog())
        paused, resumed, _ = sch.schedule(capacity_pages)
        moved += sum(r.pages for r in paused) + sum(r.pages for r in resumed)
        resident_sum += len(sch.active)
        for r in list(sch.active):
            add = min(int(tokens_per_round(r.rid, rnd)), int(lengths[r.rid]) - done[r.rid])
            done[r.rid] += add
            tokens += add
            r.pages = -(-done[r.rid] // page)
            if done[r.rid] >= lengths[r.rid]:
                sch.finish(r)
                r.pages = 0
        rnd += 1
    return {"rounds": rnd, "tokens": tokens, "pages_moved": moved,
            "pages_moved_per_1k_tokens": 1000.0 * moved / max(tokens, 1),
            "mean_resident": resident_sum / max(rnd, 1)}
