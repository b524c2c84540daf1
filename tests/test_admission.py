"""The host-side AIMD admission stub: the rule on forced utilisation / backlog
traces, pause and resume that keep a request's state, and a rollout
simulation under KV pressure (CPU only)."""

import math

import numpy as np

from self_sparse_speculative_amd.admission import AIMDAdmission, Request, simulate


def test_additive_increase_multiplicative_decrease_on_a_forced_trace():
    a = AIMDAdmission(max_limit=100, min_limit=1, low=0.75, high=0.90, backlog_limit=50)
    trace = [(0.5, 0)] * 5 + [(0.95, 0)] + [(0.5, 0)] * 3 + [(0.8, 0)] + [(0.99, 0)] * 2 + [(0.5, 60), (0.5, 0)]
    got = [a.control(u, bl) for u, bl in trace]
    #          room: +1 each   spike: /2  room again   between  pressure x2  backlog /2  room
    assert got == [2, 3, 4, 5, 6, 3, 4, 5, 6, 6, 3, 1, 1, 2]


def test_limits_are_bounded_and_a_fixed_policy_never_moves():
    a = AIMDAdmission(max_limit=3, min_limit=2, initial_limit=2)
    assert [a.control(0.1, 0) for _ in range(4)] == [3, 3, 3, 3]
    assert [a.control(0.99, 0) for _ in range(3)] == [2, 2, 2]
    f = AIMDAdmission(max_limit=8, initial_limit=8, adaptive=False)
    assert [f.control(u, 0) for u in (0.1, 0.99, 0.5)] == [8, 8, 8]


def test_pause_and_resume_keep_state_and_order():
    a = AIMDAdmission(max_limit=10, initial_limit=4)
    reqs = [Request(i, pages=0, state={"tokens": [i, i + 1], "pending": 100 + i}) for i in range(6)]
    snap = [dict(r.state) for r in reqs]
    for r in reqs:
        a.submit(r)
    _, _, adm = a.schedule(capacity_pages=100)
    assert [r.rid for r in adm] == [0, 1, 2, 3] and a.in_flight() == 4
    for r, p in zip(a.active, (30, 30, 30, 30)):
        r.pages = p  # the requests grew: 120 pages on a 100-page GPU
    paused, resumed, adm = a.schedule(capacity_pages=100)
    assert [r.rid for r in paused] == [3] and not resumed and not adm  # the newest leaves; nothing new while paused
    a.finish(reqs[0])
    paused, resumed, adm = a.schedule(capacity_pages=100)
    # the paused request resumes first, then the freed slot admits the next new one
    assert [r.rid for r in resumed] == [3] and not paused and [r.rid for r in adm] == [4]
    assert all(r.state == s for r, s in zip(reqs, snap)) and reqs[3] is a.active[-2]


def _rollout(n=256, seed=0):
    rng = np.random.default_rng(seed)
    L = np.clip(np.rint(np.exp(math.log(6144) + 0.6 * rng.standard_normal(n))), 1, 16384).astype(int) + 1024
    return L, (lambda rid, rnd: 1 + (rid * 7919 + rnd * 104729) % 6)


def test_rollout_under_kv_pressure():
    L, tau = _rollout()
    cap = 128 * 4000 // 16  # room for 128 requests of 4000 tokens
    fixed = simulate(L, tau, cap, limit=128, adaptive=False)
    aimd = simulate(L, tau, cap, limit=128, adaptive=True)
    low = simulate(L, tau, cap, limit=64, adaptive=False)
    total = int(L.sum())
    # every request finishes: paused requests resume where they stopped
    assert fixed["tokens"] == aimd["tokens"] == low["tokens"] == total
    # AIMD moves far fewer pages than a fixed high limit; a permanently low limit moves none
    # but needs more rounds (less batching)
    assert aimd["pages_moved_per_1k_tokens"] < 0.7 * fixed["pages_moved_per_1k_tokens"]
    assert low["pages_moved"] == 0 and low["rounds"] > aimd["rounds"]
