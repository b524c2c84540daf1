"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Bars: selection indices / counts and sampled tokens / decisions bit-exact;
attention max-abs 1e-5 for float32 inputs; 2e-2 relative per output vector
for bfloat16 K/V with float32 accumulation; scores 1e-5 abs (float32) and
2e-2 of the per-(sequence, KV head) maximum (bfloat16).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch
from tests.gpu_util import (nsel_cap, rel_err_rows, run_draft_steps, run_sample, run_select, run_verify,
                            to_dev)

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2

_cache = {}


def _batch(key, cid, parts=("kv", "q", "scores", "logits"), **ov):
    if key not in _cache:
        cfg = get_config(cid, **ov)
        print(f"[gen] {key}: {cfg.name} B={cfg.B} parts={parts}", flush=True)
        b = make_batch(cfg, parts=parts)
        _cache[key] = (cfg, b, to_dev(b))
    return _cache[key]


def _oracle_idx(cfg, batch, scores, b, kv):
    return oracle.select(scores[b, kv], int(batch.ctx_len[b]), cfg.s_num, cfg.s_den, cfg.window)


def _check_select(cfg, batch, scores_np, idx, n_sel, units):
    idx = idx.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    for b, kv in units:
        ref = _oracle_idx(cfg, batch, scores_np, b, kv)
        assert n_sel[b] == len(ref), (b, kv)
        assert np.array_equal(idx[b, kv, :n_sel[b]], ref), (b, kv)


# ----------------------------------------------------------------- select

@pytest.mark.parametrize("key,cid,ov", [
    ("c1", 1, {}),
    ("c2s", 2, {"B": 16}),
    ("c3s", 3, {"B": 12}),
    ("c5s", 5, {"B": 6}),
])
def test_select_matches_oracle(key, cid, ov):
    cfg, batch, t = _batch(key + "-sel", cid, parts=("scores",), **ov)
    idx, n_sel = run_select(cfg, batch, t)
    torch.cuda.synchronize()
    units = [(b, kv) for b in range(cfg.B) for kv in range(cfg.Hkv)]
    _check_select(cfg, batch, batch.scores, idx, n_sel, units)


@pytest.mark.parametrize("long_row", [40000, 24000])
def test_select_edge_cases(long_row):
    # long rows take the sampled-threshold path; its fallback (the streaming
    # passes) on the 3000-key tie bucket
    cfg = get_config(2, B=7, Hkv=2)
    rng = np.random.default_rng(7)
    L = np.array([1, 5, 64, 65, 200, long_row, 1000], dtype=np.int32)  # window 64
    stride = int(L.max())
    sc = np.zeros((7, 2, stride), np.float32)
    sc[0] = 0.0
    sc[1, :, :5] = [-0.0, 0.0, -0.0, 0.0, 1.0]
    sc[2, 0, :64] = rng.integers(0, 3, 64)
    sc[3, 0, :65] = np.inf
    sc[3, 1, :65] = -np.inf
    sc[4, :, :200] = rng.integers(0, 4, (2, 200)).astype(np.float32)  # heavy ties
    sc[4, 1, 7] = -0.0
    sc[5, :, :long_row] = rng.random((2, long_row)).astype(np.float32)
    sc[5, 0, 100:200] = 0.5  # ties in the long row
    sc[6, :, :1000] = (rng.integers(0, 2, (2, 1000)) * 2 - 1) * np.float32(1e-38)  # denormal-range signs
    sc[5, 1, :3000] = 0.25  # a tie bucket larger than the compaction capacity
    dev = torch.device("cuda")
    for s_num, s_den in [(1, 20), (1, 2), (1, 1), (0, 1), (7, 9)]:
        nc = s3r.budget(stride, s_num, s_den, cfg.window)
        idx, n_sel = s3r.select(torch.from_numpy(sc).to(dev), torch.from_numpy(L).to(dev), stride, s_num, s_den,
                                cfg.window, nsel_cap=max(1, nc))
        torch.cuda.synchronize()
        idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
        for b in range(7):
            for kv in range(2):
                ref = oracle.select(sc[b, kv], int(L[b]), s_num, s_den, cfg.window)
                assert n_sel[b] == len(ref)
                assert np.array_equal(idx[b, kv, :n_sel[b]], ref), (s_num, s_den, b, kv)


def test_select_sampled_path_falls_back_exactly():
    """Rows built against the sampled-threshold path: the sample sees only large keys (too few
    kept keys above its threshold), only small keys (more than the list holds), or nothing but
    ties. Each row must fall back and still match the oracle."""
    cfg = get_config(5, B=4, Hkv=2)
    L = 24576
    ncand = L - cfg.window
    nrun = min(ncand // 128, 160)  # the sample the kernel takes: runs of 16 every `stride` positions
    stride_s = ncand // nrun
    j = np.arange(L)
    sampled = (j < nrun * stride_s) & (j % stride_s < 16)
    rng = np.random.default_rng(12)
    sc = np.empty((4, 2, L), np.float32)
    sc[0] = np.where(sampled, 10.0 + rng.random(L), rng.random(L))   # the sample overstates the threshold
    sc[1] = np.where(sampled, rng.random(L), 10.0 + rng.random(L))   # the sample understates it
    sc[2] = 0.5                                                       # every key tied
    sc[3] = rng.random((2, L))                                        # the plain case
    ctx = np.full(4, L, dtype=np.int32)
    for s_num, s_den in [(1, 20), (1, 50), (1, 10), (1, 5)]:
        cap = s3r.budget(L, s_num, s_den, cfg.window)
        idx, n_sel = s3r.select(torch.from_numpy(sc).cuda(), torch.from_numpy(ctx).cuda(), L, s_num, s_den,
                                cfg.window, nsel_cap=cap)
        torch.cuda.synchronize()
        idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
        for b in range(4):
            for kv in range(2):
                ref = oracle.select(sc[b, kv], L, s_num, s_den, cfg.window)
                assert n_sel[b] == len(ref) and np.array_equal(idx[b, kv, :n_sel[b]], ref), (s_num, b, kv)


def test_select_rows_around_the_sampled_path_limits():
    """The sampled path holds 16-bit positions and a list sized for the largest row: a row of
    70000 positions (beyond it), one of exactly 65536 candidates (its last position is 65535),
    shorter rows, and a budget of 1/5 whose list would outgrow the largest capacity. Every kept
    set must match the oracle."""
    window = 64
    L = np.array([70000, 65536 + window, 65000, 24576, 3000], np.int32)
    max_l = int(L.max())
    rng = np.random.default_rng(21)
    sc = rng.random((len(L), 2, max_l), dtype=np.float32)
    for s_num, s_den in [(1, 20), (1, 10), (1, 5)]:
        cap = s3r.budget(max_l, s_num, s_den, window)
        idx, n_sel = s3r.select(torch.from_numpy(sc).cuda(), torch.from_numpy(L).cuda(), max_l, s_num, s_den,
                                window, nsel_cap=cap)
        torch.cuda.synchronize()
        idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
        for b in range(len(L)):
            for kv in range(2):
                ref = oracle.select(sc[b, kv], int(L[b]), s_num, s_den, window)
                assert n_sel[b] == len(ref) and np.array_equal(idx[b, kv, :n_sel[b]], ref), (s_num, s_den, b, kv)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_randomised_rows_and_budgets(seed):
    """Rows of 2000-30000 positions at budgets from 1/50 to 1/3, with score shapes that stress the
    sampled threshold: uniform, heavy-tailed, a few distinct values (ties), rising with position,
    a sawtooth of the sample's period, and spikes. Every kept set matches the oracle."""
    rng = np.random.default_rng(100 + seed)
    B, Hkv, window = 12, 2, 64
    L = rng.integers(2000, 30000, size=B).astype(np.int32)
    M = int(L.max())
    sc = np.empty((B, Hkv, M), np.float32)
    j = np.arange(M)
    shapes = [
        lambda: rng.random(M),
        lambda: rng.standard_cauchy(M),
        lambda: rng.integers(0, 5, M) / 4.0,
        lambda: j / M + 1e-3 * rng.random(M),
        lambda: (j % 153) / 153.0,
        lambda: np.where(rng.random(M) < 0.01, 100.0, 1e-3 * rng.random(M)),
    ]
    for b in range(B):
        for kv in range(Hkv):
            sc[b, kv] = shapes[(b * Hkv + kv) % len(shapes)]().astype(np.float32)
    budgets = [(1, 50), (1, 20), (1, 10), (1, 5), (1, 3)]
    for s_num, s_den in (budgets[seed], budgets[(seed + 2) % 5], budgets[(seed + 4) % 5]):
        cap = s3r.budget(M, s_num, s_den, window)
        idx, n_sel = s3r.select(torch.from_numpy(sc).cuda(), torch.from_numpy(L).cuda(), M, s_num, s_den, window,
                                nsel_cap=cap)
        torch.cuda.synchronize()
        idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
        for b in range(B):
            for kv in range(Hkv):
                ref = oracle.select(sc[b, kv], int(L[b]), s_num, s_den, window)
                assert n_sel[b] == len(ref) and np.array_equal(idx[b, kv, :n_sel[b]], ref), (s_num, s_den, b, kv)


# ----------------------------------------------------------------- draft

def _draft_case(cfg, batch, t, steps, seqs, tol, absolute):
    idx, n_sel = run_select(cfg, batch, t)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel)
    torch.cuda.synchronize()
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    worst = 0.0
    for j in steps:
        o, lse = outs[j - 1][0].cpu().numpy(), outs[j - 1][1].cpu().numpy()
        for b in seqs:
            L = int(batch.ctx_len[b])
            ro, rl = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                          idx_np[b], int(ns[b]), L, L + j, float(batch.scale))
            if absolute:
                err = float(np.abs(o[b] - ro).max())
            else:
                err = rel_err_rows(o[b], ro)
            worst = max(worst, err)
            assert err <= tol, (j, b, err)
            assert np.abs(lse[b] - rl).max() <= (1e-5 if absolute else 2e-3), (j, b)
    print(f"draft worst error {worst:.3g}")


def test_draft_c1_f32():
    cfg, batch, t = _batch("c1", 1)
    _draft_case(cfg, batch, t, range(1, cfg.k + 1), range(cfg.B), TOL_F32, True)


@pytest.mark.parametrize("key,cid,ov", [("c2d", 2, {"B": 6}), ("c3d", 3, {"B": 5})])
def test_draft_bf16(key, cid, ov):
    cfg, batch, t = _batch(key, cid, **ov)
    _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_BF16, False)


@pytest.mark.parametrize("G", [1, 3, 6, 16])
def test_draft_bf16_group_sizes(G):
    # head groups the vector path does not cover; lists of up to 3000 positions span two splits
    cfg, batch, t = _batch(f"c2g{G}", 2, B=3, Hq=2 * G, Hkv=2, lengths=("uniform", 3000, 30000), s_num=1, s_den=10)
    _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_BF16, False)


@pytest.mark.parametrize("B", [1, 5, 256, 1025, 3000])
def test_length_order_is_the_stable_descending_sort(B):
    rng = np.random.default_rng(B)
    for L in (rng.integers(1, 40, size=B), rng.integers(1, 1 << 30, size=B), np.full(B, 7)):
        L = L.astype(np.int32)
        got = s3r.length_order(torch.from_numpy(L).cuda()).cpu().numpy()
        assert np.array_equal(got, np.argsort(-L.astype(np.int64), kind="stable")), B


def test_select_writes_the_dispatch_order():
    # s3r_select forms the longest-first order in its own launch; s3r_select_grouped through the
    # order kernel; neither changes the kept sets
    rng = np.random.default_rng(8)
    B, Hkv, M = 600, 2, 3000
    L = rng.choice([100, 777, 2048, 2999, 3000], B).astype(np.int32)  # many ties
    sc = torch.from_numpy(rng.random((B, Hkv, M), dtype=np.float32)).cuda()
    ctx = torch.from_numpy(L).cuda()
    want = np.argsort(-L.astype(np.int64), kind="stable")
    idx0, n0 = s3r.select(sc, ctx, M, 1, 20, 64)
    order = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    idx1, n1 = s3r.select(sc, ctx, M, 1, 20, 64, order=order)
    assert np.array_equal(order.cpu().numpy(), want)
    assert torch.equal(n0, n1) and all(torch.equal(idx0[b, :, :n0[b]], idx1[b, :, :n0[b]]) for b in range(B))
    order.fill_(-1)
    g0, gn0 = s3r.select_grouped(sc, ctx, M, 1, 20, 64, unit=16)
    g1, gn1 = s3r.select_grouped(sc, ctx, M, 1, 20, 64, unit=16, order=order)
    assert np.array_equal(order.cpu().numpy(), want)
    assert torch.equal(gn0, gn1) and all(torch.equal(g0[b, :, :gn0[b]], g1[b, :, :gn0[b]]) for b in range(B))


@pytest.mark.parametrize("key,cid,ov", [("c1", 1, {}), ("c3d", 3, {"B": 5}), ("c2d", 2, {"B": 6})])
def test_draft_dispatch_order_changes_no_result(key, cid, ov):
    # the vector path (c1) and the MFMA path, with the longest-first order and a shuffled one:
    # every output and lse bit-identical to the launch without an order
    cfg, batch, t = _batch(key, cid, **ov)
    idx, n_sel = run_select(cfg, batch, t)
    plain = run_draft_steps(cfg, batch, t, idx, n_sel)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(cfg.B).astype(np.int32)).cuda()
    for order in (s3r.length_order(t["ctx_len"]), perm):
        got = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
        torch.cuda.synchronize()
        for (o0, l0), (o1, l1) in zip(plain, got):
            assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("key,cid,ov", [("c1", 1, {}), ("c2d", 2, {"B": 6})])
def test_draft_nothing_attended(key, cid, ov):
    # no kept position and no position of this round: output 0, lse = -inf (both kernel paths)
    cfg, batch, t = _batch(key, cid, **ov)
    idx = torch.zeros((cfg.B, cfg.Hkv, 4), dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((cfg.B,), dtype=torch.int32, device="cuda")
    out = torch.full((cfg.B, cfg.Hq, cfg.D), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((cfg.B, cfg.Hq), 7.0, dtype=torch.float32, device="cuda")
    s3r.sparse_decode_attn(t["q_draft"][0], t["kv"], idx, n_sel, t["ctx_len"], t["ctx_len"], float(batch.scale), 4,
                           out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out == 0).all() and torch.isneginf(lse).all()
    ro, rl = oracle.sparse_decode(batch.q_draft[0, 0], batch.k_pages, batch.v_pages, batch.block_table[0],
                                  np.zeros((cfg.Hkv, 4), np.int32), 0, int(batch.ctx_len[0]), int(batch.ctx_len[0]),
                                  float(batch.scale))
    assert (ro == 0).all() and np.isneginf(rl).all()


def test_draft_full_budget_is_dense():
    cfg, batch, t = _batch("c2full", 2, B=3, lengths=("uniform", 300, 700), s_num=1, s_den=1)
    idx, n_sel = run_select(cfg, batch, t)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel)
    torch.cuda.synchronize()
    for j in (1, cfg.k):
        o = outs[j - 1][0].cpu().numpy()
        for b in range(cfg.B):
            L = int(batch.ctx_len[b])
            ro, _ = oracle.dense_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                        L + j, float(batch.scale))
            assert rel_err_rows(o[b], ro) <= TOL_BF16


# ----------------------------------------------------------------- verify

def _verify_case(cfg, batch, t, seqs, absolute):
    out, lse, sc = run_verify(cfg, batch, t)
    torch.cuda.synchronize()
    out, lse, sc = out.cpu().numpy(), lse.cpu().numpy(), sc.cpu().numpy()
    worst_o = worst_s = 0.0
    for b in seqs:
        S = int(batch.seq_len[b])
        ro, rl, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                   float(batch.scale))
        if absolute:
            eo = float(np.abs(out[b] - ro).max())
            es = float(np.abs(sc[b, :, :S] - rs).max())
            assert eo <= TOL_F32 and es <= TOL_F32, (b, eo, es)
            assert np.abs(lse[b] - rl).max() <= TOL_F32
        else:
            eo = rel_err_rows(out[b], ro)
            es = float((np.abs(sc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max())
            assert eo <= TOL_BF16 and es <= TOL_BF16, (b, eo, es)
            assert np.abs(lse[b] - rl).max() <= 2e-3
        np.testing.assert_allclose(sc[b, :, :S].sum(axis=1), cfg.G * (cfg.k + 1), rtol=1e-3)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    print(f"verify worst out error {worst_o:.3g}, scores error {worst_s:.3g}")


def test_verify_c1_f32():
    cfg, batch, t = _batch("c1", 1)
    _verify_case(cfg, batch, t, range(cfg.B), True)


def test_verify_k0_f32_is_one_decoding_step():
    cfg, batch, t = _batch("c1k0", 1, parts=("kv", "q"), k=0)
    _verify_case(cfg, batch, t, range(cfg.B), True)


@pytest.mark.parametrize("key,cid,ov", [
    ("c2v", 2, {"B": 4}),                       # G=2, 14 rows (one row tile)
    ("c3v", 3, {"B": 3}),                       # G=4, 28 rows (two row tiles)
    ("c5k2", 5, {"B": 2, "k": 2, "lengths": ("uniform", 900, 3000)}),   # 12 rows
    ("c5k8", 5, {"B": 2, "k": 8, "lengths": ("uniform", 900, 3000)}),   # 36 rows (three row tiles)
    ("c3k15", 3, {"B": 2, "k": 15, "lengths": ("uniform", 100, 2100)}),  # 64 rows (four row tiles)
    ("c5k0", 5, {"B": 3, "k": 0, "lengths": ("uniform", 900, 9000)}),    # k = 0: one dense decoding step
    # long contexts: 16-19 splits per (sequence, KV head)
    ("c3long", 3, {"B": 2, "lengths": ("uniform", 62000, 66000)}),
    ("c3xlong", 3, {"B": 1, "lengths": ("uniform", 75000, 76000)}),
    ("c3k15long", 3, {"B": 1, "k": 15, "lengths": ("uniform", 40000, 41000)}),
])
def test_verify_bf16(key, cid, ov):
    cfg, batch, t = _batch(key, cid, parts=("kv", "q"), **ov)
    _verify_case(cfg, batch, t, range(cfg.B), False)


def test_verify_generic_bf16_d64_and_f32_d128():
    for key, ov in [("g64", {"D": 64, "dtype": "bf16"}), ("g128", {"D": 128, "dtype": "f32"})]:
        cfg, batch, t = _batch(key, 1, parts=("kv", "q", "scores"), B=2, Hq=8, Hkv=2,
                               lengths=("uniform", 300, 600), **ov)
        _verify_case(cfg, batch, t, range(cfg.B), ov["dtype"] == "f32")
        _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_F32 if ov["dtype"] == "f32" else TOL_BF16,
                    ov["dtype"] == "f32")


def test_ragged_short_contexts():
    L = [1, 2, 15, 16, 17, 33, 63, 64, 65, 1000]
    cfg = get_config(3, B=len(L))
    batch = make_batch(cfg, lengths=np.array(L, np.int32))
    t = to_dev(batch)
    _verify_case(cfg, batch, t, range(cfg.B), False)
    _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_BF16, False)
    idx, n_sel = run_select(cfg, batch, t)
    torch.cuda.synchronize()
    _check_select(cfg, batch, batch.scores, idx, n_sel, [(b, kv) for b in range(cfg.B) for kv in range(cfg.Hkv)])


def test_split_and_selection_path_boundaries():
    # verification lengths S = L + 7 at and around the split size (4096: one split or two;
    # 8192 and 8193: two even splits or three; 12288), and selection rows of 2047, 2048 and
    # 2049 candidates (L - 64), where the sampled-threshold path begins
    L = [4088, 4089, 4090, 8185, 8186, 12281, 2111, 2112, 2113]
    cfg = get_config(3, B=len(L))
    batch = make_batch(cfg, lengths=np.array(L, np.int32))
    t = to_dev(batch)
    print(f"[boundaries] S = {list(batch.seq_len)}", flush=True)
    _verify_case(cfg, batch, t, range(cfg.B), False)
    _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_BF16, False)
    idx, n_sel = run_select(cfg, batch, t)
    torch.cuda.synchronize()
    _check_select(cfg, batch, batch.scores, idx, n_sel, [(b, kv) for b in range(cfg.B) for kv in range(cfg.Hkv)])
    # the page-score form on the same lengths: its rows equal the position form's, bit for bit
    ms = int(batch.seq_len.max())
    o1, l1, _ = run_verify(cfg, batch, t)
    o2, l2, pg = s3r.verify_attn_pages(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), ms)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    pg = pg.cpu().numpy()
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        _, _, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                 float(batch.scale))
        ref = oracle.page_scores(rs, S)
        err = float((np.abs(pg[b, :, :ref.shape[1]] - ref).max(axis=1) / ref.max(axis=1)).max())
        assert err <= TOL_BF16, (b, err)


# ----------------------------------------------------------------- sampling

def _check_sample(cfg, batch, toks, nout, acc, T, seqs):
    toks, nout, acc = toks.cpu().numpy(), nout.cpu().numpy(), acc.cpu().numpy()
    for b in seqs:
        rt, rn, ra = oracle.spec_sample(batch.zt[b], batch.zd[b], batch.d[b], batch.u[b], T)
        assert nout[b] == rn, b
        assert np.array_equal(toks[b], rt), (b, toks[b], rt)
        assert np.array_equal(acc[b], ra), b


@pytest.mark.parametrize("key,cid,ov", [("c1", 1, {}), ("c2smp", 2, {"B": 64}), ("c5smp", 5, {"B": 32, "noise_std": 0.6})])
def test_spec_sample_bit_exact(key, cid, ov):
    parts = ("kv", "q", "scores", "logits") if key == "c1" else ("logits",)
    cfg, batch, t = _batch(key, cid, parts=parts, **ov)
    toks, nout, acc = run_sample(cfg, batch, t)
    torch.cuda.synchronize()
    _check_sample(cfg, batch, toks, nout, acc, batch.temperature, range(cfg.B))
    print(f"mean tokens per round {nout.float().mean().item():.3f}")


@pytest.mark.parametrize("T", [0.7, 1.6])
def test_spec_sample_other_temperatures(T):
    # the temperature divides every logit before the softmax, on both the target and the draft rows
    cfg, batch, t = _batch("c2smp", 2, parts=("logits",), B=64)
    toks, nout, acc = run_sample(cfg, batch, t, temperature=T)
    torch.cuda.synchronize()
    _check_sample(cfg, batch, toks, nout, acc, np.float32(T), range(cfg.B))


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_spec_sample_without_drafts(T):
    # k = 0: plain decoding, one token per sequence drawn from p_0 with u[0] (greedy: its argmax)
    cfg, batch, t = _batch("c2smp", 2, parts=("logits",), B=64)
    zt0 = t["zt"][:, :1].contiguous()
    u0 = t["u"][:, :1].contiguous()
    empty_zd = torch.empty((cfg.B, 0, zt0.shape[2]), dtype=torch.float32, device="cuda")
    empty_d = torch.empty((cfg.B, 0), dtype=torch.int32, device="cuda")
    toks, nout, acc = s3r.spec_sample(zt0, empty_zd, empty_d, u0, T)
    torch.cuda.synchronize()
    assert acc is None
    toks, nout = toks.cpu().numpy(), nout.cpu().numpy()
    for b in range(cfg.B):
        rt, rn, _ = oracle.spec_sample(batch.zt[b, :1], batch.zd[b, :0], batch.d[b, :0], batch.u[b, :1], np.float32(T))
        assert nout[b] == rn == 1 and np.array_equal(toks[b], rt), (b, toks[b], rt)


def test_spec_sample_greedy_and_identical():
    cfg, batch, t = _batch("c2smp", 2, parts=("logits",), B=64)
    toks, nout, acc = run_sample(cfg, batch, t, temperature=0.0)
    torch.cuda.synchronize()
    _check_sample(cfg, batch, toks, nout, acc, np.float32(0.0), range(cfg.B))
    zt = t["zt"]
    toks, nout, acc = s3r.spec_sample(zt, zt[:, :cfg.k].contiguous(), t["d"], t["u"], 1.0)
    torch.cuda.synchronize()
    assert (nout.cpu().numpy() == cfg.k + 1).all()
    assert (acc.cpu().numpy() == 1).all()


def test_spec_sample_greedy_with_tied_maxima():
    # integer logits: every row's maximum is taken by several tokens, so the greedy decisions
    # and outputs rest on the first-index rule alone; drafts are the first argmax, a later tied
    # token or a random one
    rng = np.random.default_rng(31)
    B, k, V = 48, 6, 4099
    zt = rng.integers(0, 3, (B, k + 1, V)).astype(np.float32)
    zd = rng.integers(0, 3, (B, k, V)).astype(np.float32)
    d = np.empty((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            tied = np.flatnonzero(zt[b, i] == zt[b, i].max())
            d[b, i] = (tied[0], tied[-1], rng.integers(0, V))[rng.integers(0, 3) if b % 4 else 0]
    u = rng.random((B, k + 1), dtype=np.float32)
    dev = torch.device("cuda")
    toks, nout, acc = s3r.spec_sample(torch.from_numpy(zt).to(dev), torch.from_numpy(zd).to(dev),
                                      torch.from_numpy(d).to(dev), torch.from_numpy(u).to(dev), 0.0)
    torch.cuda.synchronize()
    toks, nout = toks.cpu().numpy(), nout.cpu().numpy()
    full = 0
    for b in range(B):
        rt, rn, _ = oracle.spec_sample(zt[b], zd[b], d[b], u[b], np.float32(0.0))
        assert nout[b] == rn and np.array_equal(toks[b], rt), (b, toks[b], rt)
        full += int(rn == k + 1)
    assert full > 0 and int(nout.min()) == 1  # both whole acceptance and an early rejection occur


def test_spec_sample_chi_square_on_gpu():
    from scipy import stats
    V, k, n = 16, 3, 400_000
    rng = np.random.default_rng(5)
    zt1 = (1.5 * rng.standard_normal((k + 1, V))).astype(np.float32)
    zd1 = (zt1[:k] + rng.standard_normal((k, V))).astype(np.float32)
    P = [oracle.softmax_t(zt1[i], 1.0) for i in range(k + 1)]
    Q = [oracle.softmax_t(zd1[i], 1.0) for i in range(k)]
    d = np.stack([np.minimum(np.searchsorted(np.cumsum(Q[i]), rng.random(n) * np.cumsum(Q[i])[-1], side="right"), V - 1)
                  for i in range(k)], axis=1).astype(np.int32)
    u = ((rng.integers(0, 1 << 32, size=(n, k + 1), dtype=np.uint64) >> np.uint64(8)).astype(np.float32)
         * np.float32(2.0 ** -24))
    dev = torch.device("cuda")
    step = 50_000  # batch per call (the ABI takes at most 65535 sequences)
    zt = torch.from_numpy(np.broadcast_to(zt1, (step, k + 1, V)).copy()).to(dev)
    zd = torch.from_numpy(np.broadcast_to(zd1, (step, k, V)).copy()).to(dev)
    toks, nout = [], []
    for c in range(0, n, step):
        tk, no, _ = s3r.spec_sample(zt, zd, torch.from_numpy(d[c:c + step]).to(dev),
                                    torch.from_numpy(u[c:c + step]).to(dev), 1.0)
        toks.append(tk.cpu().numpy())
        nout.append(no.cpu().numpy())
    toks, nout = np.concatenate(toks), np.concatenate(nout)
    for i in range(k + 1):
        sel = nout > i
        counts = np.bincount(toks[sel, i], minlength=V)
        pv = stats.chisquare(counts, P[i] * sel.sum()).pvalue
        assert pv > 1e-3, (i, pv)


# ----------------------------------------------------------------- rollout config

@pytest.mark.parametrize("layer", [0, 27])
def test_rollout_config_round(layer):
    """Config 4 (Qwen3-1.7B shapes, 1024-token prompt prefix page-aliased across the 8 responses
    of a prompt, lognormal response lengths): two prompts x 8 responses, first and last of the 28
    layers, every step of the round against the oracle."""
    cfg = get_config(4, B=16)
    batch = make_batch(cfg, layer=layer)
    shared = 1024 // cfg.page
    for g in range(2):
        rows = batch.block_table[8 * g:8 * g + 8, :shared]
        assert (rows == rows[0]).all()  # the prefix pages really are shared
    assert not np.array_equal(batch.block_table[0, :shared], batch.block_table[8, :shared])
    t = to_dev(batch)
    idx, n_sel = run_select(cfg, batch, t)
    torch.cuda.synchronize()
    _check_select(cfg, batch, batch.scores, idx, n_sel, [(b, kv) for b in range(cfg.B) for kv in range(cfg.Hkv)])
    _draft_case(cfg, batch, t, [1, cfg.k], range(cfg.B), TOL_BF16, False)
    _verify_case(cfg, batch, t, range(cfg.B), False)
    toks, nout, acc = run_sample(cfg, batch, t)
    torch.cuda.synchronize()
    _check_sample(cfg, batch, toks, nout, acc, batch.temperature, range(cfg.B))


# ----------------------------------------------------------------- robustness

def test_large_batch_of_short_contexts():
    """1500 sequences of 20-400 positions (Qwen3-1.7B head shapes, a 4096-token vocabulary):
    grids with many small workgroups; every step on a sample of sequences, sampling on all,
    against the oracle."""
    cfg, batch, t = _batch("c2bigB", 2, B=1500, lengths=("uniform", 20, 400), V=4096)
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    idx, n_sel = run_select(cfg, batch, t, order=order)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), np.argsort(-batch.ctx_len.astype(np.int64), kind="stable"))
    rng = np.random.default_rng(3)
    seqs = sorted(set(int(x) for x in rng.integers(cfg.B, size=12)) | {0, cfg.B - 1})
    _check_select(cfg, batch, batch.scores, idx, n_sel, [(b, kv) for b in seqs for kv in range(cfg.Hkv)])
    outs = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
    torch.cuda.synchronize()
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    for j in (1, cfg.k):
        o = outs[j - 1][0].cpu().numpy()
        for b in seqs:
            L = int(batch.ctx_len[b])
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         idx_np[b], int(ns[b]), L, L + j, float(batch.scale))
            assert rel_err_rows(o[b], ro) <= TOL_BF16, (j, b)
    _verify_case(cfg, batch, t, seqs, False)
    toks, nout, acc = run_sample(cfg, batch, t)
    torch.cuda.synchronize()
    _check_sample(cfg, batch, toks, nout, acc, batch.temperature, range(cfg.B))



def test_determinism_and_poisoned_workspace():
    cfg, batch, t = _batch("c2v", 2, parts=("kv", "q"), B=4)
    results = []
    for trial in range(2):
        ws = s3r.Workspace()
        for name, nb in [("verify", s3r.verify_workspace_bytes(cfg.B, cfg.k, cfg.Hq, cfg.Hkv, cfg.D, 1,
                                                               int(batch.seq_len.max())))]:
            ws.get(name, nb).fill_(0xFF)  # NaN patterns everywhere
        out, lse, sc = s3r.verify_attn(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale),
                                       int(batch.seq_len.max()), ws=ws)
        torch.cuda.synchronize()
        results.append((out.cpu().numpy(), lse.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(results[0][0], results[1][0]) and np.array_equal(results[0][1], results[1][1])
    for b in range(cfg.B):
        S = int(batch.seq_len[b])  # entries at and beyond seq_len are not written
        assert np.array_equal(results[0][2][b, :, :S], results[1][2][b, :, :S])
        assert np.isfinite(results[0][2][b, :, :S]).all()
    assert np.isfinite(results[0][0]).all()


@pytest.mark.parametrize("key,ov", [("c2v", {"B": 4}), ("c3long", {"B": 2, "lengths": ("uniform", 62000, 66000)})])
def test_verify_without_scores_matches(key, ov):
    # the output rows and lse do not depend on whether scores are requested
    cfg, batch, t = _batch(key, 2 if key == "c2v" else 3, parts=("kv", "q"), **ov)
    o1, l1, _ = run_verify(cfg, batch, t)
    o2, l2, s2 = run_verify(cfg, batch, t, want_scores=False)
    torch.cuda.synchronize()
    assert s2 is None
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("key,cid,ov", [("c2v", 2, {"B": 4}), ("c5k8", 5, {"B": 2, "k": 8, "lengths": ("uniform", 900, 3000)}),
                                        ("g64", 1, {"D": 64, "dtype": "bf16", "B": 2, "Hq": 8, "Hkv": 2,
                                                    "lengths": ("uniform", 300, 600)})])
def test_verify_deferred_scores_on_a_second_stream(key, cid, ov):
    # output rows now, scores later on another stream: bit-identical to the one-call form
    cfg, batch, t = _batch(key, cid, parts=("kv", "q", "scores") if key == "g64" else ("kv", "q"), **ov)
    ms = int(batch.seq_len.max())
    o1, l1, s1 = run_verify(cfg, batch, t)
    ws = s3r.Workspace()
    o2, l2 = s3r.verify_attn_deferred(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), ms, ws=ws)
    done = torch.cuda.Event()
    done.record()
    side = torch.cuda.Stream()
    side.wait_event(done)
    with torch.cuda.stream(side):
        s2 = s3r.verify_scores(t["kv"], t["seq_len"], cfg.B, cfg.k, cfg.Hq, cfg.D, ms, ws=ws,
                               stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        assert torch.equal(s1[b, :, :S], s2[b, :, :S]), b


def test_invalid_arguments_raise():
    cfg, batch, t = _batch("c1", 1)
    with pytest.raises(s3r.S3RError):
        s3r.select(t["scores"], t["ctx_len"], int(batch.ctx_len.max()), 1, 0, 16)
    with pytest.raises(s3r.S3RError):
        s3r.verify_attn(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), 3)


# ----------------------------------------------------------------- full size, sampled

@pytest.mark.slow
def test_full_size_24k_round_sampled():
    """The benchmark's launch configuration (Qwen3-8B shapes, B=128, 24K context, s=0.05, k=6):
    select on all units is checked on a sample, draft and verify on sampled sequences, sampling
    on every sequence."""
    cfg, batch, t = _batch("c5full", 5)
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")  # as the benchmark: dispatch order from select
    idx, n_sel = run_select(cfg, batch, t, order=order)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
    vout, vlse, vsc = run_verify(cfg, batch, t)
    toks, nout, acc = run_sample(cfg, batch, t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    units = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.Hkv))) for _ in range(24)]
    _check_select(cfg, batch, batch.scores, idx, n_sel, units)
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    for b in [0, 77]:
        L = int(batch.ctx_len[b])
        for j in (1, cfg.k):
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         idx_np[b], int(ns[b]), L, L + j, float(batch.scale))
            assert rel_err_rows(outs[j - 1][0][b].cpu().numpy(), ro) <= TOL_BF16
    vout, vsc = vout.cpu().numpy(), vsc.cpu().numpy()
    for b in [5]:
        S = int(batch.seq_len[b])
        ro, rl, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                   float(batch.scale))
        assert rel_err_rows(vout[b], ro) <= TOL_BF16
        assert (np.abs(vsc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max() <= TOL_BF16
    _check_sample(cfg, batch, toks, nout, acc, batch.temperature, range(cfg.B))
    # the verify scores feed the next selection: bit-exact on the same array
    idx2, n2 = run_select(cfg, batch, t, scores=torch.from_numpy(vsc).cuda())
    torch.cuda.synchronize()
    _check_select(cfg, batch, vsc, idx2, n2, units[:8])


def test_tp2_rank_share_at_24k():
    """One tensor-parallel rank's share of Qwen3-8B at the 24K workload: 16 query heads over 4 KV heads
    (half of 32 / 8), the shape one GPU holds when the heads are split over two; every step of the
    round against the oracle on sampled units, sampling on every sequence."""
    cfg, batch, t = _batch("c5tp2", 5, Hq=16, Hkv=4, B=16)
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    idx, n_sel = run_select(cfg, batch, t, order=order)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
    vout, vlse, vsc = run_verify(cfg, batch, t)
    toks, nout, acc = run_sample(cfg, batch, t)
    torch.cuda.synchronize()
    _check_select(cfg, batch, batch.scores, idx, n_sel, [(b, kv) for b in range(0, cfg.B, 5) for kv in range(cfg.Hkv)])
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    vout, vsc = vout.cpu().numpy(), vsc.cpu().numpy()
    for b in [0, cfg.B - 1]:
        L, S = int(batch.ctx_len[b]), int(batch.seq_len[b])
        for j in (1, cfg.k):
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         idx_np[b], int(ns[b]), L, L + j, float(batch.scale))
            assert rel_err_rows(outs[j - 1][0][b].cpu().numpy(), ro) <= TOL_BF16
        ro, rl, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                   float(batch.scale))
        assert rel_err_rows(vout[b], ro) <= TOL_BF16
        assert (np.abs(vsc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max() <= TOL_BF16
    _check_sample(cfg, batch, toks, nout, acc, batch.temperature, range(cfg.B))
