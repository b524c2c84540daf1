"""GPU parity of the selection variants (whole pages; one kept set per sequence
from all KV heads) through the C ABI: kept positions and counts bit-exact
against the oracle on the same score arrays, and the draft step over
page-granular selections within the attention tolerances."""

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch
from tests.gpu_util import rel_err_rows, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = [(16, False), (16, True), (1, True)]


def _check(cfg, scores_np, ctx_np, unit, all_heads, s_num=None, s_den=None, window=None):
    s_num = cfg.s_num if s_num is None else s_num
    s_den = cfg.s_den if s_den is None else s_den
    window = cfg.window if window is None else window
    B, Hkv, _ = scores_np.shape
    max_ctx = int(ctx_np.max())
    order = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    idx, n_sel = s3r.select_grouped(torch.from_numpy(scores_np).cuda(), torch.from_numpy(ctx_np).cuda(), max_ctx,
                                    s_num, s_den, window, unit=unit, all_heads=all_heads, order=order)
    torch.cuda.synchronize()
    idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
    # the draft steps' dispatch order, written in the same launch: longest first, ties by index
    assert np.array_equal(order.cpu().numpy(), np.argsort(-ctx_np.astype(np.int64), kind="stable"))
    for b in range(B):
        L = int(ctx_np[b])
        ref = oracle.select_grouped(scores_np[b], L, s_num, s_den, window, unit, all_heads)
        assert n_sel[b] == len(ref[0]) == oracle.grouped_count(L, s_num, s_den, window, unit), (b, L)
        for h in range(Hkv):
            assert np.array_equal(idx[b, h, :n_sel[b]], ref[h]), (b, h, L, unit, all_heads)
    return idx, n_sel


@pytest.mark.parametrize("unit,all_heads", VARIANTS)
@pytest.mark.parametrize("cid,ov", [(1, {}), (3, {"B": 6, "lengths": ("uniform", 3000, 9000)}),
                                    (5, {"B": 2})])
def test_variants_match_oracle_on_generator_scores(cid, ov, unit, all_heads):
    cfg = get_config(cid, **ov)
    b = make_batch(cfg, parts=("scores",))
    print(f"[variants] cfg{cid} B={cfg.B} unit={unit} all_heads={all_heads}", flush=True)
    _check(cfg, b.scores, b.ctx_len, unit, all_heads)


@pytest.mark.parametrize("unit,all_heads", VARIANTS)
def test_variants_tie_heavy_and_edge_lengths(unit, all_heads):
    cfg = get_config(1, B=9, Hkv=3)
    rng = np.random.default_rng(11)
    ctx = np.array([1, 7, 15, 16, 17, 40, 17, 511, 2000], dtype=np.int32)  # a tie: the order keeps index order
    sc = rng.integers(0, 4, size=(9, 3, 2000)).astype(np.float32)  # equal page sums everywhere
    sc[0, :, :5] = -0.0
    for (sn, sd, W) in ((1, 20, 16), (1, 5, 0), (1, 1, 16), (1, 3, 40)):
        _check(cfg, sc, ctx, unit, all_heads, sn, sd, W)


@pytest.mark.parametrize("unit,all_heads", VARIANTS)
def test_variants_on_long_rows(unit, all_heads):
    # 33K-50K positions: more than 2048 candidate pages, so the page keys and the summed
    # position keys both take the sampled-threshold path, at two budgets
    cfg = get_config(3, B=3, Hkv=2)
    rng = np.random.default_rng(12)
    ctx = np.array([33000, 41234, 50000], dtype=np.int32)
    sc = rng.random((3, 2, 50000), dtype=np.float32)
    for (sn, sd) in ((1, 20), (1, 5)):
        _check(cfg, sc, ctx, unit, all_heads, sn, sd, 64)


def test_draft_over_page_selection():
    cfg = get_config(3, B=4, lengths=("uniform", 2000, 6000))
    b = make_batch(cfg, parts=("kv", "q", "scores"))
    t = to_dev(b)
    max_ctx = int(b.ctx_len.max())
    idx, n_sel = s3r.select_grouped(t["scores"], t["ctx_len"], max_ctx, cfg.s_num, cfg.s_den, cfg.window, unit=16)
    max_attend = s3r.select_grouped_capacity(max_ctx, cfg.s_num, cfg.s_den, cfg.window, 16) + cfg.k
    outs = []
    for j in (1, cfg.k):
        o, _ = s3r.sparse_decode_attn(t["q_draft"][j - 1], t["kv"], idx, n_sel, t["ctx_len"], t["ctx_len"] + j,
                                      float(b.scale), max_attend)
        outs.append((j, o))
    torch.cuda.synchronize()
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    for j, o in outs:
        o = o.cpu().numpy()
        for s in range(cfg.B):
            L = int(b.ctx_len[s])
            ro, _ = oracle.sparse_decode(b.q_draft[j - 1, s], b.k_pages, b.v_pages, b.block_table[s], idx_np[s],
                                         int(ns[s]), L, L + j, float(b.scale))
            assert rel_err_rows(o[s], ro) <= 2e-2
