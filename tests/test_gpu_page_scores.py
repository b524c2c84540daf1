"""GPU parity of the page-score form: s3r_verify_attn_pages (output rows and lse
bit-identical to s3r_verify_attn, page scores against the oracle's sums of its
position scores) and s3r_select_pages (bit-exact against the oracle's whole-page
rule on the same page-score array), one call at a time and through the round
driver. Bars: 2e-2 of the largest page score of each (sequence, KV head) for
bfloat16, 1e-5 absolute for float32; selection bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch, make_round_inputs
from tests.gpu_util import rel_err_rows, run_verify, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("f32 D=64 (generic)", 1, {}, None),
    ("bf16 D=64 (generic)", 1, {"D": 64, "dtype": "bf16", "Hq": 8, "Hkv": 2, "B": 2}, ("uniform", 300, 600)),
    ("qwen3-1.7b 14 rows", 2, {"B": 4}, None),
    ("qwen3-8b 28 rows", 3, {"B": 3}, None),
    ("k=2 12 rows", 5, {"B": 2, "k": 2}, ("uniform", 900, 3000)),
    ("k=8 36 rows (queries in LDS)", 5, {"B": 2, "k": 8}, ("uniform", 900, 3000)),
    ("k=15 64 rows", 3, {"B": 2, "k": 15}, ("uniform", 100, 2100)),
    ("24K, 7 splits", 5, {"B": 2}, None),
    ("24K k=2, 7 splits", 5, {"B": 2, "k": 2}, None),
    ("24K k=4, 7 splits", 5, {"B": 2, "k": 4}, None),
    ("24K k=8, 7 splits (queries in LDS)", 5, {"B": 2, "k": 8}, None),
    ("62K-66K, 16 splits", 3, {"B": 2}, ("uniform", 62000, 66000)),
]


def _page_case(cfg, batch, t):
    ms = int(batch.seq_len.max())
    o1, l1, _ = run_verify(cfg, batch, t)
    o2, l2, pg = s3r.verify_attn_pages(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), ms)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)  # the same rows, bit for bit
    pg = pg.cpu().numpy()
    worst = 0.0
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        _, _, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                 float(batch.scale))
        ref = oracle.page_scores(rs, S)
        got = pg[b, :, :ref.shape[1]]
        if cfg.dtype == "f32":
            err = float(np.abs(got - ref).max())
            assert err <= 1e-5, (b, err)
        else:
            err = float((np.abs(got - ref).max(axis=1) / ref.max(axis=1)).max())
            assert err <= 2e-2, (b, err)
        np.testing.assert_allclose(got.sum(axis=1), cfg.G * (cfg.k + 1), rtol=1e-3)
        worst = max(worst, err)
    print(f"page scores worst error {worst:.3g}", flush=True)
    return pg


@pytest.mark.parametrize("name,cid,ov,lengths", CASES, ids=[c[0] for c in CASES])
def test_verify_page_scores_match_oracle(name, cid, ov, lengths):
    if lengths is not None:
        ov = {**ov, "lengths": lengths}
    cfg = get_config(cid, **ov)
    print(f"[pages] {name}: B={cfg.B} k={cfg.k} G={cfg.G}", flush=True)
    batch = make_batch(cfg, parts=("kv", "q"))
    _page_case(cfg, batch, to_dev(batch))


def test_verify_page_scores_ragged_short_contexts():
    L = [1, 2, 15, 16, 17, 33, 63, 64, 65, 1000]
    cfg = get_config(3, B=len(L))
    batch = make_batch(cfg, lengths=np.array(L, np.int32), parts=("kv", "q"))
    _page_case(cfg, batch, to_dev(batch))


@pytest.mark.parametrize("all_heads", [False, True])
@pytest.mark.parametrize("cid,ov", [(3, {"B": 12}), (5, {"B": 4}), (2, {"B": 16, "lengths": ("uniform", 20, 3000)})])
def test_select_pages_matches_oracle_on_verify_page_scores(cid, ov, all_heads):
    cfg = get_config(cid, **ov)
    batch = make_batch(cfg, parts=("kv", "q"))
    t = to_dev(batch)
    ms = int(batch.seq_len.max())
    _, _, pg = s3r.verify_attn_pages(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), ms)
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    idx, n_sel = s3r.select_pages(pg, t["ctx_len"], int(batch.ctx_len.max()), cfg.s_num, cfg.s_den, cfg.window,
                                  all_heads=all_heads, order=order)
    torch.cuda.synchronize()
    pg, idx, n_sel = pg.cpu().numpy(), idx.cpu().numpy(), n_sel.cpu().numpy()
    assert np.array_equal(order.cpu().numpy(), np.argsort(-batch.ctx_len.astype(np.int64), kind="stable"))
    for b in range(cfg.B):
        L = int(batch.ctx_len[b])
        refs = oracle.select_by_page_scores(pg[b], L, cfg.s_num, cfg.s_den, cfg.window, all_heads)
        for h in range(cfg.Hkv):
            assert n_sel[b] == len(refs[h]) and np.array_equal(idx[b, h, :n_sel[b]], refs[h]), (b, h)


@pytest.mark.parametrize("cid,B,lo,hi,R,all_heads", [(3, 3, 4000, 5000, 3, False), (2, 3, 300, 700, 3, True),
                                                     (1, 2, 480, 512, 3, False)])
def test_rounds_with_page_scores_match_oracle_loop(cid, B, lo, hi, R, all_heads):
    from self_sparse_speculative_amd.driver import RoundDriver
    from tests.gpu_util import to_dev_storage
    cfg = get_config(cid, B=B)
    k = cfg.k
    L0 = np.random.default_rng(19).integers(lo, hi + 1, size=B).astype(np.int64)
    b = make_batch(cfg, lengths=L0 + (R - 1) * (k + 1), parts=("kv", "scores"))
    t = to_dev(b)
    max_len = int(L0.max()) + R * (k + 1)
    npg = (max_len + 15) // 16
    drv = RoundDriver(t["kv"], torch.from_numpy(L0.astype(np.int32)).cuda(), t["scores"][:, :, :npg].contiguous(),
                      k=k, Hq=cfg.Hq, V=cfg.V, s_num=cfg.s_num, s_den=cfg.s_den, window=cfg.window,
                      scale=float(b.scale), temperature=float(b.temperature), max_len=max_len,
                      select_all_heads=all_heads, page_scores=True)
    bt, scale, T = b.block_table, float(b.scale), b.temperature
    kp, vp = b.k_pages.copy(), b.v_pages.copy()
    L = L0.copy()
    bf16 = cfg.dtype == "bf16"
    for r in range(R):
        print(f"[page rounds] cfg{cid} round {r} L={L.tolist()}", flush=True)
        ri = make_round_inputs(cfg, r, B=B)
        pg_in = drv.scores.cpu().numpy()
        drv.set_inputs(to_dev_storage(ri.q_draft), to_dev_storage(ri.k_draft), to_dev_storage(ri.v_draft),
                       to_dev_storage(ri.q_verify), to_dev_storage(ri.k_block), to_dev_storage(ri.v_block),
                       torch.from_numpy(ri.zt).cuda(), torch.from_numpy(ri.zd).cuda(), torch.from_numpy(ri.d).cuda(),
                       torch.from_numpy(ri.u).cuda())
        drv.step()
        torch.cuda.synchronize()
        idx, nsel = drv.idx.cpu().numpy(), drv.n_sel.cpu().numpy()
        dout, vout, pg_out = drv.draft_out.cpu().numpy(), drv.ver_out.cpu().numpy(), drv.scores.cpu().numpy()
        toks, nout = drv.tokens.cpu().numpy(), drv.n_out.cpu().numpy()
        for s in range(B):
            Ls = int(L[s])
            refs = oracle.select_by_page_scores(pg_in[s], Ls, cfg.s_num, cfg.s_den, cfg.window, all_heads)
            for h in range(cfg.Hkv):
                assert nsel[s] == len(refs[h]) and np.array_equal(idx[s, h, :nsel[s]], refs[h]), (r, s, h)
            for j in range(1, k + 1):
                oracle.kv_append(kp, vp, bt[s], Ls + j - 1, ri.k_draft[j - 1, s][None], ri.v_draft[j - 1, s][None])
                o, _ = oracle.sparse_decode(ri.q_draft[j - 1, s], kp, vp, bt[s], idx[s], int(nsel[s]), Ls, Ls + j, scale)
                assert (rel_err_rows(dout[j - 1, s], o) <= 2e-2) if bf16 else (np.abs(dout[j - 1, s] - o).max() <= 1e-5)
            oracle.kv_append(kp, vp, bt[s], Ls, ri.k_block[s], ri.v_block[s])
            S = Ls + k + 1
            vo, _, vs = oracle.verify(ri.q_verify[s], kp, vp, bt[s], S, k, scale)
            ref = oracle.page_scores(vs, S)
            got = pg_out[s, :, :ref.shape[1]]
            if bf16:
                assert rel_err_rows(vout[s], vo) <= 2e-2
                assert (np.abs(got - ref).max(axis=1) / ref.max(axis=1)).max() <= 2e-2
            else:
                assert np.abs(vout[s] - vo).max() <= 1e-5 and np.abs(got - ref).max() <= 1e-5
            rt, rn, _ = oracle.spec_sample(ri.zt[s], ri.zd[s], ri.d[s], ri.u[s], T)
            assert int(nout[s]) == rn and np.array_equal(toks[s], rt)
            L[s] = Ls + rn
