"""GPU parity of the multi-round pieces through the C ABI: K/V append and round
commit against the oracle, several rounds in a row against the oracle's own
loop, and one round captured in a HIP graph and replayed against eager rounds.

Bars as for the single-round parity tests: append, commit, selection and
sampling bit-exact; attention within 1e-5 (float32) or 2e-2 relative per
output vector (bfloat16); scores 1e-5 abs / 2e-2 of the row maximum.
"""

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch, make_round_inputs
from self_sparse_speculative_amd.driver import RoundDriver
from tests.gpu_util import rel_err_rows, to_dev, to_dev_storage
from tests.poison import bits, poison_from

pytestmark = pytest.mark.gpu


def _host_pages(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("cid,D", [(1, 64), (3, 128)])
def test_kv_append_matches_oracle(cid, D):
    cfg = get_config(cid, B=5, D=D, lengths=("fixed", 100), k=3)
    b = make_batch(cfg, parts=("kv",))
    t = to_dev(b)
    kv = t["kv"]
    max_pos = int(b.block_table.shape[1]) * 16
    rng = np.random.default_rng(7)
    n = 7
    pos = np.array([0, 13, 60, 95, max_pos - 3], dtype=np.int32)  # page crossings; the last runs off its table
    sd = b.k_pages.dtype
    if sd == np.uint16:
        kr = rng.integers(0, 1 << 16, size=(5, n, cfg.Hkv, D), dtype=np.uint16)
        vr = rng.integers(0, 1 << 16, size=(5, n, cfg.Hkv, D), dtype=np.uint16)
    else:
        kr = rng.standard_normal((5, n, cfg.Hkv, D)).astype(np.float32)
        vr = rng.standard_normal((5, n, cfg.Hkv, D)).astype(np.float32)
    print(f"[append] cfg{cid} D={D} pos={pos.tolist()}", flush=True)
    s3r.kv_append(to_dev_storage(kr), to_dev_storage(vr), kv, torch.from_numpy(pos).cuda(), max_pos)
    torch.cuda.synchronize()
    kp, vp = b.k_pages.copy(), b.v_pages.copy()
    for s in range(5):
        keep = min(n, max_pos - int(pos[s]))  # rows past the table are skipped
        oracle.kv_append(kp, vp, b.block_table[s], int(pos[s]), kr[s, :keep], vr[s, :keep])
    assert np.array_equal(_host_pages(kv.k_pages), kp)
    assert np.array_equal(_host_pages(kv.v_pages), vp)


def test_commit_matches_oracle():
    k, B = 6, 300
    rng = np.random.default_rng(8)
    L = rng.integers(1, 30000, size=B).astype(np.int32)
    n_out = rng.integers(1, k + 2, size=B).astype(np.int32)
    n_out[17] = 0  # not a round's output: left as it is
    tokens = rng.integers(0, 151936, size=(B, k + 1)).astype(np.int32)
    ctx = torch.from_numpy(L).cuda()
    pending = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    cur = torch.full((k, B), -5, dtype=torch.int32, device="cuda")
    seq = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    ver = torch.full((1,), 11, dtype=torch.int64, device="cuda")
    s3r.commit(torch.from_numpy(n_out).cuda(), torch.from_numpy(tokens).cuda(), ctx, pending=pending, cur_len=cur,
               seq_len=seq, verified=ver)
    torch.cuda.synchronize()
    ctx, pending, cur, seq = ctx.cpu().numpy(), pending.cpu().numpy(), cur.cpu().numpy(), seq.cpu().numpy()
    total = 11
    for b in range(B):
        if n_out[b] == 0:
            assert ctx[b] == L[b] and pending[b] == -5 and seq[b] == -5 and (cur[:, b] == -5).all()
            continue
        L1, pend, cl, sl = oracle.commit(int(L[b]), int(n_out[b]), tokens[b], k)
        assert ctx[b] == L1 and pending[b] == pend and seq[b] == sl and cur[:, b].tolist() == cl
        total += int(n_out[b])
    assert int(ver.item()) == total


def _setup(cfg, L0, R, unit=1, all_heads=False):
    """The cache with room for R rounds, first-round scores, and the driver over it."""
    k = cfg.k
    b = make_batch(cfg, lengths=L0 + (R - 1) * (k + 1), parts=("kv", "scores"))
    t = to_dev(b)
    ctx = torch.from_numpy(L0.astype(np.int32)).cuda()
    max_len = int(L0.max()) + R * (k + 1)
    assert int(b.seq_len.max()) == max_len
    drv = RoundDriver(t["kv"], ctx, t["scores"], k=k, Hq=cfg.Hq, V=cfg.V, s_num=cfg.s_num, s_den=cfg.s_den,
                      window=cfg.window, scale=float(b.scale), temperature=float(b.temperature), max_len=max_len,
                      select_unit=unit, select_all_heads=all_heads)
    return b, drv


def _set_round(drv, ri):
    drv.set_inputs(to_dev_storage(ri.q_draft), to_dev_storage(ri.k_draft), to_dev_storage(ri.v_draft),
                   to_dev_storage(ri.q_verify), to_dev_storage(ri.k_block), to_dev_storage(ri.v_block),
                   torch.from_numpy(ri.zt).cuda(), torch.from_numpy(ri.zd).cuda(), torch.from_numpy(ri.d).cuda(),
                   torch.from_numpy(ri.u).cuda())


@pytest.mark.parametrize("cid,B,lo,hi,R,unit,all_heads,poison", [
    (1, 2, 480, 512, 4, 1, False, False), (2, 3, 300, 700, 3, 1, False, False),
    (2, 3, 300, 700, 3, 16, True, False), (1, 2, 480, 512, 3, 16, False, False),
    # every position the run has not written yet holds NaN / Inf patterns (a pooled cache)
    (3, 3, 4000, 5000, 3, 1, False, True), (1, 2, 480, 512, 3, 1, False, True)])
def test_rounds_match_oracle_loop(cid, B, lo, hi, R, unit, all_heads, poison):
    cfg = get_config(cid, B=B)
    L0 = np.random.default_rng(9).integers(lo, hi + 1, size=B).astype(np.int64)
    b, drv = _setup(cfg, L0, R, unit, all_heads)
    if poison:
        # up to the end of each sequence's own pages (the rest of a shorter row maps to page 0)
        poison_from(b.k_pages, b.v_pages, b.block_table, L0, (b.seq_len.astype(np.int64) + 15) // 16 * 16)
        drv.kv.k_pages.copy_(to_dev_storage(b.k_pages))
        drv.kv.v_pages.copy_(to_dev_storage(b.v_pages))
    k, bt, scale, T = cfg.k, b.block_table, float(b.scale), b.temperature
    bf16 = cfg.dtype == "bf16"
    kp, vp = b.k_pages.copy(), b.v_pages.copy()
    L = L0.copy()
    total = 0
    for r in range(R):
        print(f"[rounds] cfg{cid} round {r} L={L.tolist()}", flush=True)
        ri = make_round_inputs(cfg, r, B=B)
        sc_in = drv.scores.cpu().numpy()
        _set_round(drv, ri)
        drv.step()
        torch.cuda.synchronize()
        idx, nsel = drv.idx.cpu().numpy(), drv.n_sel.cpu().numpy()
        dout, vout = drv.draft_out.cpu().numpy(), drv.ver_out.cpu().numpy()
        sc_out, toks, nout = drv.scores.cpu().numpy(), drv.tokens.cpu().numpy(), drv.n_out.cpu().numpy()
        ctx, pend = drv.ctx_len.cpu().numpy(), drv.pending.cpu().numpy()
        cur, seq = drv.cur_len.cpu().numpy(), drv.seq_len.cpu().numpy()
        for s in range(B):
            Ls = int(L[s])
            refs = oracle.select_grouped(sc_in[s], Ls, cfg.s_num, cfg.s_den, cfg.window, unit, all_heads)
            for h in range(cfg.Hkv):
                assert nsel[s] == len(refs[h]) and np.array_equal(idx[s, h, :nsel[s]], refs[h])
            for j in range(1, k + 1):
                oracle.kv_append(kp, vp, bt[s], Ls + j - 1, ri.k_draft[j - 1, s][None], ri.v_draft[j - 1, s][None])
                o, _ = oracle.sparse_decode(ri.q_draft[j - 1, s], kp, vp, bt[s], idx[s], int(nsel[s]), Ls, Ls + j,
                                            scale)
                if bf16:
                    assert rel_err_rows(dout[j - 1, s], o) <= 2e-2
                else:
                    assert np.abs(dout[j - 1, s] - o).max() <= 1e-5
            oracle.kv_append(kp, vp, bt[s], Ls, ri.k_block[s], ri.v_block[s])
            S = Ls + k + 1
            vo, _, vs = oracle.verify(ri.q_verify[s], kp, vp, bt[s], S, k, scale)
            if bf16:
                assert rel_err_rows(vout[s], vo) <= 2e-2
                assert (np.abs(sc_out[s, :, :S] - vs).max(axis=1) / vs.max(axis=1)).max() <= 2e-2
            else:
                assert np.abs(vout[s] - vo).max() <= 1e-5
                assert np.abs(sc_out[s, :, :S] - vs).max() <= 1e-5
            rt, rn, _ = oracle.spec_sample(ri.zt[s], ri.zd[s], ri.d[s], ri.u[s], T)
            assert int(nout[s]) == rn and np.array_equal(toks[s], rt)
            L1, pending, cl, sl = oracle.commit(Ls, rn, rt, k)
            assert ctx[s] == L1 and pend[s] == pending and cur[:, s].tolist() == cl and seq[s] == sl
            L[s] = L1
            total += rn
        assert np.array_equal(bits(_host_pages(drv.kv.k_pages)), bits(kp))
        assert np.array_equal(bits(_host_pages(drv.kv.v_pages)), bits(vp))
    assert int(drv.verified.item()) == total


def test_graph_replays_match_eager_rounds():
    cfg = get_config(3, B=2)
    R = 3
    L0 = np.array([4300, 5000], dtype=np.int64)  # two verify splits, ragged
    b_e, eager = _setup(cfg, L0, R)
    b_g, graph = _setup(cfg, L0, R)
    print("[graph] capture", flush=True)
    graph.capture()
    names = ("idx", "n_sel", "draft_out", "ver_out", "ver_lse", "scores", "tokens", "n_out", "ctx_len", "pending",
             "cur_len", "seq_len", "verified")
    for r in range(R):
        print(f"[graph] round {r}", flush=True)
        ri = make_round_inputs(cfg, r, B=2)
        _set_round(eager, ri)
        eager.step()
        torch.cuda.synchronize()
        _set_round(graph, ri)
        graph.replay()
        torch.cuda.synchronize()
        for nm in names:
            a, g = getattr(eager, nm), getattr(graph, nm)
            if nm == "idx":  # entries past n_sel are not written
                n = eager.n_sel.cpu().numpy()
                a, g = a.cpu().numpy(), g.cpu().numpy()
                assert all(np.array_equal(a[s, :, :n[s]], g[s, :, :n[s]]) for s in range(2)), (r, nm)
            else:
                assert torch.equal(a, g), (r, nm)
        assert torch.equal(eager.kv.k_pages, graph.kv.k_pages) and torch.equal(eager.kv.v_pages, graph.kv.v_pages)
