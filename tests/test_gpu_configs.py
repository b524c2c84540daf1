"""GPU parity at the launch shapes the sweep and rollout measurements time.

* verification at every draft length k = 1..8 (the sweep's 2, 4, 6, 8 and the
  adaptive draft length's rounds) on the fixed 24576-position context (7
  splits per (sequence, KV head); 8 to 36 query rows per KV head: one, two
  and three MFMA row tiles, the last with its queries in LDS);
* selection and draft steps at the sweep's largest budget (s = 1/5, k = 8:
  4916 kept positions, three draft splits merged);
* speculative sampling on every sequence of every workload (configs 1-4, the
  sweep's draft-noise and draft-length points, and the adaptive draft
  length's noise rising along the draft), bit-exact, with the
  oracle's decision margins reported per workload and required to exceed
  1e-12 (the float64 agreement of the kernel's exponential and summation
  order with the oracle's);
* the 28-layer rollout workload as the benchmark builds it (K/V pages drawn
  on the device), full batch of 256, one middle layer: selection, draft steps
  and verification for sequences of the first, a middle and the last prompt
  group, against the oracle on the pages copied back.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch
from s3r_inputs.configs import DEGRADING_NOISE
from tests.gpu_util import nsel_cap, rel_err_rows, run_draft_steps, run_select, run_verify, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
MARGIN_FLOOR = 1e-12


def _check_verify(cfg, batch, out, lse, sc, seqs):
    for b in seqs:
        S = int(batch.seq_len[b])
        ro, rl, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                   float(batch.scale))
        eo = rel_err_rows(out[b], ro)
        es = float((np.abs(sc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max())
        assert eo <= TOL_BF16 and es <= TOL_BF16, (b, eo, es)
        assert np.abs(lse[b] - rl).max() <= 2e-3
        print(f"  seq {b}: out {eo:.3g}, scores {es:.3g}", flush=True)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8])
def test_verify_sweep_draft_lengths_at_24k(k):
    cfg = get_config(5, B=2, k=k)
    print(f"[sweep verify] k={k} R={(k + 1) * cfg.G} B=2 L=24576", flush=True)
    batch = make_batch(cfg, parts=("kv", "q"))
    t = to_dev(batch)
    out, lse, sc = run_verify(cfg, batch, t)
    torch.cuda.synchronize()
    _check_verify(cfg, batch, out.cpu().numpy(), lse.cpu().numpy(), sc.cpu().numpy(), range(cfg.B))


def test_select_and_draft_at_the_largest_sweep_budget():
    cfg = get_config(5, B=2, k=8, s_num=1, s_den=5)
    print("[sweep draft] s=1/5 k=8 B=2 L=24576", flush=True)
    batch = make_batch(cfg, parts=("kv", "q", "scores"))
    t = to_dev(batch)
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    idx, n_sel = run_select(cfg, batch, t, order=order)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
    torch.cuda.synchronize()
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    for b in range(cfg.B):
        L = int(batch.ctx_len[b])
        for kv in range(cfg.Hkv):
            ref = oracle.select(batch.scores[b, kv], L, cfg.s_num, cfg.s_den, cfg.window)
            assert ns[b] == len(ref) and np.array_equal(idx_np[b, kv, :ns[b]], ref), (b, kv)
        for j in (1, cfg.k):
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         idx_np[b], int(ns[b]), L, L + j, float(batch.scale))
            assert rel_err_rows(outs[j - 1][0][b].cpu().numpy(), ro) <= TOL_BF16, (b, j)


SAMPLING_WORKLOADS = [
    ("config 1 (tiny, V=512)", 1, {}),
    ("config 2 (Qwen3-1.7B layer, B=64)", 2, {}),
    ("config 3 (Qwen3-8B layer, B=128)", 3, {}),
    ("config 4 (rollout, B=256)", 4, {}),
    ("config 5 sigma=0.1", 5, {"noise_std": 0.1}),
    ("config 5 sigma=0.3", 5, {}),
    ("config 5 sigma=0.6", 5, {"noise_std": 0.6}),
    ("config 5 k=1", 5, {"k": 1}),
    ("config 5 k=2", 5, {"k": 2}),
    ("config 5 k=4", 5, {"k": 4}),
    ("config 5 k=8", 5, {"k": 8}),
    ("config 5 k=8, noise rising along the draft", 5, {"k": 8, "noise_by_position": DEGRADING_NOISE}),
]


@pytest.mark.parametrize("name,cid,ov", SAMPLING_WORKLOADS, ids=[w[0] for w in SAMPLING_WORKLOADS])
def test_spec_sample_every_sequence_with_margins(name, cid, ov):
    cfg = get_config(cid, **ov)
    print(f"[sampling] {name}: B={cfg.B} k={cfg.k} V={cfg.V}", flush=True)
    batch = make_batch(cfg, parts=("logits",))
    dev = torch.device("cuda")
    zt, zd = torch.from_numpy(batch.zt).to(dev), torch.from_numpy(batch.zd).to(dev)
    toks, nout, acc = s3r.spec_sample(zt, zd, torch.from_numpy(batch.d).to(dev), torch.from_numpy(batch.u).to(dev),
                                      float(batch.temperature))
    torch.cuda.synchronize()
    toks, nout, acc = toks.cpu().numpy(), nout.cpu().numpy(), acc.cpu().numpy()
    T = batch.temperature

    def one(b):
        p_rows = [oracle.softmax_t(batch.zt[b, i], T) for i in range(cfg.k + 1)]
        q_rows = [oracle.softmax_t(batch.zd[b, i], T) for i in range(cfg.k)]
        rt, rn, ra = oracle.spec_decide(p_rows, q_rows, batch.d[b], batch.u[b])
        return b, rt, rn, ra, oracle.decide_margins(p_rows, q_rows, batch.d[b], batch.u[b])

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, range(cfg.B)))
    rmin = dmin = np.inf
    for b, rt, rn, ra, (rm, dm) in res:
        assert nout[b] == rn and np.array_equal(toks[b], rt) and np.array_equal(acc[b], ra), b
        rmin, dmin = min(rmin, rm), min(dmin, dm)
    print(f"[margins] {name}: {cfg.B} sequences bit-exact, {int(nout.sum())} tokens; min ratio-test margin "
          f"{rmin:.3e}, min draw margin {dmin:.3e}", flush=True)
    assert rmin > MARGIN_FLOOR and dmin > MARGIN_FLOOR


def test_spec_sample_vocabulary_not_a_multiple_of_four():
    # V = 4099: the row statistics take their scalar path (no float4 loads) and the last
    # vocabulary chunk is ragged; N(0, 3) target logits, draft = target + N(0, 0.6)
    rng = np.random.default_rng(32)
    B, k, V = 64, 6, 4099
    zt = (3.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zd = (zt[:, :k] + 0.6 * rng.standard_normal((B, k, V))).astype(np.float32)
    q_rows = [[oracle.softmax_t(zd[b, i], 1.0) for i in range(k)] for b in range(B)]
    d = np.array([[oracle.invcdf(q_rows[b][i], rng.random()) for i in range(k)] for b in range(B)], np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    dev = torch.device("cuda")
    toks, nout, acc = s3r.spec_sample(torch.from_numpy(zt).to(dev), torch.from_numpy(zd).to(dev),
                                      torch.from_numpy(d).to(dev), torch.from_numpy(u).to(dev), 1.0)
    torch.cuda.synchronize()
    toks, nout, acc = toks.cpu().numpy(), nout.cpu().numpy(), acc.cpu().numpy()
    rmin = dmin = np.inf
    for b in range(B):
        p_rows = [oracle.softmax_t(zt[b, i], 1.0) for i in range(k + 1)]
        rt, rn, ra = oracle.spec_decide(p_rows, q_rows[b], d[b], u[b])
        assert nout[b] == rn and np.array_equal(toks[b], rt) and np.array_equal(acc[b], ra), b
        rm, dm = oracle.decide_margins(p_rows, q_rows[b], d[b], u[b])
        rmin, dmin = min(rmin, rm), min(dmin, dm)
    print(f"[margins] V=4099: {B} sequences bit-exact; min ratio-test margin {rmin:.3e}, min draw margin {dmin:.3e}")
    assert rmin > MARGIN_FLOOR and dmin > MARGIN_FLOOR


def test_spec_sample_with_masked_tokens():
    # -inf logits (tokens that cannot be drawn: a masked or padded vocabulary) in the target
    # and draft rows, a different third of the vocabulary per row; exact as elsewhere
    rng = np.random.default_rng(33)
    B, k, V = 48, 6, 2048
    zt = (3.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zd = (zt[:, :k] + 0.6 * rng.standard_normal((B, k, V))).astype(np.float32)
    zt[rng.random(zt.shape) < 1 / 3] = -np.inf
    zd[rng.random(zd.shape) < 1 / 3] = -np.inf
    zt[:, :, V - 256:] = -np.inf  # a padded tail in every target row
    q_rows = [[oracle.softmax_t(zd[b, i], 1.0) for i in range(k)] for b in range(B)]
    d = np.array([[oracle.invcdf(q_rows[b][i], rng.random()) for i in range(k)] for b in range(B)], np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    dev = torch.device("cuda")
    toks, nout, acc = s3r.spec_sample(torch.from_numpy(zt).to(dev), torch.from_numpy(zd).to(dev),
                                      torch.from_numpy(d).to(dev), torch.from_numpy(u).to(dev), 1.0)
    torch.cuda.synchronize()
    toks, nout, acc = toks.cpu().numpy(), nout.cpu().numpy(), acc.cpu().numpy()
    rmin = dmin = np.inf
    for b in range(B):
        p_rows = [oracle.softmax_t(zt[b, i], 1.0) for i in range(k + 1)]
        rt, rn, ra = oracle.spec_decide(p_rows, q_rows[b], d[b], u[b])
        assert nout[b] == rn and np.array_equal(toks[b], rt) and np.array_equal(acc[b], ra), b
        emitted = toks[b, :rn]
        assert np.isfinite(zt[b, np.arange(rn), emitted][-1:]).all()  # the drawn token is never masked
        rm, dm = oracle.decide_margins(p_rows, q_rows[b], d[b], u[b])
        rmin, dmin = min(rmin, rm), min(dmin, dm)
    print(f"[margins] masked tokens: {B} sequences bit-exact; min ratio-test margin {rmin:.3e}, "
          f"min draw margin {dmin:.3e}")
    assert rmin > MARGIN_FLOOR and dmin > MARGIN_FLOOR


def test_rollout_benchmark_inputs_middle_layer():
    """The rollout workload exactly as the benchmark times it: full batch of 256 (32 prompts x 8
    responses, 1024-token prompt pages shared), pages drawn on the device, layer 14."""
    from s3r_inputs.device import draw_pages_on_device
    cfg = get_config(4)
    layer = 14
    print(f"[rollout] layer {layer}, B={cfg.B}, pages drawn on the device", flush=True)
    batch = make_batch(cfg, layer=layer, parts=("q", "scores"))
    kp, vp = draw_pages_on_device(cfg, batch.num_pages, layer, 0, torch)
    t = to_dev(batch)
    t["kv"] = s3r.PagedKV(kp, vp, torch.from_numpy(batch.block_table).cuda())
    order = torch.empty((cfg.B,), dtype=torch.int32, device="cuda")
    idx, n_sel = run_select(cfg, batch, t, order=order)
    outs = run_draft_steps(cfg, batch, t, idx, n_sel, order=order)
    vout, vlse, vsc = run_verify(cfg, batch, t)
    torch.cuda.synchronize()
    idx_np, ns = idx.cpu().numpy(), n_sel.cpu().numpy()
    vout, vlse, vsc = vout.cpu().numpy(), vlse.cpu().numpy(), vsc.cpu().numpy()
    group = cfg.lengths[5]
    seqs = [0] + list(range(16 * group, 17 * group)) + [cfg.B - 1]
    for b in seqs:
        L, S = int(batch.ctx_len[b]), int(batch.seq_len[b])
        npg = (S + 15) // 16
        rows = torch.from_numpy(batch.block_table[b, :npg].astype(np.int64)).cuda()
        hk = kp.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)
        hv = vp.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)
        bt = np.arange(npg, dtype=np.int32)
        for kv in range(cfg.Hkv):
            ref = oracle.select(batch.scores[b, kv], L, cfg.s_num, cfg.s_den, cfg.window)
            assert ns[b] == len(ref) and np.array_equal(idx_np[b, kv, :ns[b]], ref), (b, kv)
        for j in (1, cfg.k):
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], hk, hv, bt, idx_np[b], int(ns[b]), L, L + j,
                                         float(batch.scale))
            assert rel_err_rows(outs[j - 1][0][b].cpu().numpy(), ro) <= TOL_BF16, (b, j)
        ro, rl, rs = oracle.verify(batch.q_verify[b], hk, hv, bt, S, cfg.k, float(batch.scale))
        eo = rel_err_rows(vout[b], ro)
        es = float((np.abs(vsc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max())
        assert eo <= TOL_BF16 and es <= TOL_BF16, (b, eo, es)
        assert np.abs(vlse[b] - rl).max() <= 2e-3
    print(f"[rollout] {len(seqs)} sequences checked (groups 0, 16, 31)", flush=True)


def test_read_pattern_kernels_run_in_bounds_and_deterministically():
    # measurement kernels: the verification's and a draft step's reads, checksummed per workgroup
    cfg = get_config(3, B=5, lengths=("uniform", 1, 9000))
    batch = make_batch(cfg, lengths=np.array([1, 17, 4095, 4097, 9000], np.int32), parts=("kv", "scores"))
    t = to_dev(batch)
    ms = int(batch.seq_len.max())
    # workgroups past a sequence's end write nothing: the sinks start at zero
    nv = s3r.load().s3r_read_pattern_sink_words(cfg.B, cfg.Hkv, ms, 0)
    a = s3r.read_verify_pattern(t["kv"], t["seq_len"], ms, sink=torch.zeros(nv, dtype=torch.int32, device="cuda"))
    b = s3r.read_verify_pattern(t["kv"], t["seq_len"], ms, sink=torch.zeros(nv, dtype=torch.int32, device="cuda"))
    idx, n_sel = run_select(cfg, batch, t)
    cap = idx.shape[2]
    nd = s3r.load().s3r_read_pattern_sink_words(cfg.B, cfg.Hkv, cap + 1, 1)
    c = s3r.read_draft_pattern(t["kv"], idx, n_sel, t["ctx_len"], t["ctx_len"] + 1, cap + 1,
                               sink=torch.zeros(nd, dtype=torch.int32, device="cuda"))
    d = s3r.read_draft_pattern(t["kv"], idx, n_sel, t["ctx_len"], t["ctx_len"] + 1, cap + 1,
                               sink=torch.zeros(nd, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)
    # each workgroup's word is the xor of every 32-bit word it must read: pins the bytes each
    # pattern covers (the K and V blocks of a verification subtile's two pages, the rows of a
    # draft split's kept positions), computed here from the same cache arrays
    kw = batch.k_pages.view(np.uint32)
    vw = batch.v_pages.view(np.uint32)
    page_x = np.bitwise_xor.reduce(kw.reshape(kw.shape[0], cfg.Hkv, -1), axis=2) ^ \
        np.bitwise_xor.reduce(vw.reshape(vw.shape[0], cfg.Hkv, -1), axis=2)  # [page][KV head]
    chunk_v, nsplit = 4096, -(-ms // 4096)
    want = np.zeros(nv, np.uint32)
    for pair in range(cfg.B * cfg.Hkv):
        bb, kv = divmod(pair, cfg.Hkv)
        S = int(batch.seq_len[bb])
        ch = -(-(-(-S // -(-S // chunk_v))) // 32) * 32
        for split in range(nsplit):
            c0 = split * ch
            if c0 >= S:
                continue
            acc = np.uint32(0)
            for st in range(-(-(min(S, c0 + ch) - c0) // 32)):
                pa = batch.block_table[bb, (c0 >> 4) + 2 * st]
                pb = batch.block_table[bb, (c0 >> 4) + 2 * st + 1] if c0 + st * 32 + 16 < S else pa
                acc ^= page_x[pa, kv] ^ page_x[pb, kv]
            want[((pair // 8) * nsplit + split) * 8 + pair % 8] = acc
    assert np.array_equal(a.cpu().numpy().view(np.uint32), want)
    idx_h, ns_h = idx.cpu().numpy(), n_sel.cpu().numpy()
    krow = kw.reshape(kw.shape[0], cfg.Hkv, 16, -1)
    vrow = vw.reshape(vw.shape[0], cfg.Hkv, 16, -1)
    nsd = -(-(cap + 1) // 2048)
    chunk_d = -(-(-(-(cap + 1) // nsd)) // 32) * 32
    want_d = np.zeros(nd, np.uint32)
    for bb in range(cfg.B):
        L, ns = int(batch.ctx_len[bb]), int(ns_h[bb])  # kept positions per KV head of the sequence
        for kv in range(cfg.Hkv):
            pos = np.concatenate([idx_h[bb, kv, :ns], [L]]).astype(np.int64)  # kept positions + [L, L + 1)
            for split in range(nsd):
                acc = np.uint32(0)
                for p_ in pos[split * chunk_d:(split + 1) * chunk_d]:
                    pg = batch.block_table[bb, p_ >> 4]
                    acc ^= np.bitwise_xor.reduce(krow[pg, kv, p_ & 15]) ^ np.bitwise_xor.reduce(vrow[pg, kv, p_ & 15])
                want_d[(bb * cfg.Hkv + kv) * nsd + split] = acc
    assert np.array_equal(c.cpu().numpy().view(np.uint32), want_d)


@pytest.mark.parametrize("cid,ov,lengths", [
    (3, {"B": 4}, [31, 32, 4093, 9001]),                # two row tiles, ragged tails, 1-3 splits
    (2, {"B": 3}, [17, 6000, 16390]),                   # one row tile (Qwen3-1.7B rows)
    (5, {"B": 2, "k": 8}, [5000, 12287]),               # three row tiles
])
def test_verify_scores_do_not_depend_on_the_score_stride(cid, ov, lengths):
    """The finalize writes a score row with vector stores where the row start and the tile allow it
    and with single stores elsewhere: the same scores, bit for bit, for a ragged stride, a multiple
    of 4 and a multiple of 32 plus 4, and nothing written at or past a sequence's end."""
    cfg = get_config(cid, **ov)
    batch = make_batch(cfg, lengths=np.array(lengths, np.int32), parts=("kv", "q"))
    t = to_dev(batch)
    ms = int(batch.seq_len.max())
    print(f"[stride] config {cid} k={cfg.k} G={cfg.G} lengths {lengths}", flush=True)
    res = []
    for stride in (ms, (ms + 3) // 4 * 4, (ms + 31) // 32 * 32 + 4):
        sc = torch.full((cfg.B, cfg.Hkv, stride), -7.0, dtype=torch.float32, device="cuda")
        out, lse, _ = s3r.verify_attn(t["q_verify"], t["kv"], t["seq_len"], cfg.k, float(batch.scale), ms,
                                      scores=sc)
        torch.cuda.synchronize()
        sc = sc.cpu().numpy()
        for b in range(cfg.B):
            S = int(batch.seq_len[b])
            assert (sc[b, :, S:] == -7.0).all(), (stride, b)
        res.append((sc, out.cpu().numpy()))
    for sc, out in res[1:]:
        assert np.array_equal(out, res[0][1])
        for b in range(cfg.B):
            S = int(batch.seq_len[b])
            assert np.array_equal(sc[b, :, :S], res[0][0][b, :, :S]), b
    # and the scores are the oracle's
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        _, _, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                 float(batch.scale))
        assert (np.abs(res[0][0][b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max() <= 2e-2, b
