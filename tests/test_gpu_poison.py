"""Cache slots that no call may read hold NaN and Inf bit patterns here, as a
pooled cache that only s3r_kv_append writes may hold them: the slots past each
sequence's end on its last page (verification, draft steps) and the positions
after the current draft step. Results must match the oracle, which never reads
those slots, at the usual bars (2e-2 relative per output vector for bfloat16,
1e-5 for float32; selection bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
import self_sparse_speculative_amd as s3r
from s3r_inputs import get_config, make_batch
from tests.gpu_util import rel_err_rows, run_draft_steps, run_select, run_verify, to_dev
from tests.poison import poison_from

pytestmark = pytest.mark.gpu


def _pages_per_seq(batch):
    return (batch.seq_len.astype(np.int64) + 15) // 16 * 16


CASES = [
    ("mfma k=6", 3, {"k": 6}, [4100, 5003, 778, 1234]),
    ("mfma k=2", 5, {"k": 2}, [4101, 9000, 33, 2000]),
    ("mfma k=8 (queries in LDS)", 5, {"k": 8}, [4104, 8190, 40, 3001]),
    ("generic bf16 D=64", 1, {"D": 64, "dtype": "bf16", "Hq": 8, "Hkv": 2}, [300, 455, 17, 100]),
    ("generic f32 D=128", 1, {"D": 128, "dtype": "f32", "Hq": 8, "Hkv": 2}, [301, 456, 18, 99]),
]


@pytest.mark.parametrize("name,cid,ov,L", CASES, ids=[c[0] for c in CASES])
def test_slots_past_the_end_are_never_used(name, cid, ov, L):
    cfg = get_config(cid, B=len(L), **ov)
    batch = make_batch(cfg, lengths=np.array(L, np.int32))
    print(f"[poison] {name}: seq_len={batch.seq_len.tolist()}", flush=True)
    poison_from(batch.k_pages, batch.v_pages, batch.block_table, batch.seq_len, _pages_per_seq(batch))
    t = to_dev(batch)
    f32 = cfg.dtype == "f32"
    out, lse, sc = run_verify(cfg, batch, t)
    idx, n_sel = run_select(cfg, batch, t)
    drafts = run_draft_steps(cfg, batch, t, idx, n_sel)
    torch.cuda.synchronize()
    out, sc = out.cpu().numpy(), sc.cpu().numpy()
    idx, n_sel = idx.cpu().numpy(), n_sel.cpu().numpy()
    for b in range(cfg.B):
        S, Lb = int(batch.seq_len[b]), int(batch.ctx_len[b])
        ro, rl, rs = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b], S, cfg.k,
                                   float(batch.scale))
        assert np.isfinite(out[b]).all() and np.isfinite(sc[b, :, :S]).all(), b
        if f32:
            assert np.abs(out[b] - ro).max() <= 1e-5 and np.abs(sc[b, :, :S] - rs).max() <= 1e-5, b
        else:
            assert rel_err_rows(out[b], ro) <= 2e-2, b
            assert (np.abs(sc[b, :, :S] - rs).max(axis=1) / rs.max(axis=1)).max() <= 2e-2, b
        for j in (1, cfg.k):
            o = drafts[j - 1][0][b].cpu().numpy()
            ro, _ = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         idx[b], int(n_sel[b]), Lb, Lb + j, float(batch.scale))
            assert np.isfinite(o).all(), (b, j)
            assert (np.abs(o - ro).max() <= 1e-5) if f32 else (rel_err_rows(o, ro) <= 2e-2), (b, j)


@pytest.mark.parametrize("cid,ov", [(3, {}), (1, {})])
def test_first_draft_step_with_the_rest_of_the_round_unwritten(cid, ov):
    # positions L+1 .. of this round hold NaN/Inf: the first draft step reads up to L only
    cfg = get_config(cid, B=3, **ov)
    batch = make_batch(cfg, lengths=np.array([3000, 517, 64], np.int32) if cid == 3 else None)
    poison_from(batch.k_pages, batch.v_pages, batch.block_table, batch.ctx_len + 1, _pages_per_seq(batch))
    t = to_dev(batch)
    idx, n_sel = run_select(cfg, batch, t)
    cap = s3r.budget(int(batch.ctx_len.max()), cfg.s_num, cfg.s_den, cfg.window)
    o, _ = s3r.sparse_decode_attn(t["q_draft"][0], t["kv"], idx, n_sel, t["ctx_len"], t["ctx_len"] + 1,
                                  float(batch.scale), cap + cfg.k)
    torch.cuda.synchronize()
    o, idx, n_sel = o.cpu().numpy(), idx.cpu().numpy(), n_sel.cpu().numpy()
    for b in range(cfg.B):
        Lb = int(batch.ctx_len[b])
        ro, _ = oracle.sparse_decode(batch.q_draft[0, b], batch.k_pages, batch.v_pages, batch.block_table[b], idx[b],
                                     int(n_sel[b]), Lb, Lb + 1, float(batch.scale))
        assert np.isfinite(o[b]).all()
        assert (np.abs(o[b] - ro).max() <= 1e-5) if cfg.dtype == "f32" else (rel_err_rows(o[b], ro) <= 2e-2), b
