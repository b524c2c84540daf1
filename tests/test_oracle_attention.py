"""Pins of the oracle's sparse draft attention and dense block verification (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from s3r_inputs import get_config, make_batch
from s3r_inputs.gen import bf16_bits_to_f32


def _tiny(L=37, k=3, Hq=4, Hkv=2, D=8, dtype="f32", B=2, seed=0):
    cfg = get_config(1, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, k=k, lengths=("fixed", L), V=16)
    return make_batch(cfg, seed=seed, parts=("kv", "q", "scores"))


def _dense_rows(batch, b, kv, n):
    """K, V rows [n][D] of one sequence in logical order, read by explicit page walk."""
    P = batch.cfg.page
    K = np.zeros((n, batch.cfg.D))
    V = np.zeros((n, batch.cfg.D))
    for j in range(n):
        page = batch.block_table[b, j // P]
        K[j] = batch.as_f32(batch.k_pages[page, kv, j % P])
        V[j] = batch.as_f32(batch.v_pages[page, kv, j % P])
    return K, V


def _loop_attend(q, K, V, scale):
    logits = [scale * sum(float(q[d]) * float(K[j][d]) for d in range(len(q))) for j in range(len(K))]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    z = sum(e)
    o = [sum(e[j] / z * float(V[j][d]) for j in range(len(K))) for d in range(len(q))]
    return np.array(o), m + math.log(z), [x / z for x in e]


def test_sparse_decode_bruteforce():
    batch = _tiny()
    cfg = batch.cfg
    G = cfg.G
    rng = np.random.default_rng(5)
    for b in range(cfg.B):
        L = int(batch.ctx_len[b])
        idx = [np.sort(rng.choice(L, size=9, replace=False)) for _ in range(cfg.Hkv)]
        for j in range(1, cfg.k + 1):
            q = batch.as_f32(batch.q_draft[j - 1, b])
            o, lse = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages,
                                          batch.block_table[b], idx, 9, L, L + j, float(batch.scale))
            for h in range(cfg.Hq):
                K, V = _dense_rows(batch, b, h // G, L + j)
                pos = list(idx[h // G]) + list(range(L, L + j))
                ro, rl, _ = _loop_attend(q[h], K[pos], V[pos], float(batch.scale))
                np.testing.assert_allclose(o[h], ro, rtol=1e-12, atol=1e-13)
                assert abs(lse[h] - rl) < 1e-12


def test_verify_bruteforce_and_scores():
    batch = _tiny(L=21, k=2)
    cfg = batch.cfg
    G, k = cfg.G, cfg.k
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        o, lse, sc = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                   S, k, float(batch.scale))
        q = batch.as_f32(batch.q_verify[b])
        ref_sc = np.zeros((cfg.Hkv, S))
        for h in range(cfg.Hq):
            K, V = _dense_rows(batch, b, h // G, S)
            for i in range(k + 1):
                last = S - (k + 1) + i
                ro, rl, p = _loop_attend(q[i, h], K[:last + 1], V[:last + 1], float(batch.scale))
                np.testing.assert_allclose(o[i, h], ro, rtol=1e-12, atol=1e-13)
                assert abs(lse[i, h] - rl) < 1e-12
                ref_sc[h // G, :last + 1] += p
        np.testing.assert_allclose(sc, ref_sc, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dtype,G", [("f32", 2), ("bf16", 4), ("bf16", 1)])
def test_verify_matches_torch_sdpa(dtype, G):
    Hkv = 2
    batch = _tiny(L=70, k=4, Hq=Hkv * G, Hkv=Hkv, D=16, dtype=dtype)
    cfg = batch.cfg
    k = cfg.k
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        o, lse, sc = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                   S, k, float(batch.scale))
        K = np.stack([_dense_rows(batch, b, kv, S)[0] for kv in range(Hkv)])  # [Hkv][S][D]
        V = np.stack([_dense_rows(batch, b, kv, S)[1] for kv in range(Hkv)])
        q = torch.tensor(batch.as_f32(batch.q_verify[b]), dtype=torch.float64).permute(1, 0, 2)  # [Hq][k+1][D]
        Kt = torch.tensor(K).repeat_interleave(G, dim=0)
        Vt = torch.tensor(V).repeat_interleave(G, dim=0)
        rows = torch.arange(k + 1)[:, None] + (S - k - 1)
        mask = torch.arange(S)[None, :] <= rows  # [k+1][S]
        ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, attn_mask=mask, scale=float(batch.scale))
        np.testing.assert_allclose(o.transpose(1, 0, 2), ref.numpy(), rtol=1e-11, atol=1e-12)
        logits = (q @ Kt.transpose(1, 2)) * float(batch.scale)
        prob = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)  # [Hq][k+1][S]
        ref_sc = prob.sum(dim=1).reshape(Hkv, G, S).sum(dim=1)
        np.testing.assert_allclose(sc, ref_sc.numpy(), rtol=1e-11, atol=1e-13)
        ref_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
        np.testing.assert_allclose(lse.T, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_full_budget_equals_dense_decode():
    batch = _tiny(L=45, k=3)
    cfg = batch.cfg
    for b in range(cfg.B):
        L = int(batch.ctx_len[b])
        n = oracle.budget(L, 1, 1, 16)
        assert n == L
        idx = [oracle.select(batch.scores[b, kv], L, 1, 1, 16) for kv in range(cfg.Hkv)]
        for j in range(1, cfg.k + 1):
            o, lse = oracle.sparse_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages,
                                          batch.block_table[b], idx, n, L, L + j, float(batch.scale))
            od, ld = oracle.dense_decode(batch.q_draft[j - 1, b], batch.k_pages, batch.v_pages,
                                         batch.block_table[b], L + j, float(batch.scale))
            np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse, ld, rtol=1e-13)


def test_verify_k0_equals_decode_and_rows_equal_decode():
    batch = _tiny(L=40, k=0)
    cfg = batch.cfg
    for b in range(cfg.B):
        S = int(batch.seq_len[b])
        o, lse, sc = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                   S, 0, float(batch.scale))
        od, ld = oracle.dense_decode(batch.q_verify[b, 0], batch.k_pages, batch.v_pages, batch.block_table[b],
                                     S, float(batch.scale))
        np.testing.assert_allclose(o[0], od, rtol=1e-13, atol=1e-14)
    batch = _tiny(L=40, k=5)
    for b in range(batch.cfg.B):
        S = int(batch.seq_len[b])
        o, lse, sc = oracle.verify(batch.q_verify[b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                   S, 5, float(batch.scale))
        for i in range(6):
            od, ld = oracle.dense_decode(batch.q_verify[b, i], batch.k_pages, batch.v_pages, batch.block_table[b],
                                         S - 5 + i, float(batch.scale))
            np.testing.assert_allclose(o[i], od, rtol=1e-13, atol=1e-14)
        # scores of each KV head sum to G (k+1)
        np.testing.assert_allclose(sc.sum(axis=1), batch.cfg.G * 6, rtol=1e-12)


def test_single_position_and_constant_keys():
    batch = _tiny(L=33, k=2, dtype="bf16")
    cfg = batch.cfg
    b = 0
    L = int(batch.ctx_len[b])
    idx = [np.array([7]), np.array([19])]
    # one kept position and no draft positions yet (cur = L): output is that V row exactly
    o, lse = oracle.sparse_decode(batch.q_draft[0, b], batch.k_pages, batch.v_pages, batch.block_table[b],
                                  idx, 1, L, L, float(batch.scale))
    for h in range(cfg.Hq):
        _, V = _dense_rows(batch, b, h // cfg.G, L)
        assert np.array_equal(o[h], V[idx[h // cfg.G][0]])
    # constant keys: uniform weights, output is the mean of the gathered V rows
    kp = batch.k_pages.copy()
    kp[...] = kp[0, 0, 0, 0]
    sel = [np.arange(0, 30, 3), np.arange(1, 30, 3)]
    o, lse = oracle.sparse_decode(batch.q_draft[1, b], kp, batch.v_pages, batch.block_table[b],
                                  sel, 10, L, L + 2, float(batch.scale))
    for h in range(cfg.Hq):
        _, V = _dense_rows(batch, b, h // cfg.G, L + 2)
        pos = list(sel[h // cfg.G]) + [L, L + 1]
        np.testing.assert_allclose(o[h], V[pos].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = bf16_bits_to_f32(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3])
    assert vals[4] == np.float32(3.3895314e38)
    assert vals[5] == np.float32(2.0 ** -133)


def test_page_scores_are_sums_of_position_scores():
    from s3r_inputs import get_config, make_batch
    cfg = get_config(1, B=2, Hq=4, Hkv=2, D=16, k=3, lengths=("uniform", 40, 90))
    bt = make_batch(cfg, parts=("kv", "q"))
    for b in range(cfg.B):
        S = int(bt.seq_len[b])
        _, _, sc = oracle.verify(bt.q_verify[b], bt.k_pages, bt.v_pages, bt.block_table[b], S, cfg.k, float(bt.scale))
        pg = oracle.page_scores(sc, S)
        assert pg.shape == (cfg.Hkv, -(-S // 16))
        # an explicit loop over the positions
        ref = np.zeros_like(pg)
        for h in range(cfg.Hkv):
            for j in range(S):
                ref[h, j // 16] += sc[h, j]
        np.testing.assert_allclose(pg, ref, rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(pg.sum(axis=1), cfg.G * (cfg.k + 1), rtol=1e-12)
        assert np.array_equal(oracle.page_scores(sc, S, unit=1), sc[:, :S])
        # a page moves only with its own positions
        sc2 = sc.copy()
        sc2[:, 17] += 1.0
        d = oracle.page_scores(sc2, S) - pg
        assert np.allclose(d[:, 1], 1.0) and np.abs(np.delete(d, 1, axis=1)).max() == 0
