"""Pins of the oracle's multi-round pieces: K/V append into the paged cache and
the round commit (CPU only)."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cache(num_pages, Hkv, D, dtype=np.float32, seed=0):
    rng = np.random.default_rng(seed)
    if dtype == np.uint16:
        return (rng.integers(0, 1 << 16, size=(num_pages, Hkv, 16, D), dtype=np.uint16),
                rng.integers(0, 1 << 16, size=(num_pages, Hkv, 16, D), dtype=np.uint16))
    return (rng.standard_normal((num_pages, Hkv, 16, D)).astype(np.float32),
            rng.standard_normal((num_pages, Hkv, 16, D)).astype(np.float32))


def _read(pages, bt_row, j):
    """All KV heads of position j through the oracle's attention gather (pinned by the
    attention tests against torch's scaled dot product attention)."""
    return np.stack([oracle.gather(pages, bt_row, h, [j])[0] for h in range(pages.shape[1])]).astype(pages.dtype)


def test_append_reads_back_and_leaves_the_rest():
    Hkv, D = 3, 8
    kp, vp = _cache(12, Hkv, D)
    bt = np.array([[7, 2, 9, 0], [4, 11, 5, 1]])
    k0, v0 = kp.copy(), vp.copy()
    rng = np.random.default_rng(1)
    writes = {0: (13, 7), 1: (30, 5)}  # sequence -> (first position, rows): both cross a page boundary
    for b, (pos, n) in writes.items():
        kr = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        vr = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        oracle.kv_append(kp, vp, bt[b], pos, kr, vr)
        for t in range(n):
            assert np.array_equal(_read(kp, bt[b], pos + t), kr[t])
            assert np.array_equal(_read(vp, bt[b], pos + t), vr[t])
    written = set()
    for b, (pos, n) in writes.items():
        for j in range(pos, pos + n):
            written.add((int(bt[b][j // 16]), j % 16))
    for page in range(12):
        for slot in range(16):
            if (page, slot) not in written:
                assert np.array_equal(kp[page, :, slot], k0[page, :, slot])
                assert np.array_equal(vp[page, :, slot], v0[page, :, slot])


def test_append_one_at_a_time_equals_at_once_bf16():
    Hkv, D = 2, 16
    kp, vp = _cache(6, Hkv, D, np.uint16)
    kq, vq = kp.copy(), vp.copy()
    bt = np.array([3, 0, 5])
    rng = np.random.default_rng(2)
    kr = rng.integers(0, 1 << 16, size=(9, Hkv, D), dtype=np.uint16)
    vr = rng.integers(0, 1 << 16, size=(9, Hkv, D), dtype=np.uint16)
    oracle.kv_append(kp, vp, bt, 10, kr, vr)
    for t in range(9):
        oracle.kv_append(kq, vq, bt, 10 + t, kr[t:t + 1], vr[t:t + 1])
    assert np.array_equal(kp, kq) and np.array_equal(vp, vq)


def test_append_into_a_shared_page_is_seen_by_every_table():
    Hkv, D = 1, 4
    kp, vp = _cache(5, Hkv, D)
    bt = np.array([[2, 4], [2, 1]])  # both sequences map positions 0..15 to page 2
    kr = np.full((1, Hkv, D), 7.0, np.float32)
    oracle.kv_append(kp, vp, bt[0], 3, kr, kr)
    assert np.array_equal(_read(kp, bt[1], 3), kr[0])


def pin_append_against_generator(orc) -> bool:
    """The generator lays out a cache with its own code. Clear a run of positions of one
    sequence in a copy (every KV head), append the rows the attention gather reads from the
    original, and the copy must equal the original again."""
    from s3r_inputs import get_config, make_batch
    cfg = get_config(1, B=2, Hq=4, Hkv=2, D=16, k=2, lengths=("fixed", 70))
    bt = make_batch(cfg, parts=("kv",))
    ok = True
    for b, (pos, n) in ((0, (5, 30)), (1, (47, 9))):
        rows_k = np.stack([np.stack([orc.gather(bt.k_pages, bt.block_table[b], h, [j])[0] for h in range(2)])
                           for j in range(pos, pos + n)]).astype(np.float32)
        rows_v = np.stack([np.stack([orc.gather(bt.v_pages, bt.block_table[b], h, [j])[0] for h in range(2)])
                           for j in range(pos, pos + n)]).astype(np.float32)
        kp, vp = bt.k_pages.copy(), bt.v_pages.copy()
        for j in range(pos, pos + n):
            kp[bt.block_table[b][j // 16], :, j % 16, :] = 0.0
            vp[bt.block_table[b][j // 16], :, j % 16, :] = 0.0
        orc.kv_append(kp, vp, bt.block_table[b], pos, rows_k, rows_v)
        ok = ok and np.array_equal(kp, bt.k_pages) and np.array_equal(vp, bt.v_pages)
    return ok


def test_append_restores_the_generated_cache():
    assert pin_append_against_generator(oracle)


def pin_commit(orc):
    """commit() after the golden full-acceptance and first-mismatch rounds (raises on a mismatch)."""
    test_commit_after_full_acceptance_and_first_mismatch(orc)
    return True


def test_commit_after_full_acceptance_and_first_mismatch(orc=oracle):
    # full acceptance: identical draft and target rows, the bonus becomes pending
    g = json.load(open(os.path.join(GOLDEN, "full_acceptance_k6.json")))
    k = g["k"]
    rng = np.random.default_rng(3)
    zt = (1.5 * rng.standard_normal((k + 1, 20))).astype(np.float32)
    d = np.arange(k)
    tokens, n_out, _ = oracle.spec_sample(zt, zt[:k].copy(), d, np.full(k + 1, 0.3, np.float32), np.float32(1.0))
    L1, pending, cur, seq = orc.commit(100, n_out, tokens, k)
    assert L1 == 100 + k + 1 and pending == tokens[k] and cur == [L1 + j for j in range(1, k + 1)]
    assert seq == L1 + k + 1
    # first mismatch at draft 3 of 5: three accepted plus the correction
    g = json.load(open(os.path.join(GOLDEN, "first_mismatch_k5.json")))
    k = g["k"]
    zt = np.zeros((k + 1, 8), np.float32)
    zd = np.zeros((k, 8), np.float32)
    d = np.array([1, 2, 3, 4, 5])
    for i in range(k):
        zt[i, d[i]] = 5.0
        zd[i, d[i]] = 5.0
    zt[3, d[3]] = -5.0
    tokens, n_out, _ = oracle.spec_sample(zt, zd, d, np.full(k + 1, 0.5, np.float32), np.float32(1.0))
    L1, pending, cur, seq = orc.commit(40, n_out, tokens, k)
    assert n_out == g["n_out"] and L1 == 40 + g["n_out"]
    assert pending == tokens[g["n_accepted"]] and pending != d[g["n_accepted"]]
