"""Seeded generator of one layer's worth of S3R inputs.

Recipe (one independent PCG64 stream per (seed, config, layer, seq, tag)):

* context lengths L_b: fixed, uniform integers in [lo, hi], or (rollout)
  a shared prompt prefix plus a lognormal response length clipped to
  [1, clip]; the verified block adds k+1 positions, seq_len_b = L_b + k + 1;
* q, K, V ~ N(0, 1), drawn in float32, rounded to bfloat16 with
  round-to-nearest-even when the config stores bfloat16;
* the paged cache is [num_pages][Hkv][16][D]; physical page ids are a
  seeded random permutation; in the rollout config the prompt-prefix pages
  of the 8 responses of one prompt are the same physical pages;
* first-round selector scores ~ U[0, 1) (float32, exact 24-bit values);
* target logits N(0, target_std) and draft logits = target + N(0, noise_std)
  (or a noise level per draft position),
  float32;
* uniforms u_b,i = (uint32 >> 8) * 2^-24, exact in float32;
* draft tokens d_b,i are drawn from softmax(zd_b,i / T) by the Gumbel-max
  construction (argmax of zd/T plus Gumbel noise, float64), or argmax(zd) at
  T = 0. They are inputs here because the drafting forward pass that would
  sample them is outside this step;
* multi-round runs (make_round_inputs): round r draws its own queries, the
  K/V rows each draft step appends, the K/V rows of the verified block,
  logits, uniforms and draft tokens, with the same distributions, from
  streams of their own.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import Config

TAG_LEN, TAG_PAGES, TAG_QD, TAG_QV, TAG_K, TAG_V, TAG_SCORES = 1, 2, 3, 4, 5, 6, 7
TAG_ZT, TAG_ZD, TAG_U, TAG_DTOK, TAG_KP, TAG_VP = 8, 9, 10, 11, 12, 13
TAG_KD, TAG_VD, TAG_KB, TAG_VB = 14, 15, 16, 17
# The streams of round r of a multi-round run use layer ROUND_LAYER + r, far
# from the layer numbers of a model.
ROUND_LAYER = 1 << 20

_POOL_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def unit_rng(seed: int, cid: int, layer: int, seq: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, layer, seq, tag])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def exact_uniform_f32(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms on the 2^-24 grid in [0, 1): exactly representable in float32."""
    return (rng.integers(0, 1 << 32, size=shape, dtype=np.uint64) >> np.uint64(8)).astype(np.float32) * np.float32(2.0 ** -24)


def _normal(rng, shape, dtype_name):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype_name == "bf16" else x


def _store_dtype(cfg: Config):
    return np.uint16 if cfg.dtype == "bf16" else np.float32


@dataclass
class Batch:
    cfg: Config
    layer: int
    seed: int
    ctx_len: np.ndarray  # int32 [B]: committed context L_b at selection time
    seq_len: np.ndarray  # int32 [B]: L_b + k + 1 (cache length at verification)
    block_table: np.ndarray  # int32 [B][max_pages]
    num_pages: int
    k_pages: Optional[np.ndarray] = None  # [num_pages][Hkv][16][D] uint16 (bf16 bits) or float32
    v_pages: Optional[np.ndarray] = None
    q_draft: Optional[np.ndarray] = None  # [k][B][Hq][D]
    q_verify: Optional[np.ndarray] = None  # [B][k+1][Hq][D]
    scores: Optional[np.ndarray] = None  # float32 [B][Hkv][score_stride]
    zt: Optional[np.ndarray] = None  # float32 [B][k+1][V]
    zd: Optional[np.ndarray] = None  # float32 [B][k][V]
    u: Optional[np.ndarray] = None  # float32 [B][k+1]
    d: Optional[np.ndarray] = None  # int32 [B][k]
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.cfg.D))

    @property
    def temperature(self) -> np.float32:
        return np.float32(self.cfg.temperature)

    @property
    def score_stride(self) -> int:
        return int(self.seq_len.max())

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        """Storage values (bf16 bits or float32) as float32."""
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def make_lengths(cfg: Config, seed: int = 0, B: Optional[int] = None) -> np.ndarray:
    B = cfg.B if B is None else B
    kind = cfg.lengths[0]
    rng = unit_rng(seed, cfg.cid, 0, 0, TAG_LEN)
    if kind == "fixed":
        L = np.full(B, cfg.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        L = rng.integers(cfg.lengths[1], cfg.lengths[2] + 1, size=B, dtype=np.int64)
    elif kind == "rollout":
        prefix, median, sig, clip, _group = cfg.lengths[1:]
        r = np.exp(math.log(median) + sig * rng.standard_normal(B))
        r = np.clip(np.rint(r), 1, clip).astype(np.int64)
        L = prefix + r
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


def _page_plan(cfg: Config, seq_len: np.ndarray, seed: int, layer: int):
    """Block table with seeded physical page ids (shared prompt-prefix pages in the rollout config)."""
    P = cfg.page
    B = len(seq_len)
    npages = (seq_len.astype(np.int64) + P - 1) // P
    shared = 0
    group = 1
    if cfg.lengths[0] == "rollout":
        prefix, group = cfg.lengths[1], cfg.lengths[5]
        assert prefix % P == 0
        shared = prefix // P
    n_groups = (B + group - 1) // group if shared else 0
    canon = []  # canonical page list: group prefixes, then each sequence's own pages
    total = n_groups * shared + int((npages - shared).sum())
    perm = unit_rng(seed, cfg.cid, layer, 0, TAG_PAGES).permutation(total).astype(np.int32)
    bt = np.zeros((B, int(npages.max())), dtype=np.int32)
    c = 0
    prefix_pages = []
    for g in range(n_groups):
        prefix_pages.append(perm[c:c + shared])
        c += shared
    for b in range(B):
        own = int(npages[b]) - shared
        if shared:
            bt[b, :shared] = prefix_pages[b // group]
        bt[b, shared:shared + own] = perm[c:c + own]
        c += own
    assert c == total
    del canon
    return bt, total, shared, group


def _fill_kv(cfg, batch, seed, layer, threads):
    P, Hkv, D = cfg.page, cfg.Hkv, cfg.D
    sd = _store_dtype(cfg)
    kp = np.zeros((batch.num_pages, Hkv, P, D), dtype=sd)
    vp = np.zeros((batch.num_pages, Hkv, P, D), dtype=sd)
    shared_pages = batch.extra["shared_pages"]
    group = batch.extra["group"]

    def write_positions(b, start, K, V):
        # K, V: [n][Hkv][D] for positions start .. start+n-1 (start multiple of P)
        n = K.shape[0]
        npg = (n + P - 1) // P
        padn = npg * P
        if padn != n:
            K = np.concatenate([K, np.zeros((padn - n, Hkv, D), dtype=sd)])
            V = np.concatenate([V, np.zeros((padn - n, Hkv, D), dtype=sd)])
        pages = batch.block_table[b, start // P:start // P + npg]
        kp[pages] = K.reshape(npg, P, Hkv, D).transpose(0, 2, 1, 3)
        vp[pages] = V.reshape(npg, P, Hkv, D).transpose(0, 2, 1, 3)

    def do_prefix(g):
        n = shared_pages * P
        K = _normal(unit_rng(seed, cfg.cid, layer, g, TAG_KP), (n, Hkv, D), cfg.dtype)
        V = _normal(unit_rng(seed, cfg.cid, layer, g, TAG_VP), (n, Hkv, D), cfg.dtype)
        write_positions(g * group, 0, K, V)

    def do_seq(b):
        start = shared_pages * P
        n = int(batch.seq_len[b]) - start
        K = _normal(unit_rng(seed, cfg.cid, layer, b, TAG_K), (n, Hkv, D), cfg.dtype)
        V = _normal(unit_rng(seed, cfg.cid, layer, b, TAG_V), (n, Hkv, D), cfg.dtype)
        write_positions(b, start, K, V)

    B = len(batch.seq_len)
    with ThreadPoolExecutor(threads) as ex:
        if shared_pages:
            list(ex.map(do_prefix, range((B + group - 1) // group)))
        list(ex.map(do_seq, range(B)))
    batch.k_pages, batch.v_pages = kp, vp


def make_batch(cfg: Config, layer: int = 0, seed: int = 0, B: Optional[int] = None,
               parts=("kv", "q", "scores", "logits"), threads: Optional[int] = None,
               lengths: Optional[np.ndarray] = None) -> Batch:
    """Build one layer's inputs for ``cfg`` (optionally only the first ``B`` sequences).

    ``parts`` selects which arrays to draw; the lengths and block table are
    always built. ``lengths`` overrides the drawn context lengths (tests use
    it for ragged and edge cases).
    """
    threads = _POOL_THREADS if threads is None else threads
    B = cfg.B if B is None else B
    L = make_lengths(cfg, seed, B) if lengths is None else np.asarray(lengths, dtype=np.int32)
    assert len(L) == B and int(L.min()) >= 1
    seq_len = (L.astype(np.int64) + cfg.k + 1).astype(np.int32)
    bt, num_pages, shared, group = _page_plan(cfg, seq_len, seed, layer)
    batch = Batch(cfg=cfg, layer=layer, seed=seed, ctx_len=L, seq_len=seq_len,
                  block_table=bt, num_pages=num_pages,
                  extra={"shared_pages": shared, "group": group})
    k, Hq, Hkv, D, V = cfg.k, cfg.Hq, cfg.Hkv, cfg.D, cfg.V
    sd = _store_dtype(cfg)
    if "kv" in parts:
        _fill_kv(cfg, batch, seed, layer, threads)
    if "q" in parts:
        qd = np.empty((k, B, Hq, D), dtype=sd)
        qv = np.empty((B, k + 1, Hq, D), dtype=sd)
        for b in range(B):
            qd[:, b] = _normal(unit_rng(seed, cfg.cid, layer, b, TAG_QD), (k, Hq, D), cfg.dtype)
            qv[b] = _normal(unit_rng(seed, cfg.cid, layer, b, TAG_QV), (k + 1, Hq, D), cfg.dtype)
        batch.q_draft, batch.q_verify = qd, qv
    if "scores" in parts:
        stride = int(seq_len.max())
        sc = np.zeros((B, Hkv, stride), dtype=np.float32)
        for b in range(B):
            sc[b, :, :L[b]] = exact_uniform_f32(unit_rng(seed, cfg.cid, layer, b, TAG_SCORES), (Hkv, int(L[b])))
        batch.scores = sc
    if "logits" in parts:
        # logits do not depend on the layer: one sampling step per round
        batch.zt, batch.zd, batch.u, batch.d = _logits(cfg, seed, 0, B, threads)
    return batch


def _logits(cfg: Config, seed: int, layer: int, B: int, threads: int):
    """Target and draft logits, uniforms and draft tokens of one round."""
    k, V = cfg.k, cfg.V
    zt = np.empty((B, k + 1, V), dtype=np.float32)
    zd = np.empty((B, k, V), dtype=np.float32)
    u = np.empty((B, k + 1), dtype=np.float32)
    d = np.empty((B, k), dtype=np.int32)
    T = float(np.float32(cfg.temperature))

    def do_logits(b):
        zt[b] = np.float32(cfg.target_std) * unit_rng(seed, cfg.cid, layer, b, TAG_ZT).standard_normal((k + 1, V), dtype=np.float32)
        noise = unit_rng(seed, cfg.cid, layer, b, TAG_ZD).standard_normal((k, V), dtype=np.float32)
        if cfg.noise_by_position:
            sig = np.asarray(cfg.noise_by_position[:k], dtype=np.float32)[:, None]
            zd[b] = zt[b, :k] + sig * noise
        else:
            zd[b] = zt[b, :k] + np.float32(cfg.noise_std) * noise
        u[b] = exact_uniform_f32(unit_rng(seed, cfg.cid, layer, b, TAG_U), (k + 1,))
        rg = unit_rng(seed, cfg.cid, layer, b, TAG_DTOK)
        for i in range(k):
            if T > 0.0:
                e = (rg.integers(0, 1 << 53, size=V, dtype=np.int64).astype(np.float64) + 0.5) * 2.0 ** -53
                g = -np.log(-np.log(e))
                d[b, i] = int(np.argmax(zd[b, i].astype(np.float64) / T + g))
            else:
                d[b, i] = int(np.argmax(zd[b, i]))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(do_logits, range(B)))
    return zt, zd, u, d


@dataclass
class RoundInputs:
    """What the model would hand the step in round r of a multi-round run (one layer)."""
    q_draft: np.ndarray  # [k][B][Hq][D]: query of draft step j (1..k) at position L + j - 1
    k_draft: np.ndarray  # [k][B][Hkv][D]: K row draft step j appends at position L + j - 1
    v_draft: np.ndarray
    q_verify: np.ndarray  # [B][k+1][Hq][D]
    k_block: np.ndarray  # [B][k+1][Hkv][D]: K rows of the block positions L .. L + k
    v_block: np.ndarray
    zt: np.ndarray  # float32 [B][k+1][V]
    zd: np.ndarray  # float32 [B][k][V]
    u: np.ndarray  # float32 [B][k+1]
    d: np.ndarray  # int32 [B][k]


def make_round_inputs(cfg: Config, rnd: int, seed: int = 0, B: Optional[int] = None,
                      threads: Optional[int] = None) -> RoundInputs:
    """Queries, new K/V rows, logits, uniforms and draft tokens of round ``rnd``."""
    threads = _POOL_THREADS if threads is None else threads
    B = cfg.B if B is None else B
    lay = ROUND_LAYER + rnd
    k, Hq, Hkv, D = cfg.k, cfg.Hq, cfg.Hkv, cfg.D
    sd = _store_dtype(cfg)
    qd = np.empty((k, B, Hq, D), dtype=sd)
    kd = np.empty((k, B, Hkv, D), dtype=sd)
    vd = np.empty((k, B, Hkv, D), dtype=sd)
    qv = np.empty((B, k + 1, Hq, D), dtype=sd)
    kb = np.empty((B, k + 1, Hkv, D), dtype=sd)
    vb = np.empty((B, k + 1, Hkv, D), dtype=sd)
    for b in range(B):
        qd[:, b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_QD), (k, Hq, D), cfg.dtype)
        kd[:, b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_KD), (k, Hkv, D), cfg.dtype)
        vd[:, b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_VD), (k, Hkv, D), cfg.dtype)
        qv[b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_QV), (k + 1, Hq, D), cfg.dtype)
        kb[b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_KB), (k + 1, Hkv, D), cfg.dtype)
        vb[b] = _normal(unit_rng(seed, cfg.cid, lay, b, TAG_VB), (k + 1, Hkv, D), cfg.dtype)
    zt, zd, u, d = _logits(cfg, seed, lay, B, threads)
    return RoundInputs(qd, kd, vd, qv, kb, vb, zt, zd, u, d)

