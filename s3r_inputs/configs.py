"""The five synthetic workloads of the S3R attention-and-sampling step.

Shapes follow Qwen3-1.7B (Hq 16, Hkv 8, head_dim 128) and Qwen3-8B (Hq 32,
Hkv 8, head_dim 128) attention layers; the default draft length k=6 and
budget s=0.05 are the ones the S3R paper listing page uses throughout
(Table 7 caption, Figure 6 setting). The budget fraction is kept as an
integer ratio s_num/s_den so that ceil(s*L) is exact.
"""

from dataclasses import dataclass, replace
from typing import Tuple

PAGE = 16


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" or "bf16": storage dtype of q, K and V
    lengths: Tuple  # ("fixed", L) | ("uniform", lo, hi) | ("rollout", prefix, median, sigma_ln, clip, group)
    k: int
    s_num: int
    s_den: int
    window: int
    V: int
    target_std: float
    noise_std: float
    temperature: float
    layers: int = 1
    page: int = PAGE
    # per-draft-position noise (draft position i uses noise_by_position[i]); empty: noise_std everywhere
    noise_by_position: Tuple = ()

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def s(self) -> float:
        return self.s_num / self.s_den

    def max_ctx(self) -> int:
        kind = self.lengths[0]
        if kind == "fixed":
            return self.lengths[1]
        if kind == "uniform":
            return self.lengths[2]
        if kind == "rollout":
            return self.lengths[1] + self.lengths[4]
        raise ValueError(kind)


CONFIGS = {
    1: Config(1, "tiny-f32", B=2, Hq=4, Hkv=2, D=64, dtype="f32",
              lengths=("fixed", 512), k=6, s_num=1, s_den=20, window=16,
              V=512, target_std=2.0, noise_std=0.5, temperature=1.0),
    2: Config(2, "qwen3-1.7b-layer", B=64, Hq=16, Hkv=8, D=128, dtype="bf16",
              lengths=("uniform", 2048, 16384), k=6, s_num=1, s_den=20, window=64,
              V=151936, target_std=3.0, noise_std=0.3, temperature=1.0),
    3: Config(3, "qwen3-8b-layer", B=128, Hq=32, Hkv=8, D=128, dtype="bf16",
              lengths=("uniform", 4096, 24576), k=6, s_num=1, s_den=20, window=64,
              V=151936, target_std=3.0, noise_std=0.3, temperature=1.0),
    4: Config(4, "qwen3-1.7b-rollout", B=256, Hq=16, Hkv=8, D=128, dtype="bf16",
              lengths=("rollout", 1024, 6144, 0.6, 16384, 8), k=6, s_num=1, s_den=20,
              window=64, V=151936, target_std=3.0, noise_std=0.3, temperature=1.0,
              layers=28),
    5: Config(5, "qwen3-8b-24k-sweep", B=128, Hq=32, Hkv=8, D=128, dtype="bf16",
              lengths=("fixed", 24576), k=6, s_num=1, s_den=20, window=64,
              V=151936, target_std=3.0, noise_std=0.3, temperature=1.0),
}

# Budget fractions of the sweep as exact ratios: 0.02, 0.05, 0.1, 0.2.
SWEEP_S = ((1, 50), (1, 20), (1, 10), (1, 5))
SWEEP_K = (2, 4, 6, 8)
SWEEP_SIGMA = (0.1, 0.3, 0.6)


def get_config(cid: int, **overrides) -> Config:
    """Config ``cid`` with optional field overrides (e.g. a smaller B for tests)."""
    cfg = CONFIGS[cid]
    return replace(cfg, **overrides) if overrides else cfg


def sweep_variants():
    """All 48 points of the 24K sweep: s x k x draft-noise sigma."""
    base = CONFIGS[5]
    out = []
    for s_num, s_den in SWEEP_S:
        for k in SWEEP_K:
            for sig in SWEEP_SIGMA:
                out.append(replace(base, s_num=s_num, s_den=s_den, k=k, noise_std=sig))
    return out


# Draft noise rising along the draft (positions 1..8), for the adaptive draft
# length: on N(0, 3) target logits it gives about 95 % acceptance at the first
# position falling to about 70 % at the sixth, the shape the digest reports for
# Qwen3-8B (95.8 % -> 67.9 %).
DEGRADING_NOISE = (0.12, 0.28, 0.44, 0.6, 0.76, 0.92, 1.08, 1.24)
