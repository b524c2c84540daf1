"""Seeded synthetic inputs for the S3R attention-and-sampling step.

This module is shared by the CPU oracle, the tests and the benchmark. It
holds none of the method's arithmetic: it only draws random numbers, rounds
them to the storage dtype and lays them out (paged KV cache, block tables,
per-sequence lengths). Every (config, layer, sequence, stream) unit is drawn
from its own ``numpy.random.SeedSequence([config, layer, seq, tag])`` so any
unit can be regenerated on its own.

Workloads stand in for the pages' DAPO-MATH-17k rollouts on Qwen3 models
(S3R paper listing page, Table 1 and the Table 4 settings); no dataset or
weights are used.
"""

from .configs import CONFIGS, Config, get_config, sweep_variants  # noqa: F401
from .gen import (  # noqa: F401
    Batch,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_batch,
    make_round_inputs,
    unit_rng,
)
