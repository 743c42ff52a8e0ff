"""Seeded synthetic inputs for exact attention (shared by the HIP path's tests/bench and the oracle).

This module holds no attention arithmetic. It only draws seeded random numbers,
rounds them to the storage dtype (round-to-nearest-even), and describes the
workload shapes. Every tensor is generated per (batch, head) slice from its own
seed, so any slice can be regenerated on its own (the oracle can check one head
of a multi-GiB tensor without generating the rest).

Recipe (all values are exactly representable in the storage dtype, returned as
float32 arrays, so that upcasting to float64 on the oracle side and downcasting
to bf16/fp16 on the device side are both exact):

  seed of slice (tensor t, batch b, head h) = SeedSequence([31, cfg, t, b, h])
  values = sigma * standard_normal(float32, PCG64)   (sigma in {1, 0.5}: exact)
  rounded RNE to the storage dtype (bf16: integer rounding of the fp32 bits;
  fp16: numpy's float16 cast, which is RNE; fp32: unchanged)

tensor ids: Q=0, K=1, V=2, dO=4 (the output gradient of backward workloads);
ragged decode lengths use SeedSequence([31, cfg, 3]).
Paged-cache block tables are a seeded permutation of the pool's blocks,
SeedSequence([31, 2000, seed]). FP8 caches are E4M3 codes of sigma * N(0, 1)
divided by a per-tensor scale, SeedSequence([31, 3000, seed]), rounded by
torch's float8_e4m3fn cast.
"""
from .configs import CONFIGS, Config, get_config, ragged_lengths  # noqa: F401
from .gen import (  # noqa: F401
    bf16_round, fp16_round, round_to_dtype, slice_values, tensor_values, random_tensor, paged_layout,
    fp8_codes,
)
