"""The workload shapes of exact attention (prefill and GQA decode).

Shapes follow the pages' workloads: a 512-step single head; causal MHA
prefill at 4096; a one-day-at-1-second causal series (23,400 steps, 12 heads);
causal GQA prefill at ISL 32768 with group size 8; GQA decode against a
32768-token KV cache for 64 requests (uniform or ragged lengths); and the
same decode with 4 or 64 new tokens per request (speculative decoding and
prefix caching make the decode product taller, which the pages name as the
way decode moves toward compute).
"""
from dataclasses import dataclass, field
import math

import numpy as np


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    kind: str          # "prefill" | "decode"
    dtype: str         # "f32" | "f16" | "bf16"
    B: int
    H_q: int
    H_kv: int
    N_q: int
    N_kv: int
    d: int
    causal: bool
    sigma: float
    ragged: bool = False
    note: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32 (the value both sides use)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    1: Config(1, "single-head fp32 non-causal", "prefill", "f32", 1, 1, 1, 512, 512, 64, False, 1.0),
    2: Config(2, "causal MHA prefill bf16", "prefill", "bf16", 4, 32, 32, 4096, 4096, 128, True, 1.0),
    3: Config(3, "long-series causal prefill fp16", "prefill", "f16", 1, 12, 12, 23400, 23400, 64, True, 0.5,
              note="one trading day at 1 s resolution"),
    4: Config(4, "causal GQA prefill bf16", "prefill", "bf16", 1, 32, 4, 32768, 32768, 128, True, 1.0),
    5: Config(5, "GQA decode bf16 (uniform lengths)", "decode", "bf16", 64, 32, 4, 1, 32768, 128, False, 1.0),
    6: Config(5, "GQA decode bf16 (ragged lengths)", "decode", "bf16", 64, 32, 4, 1, 32768, 128, False, 1.0,
              ragged=True),
    # multi-token decode (speculative verification of 4 draft tokens) against
    # the same 32768-token caches as config 5: the keys and values are config
    # 5's, the queries are 4 per request and head, causally aligned at the end
    7: Config(5, "GQA multi-token decode bf16 (4 tokens per request)", "decode", "bf16", 64, 32, 4, 4,
              32768, 128, True, 1.0),
    # 64 new tokens per request (chunked prefill against the cache): compute-bound
    8: Config(5, "GQA multi-token decode bf16 (64 tokens per request)", "decode", "bf16", 64, 32, 4,
              64, 32768, 128, True, 1.0),
}


def get_config(key) -> Config:
    if isinstance(key, str) and key.endswith("r"):
        return CONFIGS[6]
    return CONFIGS[int(key)]


def ragged_lengths(cfg: Config) -> np.ndarray:
    """Per-request KV lengths, uniform on 1..N_kv inclusive, seed (31, cfg, 3)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([31, cfg.cid, 3])))
    return rng.integers(1, cfg.N_kv + 1, size=cfg.B).astype(np.int32)
