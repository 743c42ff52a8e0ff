"""Seeded generation and storage-dtype rounding (no attention arithmetic here)."""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# "do" is the output gradient of the backward workloads (shaped like Q); 3 is
# taken by the ragged decode lengths
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 4}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def fp16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest float16 (numpy's cast is RNE); returns float32."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f16":
        return fp16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def slice_values(cid: int, tensor: str, b: int, h: int, n: int, d: int, sigma: float,
                 dtype: str) -> np.ndarray:
    """One [n, d] slice (batch b, head h) of tensor 'q' | 'k' | 'v' | 'do' as exact float32 values."""
    x = _rng(31, cid, TENSOR_IDS[tensor], b, h).standard_normal((n, d), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return round_to_dtype(x, dtype)


def tensor_values(cfg, tensor: str, threads: int | None = None) -> np.ndarray:
    """A whole [B, H, N, d] tensor of a config as exact float32 values (threaded per slice)."""
    H = cfg.H_q if tensor in ("q", "do") else cfg.H_kv
    N = cfg.N_q if tensor in ("q", "do") else cfg.N_kv
    out = np.empty((cfg.B, H, N, cfg.d), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = slice_values(cfg.cid, tensor, b, h, N, cfg.d, cfg.sigma, cfg.dtype)

    nthr = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthr) as ex:
        list(ex.map(fill, range(cfg.B * H)))
    return out


def random_tensor(shape, seed: int, dtype: str, sigma: float = 1.0) -> np.ndarray:
    """A small ad-hoc seeded tensor (for tests that are not one of the five configs)."""
    x = _rng(31, 1000, seed).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return round_to_dtype(x, dtype)


def paged_layout(lens, block_size: int, max_blocks: int, seed: int, spare: int = 0):
    """A block table for a paged KV cache (a random allocation, no arithmetic).

    Request b needs ceil(lens[b] / block_size) logical blocks; every needed block
    gets a distinct physical block from a seeded permutation of a pool of
    sum(needed) + spare blocks. Entries past a request's needed blocks are -1.
    Returns (table int32 [B, max_blocks], num_blocks).
    """
    lens = np.asarray(lens, dtype=np.int64)
    need = (lens + block_size - 1) // block_size
    if np.any(need > max_blocks):
        raise ValueError("max_blocks too small for lens")
    num_blocks = int(need.sum()) + int(spare)
    perm = _rng(31, 2000, seed).permutation(num_blocks).astype(np.int32)
    table = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_blocks


def fp8_codes(shape, seed: int, scale: float, sigma: float = 1.0) -> np.ndarray:
    """Seeded FP8 E4M3 cache codes (uint8) for values sigma * N(0, 1) stored with a
    per-tensor dequantisation scale: codes = E4M3(x / scale), rounded to nearest
    even by torch's float8_e4m3fn cast (magnitudes are clipped to 448 first)."""
    import torch
    x = _rng(31, 3000, seed).standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    y = np.clip(x / np.float32(scale), -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
