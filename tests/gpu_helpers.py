"""Helpers shared by the GPU parity tests: seeded inputs on the device, exact
host copies for the oracle, and the tolerance rule."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import attn_inputs as A

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# max |err| on O against the float64 oracle, fp32 accumulation in every case
TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
# log-sum-exp is fp32 on every path; it only carries the rounding of fp32 sums
TOL_LSE = {"f32": 1e-4, "f16": 1e-3, "bf16": 1e-3}


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Exact upload of float32 values that are representable in `dtype`."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(TORCH_DT[dtype])


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def device_tensor(cfg, name: str, keep=(), device="cuda"):
    """Fill a [B, H, N, d] device tensor of config `cfg` slice by slice.

    Returns (tensor, {(b, h): float32 host slice for (b, h) in keep})."""
    H = cfg.H_q if name in ("q", "do") else cfg.H_kv
    N = cfg.N_q if name in ("q", "do") else cfg.N_kv
    t = torch.empty((cfg.B, H, N, cfg.d), dtype=TORCH_DT[cfg.dtype], device=device)
    keep = set(keep)
    kept = {}

    def gen(bh):
        b, h = divmod(bh, H)
        return b, h, A.slice_values(cfg.cid, name, b, h, N, cfg.d, cfg.sigma, cfg.dtype)

    with ThreadPoolExecutor(16) as ex:
        for b, h, x in ex.map(gen, range(cfg.B * H)):
            t[b, h] = torch.from_numpy(x).to(device).to(t.dtype)
            if (b, h) in keep:
                kept[(b, h)] = x
    return t, kept


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)))


def max_rel_err(got: np.ndarray, ref: np.ndarray, floor: float = 1e-3) -> float:
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def check_lse(got: np.ndarray, ref: np.ndarray, tol: float):
    """-inf must match exactly; finite entries within tol."""
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "empty-row pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), "non-finite lse"
    if fin.any():
        err = float(np.max(np.abs(got[fin] - ref[fin])))
        assert err <= tol, f"lse max err {err} > {tol}"
