"""The no-allocation decode entry point (GPU): same results as attn_decode_fwd.

attn_decode_fwd_noalloc keeps the split partials in the library's per-device
scratch array instead of a caller workspace. Two calls in a row, the second
with a smaller input, must each match attn_decode_fwd (bit for bit where both
use the same split plan, and within the bf16 tolerance where the scratch's
limit coarsens the split), and the oracle."""
import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import TOL_LSE, TOL_O, check_lse, max_abs_err
from oracle import attention_ref

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def _case(B, Hq, Hkv, Nkv, d, Nq, lens, seed, dtype="bf16", causal=False):
    q = A.random_tensor((B, Hq, Nq, d), seed, dtype)
    k = A.random_tensor((B, Hkv, Nkv, d), seed + 1, dtype)
    v = A.random_tensor((B, Hkv, Nkv, d), seed + 2, dtype)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    up = lambda x: torch.from_numpy(x).to(DEV).to(tdt)  # noqa: E731
    return q, k, v, up(q), up(k), up(v), torch.from_numpy(np.asarray(lens, np.int32)).to(DEV)


def _check(B, Hq, Hkv, Nkv, d, Nq, lens, seed, dtype="bf16", causal=False, same_bits=True):
    print(f"no-alloc decode B={B} Hq={Hq} Hkv={Hkv} Nkv={Nkv} d={d} Nq={Nq} seed={seed}", flush=True)
    q, k, v, qd, kd, vd, lens_d = _case(B, Hq, Hkv, Nkv, d, Nq, lens, seed, dtype, causal)
    o_ref, l_ref = E.attn_decode_fwd(qd, kd, vd, kv_lens=lens_d, causal=causal, return_lse=True)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    E.attn_decode_fwd_noalloc(qd, kd, vd, o, kv_lens=lens_d, lse=lse, causal=causal)
    torch.cuda.synchronize()
    if same_bits:
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    else:
        assert max_abs_err(o.float().cpu().numpy(), o_ref.float().cpu().numpy()) <= TOL_O[dtype]
    # and the oracle, on every head of the first and last request
    for b in (0, B - 1):
        ref_o, ref_l = attention_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal, d ** -0.5, kv_lens=lens[b:b + 1])
        assert max_abs_err(o[b:b + 1].float().cpu().numpy(), ref_o) <= TOL_O[dtype]
        check_lse(lse[b:b + 1].cpu().numpy(), ref_l, TOL_LSE[dtype])


def test_noalloc_decode_two_calls_second_smaller():
    _check(8, 32, 4, 5000, 128, 1, [5000, 1, 4097, 2600, 0, 77, 5000, 3333], seed=501)
    _check(3, 16, 2, 1200, 64, 3, [1200, 700, 5], seed=502, dtype="f16", causal=True)


def test_noalloc_decode_coarsened_split_then_smaller():
    """B*H_q*N_q*splits*(d+2)*4 beyond the scratch at the plan's split: the
    entry point takes fewer, longer splits (rounding may differ from
    attn_decode_fwd's), then a smaller call uses the same scratch again."""
    B, Hq, Hkv, Nq, Nkv = 16, 64, 8, 8, 32768
    assert E.attn_decode_workspace_size(B, Hq, Hkv, Nq, Nkv, 128, torch.bfloat16) > E.DECODE_SCRATCH_BYTES
    lens = np.random.default_rng(5).integers(1, Nkv + 1, size=B)
    lens[0] = Nkv
    _check(B, Hq, Hkv, Nkv, 128, Nq, lens, seed=503, causal=True, same_bits=False)
    _check(2, 8, 1, 3000, 128, 1, [3000, 1234], seed=504)
