"""GPU parity of attn_backward (dQ, dK, dV by recomputation) against the
float64 oracle of the gradients (MI355X only). The forward's O and LSE come
from attn_prefill_fwd, as they would in training."""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import to_device, to_host64
from oracle import attention_backward_ref

pytestmark = pytest.mark.gpu

# max |err| of each gradient over max |reference| of that gradient: the kernel
# rounds P, dS and O to the 16-bit type (relative 2^-9 each) and accumulates in
# fp32; 2e-2 leaves a wide margin over that.
TOL_GRAD = 2e-2


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _run(B, Hq, Hkv, Nq, Nkv, d, causal, dtype, seed):
    _announce(f"bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} causal={causal} {dtype}")
    q = A.random_tensor((B, Hq, Nq, d), seed * 4, dtype)
    k = A.random_tensor((B, Hkv, Nkv, d), seed * 4 + 1, dtype)
    v = A.random_tensor((B, Hkv, Nkv, d), seed * 4 + 2, dtype)
    do = A.random_tensor((B, Hq, Nq, d), seed * 4 + 3, dtype)
    scale = float(np.float32(1 / math.sqrt(d)))
    qd, kd, vd, gd = (to_device(x, dtype) for x in (q, k, v, do))
    o, lse = E.attn_prefill_fwd(qd, kd, vd, causal=causal, scale=scale, return_lse=True)
    dq, dk, dv = E.attn_backward(qd, kd, vd, o, gd, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    refs = attention_backward_ref(q, k, v, do, causal, scale)
    errs = {}
    for name, got, ref in (("dq", dq, refs[0]), ("dk", dk, refs[1]), ("dv", dv, refs[2])):
        g = to_host64(got)
        assert np.all(np.isfinite(g)), f"{name} not finite"
        if ref.size == 0:
            continue
        mx = float(np.abs(ref).max())
        err = float(np.abs(g - ref).max())
        errs[name] = (err, err / max(mx, 1e-30))
        if mx == 0.0:
            assert err == 0.0, f"{name}: expected zeros"
        else:
            assert err <= TOL_GRAD * mx, f"{name}: max|err| {err:.3e} vs max|ref| {mx:.3e}"
    print("  max|err| (absolute, relative to max|ref|):",
          {k2: f"{a:.2e}, {r:.2e}" for k2, (a, r) in errs.items()}, flush=True)
    return dq, dk, dv


BWD = [
    # B, Hq, Hkv, Nq, Nkv, d
    (1, 2, 2, 100, 100, 64),
    (2, 4, 1, 200, 300, 128),     # GQA, N_q < N_kv
    (1, 8, 2, 257, 257, 128),     # ragged tails of every tile
    (2, 2, 2, 64, 192, 64),
    (1, 4, 4, 130, 70, 128),      # N_q > N_kv: causal rows without keys
    (1, 2, 1, 1, 50, 128),        # one query row
    (1, 4, 4, 1000, 1000, 128),
    # d = 64 across several 256-key dK/dV workgroups and 256-row dQ blocks,
    # N_q != N_kv both ways
    (1, 4, 2, 700, 900, 64),
    (2, 2, 2, 900, 700, 64),
    (1, 2, 1, 600, 600, 64),
    # (batch, head) unit counts around the work order's groups of 32: 33 heads
    # (a group of 32 and one of 1), 40 (32 + 8), 7, each over several blocks
    (1, 33, 33, 300, 300, 64),
    (5, 8, 8, 300, 300, 128),
    (7, 1, 1, 520, 520, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", BWD, ids=lambda c: "x".join(map(str, c)))
def test_backward_matches_oracle(case, causal, dtype):
    seed = zlib.crc32(repr((case, causal, dtype)).encode()) % 10000
    _run(*case, causal, dtype, seed)


def test_backward_is_deterministic():
    _announce("bwd determinism")
    q = to_device(A.random_tensor((2, 8, 700, 128), 1, "bf16"), "bf16")
    k = to_device(A.random_tensor((2, 2, 700, 128), 2, "bf16"), "bf16")
    v = to_device(A.random_tensor((2, 2, 700, 128), 3, "bf16"), "bf16")
    do = to_device(A.random_tensor((2, 8, 700, 128), 4, "bf16"), "bf16")
    o, lse = E.attn_prefill_fwd(q, k, v, causal=True, return_lse=True)
    a = E.attn_backward(q, k, v, o, do, lse, causal=True)
    b = E.attn_backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_no_keys_and_no_queries():
    _announce("bwd empty sides")
    q = to_device(A.random_tensor((1, 2, 40, 64), 5, "bf16"), "bf16")
    k = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = E.attn_prefill_fwd(q, k, k, return_lse=True)
    dq = torch.full_like(q, 7.0)
    E.attn_backward(q, k, k, o, q.clone(), lse, dq=dq)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq) == 0
    # no query rows: dK and dV are zero
    q0 = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k1 = to_device(A.random_tensor((1, 2, 33, 64), 6, "bf16"), "bf16")
    lse0 = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k1, 3.0)
    dv = torch.full_like(k1, 3.0)
    E.attn_backward(q0, k1, k1, q0, q0, lse0, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0
