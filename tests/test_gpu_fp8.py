"""GPU parity of the FP8 E4M3 KV-cache decode paths (contiguous and paged)
against the float64 oracle over the dequantised cache (MI355X only)."""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import TOL_LSE, TOL_O, check_lse, max_abs_err, to_device, to_host64
from oracle import attention_fp8kv_ref, gather_paged

pytestmark = pytest.mark.gpu

KS, VS = 2.0 ** -6, 2.0 ** -5   # per-tensor dequantisation scales (cache values ~ N(0, 1))


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _fp8_case(B, Hq, Hkv, Nkv, d, lens, Nq, causal, seed, poison=False):
    _announce(f"fp8 B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} causal={causal} lens={lens}")
    q = A.random_tensor((B, Hq, Nq, d), seed * 3, "bf16")
    kc = A.fp8_codes((B, Hkv, Nkv, d), seed * 3 + 1, KS)
    vc = A.fp8_codes((B, Hkv, Nkv, d), seed * 3 + 2, VS)
    kd, vd = _u8(kc), _u8(vc)
    lens_np = None if lens is None else np.asarray(lens, np.int32)
    lens_d = None if lens is None else torch.from_numpy(lens_np).cuda()
    if poison and lens is not None:
        for b, n in enumerate(lens_np):   # 0x7F is NaN in E4M3
            kd[b, :, n:] = 0x7F
            vd[b, :, n:] = 0x7F
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = E.attn_decode_fp8_fwd(to_device(q, "bf16"), kd, vd, KS, VS, kv_lens=lens_d,
                                   causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_fp8kv_ref(q, kc, vc, KS, VS, causal, scale, kv_lens=lens_np)
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    err = max_abs_err(got, oref)
    assert err <= TOL_O["bf16"], f"max |err| {err}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE["bf16"])


FP8 = [
    # B, Hq, Hkv, Nkv, d, lens, Nq
    (2, 8, 1, 1000, 128, [1000, 3], 1),
    (3, 32, 4, 3000, 128, [3000, 1500, 7], 1),
    (2, 16, 2, 2049, 64, [2049, 1234], 1),
    (4, 24, 2, 5000, 128, [5000, 4097, 128, 129], 4),
    (2, 8, 1, 4100, 128, [4100, 2049], 9),
    (1, 8, 2, 700, 64, None, 16),
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: "x".join(map(str, (c[0], c[1], c[2], c[3], c[4], c[6]))))
def test_fp8_decode_matches_oracle(case):
    B, Hq, Hkv, Nkv, d, lens, Nq = case
    _fp8_case(B, Hq, Hkv, Nkv, d, lens, Nq, Nq > 1, zlib.crc32(repr(case).encode()) % 10000)


def test_fp8_decode_never_reads_past_kv_lens():
    _fp8_case(3, 16, 2, 3000, 128, [2999, 5, 1500], 2, True, seed=83, poison=True)


def test_fp8_decode_tracks_the_bf16_path():
    """The same dequantised cache in bf16 (exact: scales are powers of two) gives
    the same attention through the 16-bit path, within the tolerance."""
    _announce("fp8 vs bf16 cache")
    B, Hq, Hkv, N, d = 2, 16, 2, 3000, 128
    q = to_device(A.random_tensor((B, Hq, 1, d), 91, "bf16"), "bf16")
    kc = A.fp8_codes((B, Hkv, N, d), 92, KS)
    vc = A.fp8_codes((B, Hkv, N, d), 93, VS)
    kd, vd = _u8(kc), _u8(vc)
    kb = (kd.view(torch.float8_e4m3fn).float() * KS).to(torch.bfloat16)
    vb = (vd.view(torch.float8_e4m3fn).float() * VS).to(torch.bfloat16)
    o8 = E.attn_decode_fp8_fwd(q, kd, vd, KS, VS)
    o16 = E.attn_decode_fwd(q, kb, vb)
    torch.cuda.synchronize()
    assert max_abs_err(to_host64(o8), to_host64(o16)) <= 2 * TOL_O["bf16"]


@pytest.mark.parametrize("bs", [16, 64])
def test_paged_fp8_decode_matches_oracle(bs):
    B, Hq, Hkv, d, Nq = 3, 16, 2, 128, 3
    lens = np.array([2900, 17, 1300], np.int32)
    maxb = 3000 // bs + 1
    _announce(f"paged fp8 bs={bs}")
    table, nblk = A.paged_layout(lens, bs, maxb, seed=bs, spare=2)
    q = A.random_tensor((B, Hq, Nq, d), 94 + bs, "bf16")
    kp = A.fp8_codes((nblk, Hkv, bs, d), 95 + bs, KS)
    vp = A.fp8_codes((nblk, Hkv, bs, d), 96 + bs, VS)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = E.attn_decode_paged_fp8_fwd(to_device(q, "bf16"), _u8(kp), _u8(vp), KS, VS,
                                         torch.from_numpy(table).cuda(),
                                         kv_lens=torch.from_numpy(lens).cuda(), causal=True,
                                         scale=scale, return_lse=True)
    torch.cuda.synchronize()
    kc = gather_paged(kp, table, lens, bs)
    vc = gather_paged(vp, table, lens, bs)
    oref, lref = attention_fp8kv_ref(q, kc, vc, KS, VS, True, scale, kv_lens=lens)
    err = max_abs_err(to_host64(o), oref)
    assert err <= TOL_O["bf16"], f"max |err| {err}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE["bf16"])
