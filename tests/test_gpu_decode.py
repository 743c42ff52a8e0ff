"""GPU parity of attn_decode_fwd (split-KV GQA decode + LSE merge) against the
float64 oracle (MI355X only)."""
import math
import os
import sys
import zlib

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import TOL_LSE, TOL_O, check_lse, device_tensor, max_abs_err, to_device, to_host64
from oracle import attention_head_rows, attention_ref

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _decode_case(B, Hq, Hkv, Nkv, d, dtype, lens, seed, poison=False, Nq=1, causal=False):
    _announce(f"decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} {dtype} causal={causal} "
              f"lens={None if lens is None else list(lens)[:6]}")
    q = A.random_tensor((B, Hq, Nq, d), seed * 3, dtype)
    k = A.random_tensor((B, Hkv, Nkv, d), seed * 3 + 1, dtype)
    v = A.random_tensor((B, Hkv, Nkv, d), seed * 3 + 2, dtype)
    kd, vd = to_device(k, dtype), to_device(v, dtype)
    lens_d = None
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int32)
        lens_d = torch.from_numpy(lens).cuda()
        if poison:   # positions past each request's length must never be read
            for b, n in enumerate(lens):
                kd[b, :, n:] = float("nan")
                vd[b, :, n:] = float("nan")
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = E.attn_decode_fwd(to_device(q, dtype), kd, vd, kv_lens=lens_d, scale=scale,
                               causal=causal, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_ref(q, k, v, causal, scale, kv_lens=lens)
    got = to_host64(o)
    assert np.all(np.isfinite(got))
    err = max_abs_err(got, oref)
    assert err <= TOL_O[dtype], f"max |err| {err}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE[dtype])


CASES = [
    # B, Hq, Hkv, Nkv, d, lens
    (1, 8, 1, 1, 128, None), (2, 8, 1, 100, 128, None), (3, 32, 4, 1000, 128, [1000, 1, 517]),
    (2, 4, 4, 300, 64, [0, 300]), (2, 16, 1, 2049, 128, [2049, 1234]), (1, 32, 1, 700, 64, None),
    (4, 24, 2, 5000, 128, [5000, 4097, 128, 129]), (2, 2, 2, 130, 128, None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_decode_small_matches_oracle(case, dtype):
    *shape, lens = case
    _decode_case(*shape, dtype, lens, seed=zlib.crc32(repr((case, dtype)).encode()) % 10000)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_never_reads_past_kv_lens(dtype):
    _decode_case(3, 16, 2, 3000, 128, dtype, [2999, 5, 1500], seed=77, poison=True)


# multi-token decode: N_q new tokens per request (speculative verification,
# chunked prefill against a cache), bottom-right causal alignment per request
MULTI = [
    # B, Hq, Hkv, Nkv, d, Nq, lens
    (2, 8, 1, 1000, 128, 4, [1000, 3]),          # request 1: fewer keys than queries
    (3, 32, 4, 3000, 128, 7, [3000, 1500, 7]),
    (2, 4, 4, 500, 64, 16, None),                # G * N_q = 16: one full column group
    (1, 16, 2, 2500, 128, 33, None),             # 264 columns: ragged last group
    (2, 8, 1, 4100, 128, 64, [4100, 2049]),      # 512 columns per KV head
    (2, 2, 1, 5000, 64, 2, [4999, 130]),
    (1, 8, 8, 64, 128, 64, None),                # N_q == N_kv: plain causal prefill
    (2, 8, 2, 1500, 64, 5, [1500, 700]),         # d = 64, 20 columns: two groups per wavefront
    (1, 8, 1, 900, 64, 9, None),                 # d = 64, 72 columns: four groups per wavefront
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", MULTI, ids=lambda c: "x".join(map(str, c[:6])))
def test_decode_multi_token_matches_oracle(case, dtype, causal):
    B, Hq, Hkv, Nkv, d, Nq, lens = case
    _decode_case(B, Hq, Hkv, Nkv, d, dtype, lens,
                 seed=zlib.crc32(repr((case, dtype, causal)).encode()) % 10000, Nq=Nq,
                 causal=causal)


@pytest.mark.parametrize("Nq", [3, 16])
def test_decode_multi_token_never_reads_past_kv_lens(Nq):
    _decode_case(3, 16, 2, 3000, 128, "bf16", [2999, 5, 1500], seed=78, poison=True, Nq=Nq,
                 causal=True)


def test_decode_multi_token_agrees_with_prefill():
    """N_q new tokens against a full cache: the decode path and the prefill path
    compute the same causal attention (each against the oracle's tolerance)."""
    _announce("decode vs prefill, B=2 Hq=16 Hkv=2 Nq=8 Nkv=3000")
    q = to_device(A.random_tensor((2, 16, 8, 128), 11, "bf16"), "bf16")
    k = to_device(A.random_tensor((2, 2, 3000, 128), 12, "bf16"), "bf16")
    v = to_device(A.random_tensor((2, 2, 3000, 128), 13, "bf16"), "bf16")
    od, ld = E.attn_decode_fwd(q, k, v, causal=True, return_lse=True)
    op, lp = E.attn_prefill_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert max_abs_err(to_host64(od), to_host64(op)) <= 2 * TOL_O["bf16"]
    assert float((ld - lp).abs().max()) <= 2 * TOL_LSE["bf16"]


def test_decode_causal_flag_is_a_no_op_for_one_query():
    q = to_device(A.random_tensor((2, 8, 1, 128), 5, "bf16"), "bf16")
    k = to_device(A.random_tensor((2, 1, 333, 128), 6, "bf16"), "bf16")
    v = to_device(A.random_tensor((2, 1, 333, 128), 7, "bf16"), "bf16")
    o1 = E.attn_decode_fwd(q, k, v, causal=False)
    o2 = E.attn_decode_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.slow
@pytest.mark.parametrize("ragged", [False, True])
def test_decode_config5_full_size(ragged):
    """Config 5 (B=64, H_q=32, H_kv=4, KV 32768, bf16), every query head checked."""
    cfg = A.CONFIGS[6 if ragged else 5]
    _announce(cfg.name)
    lens = A.ragged_lengths(cfg) if ragged else np.full(cfg.B, cfg.N_kv, np.int32)
    kv_keep = [(b, g) for b in range(cfg.B) for g in range(cfg.H_kv)]
    q, qk = device_tensor(cfg, "q", keep=[(b, h) for b in range(cfg.B) for h in range(cfg.H_q)])
    k, kk = device_tensor(cfg, "k", keep=kv_keep)
    v, vk = device_tensor(cfg, "v", keep=kv_keep)
    lens_d = torch.from_numpy(lens).cuda()
    o, lse = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    og = to_host64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(cfg.B):
        for h in range(cfg.H_q):
            g = h // cfg.G
            oref, lref = attention_head_rows(qk[(b, h)], [0], 1, kk[(b, g)], vk[(b, g)], False,
                                             cfg.scale, n=int(lens[b]))
            err = max_abs_err(og[b, h], oref)
            worst = max(worst, err)
            assert err <= TOL_O[cfg.dtype], f"(b={b}, h={h}) max |err| {err}"
            check_lse(lg[b, h], lref, TOL_LSE[cfg.dtype])
    print(f"{cfg.name}: worst max|err| = {worst:.3e}", flush=True)


@pytest.mark.parametrize("chunk", [128, 384, 1024, 8192])
def test_decode_split_size_does_not_change_the_result(chunk, tune):
    """The split of the KV sequence is a performance choice only: every split size
    matches the oracle (and so each other) within the tolerance."""
    tune(decode_chunk=chunk)
    _decode_case(3, 16, 2, 5000, 128, "bf16", [5000, 1, 2600], seed=91)
    _decode_case(2, 8, 2, 3000, 128, "bf16", [3000, 2000], seed=92, Nq=5, causal=True)


@pytest.mark.parametrize("groups", ["1", "2", "4"])
def test_decode_column_groups_per_wavefront_agree(groups, tune):
    """How many 16-column groups one wavefront serves is a performance choice:
    every setting matches the oracle."""
    tune(decode_groups=groups)
    _decode_case(2, 16, 2, 2100, 128, "bf16", [2100, 999], seed=93, Nq=6, causal=True)
    _decode_case(2, 8, 2, 1100, 64, "f16", [1100, 64], seed=94, Nq=3, causal=True)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", MULTI, ids=lambda c: "x".join(map(str, c[:6])))
def test_decode_rows_mode_matches_oracle(case, dtype, causal, tune):
    """Multi-token decode through the prefill kernel in rows mode (forced here;
    chosen automatically for many rows per KV head and many KV heads)."""
    tune(decode_rows_mode=1)
    B, Hq, Hkv, Nkv, d, Nq, lens = case
    _decode_case(B, Hq, Hkv, Nkv, d, dtype, lens,
                 seed=zlib.crc32(repr((case, dtype, causal, "rows")).encode()) % 10000, Nq=Nq,
                 causal=causal)


def test_decode_rows_mode_chosen_for_tall_batches():
    """64 requests x 4 KV heads x (8 heads x 16 tokens) rows: rows mode by default."""
    lens = np.random.default_rng(3).integers(1, 2001, size=64).astype(np.int32)
    _decode_case(64, 32, 4, 2000, 128, "bf16", lens, seed=95, Nq=16, causal=True)


@pytest.mark.parametrize("form", ["4", "5"], ids=["ring", "staged"])
@pytest.mark.parametrize("case", [MULTI[2], MULTI[4], MULTI[7]], ids=lambda c: "x".join(map(str, c[:6])))
def test_decode_rows_mode_both_kernel_forms(case, form, tune):
    """Rows mode through either form of the prefill kernel (K/V tiles streamed
    by direct loads, or staged through registers)."""
    tune(decode_rows_mode=1)
    tune(prefill_variant=form)
    B, Hq, Hkv, Nkv, d, Nq, lens = case
    _decode_case(B, Hq, Hkv, Nkv, d, "bf16", lens,
                 seed=zlib.crc32(repr((case, form)).encode()) % 10000, Nq=Nq, causal=True)


@pytest.mark.parametrize("mix", ["uniform", "ragged", "short"])
def test_decode_device_chosen_split_matches_oracle(mix):
    """Enough (request, KV head) pairs that the grid is full: the kernels then
    raise the split size on the device from the actual lengths (to about one
    unit per wavefront), and the merge must find the same splits. "short":
    requests of at most 600 keys in an 8192-position cache, where the split
    stays at the plan's finest (128 keys) and each request spreads over
    several wavefronts."""
    rng = np.random.default_rng(7)
    lens = {"uniform": None, "ragged": rng.integers(1, 8193, size=40),
            "short": rng.integers(1, 601, size=40)}[mix]
    _decode_case(40, 32, 4, 8192, 64, "bf16", lens, seed=96)
    _decode_case(40, 32, 4, 8192, 64, "bf16", lens, seed=97, Nq=3, causal=True)


@pytest.mark.parametrize("chunk", [0, 128], ids=["plan", "fine"])
def test_decode_workspace_contents_do_not_matter(chunk, tune):
    """The workspace needs no initialisation: filled with NaN bytes beforehand
    it gives the same bits as a zeroed one (ragged lengths, so most rows use
    fewer splits than the workspace holds; 128-key splits give more than 16
    partials per row)."""
    if chunk:
        tune(decode_chunk=chunk)
    B, Hq, Hkv, N, d = 6, 16, 2, 3000, 128
    q = to_device(A.random_tensor((B, Hq, 1, d), 601, "bf16"), "bf16")
    k = to_device(A.random_tensor((B, Hkv, N, d), 602, "bf16"), "bf16")
    v = to_device(A.random_tensor((B, Hkv, N, d), 603, "bf16"), "bf16")
    lens = torch.tensor([3000, 1, 2049, 0, 700, 2999], dtype=torch.int32, device="cuda")
    size = E.attn_decode_workspace_size(B, Hq, Hkv, 1, N, d, torch.bfloat16)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((size,), fill, dtype=torch.uint8, device="cuda")
        o, lse = E.attn_decode_fwd(q, k, v, kv_lens=lens, workspace=ws, return_lse=True)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[1][0]).all()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
