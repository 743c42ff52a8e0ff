"""GPU parity of attn_prefill_fwd against the float64 oracle (MI355X only)."""
import math
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


def _run_small(B, Hq, Hkv, Nq, Nkv, d, dtype, causal, seed, sigma=1.0, scale=None):
    _announce(f"prefill B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} {dtype} causal={causal}")
    q = A.random_tensor((B, Hq, Nq, d), seed * 3 + 0, dtype, sigma)
    k = A.random_tensor((B, Hkv, Nkv, d), seed * 3 + 1, dtype, sigma)
    v = A.random_tensor((B, Hkv, Nkv, d), seed * 3 + 2, dtype, sigma)
    scale = float(np.float32(1 / math.sqrt(d))) if scale is None else scale
    o, lse = E.attn_prefill_fwd(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                                causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_ref(q, k, v, causal, scale)
    err = max_abs_err(to_host64(o), oref)
    assert err <= TOL_O[dtype], f"max |err| {err} > {TOL_O[dtype]}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE[dtype])
    return err


SMALL = [
    # B, Hq, Hkv, Nq, Nkv, d
    (1, 1, 1, 1, 1, 64), (1, 2, 1, 17, 17, 64), (2, 2, 2, 63, 63, 128), (1, 1, 1, 64, 64, 128),
    (1, 4, 2, 65, 65, 64), (1, 2, 2, 127, 127, 128), (2, 8, 1, 129, 129, 128),
    (1, 8, 2, 200, 200, 64), (1, 4, 4, 1000, 1000, 128),
    # rectangular: queries at the end of a longer key sequence, and more queries than keys
    (1, 2, 1, 37, 300, 128), (1, 2, 2, 130, 70, 64), (2, 4, 2, 1, 257, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_prefill_small_matches_oracle(shape, causal, dtype):
    _run_small(*shape, dtype, causal, seed=zlib.crc32(repr((shape, causal, dtype)).encode()) % 10000)


# One work item per workgroup (too few items for the persistent grid): the
# work order deals (batch, head) units in groups of 32, block-major; these unit
# counts leave a partial group (33, 40, 70), a group that is not a multiple of
# 8 (7, 12, 33) and one that is (32, 40's first), with several query blocks.
ONE_ITEM_GRIDS = [
    # B, Hq, Hkv, Nq, Nkv, d, dtype
    (1, 33, 3, 300, 300, 64, "f16"),
    (5, 8, 2, 520, 520, 128, "bf16"),
    (7, 1, 1, 300, 300, 64, "bf16"),
    (1, 12, 12, 400, 400, 64, "f16"),
    (2, 35, 5, 260, 300, 128, "bf16"),
    (1, 32, 4, 600, 600, 128, "f16"),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", ONE_ITEM_GRIDS, ids=lambda c: "x".join(map(str, c)))
def test_prefill_one_item_grid_work_order(case, causal):
    B, Hq, Hkv, Nq, Nkv, d, dtype = case
    _run_small(B, Hq, Hkv, Nq, Nkv, d, dtype, causal,
               seed=zlib.crc32(repr((case, causal, "order")).encode()) % 10000)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_prefill_no_keys_gives_zero_and_neg_inf(dtype):
    q = to_device(A.random_tensor((1, 2, 5, 64), 1, dtype), dtype)
    k = torch.empty((1, 1, 0, 64), dtype=q.dtype, device="cuda")
    o, lse = E.attn_prefill_fwd(q, k, k.clone(), causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_prefill_empty_batch_is_noop():
    q = torch.empty((0, 2, 5, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 2, 5, 64), dtype=torch.bfloat16, device="cuda")
    o = E.attn_prefill_fwd(q, k, k.clone())
    assert o.shape == q.shape


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_masked_positions_do_not_leak_bit_exact(d):
    """Perturbing keys/values at positions >= j with large finite values leaves
    causal rows < j bit-identical (at d = 64 too, where rows j..j+9 share a
    wavefront with rows below j and their scores overflow the first pass of
    the softmax step)."""
    _announce(f"prefill masked-position bit identity d={d}")
    B, H, N, j = 1, 2, 300, 150
    q = to_device(A.random_tensor((B, H, N, d), 11, "bf16"), "bf16")
    k = to_device(A.random_tensor((B, H, N, d), 12, "bf16"), "bf16")
    v = to_device(A.random_tensor((B, H, N, d), 13, "bf16"), "bf16")
    o1 = E.attn_prefill_fwd(q, k, v, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, j:] = 3.0e4
    v2[:, :, j:] = -1.0e30
    o2 = E.attn_prefill_fwd(q, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :j], o2[:, :, :j])


def test_prefill_reads_nothing_outside_its_tensors():
    """Tensors placed inside NaN-filled allocations: outputs stay finite and equal."""
    _announce("prefill NaN guard bands")
    B, Hq, Hkv, N, d = 1, 4, 2, 97, 64
    dt = "f16"
    host = [A.random_tensor((B, h, N, d), 20 + i, dt) for i, h in enumerate((Hq, Hkv, Hkv))]
    clean = [to_device(x, dt) for x in host]
    guarded = []
    for x in clean:
        buf = torch.full((x.numel() + 8192,), float("nan"), dtype=x.dtype, device="cuda")
        view = buf[4096:4096 + x.numel()].view(x.shape)
        view.copy_(x)
        guarded.append(view)
    for causal in (False, True):
        o1 = E.attn_prefill_fwd(*clean, causal=causal)
        o2 = E.attn_prefill_fwd(*guarded, causal=causal)
        torch.cuda.synchronize()
        assert torch.isfinite(o2).all()
        assert torch.equal(o1, o2)


def test_prefill_config1_full():
    cfg = A.CONFIGS[1]
    _announce(cfg.name)
    q, k, v = (A.tensor_values(cfg, t) for t in "qkv")
    o, lse = E.attn_prefill_fwd(to_device(q, "f32"), to_device(k, "f32"), to_device(v, "f32"),
                                causal=cfg.causal, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_ref(q, k, v, cfg.causal, cfg.scale)
    err = max_abs_err(to_host64(o), oref)
    assert err <= 1e-4, err
    check_lse(lse.cpu().numpy().astype(np.float64), lref, 1e-4)


def _sample_rows(N, rng, extra=48, item_rows=(128, 256)):
    """Rows 0, 1, the last two, the middle, both sides of every boundary between
    work items (multiples of the 128- and 256-row query blocks, where a
    persistent workgroup hands over to its next item), tile edges near both
    ends, and random rows."""
    base = {0, 1, N - 1, N - 2, N // 2}
    for t in (63, 64, 65, 127, 128, 129, 255, 256):
        base.update(x for x in (t, N - t) if 0 <= x < N)
    for bm in item_rows:
        for edge in range(bm, N, bm):
            base.update((edge - 1, edge))
    base.update(rng.integers(0, N, size=extra).tolist())
    return np.array(sorted(base))


@pytest.mark.slow
@pytest.mark.parametrize("cid", [2, 3, 4])
def test_prefill_full_size_sampled(cid):
    """Full-size configs in the benchmark's launch configuration; every head is
    checked on sampled rows (every work-item boundary, tile edges, ends, random
    rows)."""
    cfg = A.CONFIGS[cid]
    _announce(f"config {cid}: {cfg.name}")
    rng = np.random.default_rng(cid)
    G = cfg.G
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H_q)]
    q, qk = device_tensor(cfg, "q", keep=heads)
    k, kk = device_tensor(cfg, "k", keep=[(b, h // G) for b, h in heads])
    v, vk = device_tensor(cfg, "v", keep=[(b, h // G) for b, h in heads])
    o, lse = E.attn_prefill_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    worst = 0.0
    for (b, h) in heads:
        rows = _sample_rows(cfg.N_q, rng, extra=16)
        oref, lref = attention_head_rows(qk[(b, h)][rows], rows, cfg.N_q, kk[(b, h // G)],
                                         vk[(b, h // G)], cfg.causal, cfg.scale)
        got = o[b, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        err = max_abs_err(got, oref)
        worst = max(worst, err)
        assert err <= TOL_O[cfg.dtype], f"(b={b}, h={h}) max |err| {err}"
        check_lse(lse[b, h, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64), lref,
                  TOL_LSE[cfg.dtype])
    print(f"config {cid}: worst sampled max|err| = {worst:.3e}", flush=True)


# more work items than workgroups: a persistent grid walks several items per
# workgroup (d = 128: one workgroup per compute unit; d = 64: three)
MANY_ITEMS = [(2, 64, 64, 700, 700, 128), (4, 64, 16, 500, 500, 64), (1, 48, 8, 1100, 2000, 128)]


@pytest.mark.parametrize("form", [None, "4", "5"], ids=["default", "ring", "staged"])
@pytest.mark.parametrize("slots", [None, "16", "8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", MANY_ITEMS, ids=lambda s: "x".join(map(str, s)))
def test_prefill_persistent_grid_many_items(shape, causal, slots, form, tune):
    """Several items per workgroup: a persistent grid of 8 or 16 workgroups (or
    the automatic choice) walks every query block exactly once, with the K/V
    tiles staged through registers or streamed by direct loads across items."""
    if slots is not None:
        tune(prefill_slots=slots)
    if form is not None:
        tune(prefill_variant=form)
    _run_small(*shape, "bf16", causal, seed=zlib.crc32(repr((shape, causal)).encode()) % 10000)


@pytest.mark.parametrize("variant", ["1", "2", "3", "4", "5"])
def test_prefill_variants_match_oracle(variant, tune):
    """Every alternative kernel behind the prefill_variant knob (tuning only) meets
    the same bar as the default."""
    tune(prefill_variant=variant)
    for i, (shape, causal, dtype) in enumerate([
            ((1, 4, 2, 300, 300, 128), True, "bf16"), ((2, 2, 2, 129, 257, 64), True, "f16"),
            ((1, 8, 8, 200, 200, 128), False, "f16"), ((1, 2, 1, 70, 30, 64), True, "bf16")]):
        _run_small(*shape, dtype, causal, seed=100 + 10 * int(variant) + i)


@pytest.mark.parametrize("rising", [True, False], ids=["rising", "falling"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (64, "bf16"), (128, "bf16")])
def test_prefill_rescales_when_scores_grow_along_the_keys(d, dtype, causal, rising):
    """Key norms grow by 1.5x per 64 keys (or shrink): with rising scores every
    tile's maximum exceeds the row's reference by more than the lazy-rescale
    margin, so the rescale path runs on most tiles (at d = 64 also the fallback
    from the max-free fast path); with falling scores it almost never does."""
    B, H, N = 1, 4, 700
    seed = zlib.crc32(repr((d, dtype, causal, rising)).encode()) % 10000
    _announce(f"prefill growing scores d={d} {dtype} causal={causal} rising={rising}")
    q = A.random_tensor((B, H, N, d), seed * 3, dtype)
    k = A.random_tensor((B, H, N, d), seed * 3 + 1, dtype)
    v = A.random_tensor((B, H, N, d), seed * 3 + 2, dtype)
    f = 1.5 ** (np.arange(N) / 64.0)
    if not rising:
        f = f[::-1]
    k = A.round_to_dtype((k * f[None, None, :, None].astype(np.float32)).astype(np.float32), dtype)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = E.attn_prefill_fwd(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                                causal=causal, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    oref, lref = attention_ref(q, k, v, causal, scale)
    err = max_abs_err(to_host64(o), oref)
    assert err <= TOL_O[dtype], f"max |err| {err}"
    check_lse(lse.cpu().numpy().astype(np.float64), lref, TOL_LSE[dtype])
