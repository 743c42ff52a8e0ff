"""Full-size parity of the workloads that bench.py times beside the headline
prefill: multi-token decode (4 and 64 new tokens per request), paged and FP8
decode against config 5's 32768-token cache, and the backward pass of config
2 (plus a GQA backward of 32 query heads over 4 KV heads). Each runs in the
benchmark's launch configuration on the whole batch; the float64 oracle then
checks sampled heads one by one (MI355X only)."""
import sys

import numpy as np
import pytest
import torch

import attn_inputs as A
import exact_attention_31_amd as E
from gpu_helpers import TOL_LSE, TOL_O, check_lse, device_tensor, max_abs_err, to_host64
from oracle import attention_backward_ref, attention_fp8kv_ref, attention_head_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# requests whose KV heads are kept on the host for the oracle (first, last, two inside)
SAMPLED_REQUESTS = (0, 13, 38, 63)


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def c5_cache():
    """Config 5's K and V caches on the device (bf16, [64, 4, 32768, 128]) and
    the host copies of the sampled requests' KV heads."""
    cfg = A.CONFIGS[5]
    _announce("config 5 cache")
    keep = [(b, g) for b in SAMPLED_REQUESTS for g in range(cfg.H_kv)]
    k, kk = device_tensor(cfg, "k", keep=keep)
    v, vk = device_tensor(cfg, "v", keep=keep)
    yield cfg, k, v, kk, vk
    del k, v
    torch.cuda.empty_cache()


def _sampled_heads(cfg):
    """Two query heads of every KV head of every sampled request."""
    G = cfg.G
    return [(b, g * G + j) for b in SAMPLED_REQUESTS for g in range(cfg.H_kv) for j in (0, G - 1)]


@pytest.mark.parametrize("cid", [7, 8])
def test_decode_multi_token_full_size_sampled(c5_cache, cid):
    """4 and 64 new tokens per request, causal (bottom-right) against the full
    cache: the 4-token step runs the split-KV kernels, the 64-token step the
    prefill kernel in rows mode."""
    _, k, v, kk, vk = c5_cache
    cfg = A.CONFIGS[cid]
    _announce(cfg.name)
    heads = _sampled_heads(cfg)
    q, qk = device_tensor(cfg, "q", keep=heads)
    lens_d = torch.full((cfg.B,), cfg.N_kv, dtype=torch.int32, device="cuda")
    o, lse = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal,
                               return_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(cfg.N_q)
    worst = 0.0
    for b, h in heads:
        g = h // cfg.G
        oref, lref = attention_head_rows(qk[(b, h)], rows, cfg.N_q, kk[(b, g)], vk[(b, g)],
                                         cfg.causal, cfg.scale)
        err = max_abs_err(to_host64(o[b, h]), oref)
        worst = max(worst, err)
        assert err <= TOL_O[cfg.dtype], f"(b={b}, h={h}) max |err| {err}"
        check_lse(lse[b, h].cpu().numpy().astype(np.float64), lref, TOL_LSE[cfg.dtype])
    print(f"{cfg.name}: worst sampled max|err| = {worst:.3e}", flush=True)


def test_paged_decode_config5_full_size(c5_cache, tune):
    """Config 5 through a paged cache of 16-position blocks scattered over a
    pool in a seeded order (the benchmark's layout): the same bits as the
    contiguous path on every head, and the oracle on the sampled ones."""
    cfg, k, v, kk, vk = c5_cache
    _announce("config 5, paged, block 16")
    B, H_kv, N, d = k.shape
    bs = 16
    nb = N // bs
    lens = np.full(B, N, np.int32)
    table, nblk = A.paged_layout(lens, bs, nb, seed=5)
    perm = torch.from_numpy(table.reshape(-1).astype(np.int64)).cuda()
    kp = torch.empty((nblk, H_kv, bs, d), dtype=k.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = k.reshape(B, H_kv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, bs, d)
    vp[perm] = v.reshape(B, H_kv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, bs, d)
    heads = _sampled_heads(cfg)
    q, qk = device_tensor(cfg, "q", keep=heads)
    lens_d = torch.from_numpy(lens).cuda()
    o, lse = E.attn_decode_paged_fwd(q, kp, vp, torch.from_numpy(table).cuda(), kv_lens=lens_d,
                                     scale=cfg.scale, return_lse=True)
    # paged caches keep 2048-key splits; the contiguous path, held to the same
    # split, must give the same bits
    tune(decode_chunk=2048)
    oc, lc = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    del kp, vp
    for b, h in heads:
        g = h // cfg.G
        oref, lref = attention_head_rows(qk[(b, h)], np.arange(1), 1, kk[(b, g)], vk[(b, g)], False,
                                         cfg.scale)
        err = max_abs_err(to_host64(o[b, h]), oref)
        assert err <= TOL_O[cfg.dtype], f"(b={b}, h={h}) max |err| {err}"
        check_lse(lse[b, h].cpu().numpy().astype(np.float64), lref, TOL_LSE[cfg.dtype])


def test_fp8_decode_config5_full_size_sampled(c5_cache):
    """Config 5's cache as FP8 E4M3 codes with per-tensor scales 2^-6 (the
    benchmark's setting); the oracle dequantises the same codes."""
    cfg, k, v, _, _ = c5_cache
    _announce("config 5, FP8 E4M3 cache")
    k_scale = v_scale = 2.0 ** -6
    kc = (k.float() / k_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (v.float() / v_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    heads = _sampled_heads(cfg)
    q, qk = device_tensor(cfg, "q", keep=heads)
    lens_d = torch.full((cfg.B,), cfg.N_kv, dtype=torch.int32, device="cuda")
    o, lse = E.attn_decode_fp8_fwd(q, kc, vc, k_scale, v_scale, kv_lens=lens_d, scale=cfg.scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    worst = 0.0
    for b, h in heads:
        g = h // cfg.G
        kcode = kc[b, g].cpu().numpy()[None, None]
        vcode = vc[b, g].cpu().numpy()[None, None]
        oref, lref = attention_fp8kv_ref(qk[(b, h)][None, None], kcode, vcode, k_scale, v_scale, False,
                                         cfg.scale)
        err = max_abs_err(to_host64(o[b, h]), oref[0, 0])
        worst = max(worst, err)
        assert err <= TOL_O[cfg.dtype], f"(b={b}, h={h}) max |err| {err}"
        check_lse(lse[b, h].cpu().numpy().astype(np.float64), lref[0, 0], TOL_LSE[cfg.dtype])
    print(f"fp8 decode: worst sampled max|err| = {worst:.3e}", flush=True)


def test_backward_config2_full_size_sampled():
    """The backward pass of config 2 (causal MHA bf16, 4 x 32 heads of 4096 rows)
    with a seeded output gradient; whole heads of dQ, dK and dV checked for a
    sample of (batch, head) pairs. Tolerance as for the small cases: max |err|
    of each gradient within 2e-2 of its largest reference entry."""
    cfg = A.CONFIGS[2]
    _announce("config 2, backward")
    rng = np.random.default_rng(2)
    picks = rng.choice(cfg.B * cfg.H_q, size=16, replace=False)
    heads = sorted({(0, 0), (cfg.B - 1, cfg.H_q - 1)} | {divmod(int(x), cfg.H_q) for x in picks})
    assert len(heads) >= 16
    q, qk = device_tensor(cfg, "q", keep=heads)
    k, kk = device_tensor(cfg, "k", keep=heads)
    v, vk = device_tensor(cfg, "v", keep=heads)
    do, dok = device_tensor(cfg, "do", keep=heads)
    o, lse = E.attn_prefill_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, return_lse=True)
    dq, dk, dv = E.attn_backward(q, k, v, o, do, lse, causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    for b, h in heads:
        errs = []
        refs = attention_backward_ref(qk[(b, h)][None, None], kk[(b, h)][None, None],
                                      vk[(b, h)][None, None], dok[(b, h)][None, None], cfg.causal,
                                      cfg.scale)
        for name, got, ref in (("dq", dq, refs[0]), ("dk", dk, refs[1]), ("dv", dv, refs[2])):
            g = to_host64(got[b, h])
            r = ref[0, 0]
            mx = float(np.abs(r).max())
            err = float(np.abs(g - r).max())
            assert np.all(np.isfinite(g)), f"{name} (b={b}, h={h}) not finite"
            assert err <= 2e-2 * mx, f"{name} (b={b}, h={h}): max|err| {err:.3e} vs max|ref| {mx:.3e}"
            errs.append(f"{name} {err:.2e} ({err / mx:.2e} of max|ref|)")
        print(f"  (b={b}, h={h}) ok: " + ", ".join(errs), flush=True)


def test_backward_gqa_sampled_kv_heads():
    """The backward of a causal GQA prefill (bf16, 32 query heads over 4 KV heads,
    N=2048, d=128): dK and dV of a KV head sum the contributions of its 8 query
    heads. Two KV heads are checked whole (dK, dV, and dQ of their 16 query
    heads) against the float64 oracle; relative tolerance as for config 2."""
    _announce("GQA backward 1x32/4x2048x128 causal")
    B, Hq, Hkv, N, d = 1, 32, 4, 2048, 128
    G = Hq // Hkv
    q = A.random_tensor((B, Hq, N, d), 901, "bf16")
    k = A.random_tensor((B, Hkv, N, d), 902, "bf16")
    v = A.random_tensor((B, Hkv, N, d), 903, "bf16")
    do = A.random_tensor((B, Hq, N, d), 904, "bf16")
    scale = float(np.float32(d ** -0.5))
    dev = [torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v, do)]
    o, lse = E.attn_prefill_fwd(dev[0], dev[1], dev[2], causal=True, scale=scale, return_lse=True)
    dq, dk, dv = E.attn_backward(dev[0], dev[1], dev[2], o, dev[3], lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    for g in (0, Hkv - 1):
        hs = slice(g * G, (g + 1) * G)
        rq, rk, rv = attention_backward_ref(q[:, hs], k[:, g:g + 1], v[:, g:g + 1], do[:, hs], True, scale)
        errs = []
        for name, got, ref in (("dq", dq[:, hs], rq), ("dk", dk[:, g:g + 1], rk), ("dv", dv[:, g:g + 1], rv)):
            gh = to_host64(got)
            mx = float(np.abs(ref).max())
            err = float(np.abs(gh - ref).max())
            assert np.all(np.isfinite(gh)), f"{name} (kv head {g}) not finite"
            assert err <= 2e-2 * mx, f"{name} (kv head {g}): max|err| {err:.3e} vs max|ref| {mx:.3e}"
            errs.append(f"{name} {err:.2e} ({err / mx:.2e} of max|ref|)")
        print(f"  kv head {g} ok: " + ", ".join(errs), flush=True)
