"""Benchmark: prefill attention TFLOP/s and decode KV GB/s on one MI355X.

Default run (one JSON line on stdout):
  * the step timed for `value` is one causal MHA prefill, bf16, B=4, H=32,
    N=4096, d=128 (inputs resident in HBM), in TFLOP/s of algorithmic work
    (4*d FLOP per visible query-key pair per query head);
  * the decode half of the metric is timed the same way on GQA decode, bf16,
    B=64, H_q=32, H_kv=4, d=128, 32768 cached tokens per request, in GB/s of
    K and V bytes read, and reported under "decode";
  * "roofline" relates the prefill kernel's rate (from HIP events on its launch
    stream) to the bf16 MFMA peak; "decode_roofline" relates decode to HBM peak;
  * "decode_multi_token" times the same caches with 4 new tokens per request
    (causal, bottom-right aligned), as a speculative-decoding verifier sees it,
    and "decode_multi_token_64" with 64 (compute-bound, in TFLOP/s);
  * "decode_paged" times the same caches cut into 16-position blocks scattered
    over a pool and read through a block table;
  * "decode_fp8" times the same caches stored as FP8 E4M3 codes (half the bytes);
  * "backward" times the gradient of the prefill workload (dQ, dK, dV) in
    TFLOP/s of 10*d FLOP per visible pair per head;
  * "cpu_baseline" times the float64 oracle on a bounded sample of the prefill
    workload on this host's cores.
`--all` also times the other three workloads (fp32 single head, the 23,400-step
fp16 series, causal GQA prefill at 32768) and ragged decode.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16BIT = 2500.0   # TFLOP/s, dense bf16/fp16 MFMA, MI355X
PEAK_MFMA_F32 = 157.3      # TFLOP/s, fp32 matrix
PEAK_HBM = 8000.0          # GB/s, HBM3E

# Context figures the pages print (quoted, with our recomputed values beside them).
PAGE_CONTEXT = {
    "prefill_ai_G8_ISL32768_as_printed": "~15,990 FLOP/B (formula 2*G*ISL/(G+1) gives 58,254.2)",
    "decode_ai_G8_KVSL32768_as_printed": "~15.99 per FP8 KV element (formula gives 15.996)",
    "decode_speedup_G1_to_G8_as_printed": "about 2x (FP8 KV cache, hardware not named)",
    "fp16_score_matrix_23400_steps_12_heads_as_printed": "about 12.9 GB (23400^2*12*2 B = 13.14 GB)",
}


def visible_pairs(N_q: int, n: int, causal: bool) -> int:
    """Visible (query, key) pairs for one head, bottom-right causal alignment (closed form)."""
    if not causal:
        return N_q * n
    off = n - N_q
    # rows i with i + off + 1 in [1, n]: count min(n, i + off + 1) for i + off + 1 > 0
    total = 0
    i0 = max(0, -off)  # first row that sees any key
    i1 = min(N_q, n - off)  # rows below i1 see a prefix shorter than n
    if i1 > i0:
        a, b = i0 + off + 1, i1 - 1 + off + 1
        total += (a + b) * (i1 - i0) // 2
    if N_q > max(i1, i0):
        total += n * (N_q - max(i1, i0))
    return total


def prefill_flops(cfg) -> int:
    return 4 * cfg.d * cfg.B * cfg.H_q * visible_pairs(cfg.N_q, cfg.N_kv, cfg.causal)


def decode_kv_bytes(cfg, lens) -> int:
    es = 2 if cfg.dtype in ("bf16", "f16") else 4
    return int(np.sum(lens, dtype=np.int64)) * cfg.H_kv * cfg.d * 2 * es


def make_device_tensor(cfg, name, torch, threads=16):
    import attn_inputs as A
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    H = cfg.H_q if name in ("q", "do") else cfg.H_kv
    N = cfg.N_q if name in ("q", "do") else cfg.N_kv
    t = torch.empty((cfg.B, H, N, cfg.d), dtype=dt, device="cuda")

    def gen(bh):
        b, h = divmod(bh, H)
        return b, h, A.slice_values(cfg.cid, name, b, h, N, cfg.d, cfg.sigma, cfg.dtype)

    with ThreadPoolExecutor(threads) as ex:
        for b, h, x in ex.map(gen, range(cfg.B * H)):
            t[b, h] = torch.from_numpy(x).to("cuda").to(dt)
    return t


def time_launches(fn, steps, warmup, torch):
    """Warm up, then time exactly `steps` calls with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def bench_prefill(cfg, steps, warmup, torch, E):
    q = make_device_tensor(cfg, "q", torch)
    k = make_device_tensor(cfg, "k", torch)
    v = make_device_tensor(cfg, "v", torch)
    o = torch.empty_like(q)
    t_first = time.perf_counter()
    E.attn_prefill_fwd(q, k, v, o, causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t_first) * 1e3
    ms, wall = time_launches(lambda: E.attn_prefill_fwd(q, k, v, o, causal=cfg.causal, scale=cfg.scale),
                             steps, warmup, torch)
    flops = prefill_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_F32 if cfg.dtype == "f32" else PEAK_MFMA_16BIT
    del q, k, v, o
    return {"config": cfg.cid, "name": cfg.name, "ms": ms, "tflops": tflops, "flops": flops,
            "frac_of_peak": tflops / peak, "peak_tflops": peak, "first_call_ms": first_ms,
            "wall_s": wall}


def bench_decode(cfg, steps, warmup, torch, E, ragged=False, cache=None):
    """Time one decode step (split + merge kernels). `cache` = (k, v) device tensors
    of this config's shape to reuse (configs that share caches share seeds)."""
    import attn_inputs as A
    lens = A.ragged_lengths(cfg) if ragged else np.full(cfg.B, cfg.N_kv, np.int32)
    q = make_device_tensor(cfg, "q", torch)
    if cache is None:
        cache = (make_device_tensor(cfg, "k", torch), make_device_tensor(cfg, "v", torch))
    k, v = cache
    o = torch.empty_like(q)
    lens_d = torch.from_numpy(lens).cuda()
    ws = torch.empty(E.attn_decode_workspace_size(cfg.B, cfg.H_q, cfg.H_kv, cfg.N_q, cfg.N_kv, cfg.d,
                                                  q.dtype),
                     dtype=torch.uint8, device="cuda")

    def call():
        E.attn_decode_fwd(q, k, v, o, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal, workspace=ws)

    ms, wall = time_launches(call, steps, warmup, torch)
    nbytes = decode_kv_bytes(cfg, lens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = 4 * cfg.d * cfg.H_q * sum(visible_pairs(cfg.N_q, int(n), cfg.causal) for n in lens)
    del q, o, ws
    key = "5r" if ragged else (cfg.cid if cfg.N_q == 1 else f"{cfg.cid}x{cfg.N_q}")
    return {"config": key, "name": cfg.name, "ms": ms, "kv_bytes": nbytes,
            "gb_per_s": gbs, "frac_of_peak": gbs / PEAK_HBM, "peak_gb_per_s": PEAK_HBM,
            "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12, "wall_s": wall}, cache


def bench_decode_paged(cfg, steps, warmup, torch, E, cache, block_size=16):
    """Decode over a paged copy of `cache`: its 16-position blocks are scattered
    over a pool in a seeded random order and addressed through a block table."""
    import attn_inputs as A
    k, v = cache
    B, H_kv, N, d = k.shape
    nb = N // block_size
    lens = np.full(B, N, np.int32)
    table, nblk = A.paged_layout(lens, block_size, nb, seed=5)
    perm = torch.from_numpy(table.reshape(-1).astype(np.int64)).cuda()
    kp = torch.empty((nblk, H_kv, block_size, d), dtype=k.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = k.reshape(B, H_kv, nb, block_size, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, block_size, d)
    vp[perm] = v.reshape(B, H_kv, nb, block_size, d).permute(0, 2, 1, 3, 4).reshape(-1, H_kv, block_size, d)
    table_d = torch.from_numpy(table).cuda()
    q = make_device_tensor(cfg, "q", torch)
    o = torch.empty_like(q)
    lens_d = torch.from_numpy(lens).cuda()
    ws = torch.empty(E.attn_decode_paged_workspace_size(B, cfg.H_q, H_kv, cfg.N_q, nb, block_size, d,
                                                        q.dtype), dtype=torch.uint8, device="cuda")

    def call():
        E.attn_decode_paged_fwd(q, kp, vp, table_d, o, kv_lens=lens_d, scale=cfg.scale,
                                causal=cfg.causal, workspace=ws)

    ms, wall = time_launches(call, steps, warmup, torch)
    # the same logical cache through the contiguous path, held to the paged
    # path's 2048-key splits, gives the same bits
    with E.tuning(decode_chunk=2048):
        oc = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal)
        torch.cuda.synchronize()
    same = bool(torch.equal(o, oc))
    nbytes = decode_kv_bytes(cfg, lens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del kp, vp, q, o, ws, oc
    return {"config": f"{cfg.cid}-paged{block_size}", "name": cfg.name + f", paged, block {block_size}",
            "ms": ms, "kv_bytes": nbytes, "gb_per_s": gbs, "frac_of_peak": gbs / PEAK_HBM,
            "peak_gb_per_s": PEAK_HBM, "wall_s": wall, "equals_contiguous": same}


def bench_decode_fp8(cfg, steps, warmup, torch, E, cache, k_scale=2.0 ** -6, v_scale=2.0 ** -6):
    """Decode over an FP8 E4M3 copy of `cache` (codes = E4M3(value / scale),
    per-tensor scales); bytes counted are the FP8 bytes read."""
    import attn_inputs as A
    k, v = cache
    B, H_kv, N, d = k.shape
    kc = (k.float() / k_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (v.float() / v_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    lens = np.full(B, N, np.int32)
    q = make_device_tensor(cfg, "q", torch)
    o = torch.empty_like(q)
    lens_d = torch.from_numpy(lens).cuda()
    ws = torch.empty(E.attn_decode_workspace_size(B, cfg.H_q, H_kv, cfg.N_q, N, d, q.dtype),
                     dtype=torch.uint8, device="cuda")

    def call():
        E.attn_decode_fp8_fwd(q, kc, vc, k_scale, v_scale, o, kv_lens=lens_d, scale=cfg.scale,
                              causal=cfg.causal, workspace=ws)

    ms, wall = time_launches(call, steps, warmup, torch)
    nbytes = decode_kv_bytes(cfg, lens) // 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    # what the quantisation costs: the same step over the unquantised bf16 cache
    o16 = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal)
    diff = (o.float() - o16.float()).abs()
    err = {"max_abs_diff_vs_bf16_cache": float(diff.max()),
           "mean_abs_diff_vs_bf16_cache": float(diff.mean()),
           "mean_abs_output": float(o16.float().abs().mean())}
    del kc, vc, q, o, ws, o16, diff
    return {"config": f"{cfg.cid}-fp8", "name": cfg.name + ", FP8 E4M3 cache", "ms": ms,
            "kv_bytes": nbytes, "gb_per_s": gbs, "frac_of_peak": gbs / PEAK_HBM,
            "peak_gb_per_s": PEAK_HBM, "wall_s": wall, **err}


def bench_backward(cfg, steps, warmup, torch, E):
    """Time one backward pass (Delta prep, dK/dV, dQ) of a prefill workload, given
    the forward's O and LSE; TFLOP/s of 10*d FLOP per visible pair per head (the
    five products of the gradient; the recomputation adds 4*d more)."""
    q = make_device_tensor(cfg, "q", torch)
    k = make_device_tensor(cfg, "k", torch)
    v = make_device_tensor(cfg, "v", torch)
    o, lse = E.attn_prefill_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, return_lse=True)
    do = make_device_tensor(cfg, "do", torch)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(E.attn_backward_workspace_size(cfg.B, cfg.H_q, cfg.H_kv, cfg.N_q, cfg.N_kv, cfg.d,
                                                    q.dtype), dtype=torch.uint8, device="cuda")

    def call():
        E.attn_backward(q, k, v, o, do, lse, dq, dk, dv, causal=cfg.causal, scale=cfg.scale,
                        workspace=ws)

    ms, wall = time_launches(call, steps, warmup, torch)
    flops = prefill_flops(cfg) * 10 // 4
    tflops = flops / (ms * 1e-3) / 1e12
    # Q, K, V, O, dO read and dQ, dK, dV written once each, plus the LSE
    nbytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, do, dq, dk, dv))
    nbytes += lse.numel() * lse.element_size()
    del q, k, v, o, do, dq, dk, dv, ws
    return {"config": f"{cfg.cid}-bwd", "name": cfg.name + ", backward", "ms": ms, "flops": flops,
            "tflops": tflops, "frac_of_peak": tflops / PEAK_MFMA_16BIT, "peak_tflops": PEAK_MFMA_16BIT,
            "bytes": nbytes, "wall_s": wall}


def library_gemm_tflops(torch, n=8192, steps=20):
    """A plain bf16 GEMM through torch (hipBLASLt) on this GPU: the practical
    matrix-core rate under the card's power limit, reported beside the nominal peak."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms, _ = time_launches(lambda: torch.matmul(a, b), steps, 30, torch)
    del a, b
    return 2 * n ** 3 / (ms * 1e-3) / 1e12


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size (torch's copy kernel): the
    HBM counters read for it calibrate the FETCH_SIZE / WRITE_SIZE scale."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"copy_bytes": nbytes, "reps": reps}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(name: str) -> str:
    import hashlib
    path = os.path.join(ROOT, "exact_attention_31_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel source changed after they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash(rec["source"]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, budget_s=15.0):
    """The float64 oracle on a bounded sample of the prefill workload (whole heads)."""
    import attn_inputs as A
    from oracle import attention_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = 1
    heads_done, elapsed = 0, 0.0
    t_start = time.perf_counter()
    while elapsed < budget_s and heads_done < cfg.B * cfg.H_q:
        b, h = divmod(heads_done, cfg.H_q)
        q = A.slice_values(cfg.cid, "q", b, h, cfg.N_q, cfg.d, cfg.sigma, cfg.dtype)
        g = h // cfg.G
        k = A.slice_values(cfg.cid, "k", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
        v = A.slice_values(cfg.cid, "v", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
        t0 = time.perf_counter()
        attention_ref(q[None, None], k[None, None], v[None, None], cfg.causal, cfg.scale)
        elapsed += time.perf_counter() - t0
        heads_done += 1
        if time.perf_counter() - t_start > 4 * budget_s:
            break
    flops = 4 * cfg.d * heads_done * visible_pairs(cfg.N_q, cfg.N_kv, cfg.causal)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads_done} of {cfg.B * cfg.H_q} heads (full {cfg.N_q}-row causal heads, "
                      f"float64 numpy, {elapsed:.1f} s)",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_decode(cfg, budget_s=5.0):
    """The float64 oracle on a bounded sample of the decode workload: whole
    requests (all KV heads, each with its G query heads), KV bytes per second
    counted as the GPU's (the cache's 16-bit bytes)."""
    import attn_inputs as A
    from oracle import attention_head_rows
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = 1
    done, elapsed = 0, 0.0
    t_start = time.perf_counter()
    while elapsed < budget_s and done < cfg.B:
        b = done
        for g in range(cfg.H_kv):
            k = A.slice_values(cfg.cid, "k", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
            v = A.slice_values(cfg.cid, "v", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
            qs = [A.slice_values(cfg.cid, "q", b, g * cfg.G + j, cfg.N_q, cfg.d, cfg.sigma, cfg.dtype)
                  for j in range(cfg.G)]
            t0 = time.perf_counter()
            for q in qs:
                attention_head_rows(q, np.arange(cfg.N_q), cfg.N_q, k, v, cfg.causal, cfg.scale)
            elapsed += time.perf_counter() - t0
        done += 1
        if time.perf_counter() - t_start > 6 * budget_s:
            break
    nbytes = done * cfg.H_kv * cfg.N_kv * cfg.d * 2 * 2
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cfg.B} requests (all {cfg.H_kv} KV heads x {cfg.G} query heads, "
                      f"{cfg.N_kv} keys each, float64 numpy, {elapsed:.1f} s)"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed launches first (the clocks ramp during the first ~50 ms)")
    ap.add_argument("--all", action="store_true", help="also time configs 1, 3, 4 and ragged decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_ragged", "decode_multi",
                                       "decode_paged", "decode_fp8", "backward"], default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              f"multi-GPU path.", file=sys.stderr)
        return 2

    import torch
    import attn_inputs as A
    import exact_attention_31_amd as E
    E.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 3
    props = torch.cuda.get_device_properties(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)), flush=True)
        return 0

    res = {}
    if args.only in (None, "prefill"):
        res["prefill"] = bench_prefill(A.CONFIGS[2], args.steps, args.warmup, torch, E)
        print(f"# prefill c2: {res['prefill']['ms']:.3f} ms  {res['prefill']['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    if args.only in (None, "prefill"):
        res["gemm"] = library_gemm_tflops(torch)
        print(f"# bf16 8192^3 GEMM (torch/hipBLASLt): {res['gemm']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if args.only in (None, "backward"):
        r = bench_backward(A.CONFIGS[2], args.steps, args.warmup, torch, E)
        print(f"# backward c2: {r['ms']:.3f} ms  {r['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        res["backward"] = r
    cache = None
    if args.only in (None, "decode"):
        res["decode"], cache = bench_decode(A.CONFIGS[5], args.steps, args.warmup, torch, E)
        print(f"# decode c5: {res['decode']['ms']:.3f} ms  {res['decode']['gb_per_s']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if args.only in (None, "decode_multi"):
        r, cache = bench_decode(A.CONFIGS[7], args.steps, args.warmup, torch, E, cache=cache)
        print(f"# decode c5, 4 tokens: {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s  "
              f"{r['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        res["decode_multi"] = r
        if args.only == "decode_multi":
            res["decode"] = r
            res["decode_label"] = ("GQA multi-token decode, bf16, B=64, 4 new tokens per request "
                                   "(causal), H_q=32, H_kv=4, d=128, KV 32768")
        r, cache = bench_decode(A.CONFIGS[8], args.steps, args.warmup, torch, E, cache=cache)
        print(f"# decode c5, 64 tokens: {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s  "
              f"{r['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        res["decode_multi64"] = r
    if args.only in (None, "decode_paged"):
        if cache is None:
            _, cache = bench_decode(A.CONFIGS[5], 1, 1, torch, E)
        r = bench_decode_paged(A.CONFIGS[5], args.steps, args.warmup, torch, E, cache)
        print(f"# decode c5 paged (block 16): {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s  "
              f"same bits as contiguous: {r['equals_contiguous']}", file=sys.stderr, flush=True)
        res["decode_paged"] = r
        if args.only == "decode_paged":
            res["decode"] = r
            res["decode_label"] = ("GQA decode over a paged cache (block 16), bf16, B=64, H_q=32, "
                                   "H_kv=4, d=128, KV 32768")
    if args.only in (None, "decode_fp8"):
        if cache is None:
            _, cache = bench_decode(A.CONFIGS[5], 1, 1, torch, E)
        r = bench_decode_fp8(A.CONFIGS[5], args.steps, args.warmup, torch, E, cache)
        print(f"# decode c5 FP8 cache: {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s",
              file=sys.stderr, flush=True)
        res["decode_fp8"] = r
        if args.only == "decode_fp8":
            res["decode"] = r
            res["decode_label"] = ("GQA decode over an FP8 E4M3 cache, bf16 queries, B=64, H_q=32, "
                                   "H_kv=4, d=128, KV 32768")
    extra = []
    if args.only == "decode_ragged":
        r, cache = bench_decode(A.CONFIGS[6], args.steps, args.warmup, torch, E, ragged=True)
        print(f"# decode c5 ragged: {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s", file=sys.stderr, flush=True)
        res["decode"] = r
        res["decode_label"] = ("GQA decode, bf16, B=64, H_q=32, H_kv=4, d=128, KV lengths "
                               "uniform on 1..32768")
    if args.all:
        for cid in (1, 3, 4):
            r = bench_prefill(A.CONFIGS[cid], max(5, args.steps // 5) if cid == 4 else args.steps,
                              args.warmup, torch, E)
            extra.append(r)
            print(f"# prefill c{cid}: {r['ms']:.3f} ms  {r['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        r, cache = bench_decode(A.CONFIGS[6], args.steps, args.warmup, torch, E, ragged=True,
                                cache=cache)
        extra.append(r)
        print(f"# decode c5 ragged: {r['ms']:.3f} ms  {r['gb_per_s']:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu and "prefill" in res:
        cpu = cpu_baseline(A.CONFIGS[2], args.cpu_budget)
    cpu_dec = None
    if not args.no_cpu and "decode" in res and "decode_label" not in res:
        cpu_dec = cpu_baseline_decode(A.CONFIGS[5], max(2.0, args.cpu_budget / 3))

    p = res.get("prefill")
    d = res.get("decode")
    if p is None and d is None:   # --only backward: its own line
        p = dict(res["backward"], first_call_ms=0.0)
    main_r = p if p is not None else d
    line = {
        "metric": "prefill attention TFLOP/s and decode KV GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(p["tflops"], 3) if p else round(d["gb_per_s"], 3),
        "unit": "TFLOP/s" if p else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_r["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "causal MHA prefill, bf16, B=4, H_q=H_kv=32, N=4096, d=128"
                   if p else res.get("decode_label",
                                     "GQA decode, bf16, B=64, H_q=32, H_kv=4, d=128, KV 32768"),
                   "B": 4 if p else 64, "seq_len": 4096 if p else 32768, "head_dim": 128,
                   "causal": bool(p), "parallelism": "single GPU"},
    }
    if p:
        line["roofline"] = {"bound": "mfma", "achieved": round(p["tflops"], 3), "peak": PEAK_MFMA_16BIT,
                            "unit": "TFLOP/s", "frac": round(p["tflops"] / PEAK_MFMA_16BIT, 4),
                            "traffic": measured_traffic("prefill"),
                            "kernel": "prefill16_kernel<BF16,128,causal> (persistent grid)",
                            "work_per_launch": p["flops"]}
        if "gemm" in res:
            line["roofline"]["library_gemm_tflops"] = round(res["gemm"], 1)
            line["roofline"]["frac_of_library_gemm"] = round(p["tflops"] / res["gemm"], 4)
    if d:
        line["decode"] = {"workload": res.get("decode_label", "GQA decode, bf16, B=64, H_q=32, H_kv=4 "
                                                              "(G=8), d=128, KV 32768 per request"),
                          "ms_per_step": round(d["ms"], 5),
                          "value": round(d["gb_per_s"], 2), "unit": "GB/s",
                          "frac_of_hbm_peak": round(d["frac_of_peak"], 4)}
        if cpu_dec is not None:
            line["decode"]["cpu_baseline"] = cpu_dec
        line["decode_roofline"] = {"bound": "hbm", "achieved": round(d["gb_per_s"], 2), "peak": PEAK_HBM,
                                   "unit": "GB/s", "frac": round(d["frac_of_peak"], 4),
                                   # counters were taken on the plain decode workload only
                                   "traffic": None if "decode_label" in res else measured_traffic("decode"),
                                   "kernel": "decode_split_kernel + decode_merge_kernel (one step)",
                                   "work_per_launch": d["kv_bytes"]}
    dm = res.get("decode_multi")
    if dm and dm is not d:
        line["decode_multi_token"] = {
            "workload": "GQA multi-token decode, bf16, B=64, 4 new tokens per request (causal, "
                        "bottom-right), H_q=32, H_kv=4 (G=8), d=128, KV 32768 per request",
            "ms_per_step": round(dm["ms"], 5), "value": round(dm["gb_per_s"], 2), "unit": "GB/s",
            "frac_of_hbm_peak": round(dm["frac_of_peak"], 4), "tflops": round(dm["tflops"], 2),
            "kernel": "decode_split_kernel + decode_merge_kernel (one step)"}
    dm64 = res.get("decode_multi64")
    if dm64:
        line["decode_multi_token_64"] = {
            "workload": "GQA multi-token decode, bf16, B=64, 64 new tokens per request (causal, "
                        "bottom-right), H_q=32, H_kv=4 (G=8), d=128, KV 32768 per request",
            "ms_per_step": round(dm64["ms"], 5), "value": round(dm64["tflops"], 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(dm64["tflops"] / PEAK_MFMA_16BIT, 4),
            "kv_gb_per_s": round(dm64["gb_per_s"], 2),
            "kernel": "prefill16_kernel in rows mode (one step)"}
    dp = res.get("decode_paged")
    if dp and dp is not d:
        line["decode_paged"] = {
            "workload": "GQA decode over a paged cache (16-position blocks scattered over a pool "
                        "in random order), bf16, B=64, H_q=32, H_kv=4, d=128, KV 32768 per request",
            "ms_per_step": round(dp["ms"], 5), "value": round(dp["gb_per_s"], 2), "unit": "GB/s",
            "frac_of_hbm_peak": round(dp["frac_of_peak"], 4),
            "equals_contiguous": dp["equals_contiguous"],
            "kernel": "decode_split_kernel<paged> + decode_merge_kernel (one step)"}
    df8 = res.get("decode_fp8")
    if df8 and df8 is not d:
        line["decode_fp8"] = {
            "workload": "GQA decode over an FP8 E4M3 cache (per-tensor scales), bf16 queries and "
                        "output, B=64, H_q=32, H_kv=4, d=128, KV 32768 per request",
            "ms_per_step": round(df8["ms"], 5), "value": round(df8["gb_per_s"], 2), "unit": "GB/s",
            "frac_of_hbm_peak": round(df8["frac_of_peak"], 4),
            "max_abs_diff_vs_bf16_cache": round(df8["max_abs_diff_vs_bf16_cache"], 6),
            "mean_abs_diff_vs_bf16_cache": round(df8["mean_abs_diff_vs_bf16_cache"], 6),
            "mean_abs_output": round(df8["mean_abs_output"], 6),
            "kernel": "decode_split_kernel<fp8> + decode_merge_kernel (one step)"}
    bw = res.get("backward")
    if bw:
        line["backward"] = {
            "workload": "backward of causal MHA prefill, bf16, B=4, H_q=H_kv=32, N=4096, d=128 "
                        "(given the forward's O and LSE)",
            "ms_per_step": round(bw["ms"], 5), "value": round(bw["tflops"], 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(bw["frac_of_peak"], 4), "work_per_launch": bw["flops"],
            # Q, K, V, O, dO and the LSE read once, dQ, dK, dV written once
            "algorithmic_bytes": bw["bytes"],
            "traffic": measured_traffic("backward"),
            "kernel": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel (one step)"}
    if p:
        line["prefill_first_call_ms"] = round(p["first_call_ms"], 3)
    if cpu:
        line["cpu_baseline"] = cpu
    if extra:
        line["other_workloads"] = [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                                   for r in extra]
    line["device"] = {"name": props.name, "cus": props.multi_processor_count,
                      "arch": getattr(props, "gcnArchName", "")}
    line["page_context"] = PAGE_CONTEXT
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
