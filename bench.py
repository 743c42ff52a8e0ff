"""Benchmark: prefill attention TFLOP/s and decode KV GB/s on one MI355X.

The default run times every workload and prints one JSON line on stdout:
  * the headline (`value`, `ms_per_step`, `roofline`, `cpu_baseline`) is the
    largest single-GPU prefill workload: causal GQA prefill, bf16, B=1,
    H_q=32, H_kv=4 (G=8), N=32768, d=128, in TFLOP/s of algorithmic work
    (4*d FLOP per visible query-key pair per query head), inputs resident in
    HBM; one step is one attn_prefill_fwd launch;
  * `workloads` holds every workload with its own timing and roofline
    fraction: the fp32 single head, causal MHA prefill (B=4, H=32, N=4096,
    d=128), the 23,400-step fp16 series, the GQA prefill above, GQA decode
    (B=64, H_q=32, H_kv=4, d=128, KV 32768: uniform lengths, ragged lengths,
    4 and 64 new tokens per request, a paged cache, an FP8 cache) and the
    backward of the MHA prefill;
  * timing uses HIP events on the launch stream: the mean (= ms_per_step)
    over K back-to-back launches between one pair of events, then p50, p90,
    min and max from a second pass with a pair of events around each launch;
    warm-up runs at least --warmup launches and at least --min-warmup-ms of
    GPU work (the clocks ramp during the first ~50 ms);
  * `cpu_baseline` objects time the float64 oracle on this host's cores, on
    whole heads (or requests) of the workload for a bounded time; where only
    a sample fits, the rate is extrapolated to the whole workload and says so.
`--only A,B` times only those workloads (the first is the line's headline);
`--traffic-from DIR` turns rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs into
profiles/traffic.json; `--copy-calibration` runs the copy those counters are
calibrated against.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16BIT = 2500.0   # TFLOP/s, dense bf16/fp16 MFMA, MI355X
PEAK_MFMA_F32 = 157.3      # TFLOP/s, fp32 matrix
PEAK_HBM = 8000.0          # GB/s, HBM3E

METRIC = "prefill attention TFLOP/s and decode KV GB/s, as % of MI355X MFMA/HBM peak"

# Context figures the pages print (quoted, with our recomputed values beside them).
PAGE_CONTEXT = {
    "prefill_ai_G8_ISL32768_as_printed": "~15,990 FLOP/B (formula 2*G*ISL/(G+1) gives 58,254.2)",
    "decode_ai_G8_KVSL32768_as_printed": "~15.99 per FP8 KV element (formula gives 15.996)",
    "decode_speedup_G1_to_G8_as_printed": "about 2x (FP8 KV cache, hardware not named)",
    "fp16_score_matrix_23400_steps_12_heads_as_printed": "about 12.9 GB (23400^2*12*2 B = 13.14 GB)",
}

# workload name -> (config id, description); decode variants share config 5's caches
WORKLOADS = {
    "prefill_c4": (4, "causal GQA prefill, bf16, B=1, H_q=32, H_kv=4 (G=8), N=32768, d=128"),
    "prefill_c2": (2, "causal MHA prefill, bf16, B=4, H_q=H_kv=32, N=4096, d=128"),
    "prefill_c3": (3, "causal prefill of a 23,400-step series, fp16, B=1, H=12, N=23400, d=64"),
    "prefill_c1": (1, "single-head attention, fp32, non-causal, B=1, H=1, N=512, d=64"),
    "backward_c2": (2, "backward of causal MHA prefill, bf16, B=4, H_q=H_kv=32, N=4096, d=128 "
                       "(given the forward's O and LSE)"),
    "decode_c5": (5, "GQA decode, bf16, B=64, H_q=32, H_kv=4 (G=8), d=128, KV 32768 per request"),
    "decode_c5_ragged": (6, "GQA decode, bf16, B=64, H_q=32, H_kv=4 (G=8), d=128, KV lengths uniform "
                            "on 1..32768 (seeded)"),
    "decode_c5_4tok": (7, "GQA multi-token decode, bf16, B=64, 4 new tokens per request (causal, "
                          "bottom-right), H_q=32, H_kv=4, d=128, KV 32768 per request"),
    "decode_c5_64tok": (8, "GQA multi-token decode, bf16, B=64, 64 new tokens per request (causal, "
                           "bottom-right), H_q=32, H_kv=4, d=128, KV 32768 per request"),
    "decode_c5_paged": (5, "GQA decode over a paged cache (16-position blocks scattered over a pool in "
                           "random order), bf16, B=64, H_q=32, H_kv=4, d=128, KV 32768 per request"),
    "decode_c5_fp8": (5, "GQA decode over an FP8 E4M3 cache (per-tensor scales), bf16 queries and "
                         "output, B=64, H_q=32, H_kv=4, d=128, KV 32768 per request"),
}
DEFAULT_ORDER = ["prefill_c4", "prefill_c2", "prefill_c3", "prefill_c1", "backward_c2", "decode_c5",
                 "decode_c5_ragged", "decode_c5_4tok", "decode_c5_64tok", "decode_c5_paged",
                 "decode_c5_fp8"]

# kernels each workload's step launches (names as the profiler reports them)
STEP_KERNELS = {
    "prefill": ["prefill16_kernel", "prefill16_ring_kernel", "prefill32_kernel"],
    "decode": ["decode_split_kernel", "decode_merge_kernel", "prefill16_kernel", "prefill16_ring_kernel"],
    "backward": ["bwd_dq_kernel", "bwd_dkdv_kernel"],
}
KERNEL_SOURCES = {"prefill": ["prefill.hip"], "decode": ["decode.hip", "prefill.hip"],
                  "backward": ["backward.hip"]}


def visible_pairs(N_q: int, n: int, causal: bool) -> int:
    """Visible (query, key) pairs for one head, bottom-right causal alignment (closed form)."""
    if not causal:
        return N_q * n
    off = n - N_q
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


def prefill_bytes(cfg) -> int:
    """Algorithmic bytes of one prefill launch: Q, K, V read once, O written once."""
    es = 4 if cfg.dtype == "f32" else 2
    return es * cfg.d * (2 * cfg.B * cfg.H_q * cfg.N_q + 2 * cfg.B * cfg.H_kv * cfg.N_kv)


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


def time_launches(fn, steps, warmup, torch, min_warmup_ms=200.0):
    """Warm up (at least `warmup` calls and `min_warmup_ms` of wall time), then
    time exactly `steps` back-to-back calls between one pair of HIP events on the
    current stream (the stream the library launches on): their mean is the step
    time. A second pass of `steps` calls, each between its own pair of events,
    gives the per-launch distribution (p50, p90, min, max); the events recorded
    between launches cost a few microseconds each, so that pass is not used for
    the mean."""
    stream = torch.cuda.current_stream()
    n_warm = 0
    t0 = time.perf_counter()
    while n_warm < warmup:
        fn()
        n_warm += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_warmup_ms:
        for _ in range(4):
            fn()
        n_warm += 4
        torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t1 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    mean = start.elapsed_time(end) / steps
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    events[0].record(stream)
    for i in range(steps):
        fn()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [events[i].elapsed_time(events[i + 1]) for i in range(steps)]
    srt = sorted(per)

    def pct(p):
        return srt[min(len(srt) - 1, max(0, int(math.ceil(p * len(srt))) - 1))]

    return {"mean_ms": mean, "p50_ms": statistics.median(per), "p90_ms": pct(0.9),
            "min_ms": srt[0], "max_ms": srt[-1], "per_launch_mean_ms": sum(per) / len(per),
            "launches": steps, "warmup_launches": n_warm, "warmup_ms": round(warm_ms, 1),
            "wall_s": round(wall, 3)}


def _rate(work, ms, scale):
    return work / (ms * 1e-3) / scale


def _timing_out(t):
    return {k: (round(v, 5) if isinstance(v, float) else v) for k, v in t.items()}


def kernel_source_hash(name: str) -> str:
    path = os.path.join(ROOT, "exact_attention_31_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(workload: str):
    """HBM bytes per step from the committed counter runs, or None when a kernel
    source the step runs changed after they were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    for src, h in rec.get("sources", {}).items():
        if kernel_source_hash(src) != h:
            return None
    return rec.get("bytes_per_step")


# ------------------------------------------------------------------ workloads
def bench_prefill(name, cfg, args, torch, E):
    q = make_device_tensor(cfg, "q", torch)
    k = make_device_tensor(cfg, "k", torch)
    v = make_device_tensor(cfg, "v", torch)
    o = torch.empty_like(q)
    torch.cuda.synchronize()
    t_first = time.perf_counter()
    E.attn_prefill_fwd(q, k, v, o, causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t_first) * 1e3
    t = time_launches(lambda: E.attn_prefill_fwd(q, k, v, o, causal=cfg.causal, scale=cfg.scale),
                      args.steps, args.warmup, torch, args.min_warmup_ms)
    del q, k, v, o
    flops = prefill_flops(cfg)
    f32 = cfg.dtype == "f32"
    peak = PEAK_MFMA_F32 if f32 else PEAK_MFMA_16BIT
    tf = _rate(flops, t["mean_ms"], 1e12)
    kern = ("prefill32_kernel" if f32 else
            ("prefill16_ring_kernel" if cfg.d == 64 else "prefill16_kernel (persistent grid)"))
    return {"workload": WORKLOADS[name][1], "timing": _timing_out(t), "first_call_ms": round(first_ms, 3),
            "value": round(tf, 3), "unit": "TFLOP/s", "value_p50": round(_rate(flops, t["p50_ms"], 1e12), 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(tf / peak, 4), "traffic": measured_traffic(name),
                         "algorithmic_bytes": prefill_bytes(cfg), "work_per_launch": flops,
                         "kernel": kern + (", fp32 matrix peak" if f32 else "")}}


def bench_backward(name, cfg, args, torch, E):
    """One backward pass (prep, dK/dV, dQ) given the forward's O and LSE;
    TFLOP/s of 10*d FLOP per visible pair per head (the five products of the
    gradient; the recomputation adds 4*d more)."""
    q = make_device_tensor(cfg, "q", torch)
    k = make_device_tensor(cfg, "k", torch)
    v = make_device_tensor(cfg, "v", torch)
    o, lse = E.attn_prefill_fwd(q, k, v, causal=cfg.causal, scale=cfg.scale, return_lse=True)
    do = make_device_tensor(cfg, "do", torch)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(E.attn_backward_workspace_size(cfg.B, cfg.H_q, cfg.H_kv, cfg.N_q, cfg.N_kv, cfg.d,
                                                    q.dtype), dtype=torch.uint8, device="cuda")

    def call():
        E.attn_backward(q, k, v, o, do, lse, dq, dk, dv, causal=cfg.causal, scale=cfg.scale, workspace=ws)

    t = time_launches(call, args.steps, args.warmup, torch, args.min_warmup_ms)
    flops = prefill_flops(cfg) * 10 // 4
    # Q, K, V, O, dO and the LSE read once, dQ, dK, dV written once
    nbytes = sum(x.numel() * x.element_size() for x in (q, k, v, o, do, dq, dk, dv))
    nbytes += lse.numel() * lse.element_size()
    del q, k, v, o, do, dq, dk, dv, ws
    tf = _rate(flops, t["mean_ms"], 1e12)
    return {"workload": WORKLOADS[name][1], "timing": _timing_out(t), "value": round(tf, 3),
            "unit": "TFLOP/s", "value_p50": round(_rate(flops, t["p50_ms"], 1e12), 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_16BIT, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_MFMA_16BIT, 4), "traffic": measured_traffic(name),
                         "algorithmic_bytes": nbytes, "work_per_launch": flops,
                         "kernel": "bwd_dq_kernel + bwd_dkdv_kernel (one step)"}}


class DecodeCache:
    """Config 5's K and V caches on the device, generated once and shared."""

    def __init__(self, torch):
        import attn_inputs as A
        cfg = A.CONFIGS[5]
        self.k = make_device_tensor(cfg, "k", torch)
        self.v = make_device_tensor(cfg, "v", torch)


def _decode_result(name, t, nbytes, flops, extra=None, compute_bound=False):
    gbs = _rate(nbytes, t["mean_ms"], 1e9)
    tf = _rate(flops, t["mean_ms"], 1e12)
    r = {"workload": WORKLOADS[name][1], "timing": _timing_out(t), "kv_bytes": nbytes}
    if compute_bound:
        r.update({"value": round(tf, 3), "unit": "TFLOP/s", "kv_gb_per_s": round(gbs, 2),
                  "value_p50": round(_rate(flops, t["p50_ms"], 1e12), 3),
                  "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_MFMA_16BIT,
                               "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_16BIT, 4),
                               "traffic": measured_traffic(name), "work_per_launch": flops,
                               "kernel": "prefill kernel in rows mode (one step)"}})
    else:
        r.update({"value": round(gbs, 2), "unit": "GB/s", "tflops": round(tf, 3),
                  "value_p50": round(_rate(nbytes, t["p50_ms"], 1e9), 2),
                  "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM, 4), "traffic": measured_traffic(name),
                               "work_per_launch": nbytes,
                               "kernel": "decode_split_kernel + decode_merge_kernel (one step)"}})
    if extra:
        r.update(extra)
    return r


def bench_decode(name, cfg, args, torch, E, cache):
    import attn_inputs as A
    lens = A.ragged_lengths(cfg) if cfg.ragged else np.full(cfg.B, cfg.N_kv, np.int32)
    q = make_device_tensor(cfg, "q", torch)
    o = torch.empty_like(q)
    lens_d = torch.from_numpy(lens).cuda()
    ws = torch.empty(E.attn_decode_workspace_size(cfg.B, cfg.H_q, cfg.H_kv, cfg.N_q, cfg.N_kv, cfg.d,
                                                  q.dtype), dtype=torch.uint8, device="cuda")

    def call():
        E.attn_decode_fwd(q, cache.k, cache.v, o, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal,
                          workspace=ws)

    t = time_launches(call, args.steps, args.warmup, torch, args.min_warmup_ms)
    del q, o, ws
    nbytes = decode_kv_bytes(cfg, lens)
    flops = 4 * cfg.d * cfg.H_q * sum(visible_pairs(cfg.N_q, int(n), cfg.causal) for n in lens)
    return _decode_result(name, t, nbytes, flops, compute_bound=cfg.N_q >= 64)


def bench_decode_paged(name, cfg, args, torch, E, cache, block_size=16):
    """Decode over a paged copy of the cache: its 16-position blocks are
    scattered over a pool in a seeded random order and addressed through a
    block table."""
    import attn_inputs as A
    k, v = cache.k, cache.v
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
        E.attn_decode_paged_fwd(q, kp, vp, table_d, o, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal,
                                workspace=ws)

    t = time_launches(call, args.steps, args.warmup, torch, args.min_warmup_ms)
    # the same logical cache through the contiguous path, held to the paged
    # path's 2048-key splits, gives the same bits
    with E.tuning(decode_chunk=2048):
        oc = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal)
        torch.cuda.synchronize()
    same = bool(torch.equal(o, oc))
    del kp, vp, q, o, ws, oc
    nbytes = decode_kv_bytes(cfg, lens)
    r = _decode_result(name, t, nbytes, 4 * cfg.d * cfg.H_q * B * N, {"equals_contiguous": same})
    r["roofline"]["kernel"] = "decode_split_kernel<paged> + decode_merge_kernel (one step)"
    return r


def bench_decode_fp8(name, cfg, args, torch, E, cache, k_scale=2.0 ** -6, v_scale=2.0 ** -6):
    """Decode over an FP8 E4M3 copy of the cache (codes = E4M3(value / scale),
    per-tensor scales); bytes counted are the FP8 bytes read."""
    k, v = cache.k, cache.v
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

    t = time_launches(call, args.steps, args.warmup, torch, args.min_warmup_ms)
    # what the quantisation costs: the same step over the unquantised bf16 cache
    o16 = E.attn_decode_fwd(q, k, v, kv_lens=lens_d, scale=cfg.scale, causal=cfg.causal)
    diff = (o.float() - o16.float()).abs()
    err = {"max_abs_diff_vs_bf16_cache": round(float(diff.max()), 6),
           "mean_abs_diff_vs_bf16_cache": round(float(diff.mean()), 6),
           "mean_abs_output": round(float(o16.float().abs().mean()), 6)}
    del kc, vc, q, o, ws, o16, diff
    nbytes = decode_kv_bytes(cfg, lens) // 2
    r = _decode_result(name, t, nbytes, 4 * cfg.d * cfg.H_q * B * N, err)
    r["roofline"]["kernel"] = "decode_split_kernel<fp8> + decode_merge_kernel (one step)"
    return r


def library_gemm_tflops(torch, args, n=8192):
    """A plain bf16 GEMM through torch (hipBLASLt) on this GPU: the practical
    matrix-core rate under the card's power limit, reported beside the nominal peak."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    t = time_launches(lambda: torch.matmul(a, b), 20, 30, torch, args.min_warmup_ms)
    del a, b
    return {"tflops_mean": round(_rate(2 * n ** 3, t["mean_ms"], 1e12), 1),
            "tflops_p50": round(_rate(2 * n ** 3, t["p50_ms"], 1e12), 1), "shape": f"{n}^3 bf16"}


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size (torch's copy kernel): the
    HBM counters read for it calibrate the FETCH_SIZE / WRITE_SIZE scale."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"copy_bytes": nbytes, "reps": reps}


# ------------------------------------------------------------- CPU baselines
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline_prefill(cfg, budget_s):
    """The float64 oracle on whole heads of a prefill workload for about
    `budget_s` seconds on this host's cores; the rate is extrapolated to the
    whole workload when not every head fits."""
    import attn_inputs as A
    from oracle import attention_ref
    heads = cfg.B * cfg.H_q
    done, elapsed = 0, 0.0
    while done < heads and (done == 0 or elapsed < budget_s):
        b, h = divmod(done, cfg.H_q)
        q = A.slice_values(cfg.cid, "q", b, h, cfg.N_q, cfg.d, cfg.sigma, cfg.dtype)
        g = h // cfg.G
        k = A.slice_values(cfg.cid, "k", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
        v = A.slice_values(cfg.cid, "v", b, g, cfg.N_kv, cfg.d, cfg.sigma, cfg.dtype)
        t0 = time.perf_counter()
        attention_ref(q[None, None], k[None, None], v[None, None], cfg.causal, cfg.scale)
        elapsed += time.perf_counter() - t0
        done += 1
    flops = 4 * cfg.d * done * visible_pairs(cfg.N_q, cfg.N_kv, cfg.causal)
    rate = flops / elapsed
    full = done == heads
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(_blas_threads()), "kind": "oracle",
            "sample": f"{done} of {heads} heads (whole {cfg.N_q}-row heads, float64 numpy, "
                      f"{elapsed:.1f} s)" + ("" if full else "; whole-workload time extrapolated"),
            "extrapolated": not full,
            "workload_seconds": round(elapsed if full else prefill_flops(cfg) / rate, 2),
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_decode(cfg, budget_s):
    """The float64 oracle on whole requests of the decode workload (all KV
    heads, each with its G query heads) for about `budget_s` seconds; KV bytes
    per second counted as the GPU's (the cache's 16-bit bytes)."""
    import attn_inputs as A
    from oracle import attention_head_rows
    done, elapsed = 0, 0.0
    while done < cfg.B and (done == 0 or elapsed < budget_s):
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
    nbytes = done * cfg.H_kv * cfg.N_kv * cfg.d * 2 * 2
    rate = nbytes / elapsed
    full = done == cfg.B
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": int(_blas_threads()), "kind": "oracle",
            "sample": f"{done} of {cfg.B} requests (all {cfg.H_kv} KV heads x {cfg.G} query heads, "
                      f"{cfg.N_kv} keys each, float64 numpy, {elapsed:.1f} s)"
                      + ("" if full else "; whole-workload time extrapolated"),
            "extrapolated": not full,
            "workload_seconds": round(decode_kv_bytes(cfg, [cfg.N_kv] * cfg.B) / rate, 2)}


# ------------------------------------------------------------ traffic counters
def _counter_rows(path):
    """(kernel name, counter value) per dispatch from one rocprofv3 counter-collection CSV."""
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            val = row.get("Counter_Value") or row.get("Counter-Value")
            if name and val not in (None, ""):
                yield name, float(val)


def _kernel_base(name: str) -> str:
    """'void attn::(anonymous namespace)::prefill16_kernel<...>(...)' -> 'prefill16_kernel'."""
    n = name.replace("(anonymous namespace)", "").split("<")[0].split("(")[0]
    return n.split("::")[-1].replace("void ", "").strip()


def _per_kernel_median(rows, keep):
    vals = {}
    for name, val in rows:
        base = _kernel_base(name)
        if base in keep:
            vals.setdefault(base, []).append(val)
    return {k: statistics.median(v) for k, v in vals.items()}


def traffic_from(root: str) -> dict:
    """Reduce rocprofv3 FETCH_SIZE / WRITE_SIZE runs under `root` (folders
    <workload>_FETCH_SIZE and <workload>_WRITE_SIZE, plus copy_FETCH_SIZE and
    copy_WRITE_SIZE for the 1 GiB calibration copy) to bytes per step, and
    write profiles/traffic.json."""
    def counters(folder):
        files = glob.glob(os.path.join(root, folder, "**", "*counter_collection.csv"), recursive=True)
        rows = []
        for p in files:
            rows.extend(_counter_rows(p))
        return rows

    copy_f = [v for n, v in counters("copy_FETCH_SIZE") if "copy" in n.lower()]
    copy_w = [v for n, v in counters("copy_WRITE_SIZE") if "copy" in n.lower()]
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy found under " + root)
    gib_kib = (1 << 30) / 1024
    fscale, wscale = gib_kib / statistics.median(copy_f), gib_kib / statistics.median(copy_w)
    out = {"calibration": {"copy_bytes": 1 << 30, "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
                           "copy_fetch_kib": statistics.median(copy_f), "copy_write_kib": statistics.median(copy_w),
                           "note": "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) read for a 1 GiB device copy; "
                                   "scale = 1 GiB / reading"},
           "workloads": {}}
    for name in WORKLOADS:
        kind = name.split("_")[0]
        keep = set(STEP_KERNELS[kind])
        fk = _per_kernel_median(counters(name + "_FETCH_SIZE"), keep)
        wk = _per_kernel_median(counters(name + "_WRITE_SIZE"), keep)
        if not fk or not wk:
            continue
        per = {k: {"fetch_kib": fk.get(k, 0.0), "write_kib": wk.get(k, 0.0)} for k in sorted(set(fk) | set(wk))}
        total = sum(v["fetch_kib"] * fscale + v["write_kib"] * wscale for v in per.values()) * 1024
        out["workloads"][name] = {"workload": WORKLOADS[name][1], "per_kernel": per,
                                  "bytes_per_step": int(round(total)),
                                  "sources": {s: kernel_source_hash(s) for s in KERNEL_SOURCES[kind]}}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


# ----------------------------------------------------------------------- main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed launches per workload")
    ap.add_argument("--warmup", type=int, default=10, help="untimed launches first (at least)")
    ap.add_argument("--min-warmup-ms", type=float, default=200.0,
                    help="and at least this much wall time of warm-up launches per workload")
    ap.add_argument("--only", default=None,
                    help="time only these workloads (comma-separated names from: " + ", ".join(WORKLOADS) + ")")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the headline workload's CPU baseline "
                         "(the other workloads get less)")
    ap.add_argument("--no-gemm", action="store_true", help="skip the library GEMM reference")
    ap.add_argument("--gemm", action="store_true", help="time the library GEMM reference with --only too")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR", default=None,
                    help="write profiles/traffic.json from rocprofv3 counter runs under DIR and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              f"multi-GPU path.", file=sys.stderr)
        return 2
    if args.traffic_from:
        rec = traffic_from(args.traffic_from)
        print(json.dumps({k: v["bytes_per_step"] for k, v in rec["workloads"].items()}))
        return 0

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

    names = [x for x in args.only.split(",") if x] if args.only else DEFAULT_ORDER
    bad = [x for x in names if x not in WORKLOADS]
    if bad:
        print(f"unknown workload(s): {', '.join(bad)}", file=sys.stderr)
        return 2
    res = {}
    cache = None
    for name in names:
        cid = WORKLOADS[name][0]
        cfg = A.CONFIGS[cid]
        print(f"# {name}: {WORKLOADS[name][1]}", file=sys.stderr, flush=True)
        if name.startswith("prefill"):
            r = bench_prefill(name, cfg, args, torch, E)
        elif name.startswith("backward"):
            r = bench_backward(name, cfg, args, torch, E)
        else:
            if cache is None:
                cache = DecodeCache(torch)
            if name == "decode_c5_paged":
                r = bench_decode_paged(name, cfg, args, torch, E, cache)
            elif name == "decode_c5_fp8":
                r = bench_decode_fp8(name, cfg, args, torch, E, cache)
            else:
                r = bench_decode(name, cfg, args, torch, E, cache)
        t = r["timing"]
        print(f"#   mean {t['mean_ms']:.4f} ms  p50 {t['p50_ms']:.4f} ms  {r['value']} {r['unit']}  "
              f"({100 * r['roofline']['frac']:.1f}% of peak)", file=sys.stderr, flush=True)
        res[name] = r
    del cache
    torch.cuda.empty_cache()
    gemm = None if (args.no_gemm or (args.only and not args.gemm)) else library_gemm_tflops(torch, args)

    if not args.no_cpu:
        budgets = {"prefill_c4": args.cpu_budget, "prefill_c3": args.cpu_budget / 2,
                   "prefill_c2": args.cpu_budget / 2, "prefill_c1": 1.0, "decode_c5": args.cpu_budget / 3}
        for name, budget in budgets.items():
            if name in res:
                cfg = A.CONFIGS[WORKLOADS[name][0]]
                fn = cpu_baseline_decode if name.startswith("decode") else cpu_baseline_prefill
                cb = fn(cfg, budget)
                res[name]["cpu_baseline"] = cb
                print(f"# cpu baseline {name}: {cb['value']} {cb['unit']} ({cb['sample']})",
                      file=sys.stderr, flush=True)

    head_name = names[0]
    head = res[head_name]
    cfg = A.CONFIGS[WORKLOADS[head_name][0]]
    line = {
        "metric": METRIC,
        "value": head["value"], "unit": head["unit"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["timing"]["mean_ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": head["workload"], "B": cfg.B, "H_q": cfg.H_q, "H_kv": cfg.H_kv,
                   "seq_len": cfg.N_kv, "query_len": cfg.N_q, "head_dim": cfg.d, "causal": cfg.causal,
                   "parallelism": "single GPU"},
        "timing": head["timing"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if "first_call_ms" in head:
        line["first_call_ms"] = head["first_call_ms"]
    line["workloads"] = res
    if gemm:
        line["library_gemm"] = gemm
    line["device"] = {"name": props.name, "cus": props.multi_processor_count,
                      "arch": getattr(props, "gcnArchName", "")}
    line["page_context"] = PAGE_CONTEXT
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
