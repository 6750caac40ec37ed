"""Benchmark of the paged MLA latent-K path on one MI355X.

A step is one call of mla_decompress_k_paged on the bf16 decode-sized batch
(64 requests, cached lengths U{256..4096}, page_size 128, rows of 576 = 512
latent + 64 rope, W_k [16384, 512]): the paged gather into k_latent_buffer and
the up-projection into k_buffer.  Inputs are seeded synthetic data resident in
HBM before timing starts.  `value` is rows per second of whole calls.

The roofline object is for the dominant kernel, the bf16 product: its launches
are timed on their own through mla_latent_matmul (one kernel per call) over the
rows the gather produced, and `achieved` = 2*M*N*K / average launch time.  The
gather step is timed the same way through mla_gather_latent_paged.

The JSON line also carries the other rows of the path, each timed the same way:
  c2_prefill   bf16, 4 x 16384 rows, copies starting mid-cache
  c3_fp8       fp8 block-scaled form on the same shapes (quantise pass + product)
  c6_fp8_cache the same shapes read from an e4m3 cache with per-128-column scales
  c4_kv_matmul write path, 128 lognormal requests, hidden 4096 -> 2 x 8 x 128
  c2_fused_kv  K and V decompression in one call, against two separate calls
  c6_fused_kv_fp8_cache  the same from the e4m3 cache, against two calls
  c2_tp8_share one GPU's share of W_k when 8 GPUs split the heads (N = 2048)
  c5_latent_write  RMSNorm + rope rotation + scatter of 88994 new tokens'
               rows into the MLA pages (HBM-bound), and c5_latent_write_fp8
               into an e4m3 cache (codes + fp32 scale per 128 columns)
  c7_absorb    query absorption for a decode batch of 128 tokens x 128 heads
               (w_uk [128, 512, 128]; HIP-graph replay like p64/p256), and
               c7_absorb_fp8 with an e4m3 w_uk and 128x128 block scales
  p64, p256    1 and 4 newest rows per request of the decode batch (weight-bound;
               timed by HIP-graph replay over 32 weight copies, see probe_row)

Timing: HIP events recorded on the stream the library launches on (torch's
current stream), per launch and around the whole timed region, bracketed by
torch.cuda.synchronize().  The untimed warmup is W calls, continued until the
GPU has been busy for 0.2 s (its clock ramps up over the first tens of ms after
the host-side set-up); `warmup_run` reports how many calls that took.  The CPU baseline times the oracle on the host cores
on a bounded sample of the same workload and is a reported baseline only.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decompressed K rows/sec + TFLOP/s (% MFMA peak) at kv_lora_rank=512, N=16384"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
CSRC = "mla_paged_latent_page_amd/csrc/"
KERNEL_SOURCES = {
    "gemm_bf16_ring": ("decompress_bf16_ring.hip", "bf16_tile_common.hpp", "decompress_bf16.hip"),
    "gather_rows_kernel": ("gather.hip",),
    "gemm_fp8_ring": ("decompress_fp8_ring.hip", "decompress_fp8.hip", "bf16_tile_common.hpp"),
    "kv_matmul_ring": ("kv_matmul_ring.hip", "kv_matmul.hip", "bf16_tile_common.hpp"),
    "decompress_small_bf16": ("decompress_small.hip",),
    "latent_write_kernel": ("latent_write.hip",),
    "absorb_bf16": ("absorb.hip",),
    "absorb_fp8": ("absorb.hip",),
}


def source_hash(kernel):
    """Hash of the sources a kernel is built from (its own files + common.hpp)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel] + ("common.hpp", "launch.hpp"):
        with open(os.path.join(ROOT, CSRC, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


WARM_SECONDS = 0.2   # the GPU's clock ramps up over some tens of ms after host-side set-up


class Timed:
    """Run fn() warmup + steps times on the current stream with HIP events.

    The untimed warmup is `warmup` calls, continued until they have kept the
    GPU busy for warm_seconds: timed right after the inputs are built, the
    first ~30 ms of calls run several per cent slow while the clock ramps up."""

    warm_seconds = WARM_SECONDS

    def __init__(self, torch, fn, steps, warmup):
        self.torch = torch
        stream = torch.cuda.current_stream()
        w0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - w0 < Timed.warm_seconds:
            fn()
            n += 1
            if n % 8 == 0 or n == warmup:
                torch.cuda.synchronize()
        self.warmup_run = n
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(stream)
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        self.wall_s = time.perf_counter() - wall0
        self.total_ms = t0.elapsed_time(t1)
        self.launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        self.avg_launch_ms = float(np.mean(self.launch_ms))
        self.min_launch_ms = float(np.min(self.launch_ms))
        self.ms_per_step = self.total_ms / steps


def decompress_runner(torch, mp, W, case):
    dc, t = W.device_decompress(case)
    M, D, N = case.M, case.D_c, case.N
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    if case.weight_dtype == "e4m3":
        ws = torch.empty(mp.mla_decompress_k_paged_fp8_workspace_size(M, case.K), dtype=torch.uint8, device="cuda")

        def fn():
            mp.mla_decompress_k_paged_fp8(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                          t["weight_scale"], cache, case.layer_idx, lat, out, ws)
    else:
        def fn():
            mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], cache,
                                      case.layer_idx, lat, out)
    return fn


def kv_runner(torch, mp, W, case, case_v):
    """One fused K and V call (mla_decompress_kv_paged) on a case and its W_uv."""
    dc, t = W.device_decompress(case)
    _, tv = W.device_decompress(case_v)
    M, D = case.M, case.D_c
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    kout = torch.empty((M, case.N), dtype=torch.bfloat16, device="cuda")
    vout = torch.empty((M, case_v.N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)

    def fused():
        mp.mla_decompress_kv_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], tv["weight"],
                                   cache, case.layer_idx, lat, kout, vout)

    def separate():
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], cache,
                                  case.layer_idx, lat, kout)
        mp.mla_latent_matmul(lat, M, tv["weight"], vout)
    return fused, separate


def decompress_costs(case):
    """(flops, algorithmic HBM bytes) of one call: read each gathered cache row,
    write it to k_latent, write the k_buffer row, read the weight once."""
    M, N, K, D = case.M, case.N, case.K, case.D_c
    flops = 2.0 * M * N * K
    if case.weight_dtype == "e4m3":
        w_bytes = N * K + case.weight_scale.nbytes
        out_b = 2
    else:
        w_bytes = N * K * 2
        out_b = 2
    return flops, M * (2 * D * 2 + N * out_b) + w_bytes


def probe_case(W, base, newest):
    """The decode batch with only each request's `newest` last cached rows."""
    lens = base.cache.cache_lengths.astype(np.int64)
    offs = lens - newest
    bro = np.zeros(len(lens) + 1, np.uint32)
    bro[1:] = np.cumsum(np.full(len(lens), newest))
    return W.DecompressCase(f"p{newest * len(lens)}", base.cache, base.layer_idx, bro, offs.astype(np.uint32),
                            base.K, base.N, base.weight, base.weight_dtype)


def probe_row(torch, mp, W, pc, warmup, copies=32, reps=20):
    """Few-rows call timed without launch overhead: `copies` launches, each on
    its own copy of the weight (32 x 16 MiB, so every launch reads its weight
    from HBM, not from the last-level cache), captured once in a HIP graph and
    replayed `reps` times between two events.  The graph's output is checked
    against an eager call first."""
    dc, t = W.device_decompress(pc)
    M, D, N = pc.M, pc.D_c, pc.N
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    weights = [t["weight"].clone() for _ in range(copies)]

    def call(w):
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, w, cache, pc.layer_idx, lat, out)
    call(weights[0])
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w in weights[:3]:
            call(w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w in weights:
            call(w)
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.int16), eager.view(torch.int16)):
        raise RuntimeError(f"{pc.name}: graph replay differs from the eager call")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * copies)
    f, b = decompress_costs(pc)
    gbs = b / (ms * 1e-3) / 1e9
    del g
    return {"rows": M, "us_per_call": round(ms * 1e3, 3), "tflops": round(f / (ms * 1e-3) / 1e12, 2),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_from_profile("decompress_small_bf16", pc.name)),
            "kernel": "decompress_small_bf16 (gather + product in one launch)",
            "timing": f"HIP graph of {copies} launches on {copies} weight copies, replayed {reps} times"}


def absorb_row(torch, mp, W, warmup, copies=32, reps=20, fp8=False):
    """Query absorption for a decode batch (a few microseconds per call), timed
    like the few-rows probes: `copies` launches on their own copies of w_uk
    (16 MiB each, so every launch reads its weight from HBM), captured in one
    HIP graph and replayed `reps` times; checked against an eager call first."""
    c = W.c7_absorb_fp8() if fp8 else W.c7_absorb()
    t = W.device_absorb(c)
    out = torch.empty((c.T, c.H, c.out_dim), dtype=torch.bfloat16, device="cuda")
    weights = [t["w_uk_e4m3" if fp8 else "w_uk"].clone() for _ in range(copies)]

    def call(w):
        if fp8:
            mp.mla_absorb_q_fp8(t["q"], w, t["w_uk_scale"], out, d_nope=c.d_nope, copy_rope=c.copy_rope)
        else:
            mp.mla_absorb_q(t["q"], w, out, d_nope=c.d_nope, copy_rope=c.copy_rope)
    call(weights[0])
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for w in weights[:3]:
            call(w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w in weights:
            call(w)
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.int16), eager.view(torch.int16)):
        raise RuntimeError(f"{c.name}: graph replay differs from the eager call")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * copies)
    T, H, L, Dq = c.T, c.H, c.kv_latent_dim, c.q.shape[2]
    wb = H * L * c.d_nope + c.w_scale.nbytes if fp8 else H * L * c.d_nope * 2
    b = wb + T * H * Dq * 2 + T * H * c.out_dim * 2
    gbs = b / (ms * 1e-3) / 1e9
    kern = "absorb_fp8" if fp8 else "absorb_bf16"
    del g, weights
    return {"tokens": T, "heads": H, "us_per_call": round(ms * 1e3, 3),
            "tflops": round(2.0 * T * H * L * c.d_nope / (ms * 1e-3) / 1e12, 2),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_from_profile(kern, c.name)),
            "kernel": kern,
            "timing": f"HIP graph of {copies} launches on {copies} weight copies, replayed {reps} times",
            "note": "algorithmic bytes: w_uk once (16 MiB bf16, 8 MiB e4m3 + scales), the queries (nope + rope) "
                    "once, the output once"}


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def cpu_baseline(case, seconds):
    """Time the oracle on the host: the gather of every row, then the product of
    randomly chosen rows in chunks until about `seconds` have been spent on it.
    rate = rows / (product time + gather time * rows / M)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    rng = np.random.default_rng(123)
    order = rng.permutation(case.M)
    t0 = time.perf_counter()
    lat = oracle.gather(case)
    t_gather = time.perf_counter() - t0
    done, chunk, t_mm = 0, 256, 0.0
    while done < case.M and t_mm < seconds:
        rows = np.sort(order[done:done + chunk])
        t1 = time.perf_counter()
        oracle.matmul_nt(lat, case.cache.dtype, case.weight, case.weight_dtype, case.K, rows)
        t_mm += time.perf_counter() - t1
        done += len(rows)
        chunk = min(chunk * 2, 2048)
    eff = t_mm + t_gather * done / case.M
    return {"value": round(done / eff, 2), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"gather of all {case.M} rows ({t_gather:.1f} s) + up-projection of {done} random rows "
                      f"({t_mm:.1f} s); rate = rows / (product time + gather time x rows/M)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="keep warming up until the GPU has been busy this long (0: exactly --warmup calls)")
    ap.add_argument("--rows", choices=["all", "main"], default="all",
                    help="also time the other rows of the path (default) or only the main workload")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-baseline sample (0: skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    Timed.warm_seconds = args.warm_seconds
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the path is measured on a single MI355X; "
              "multi-GPU sharding is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_paged_latent_page_amd as mp
    import workloads as W

    torch.cuda.set_device(0)
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        t = Timed(torch, lambda: dst.copy_(src), 5, 1)
        print(json.dumps({"copy_bytes_each_way": src.nbytes, "ms": round(t.avg_launch_ms, 4),
                          "read_plus_write_gbs": round(2 * src.nbytes / (t.avg_launch_ms * 1e-3) / 1e9, 1)}))
        return

    # ---- main workload: bf16 decode-sized batch
    case = W.c1_decode()
    fn = decompress_runner(torch, mp, W, case)
    tm = Timed(torch, fn, args.steps, args.warmup)
    flops, alg_bytes = decompress_costs(case)
    call_tf = flops / (tm.avg_launch_ms * 1e-3) / 1e12
    print(f"[bench] c1_decode M={case.M}: {tm.avg_launch_ms:.3f} ms/call, {call_tf:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    # the two steps on their own: gather (HBM copy) and the product (dominant kernel)
    dc, t = W.device_decompress(case)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    lat = torch.empty((case.M, case.D_c), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    tg = Timed(torch, lambda: mp.mla_gather_latent_paged(t["buffer_row_offsets"], t["cache_offsets"], case.M,
                                                         cache, case.layer_idx, lat), args.steps, args.warmup)
    tp = Timed(torch, lambda: mp.mla_latent_matmul(lat, case.M, t["weight"], out), args.steps, args.warmup)
    gather_bytes = case.M * case.D_c * 2 * 2
    prod_tf = flops / (tp.avg_launch_ms * 1e-3) / 1e12
    print(f"[bench] gather {tg.avg_launch_ms:.3f} ms ({gather_bytes / tg.avg_launch_ms / 1e6:.0f} GB/s), "
          f"product {tp.avg_launch_ms:.3f} ms ({prod_tf:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    del lat, out, dc, t, cache
    rows_per_s = case.M * args.steps / (tm.total_ms * 1e-3)
    result = {
        "metric": METRIC, "value": round(rows_per_s, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_run": tm.warmup_run, "ms_per_step": round(tm.ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c1_decode: bf16 decode-sized batch, 64 requests with cached lengths "
                               "U{256..4096} copied from position 0, page_size 128, 576-wide rows "
                               "(kv_lora_rank 512 + rope 64), W_k [16384, 512]",
                   "rows": case.M, "N": case.N, "K": case.K, "page_size": 128, "seed": 1},
        "tflops": round(call_tf, 2),
        "mfma_frac": round(call_tf / PEAK_BF16_TFLOPS, 4),
        "hbm_gbs_algorithmic": round(alg_bytes / (tm.avg_launch_ms * 1e-3) / 1e9, 1),
        "roofline": roofline("mfma", prod_tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic_from_profile("gemm_bf16_ring", "c1_decode")),
        "kernel": "gemm_bf16_ring<2,4> (the product step; 2*M*N*K flop per launch)",
        "launch_ms": {"call_avg": round(tm.avg_launch_ms, 4), "call_min": round(tm.min_launch_ms, 4),
                      "product_avg": round(tp.avg_launch_ms, 4), "product_min": round(tp.min_launch_ms, 4),
                      "gather_avg": round(tg.avg_launch_ms, 4), "gather_min": round(tg.min_launch_ms, 4)},
        "gather": {"kernel": "gather_rows_kernel", "bytes_per_launch": gather_bytes,
                   "roofline": roofline("hbm", gather_bytes / (tg.avg_launch_ms * 1e-3) / 1e9, PEAK_HBM_GBS,
                                        "GB/s", traffic_from_profile("gather_rows_kernel", "c1_decode"))},
        "published_baseline": "none: the pages publish no performance numbers",
    }

    # ---- the other rows of the path
    if args.rows == "all":
        rows = {}
        steps = max(3, args.steps // 2)
        for probe_n in (1, 4):
            pc = probe_case(W, case, probe_n)
            rows[pc.name] = probe_row(torch, mp, W, pc, args.warmup)
            r = rows[pc.name]
            print(f"[bench] {pc.name}: {r['us_per_call']:.2f} us/call (graph replay), "
                  f"{r['roofline']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
        del fn
        torch.cuda.empty_cache()
        for name, make, bound in (("c2_prefill", W.c2_prefill, "mfma"), ("c3_fp8", W.c3_fp8, "hbm")):
            c = make()
            t = Timed(torch, decompress_runner(torch, mp, W, c), steps, args.warmup)
            f, b = decompress_costs(c)
            tf = f / (t.avg_launch_ms * 1e-3) / 1e12
            gbs = b / (t.avg_launch_ms * 1e-3) / 1e9
            entry = {"rows": c.M, "ms": round(t.avg_launch_ms, 4), "rows_per_s": round(c.M / (t.avg_launch_ms * 1e-3), 1),
                     "tflops": round(tf, 2), "hbm_gbs_algorithmic": round(gbs, 1)}
            if bound == "mfma":
                entry["roofline"] = roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                             traffic_from_profile("gemm_bf16_ring", name))
                entry["note"] = "time per call: gather + product (gemm_bf16_ring); traffic: the product kernel"
            else:
                entry["roofline"] = roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                             traffic_from_profile("gemm_fp8_ring", name))
                entry["fp8_mfma_frac"] = round(tf / PEAK_FP8_TFLOPS, 4)
                entry["note"] = "time per call: gather + quantise pass (gather_quant_fp8_kernel) + fp8 product (gemm_fp8_ring)"
            rows[name] = entry
            print(f"[bench] {name}: {t.avg_launch_ms:.3f} ms, {tf:.1f} TFLOP/s, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        # the prefill batch read from an e4m3 cache with per-128-column scales
        c = W.c6_fp8_cache()
        dc, tt = W.device_decompress(c)
        nblk = c.cache.scale_blocks
        f8lat = torch.empty((c.M, c.D_c), dtype=torch.uint8, device="cuda")
        f8sc = torch.empty((c.M, nblk), dtype=torch.float32, device="cuda")
        f8out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        f8cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)

        def f8_fn():
            mp.mla_decompress_k_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, tt["weight_q"],
                                                tt["weight_scale"], f8cache, c.layer_idx, f8lat, f8sc, f8out)
        t = Timed(torch, f8_fn, steps, args.warmup)
        f = 2.0 * c.M * c.N * c.K
        b = c.M * (2 * (c.D_c + nblk * 4) + c.N * 2) + c.N * c.K + c.weight_scale.nbytes
        tf = f / (t.avg_launch_ms * 1e-3) / 1e12
        gbs = b / (t.avg_launch_ms * 1e-3) / 1e9
        rows["c6_fp8_cache"] = {"rows": c.M, "ms": round(t.avg_launch_ms, 4),
                                "rows_per_s": round(c.M / (t.avg_launch_ms * 1e-3), 1), "tflops": round(tf, 2),
                                "hbm_gbs_algorithmic": round(gbs, 1), "fp8_mfma_frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                                     traffic_from_profile("gemm_fp8_ring", "c6_fp8_cache")),
                                "note": "time per call: gather of e4m3 rows and their scales (gather_rows_kernel) "
                                        "+ fp8 product on them (gemm_fp8_ring); no quantisation pass"}
        print(f"[bench] c6_fp8_cache: {t.avg_launch_ms:.3f} ms, {tf:.1f} TFLOP/s, {gbs:.0f} GB/s", file=sys.stderr,
              flush=True)
        # K and V from the same e4m3 cache in one call, against two single-projection calls
        cv8 = W.with_second_projection(c, seed=1006, N=c.N)
        wv8 = torch.from_numpy(cv8.weight_q).cuda()
        sv8 = torch.from_numpy(cv8.weight_scale).cuda()
        f8vout = torch.empty((c.M, cv8.N), dtype=torch.bfloat16, device="cuda")

        def f8kv_fn():
            mp.mla_decompress_kv_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, tt["weight_q"],
                                                 tt["weight_scale"], wv8, sv8, f8cache, c.layer_idx, f8lat, f8sc,
                                                 f8out, f8vout)

        def f8kv_separate():
            f8_fn()
            mp.mla_decompress_k_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, wv8, sv8, f8cache,
                                                c.layer_idx, f8lat, f8sc, f8vout)
        t = Timed(torch, f8kv_fn, steps, args.warmup)
        t2 = Timed(torch, f8kv_separate, steps, args.warmup)
        f = 2.0 * c.M * (c.N + cv8.N) * c.K
        b = (c.M * (2 * (c.D_c + nblk * 4) + (c.N + cv8.N) * 2) + (c.N + cv8.N) * c.K + c.weight_scale.nbytes
             + cv8.weight_scale.nbytes)
        tf = f / (t.avg_launch_ms * 1e-3) / 1e12
        gbs = b / (t.avg_launch_ms * 1e-3) / 1e9
        rows["c6_fused_kv_fp8_cache"] = {
            "rows": c.M, "ms": round(t.avg_launch_ms, 4), "separate_calls_ms": round(t2.avg_launch_ms, 4),
            "tflops": round(tf, 2), "hbm_gbs_algorithmic": round(gbs, 1), "fp8_mfma_frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                 traffic_from_profile("gemm_fp8_ring", "c6_fused_kv_fp8_cache")),
            "note": "one gather of codes and scales + one gemm_fp8_ring launch over W_k's and W_uv's N-tiles; "
                    "separate_calls_ms: two mla_decompress_k_paged_fp8_cache calls (W_k, then W_uv)"}
        print(f"[bench] c6_fused_kv_fp8_cache: {t.avg_launch_ms:.3f} ms, {gbs:.0f} GB/s; separate calls "
              f"{t2.avg_launch_ms:.3f} ms", file=sys.stderr, flush=True)
        del f8kv_fn, f8kv_separate, wv8, sv8, f8vout
        del f8_fn, f8lat, f8sc, f8out, f8cache, dc, tt
        torch.cuda.empty_cache()
        # fused K and V on the prefill batch (W_uv drawn like W_k), against the
        # same work as a K call followed by a V product on the gathered rows
        c = W.c2_prefill()
        cv = W.with_second_projection(c, seed=1002, N=c.N)
        fused, separate = kv_runner(torch, mp, W, c, cv)
        t = Timed(torch, fused, steps, args.warmup)
        t2 = Timed(torch, separate, steps, args.warmup)
        f = 2.0 * c.M * (c.N + cv.N) * c.K
        b = c.M * (2 * c.D_c * 2 + (c.N + cv.N) * 2) + (c.N + cv.N) * c.K * 2
        tf = f / (t.avg_launch_ms * 1e-3) / 1e12
        rows["c2_fused_kv"] = {"rows": c.M, "ms": round(t.avg_launch_ms, 4),
                               "separate_calls_ms": round(t2.avg_launch_ms, 4), "tflops": round(tf, 2),
                               "hbm_gbs_algorithmic": round(b / (t.avg_launch_ms * 1e-3) / 1e9, 1),
                               "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                    traffic_from_profile("gemm_bf16_ring", "c2_fused_kv")),
                               "note": "one gather + one gemm_bf16_ring launch over the N-tiles of W_k, then "
                                       "those of W_uv [16384, 512] (each XCD keeps one projection's share of "
                                       "the weight in L2 at a time); separate_calls_ms: mla_decompress_k_paged "
                                       "then mla_latent_matmul with W_uv"}
        print(f"[bench] c2_fused_kv: {t.avg_launch_ms:.3f} ms ({tf:.1f} TFLOP/s); separate calls "
              f"{t2.avg_launch_ms:.3f} ms", file=sys.stderr, flush=True)
        del fused, separate
        torch.cuda.empty_cache()
        # one GPU's share of W_k under 8-way tensor parallelism over heads: N = 2048
        ct = dataclasses.replace(c, name="c2_tp8_share", N=2048, weight=np.ascontiguousarray(c.weight[:2048]))
        t = Timed(torch, decompress_runner(torch, mp, W, ct), steps, args.warmup)
        f, b = decompress_costs(ct)
        tf = f / (t.avg_launch_ms * 1e-3) / 1e12
        rows["c2_tp8_share"] = {"rows": ct.M, "N": 2048, "ms": round(t.avg_launch_ms, 4), "tflops": round(tf, 2),
                                "hbm_gbs_algorithmic": round(b / (t.avg_launch_ms * 1e-3) / 1e9, 1),
                                "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                     traffic_from_profile("gemm_bf16_ring", "c2_tp8_share")),
                                "note": "the prefill batch against the first 16 heads of W_k (N = 2048), "
                                        "one GPU's share at 8-way tensor parallelism over heads"}
        print(f"[bench] c2_tp8_share: {t.avg_launch_ms:.3f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        kc = W.c4_kv_matmul()
        dc, tt = W.device_kv(kc)
        cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)

        def kv_fn():
            mp.kv_matmul_paged(tt["hidden"], tt["input_row_offsets"], tt["weight"], cache, kc.layer_idx)
        t = Timed(torch, kv_fn, steps, args.warmup)
        f = 2.0 * kc.T * kc.hidden_dim * kc.N
        b = kc.T * (kc.hidden_dim * 2 + kc.N * 2) + kc.weight.nbytes
        tf = f / (t.avg_launch_ms * 1e-3) / 1e12
        rows["c4_kv_matmul"] = {"tokens": kc.T, "ms": round(t.avg_launch_ms, 4), "tflops": round(tf, 2),
                                "hbm_gbs_algorithmic": round(b / (t.avg_launch_ms * 1e-3) / 1e9, 1),
                                "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                     traffic_from_profile("kv_matmul_ring", "c4_kv_matmul")),
                                "kernel": "kv_matmul_ring"}
        print(f"[bench] c4_kv_matmul: {t.avg_launch_ms:.3f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del dc, tt, cache
        torch.cuda.empty_cache()
        # the latent write path (RMSNorm + rope rotation + scatter into the MLA pages)
        lc = W.c5_latent_write()
        ldc, lt = W.device_latent_write(lc)
        lcache = mp.PagedKVCache(ldc.pool, ldc.page_table, ldc.cache_lengths)

        def lw_fn():
            mp.mla_write_latent_paged(lt["x"], lt["input_row_offsets"], lt["gamma"], lc.eps, lt["freqs"], lc.K,
                                      lcache, lc.layer_idx)
        t = Timed(torch, lw_fn, steps, args.warmup)
        D = lc.x.shape[1]
        b = lc.T * (D * 2 * 2 + (D - lc.K) * 4) + lc.K * 4
        gbs = b / (t.avg_launch_ms * 1e-3) / 1e9
        rows["c5_latent_write"] = {"tokens": lc.T, "ms": round(t.avg_launch_ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
                                   "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                                        traffic_from_profile("latent_write_kernel", "c5_latent_write")),
                                   "kernel": "latent_write_kernel",
                                   "note": "per token: read the 1152-byte row and its 256-byte rope table row, "
                                           "write the 1152-byte cache row"}
        print(f"[bench] c5_latent_write: {t.avg_launch_ms:.4f} ms, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        del ldc, lt, lcache
        # the same batch written into an e4m3 cache (codes + one fp32 scale per 128 columns)
        lc8 = W.c5_latent_write_fp8()
        ldc8, lt8 = W.device_latent_write(lc8)
        lcache8 = mp.PagedKVCache(ldc8.pool, ldc8.page_table, ldc8.cache_lengths, scales=ldc8.scales)

        def lw8_fn():
            mp.mla_write_latent_paged_fp8(lt8["x"], lt8["input_row_offsets"], lt8["gamma"], lc8.eps, lt8["freqs"],
                                          lc8.K, lcache8, lc8.layer_idx)
        t = Timed(torch, lw8_fn, steps, args.warmup)
        D = lc8.x.shape[1]
        nblk = -(-D // 128)
        b = lc8.T * (D * 2 + (D - lc8.K) * 4 + D + nblk * 4) + lc8.K * 4
        gbs = b / (t.avg_launch_ms * 1e-3) / 1e9
        rows["c5_latent_write_fp8"] = {
            "tokens": lc8.T, "ms": round(t.avg_launch_ms, 4), "hbm_gbs_algorithmic": round(gbs, 1),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                 traffic_from_profile("latent_write_kernel", "c5_latent_write_fp8")),
            "kernel": "latent_write_kernel<true>",
            "note": "per token: read the 1152-byte row and its 256-byte rope table row, write 576 e4m3 codes "
                    "and 5 fp32 scales"}
        print(f"[bench] c5_latent_write_fp8: {t.avg_launch_ms:.4f} ms, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        del ldc8, lt8, lcache8
        for name, f8 in (("c7_absorb", False), ("c7_absorb_fp8", True)):
            rows[name] = absorb_row(torch, mp, W, args.warmup, fp8=f8)
            r = rows[name]
            print(f"[bench] {name}: {r['us_per_call']:.2f} us/call (graph replay), "
                  f"{r['roofline']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
        result["rows"] = rows

    if args.cpu_seconds > 0:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
