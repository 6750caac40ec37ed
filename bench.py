"""Benchmark of the paged MLA latent-K path on one MI355X.

A step is one call of mla_decompress_k_paged on the bf16 decode-sized batch
(64 requests, cached lengths U{256..4096}, page_size 128, rows of 576 = 512
latent + 64 rope, W_k [16384, 512]): the paged gather into k_latent_buffer and
the up-projection into k_buffer.  Inputs are seeded synthetic data resident in
HBM before timing starts.  `value` is rows per second of whole calls, back to
back.

The roofline object is for the dominant kernel, the bf16 product: its launches
are timed on their own through mla_latent_matmul (one kernel per call) over the
rows the gather produced, and `achieved` = 2*M*N*K / average launch time.  The
gather step is timed the same way through mla_gather_latent_paged.

The JSON line also carries the other rows of the path (OTHER_ROWS below), each timed
the same way, or, for calls of a few microseconds, by HIP-graph replay over 32
copies of the weight (so every launch reads its weight from HBM).

Timing: HIP events recorded on the stream the library launches on (torch's
current stream), per launch and around the whole timed region, bracketed by
torch.cuda.synchronize().  The untimed warmup is W calls, continued until the
GPU has been busy for 0.2 s (its clock ramps up over the first tens of ms after
the host-side set-up).  Launch times are reported as median, mean and minimum.
`cold`: the product launch timed alone after writing a 512 MB scratch buffer
(twice the last-level cache) before each launch, median of the launches.
`peaks`: ceilings measured on the same GPU in the same run (the bf16 matrix
pipe under the product's operand pattern, HBM read and write streams, a 16 MiB
read, an empty launch).  The CPU baseline times the oracle on the host cores
on a bounded sample of the same workload and is a reported baseline only.

Profiling and records (profiles/):
  --profile ROW            run only ROW's call (steps times after warmup), for
                           rocprofv3 --kernel-trace / --pmc runs
  --traffic-from F W       with --row ROW: from the FETCH_SIZE and WRITE_SIZE
                           counter CSVs of `--profile ROW` runs, write
                           profiles/<kernel>_<row>_hbm_traffic.json (ROW copy:
                           the calibration of both counters on a 1 GiB copy)
  --counters-from CSV...   with --row ROW: summarise counter CSVs of
                           `--profile ROW` runs (matrix-pipe busy cycles, clock,
                           vector-memory unit busy, LDS busy and bank-conflict
                           stalls) into
                           profiles/<kernel>_<row>_counters.json
"""
import argparse
import csv
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
    "decompress_small_fp8_gq": ("decompress_fp8_small.hip", "decompress_fp8.hip", "bf16_tile_common.hpp"),
    "decompress_small_fp8_gc": ("decompress_fp8_small.hip", "decompress_fp8.hip", "bf16_tile_common.hpp"),
    "latent_write_kernel": ("latent_write.hip",),
    "absorb_bf16": ("absorb.hip",),
    "absorb_fp8": ("absorb.hip",),
    "__amd_rocclr_copyBuffer": (),
}
COPY_BYTES = 1 << 30


def source_hash(kernel):
    """Hash of the sources a kernel is built from (its own files + common.hpp)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel] + ("common.hpp", "launch.hpp"):
        with open(os.path.join(ROOT, CSRC, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _record(kernel, workload, kind):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_{kind}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_hash") == source_hash(kernel) else None


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from the committed counter record, if it was taken
    on the current kernel source; else None."""
    rec = _record(kernel, workload, "hbm_traffic")
    return rec.get("hbm_bytes_per_launch") if rec else None


def counters_from_profile(kernel, workload):
    """Matrix-pipe utilisation and clock from the committed counter record, if
    it was taken on the current kernel source; else None."""
    rec = _record(kernel, workload, "counters")
    if not rec:
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "clock_ghz", "ta_busy_frac", "lds_busy_frac", "lds_bank_conflict_frac")
            if k in rec}


WARM_SECONDS = 0.2   # the GPU's clock ramps up over some tens of ms after host-side set-up


class Timed:
    """Run fn() warmup + steps times on the current stream with HIP events.

    The untimed warmup is `warmup` calls, continued until they have kept the
    GPU busy for warm_seconds: timed right after the inputs are built, the
    first ~30 ms of calls run several per cent slow while the clock ramps up."""

    warm_seconds = WARM_SECONDS

    def __init__(self, torch, fn, steps, warmup):
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
        self.median_launch_ms = float(np.median(self.launch_ms))
        self.min_launch_ms = float(np.min(self.launch_ms))
        self.ms_per_step = self.total_ms / steps

    def summary(self):
        return {"median": round(self.median_launch_ms, 4), "avg": round(self.avg_launch_ms, 4),
                "min": round(self.min_launch_ms, 4)}


def graph_time(torch, call, copies, reps, warmup, check=None):
    """Average time of call(i), i < copies, captured once in a HIP graph and
    replayed `reps` times between two events; check() (if given) compares the
    graph's result with an eager run first."""
    call(0)
    torch.cuda.synchronize()
    eager = check() if check else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            call(i)
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    if check and not torch.equal(check(), eager):
        raise RuntimeError("graph replay differs from the eager call")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * copies)


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# ---------------------------------------------------------------------------
# rows: each builds its inputs and returns a Row with one call per fn(i)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Row:
    fn: object                 # fn(i): one call (i picks a weight copy where the row rotates them)
    kernel: str                # dominant kernel (the one the roofline and the records are about)
    flops: float
    bytes: float               # algorithmic HBM bytes of one call
    bound: str                 # "mfma" or "hbm"
    peak: float                # the bound's peak (TFLOP/s or GB/s)
    copies: int = 0            # > 0: timed by graph replay over this many weight copies
    check: object = None       # graph rows: returns the output to compare with an eager call
    info: dict = dataclasses.field(default_factory=dict)
    separate: object = None    # fused rows: the same work as separate calls


def decompress_costs(case):
    """(flops, algorithmic HBM bytes) of one call: read each gathered cache row,
    write it to k_latent, write the k_buffer row, read the weight once."""
    M, N, K, D = case.M, case.N, case.K, case.D_c
    flops = 2.0 * M * N * K
    w_bytes = N * K + case.weight_scale.nbytes if case.weight_dtype == "e4m3" else N * K * 2
    return flops, M * (2 * D * 2 + N * 2) + w_bytes


def decompress_row(torch, mp, W, case, bound="mfma"):
    dc, t = W.device_decompress(case)
    M, D, N = case.M, case.D_c, case.N
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    f, b = decompress_costs(case)
    if case.weight_dtype == "e4m3":
        ws = torch.empty(mp.mla_decompress_k_paged_fp8_workspace_size(M, case.K), dtype=torch.uint8, device="cuda")

        def fn(i=0):
            mp.mla_decompress_k_paged_fp8(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                          t["weight_scale"], cache, case.layer_idx, lat, out, ws)
        return Row(fn, "gemm_fp8_ring", f, b, "hbm", PEAK_HBM_GBS,
                   info={"rows": M, "note": "time per call: gather + quantise pass (gather_quant_fp8_kernel) + "
                                            "fp8 product (gemm_fp8_ring)"})

    def fn(i=0):
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], cache,
                                  case.layer_idx, lat, out)
    return Row(fn, "gemm_bf16_ring", f, b, bound, PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS,
               info={"rows": M, "N": N, "note": "time per call: gather + product (gemm_bf16_ring)"})


def product_row(torch, mp, W, case):
    """The product step alone (mla_latent_matmul: one gemm_bf16_ring launch) over
    the rows the gather produced, and the gather step alone."""
    dc, t = W.device_decompress(case)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    lat = torch.empty((case.M, case.D_c), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    mp.mla_gather_latent_paged(t["buffer_row_offsets"], t["cache_offsets"], case.M, cache, case.layer_idx, lat)

    def product(i=0):
        mp.mla_latent_matmul(lat, case.M, t["weight"], out)

    def gather(i=0):
        mp.mla_gather_latent_paged(t["buffer_row_offsets"], t["cache_offsets"], case.M, cache, case.layer_idx, lat)
    f, _ = decompress_costs(case)
    gb = case.M * case.D_c * 2 * 2
    return (Row(product, "gemm_bf16_ring", f, case.M * (case.K * 2 + case.N * 2) + case.N * case.K * 2, "mfma",
                PEAK_BF16_TFLOPS),
            Row(gather, "gather_rows_kernel", 0.0, gb, "hbm", PEAK_HBM_GBS))


def probe_case(W, base, newest):
    """The decode batch with only each request's `newest` last cached rows."""
    lens = base.cache.cache_lengths.astype(np.int64)
    offs = lens - newest
    bro = np.zeros(len(lens) + 1, np.uint32)
    bro[1:] = np.cumsum(np.full(len(lens), newest))
    return W.DecompressCase(f"p{newest * len(lens)}", base.cache, base.layer_idx, bro, offs.astype(np.uint32),
                            base.K, base.N, base.weight, base.weight_dtype)


def probe_row(torch, mp, W, pc, copies=32):
    """Few-rows call: each launch on its own copy of the weight (32 x 16 MiB, so
    every launch reads its weight from HBM, not from the last-level cache)."""
    dc, t = W.device_decompress(pc)
    M, D, N = pc.M, pc.D_c, pc.N
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    weights = [t["weight"].clone() for _ in range(copies)]

    def fn(i=0):
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, weights[i % copies], cache,
                                  pc.layer_idx, lat, out)
    f, b = decompress_costs(pc)
    return Row(fn, "decompress_small_bf16", f, b, "hbm", PEAK_HBM_GBS, copies=copies,
               check=lambda: out.view(torch.int16).clone(),
               info={"rows": M, "kernel": "decompress_small_bf16 (gather + product in one launch)"})


def fp8_probe_case(W, newest=16):
    """C3's 4 requests, the newest `newest` tokens of each (64 rows by default),
    against C3's e4m3 W_k: the decode-sized fp8 call."""
    base = W.c3_fp8()
    q = probe_case(W, base, newest)
    return dataclasses.replace(base, name=f"p{q.M}_fp8", buffer_row_offsets=q.buffer_row_offsets,
                               cache_offsets=q.cache_offsets)


def probe_row_fp8(torch, mp, W, pc, copies=32):
    """Few-rows fp8 call (gather, quantisation and product in one launch): each
    launch on its own copy of the 8 MiB weight."""
    dc, t = W.device_decompress(pc)
    M, D, N = pc.M, pc.D_c, pc.N
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    ws = torch.empty(mp.mla_decompress_k_paged_fp8_workspace_size(M, pc.K), dtype=torch.uint8, device="cuda")
    weights = [t["weight_q"].clone() for _ in range(copies)]

    def fn(i=0):
        mp.mla_decompress_k_paged_fp8(t["buffer_row_offsets"], t["cache_offsets"], M, weights[i % copies],
                                      t["weight_scale"], cache, pc.layer_idx, lat, out, ws)
    f, b = decompress_costs(pc)
    return Row(fn, "decompress_small_fp8_gq", f, b, "hbm", PEAK_HBM_GBS, copies=copies,
               check=lambda: out.view(torch.int16).clone(),
               info={"rows": M, "kernel": "decompress_small_fp8_gq (gather, quantisation and product in one launch)"})


def fp8_cache_probe_case(W, newest=16):
    """C6's 4 requests, the newest `newest` tokens of each (64 rows by default),
    from its e4m3 cache: the decode-sized fp8-cache call."""
    base = W.c6_fp8_cache()
    q = probe_case(W, base, newest)
    return dataclasses.replace(base, name=f"p{q.M}_fp8_cache", buffer_row_offsets=q.buffer_row_offsets,
                               cache_offsets=q.cache_offsets)


def fp8_cache_call_bytes(c):
    """One fp8-cache call: each row's codes and scales read and written, its
    k_buffer row written, the weight codes and scales read once."""
    return c.M * (2 * (c.D_c + c.cache.scale_blocks * 4) + c.N * 2) + c.N * c.K + c.weight_scale.nbytes


def probe_row_fp8_cache(torch, mp, W, pc, copies=32):
    """Few-rows call on the e4m3 cache (codes and scales gathered into the
    product's LDS layout and multiplied in one launch): each launch on its own
    copy of the 8 MiB weight."""
    dc, t = W.device_decompress(pc)
    M, N = pc.M, pc.N
    lat = torch.empty((M, pc.D_c), dtype=torch.uint8, device="cuda")
    sc = torch.empty((M, pc.cache.scale_blocks), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    weights = [t["weight_q"].clone() for _ in range(copies)]

    def fn(i=0):
        mp.mla_decompress_k_paged_fp8_cache(t["buffer_row_offsets"], t["cache_offsets"], M, weights[i % copies],
                                            t["weight_scale"], cache, pc.layer_idx, lat, sc, out)
    return Row(fn, "decompress_small_fp8_gc", 2.0 * M * N * pc.K, fp8_cache_call_bytes(pc), "hbm", PEAK_HBM_GBS,
               copies=copies, check=lambda: out.view(torch.int16).clone(),
               info={"rows": M, "kernel": "decompress_small_fp8_gc (codes and scales gathered and multiplied in "
                                          "one launch)"})


def absorb_row(torch, mp, W, fp8, copies=32):
    c = W.c7_absorb_fp8() if fp8 else W.c7_absorb()
    t = W.device_absorb(c)
    out = torch.empty((c.T, c.H, c.out_dim), dtype=torch.bfloat16, device="cuda")
    weights = [t["w_uk_e4m3" if fp8 else "w_uk"].clone() for _ in range(copies)]

    def fn(i=0):
        w = weights[i % copies]
        if fp8:
            mp.mla_absorb_q_fp8(t["q"], w, t["w_uk_scale"], out, d_nope=c.d_nope, copy_rope=c.copy_rope)
        else:
            mp.mla_absorb_q(t["q"], w, out, d_nope=c.d_nope, copy_rope=c.copy_rope)
    T, H, L, Dq = c.T, c.H, c.kv_latent_dim, c.q.shape[2]
    wb = H * L * c.d_nope + c.w_scale.nbytes if fp8 else H * L * c.d_nope * 2
    b = wb + T * H * Dq * 2 + T * H * c.out_dim * 2
    return Row(fn, "absorb_fp8" if fp8 else "absorb_bf16", 2.0 * T * H * L * c.d_nope, b, "hbm", PEAK_HBM_GBS,
               copies=copies, check=lambda: out.view(torch.int16).clone(),
               info={"tokens": T, "heads": H, "note": "algorithmic bytes: w_uk once (16 MiB bf16, 8 MiB e4m3 + "
                                                      "scales), the queries (nope + rope) once, the output once"})


def fp8_cache_rows(torch, mp, W):
    """The prefill batch read from an e4m3 cache (K alone, and K and V in one call)."""
    c = W.c6_fp8_cache()
    dc, tt = W.device_decompress(c)
    nblk = c.cache.scale_blocks
    lat = torch.empty((c.M, c.D_c), dtype=torch.uint8, device="cuda")
    sc = torch.empty((c.M, nblk), dtype=torch.float32, device="cuda")
    kout = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    cv = W.with_second_projection(c, seed=1006, N=c.N)
    wv = torch.from_numpy(cv.weight_q).cuda()
    sv = torch.from_numpy(cv.weight_scale).cuda()
    vout = torch.empty((c.M, cv.N), dtype=torch.bfloat16, device="cuda")

    def k_only(i=0):
        mp.mla_decompress_k_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, tt["weight_q"],
                                            tt["weight_scale"], cache, c.layer_idx, lat, sc, kout)

    def kv(i=0):
        mp.mla_decompress_kv_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, tt["weight_q"],
                                             tt["weight_scale"], wv, sv, cache, c.layer_idx, lat, sc, kout, vout)

    def kv_separate(i=0):
        k_only()
        mp.mla_decompress_k_paged_fp8_cache(tt["buffer_row_offsets"], tt["cache_offsets"], c.M, wv, sv, cache,
                                            c.layer_idx, lat, sc, vout)
    row_b = 2 * (c.D_c + nblk * 4)
    one = Row(k_only, "gemm_fp8_ring", 2.0 * c.M * c.N * c.K,
              c.M * (row_b + c.N * 2) + c.N * c.K + c.weight_scale.nbytes, "hbm", PEAK_HBM_GBS,
              info={"rows": c.M, "note": "time per call: gather of e4m3 rows and their scales (gather_rows_kernel) "
                                         "+ fp8 product on them (gemm_fp8_ring); no quantisation pass"})
    two = Row(kv, "gemm_fp8_ring", 2.0 * c.M * (c.N + cv.N) * c.K,
              c.M * (row_b + (c.N + cv.N) * 2) + (c.N + cv.N) * c.K + c.weight_scale.nbytes + cv.weight_scale.nbytes,
              "hbm", PEAK_HBM_GBS, separate=kv_separate,
              info={"rows": c.M, "note": "one gather of codes and scales + one gemm_fp8_ring launch over W_k's and "
                                         "W_uv's N-tiles; separate_calls_ms: two mla_decompress_k_paged_fp8_cache "
                                         "calls (W_k, then W_uv)"})
    return one, two


def fused_kv_row(torch, mp, W):
    """K and V decompression in one call on the prefill batch (W_uv drawn like
    W_k), against a K call followed by a V product on the gathered rows."""
    c = W.c2_prefill()
    cv = W.with_second_projection(c, seed=1002, N=c.N)
    dc, t = W.device_decompress(c)
    _, tv = W.device_decompress(cv)
    M, D = c.M, c.D_c
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    kout = torch.empty((M, c.N), dtype=torch.bfloat16, device="cuda")
    vout = torch.empty((M, cv.N), dtype=torch.bfloat16, device="cuda")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)

    def fused(i=0):
        mp.mla_decompress_kv_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], tv["weight"],
                                   cache, c.layer_idx, lat, kout, vout)

    def separate(i=0):
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], cache,
                                  c.layer_idx, lat, kout)
        mp.mla_latent_matmul(lat, M, tv["weight"], vout)
    f = 2.0 * M * (c.N + cv.N) * c.K
    b = M * (2 * D * 2 + (c.N + cv.N) * 2) + (c.N + cv.N) * c.K * 2
    return Row(fused, "gemm_bf16_ring", f, b, "mfma", PEAK_BF16_TFLOPS, separate=separate,
               info={"rows": M, "note": "one gather + one gemm_bf16_ring launch over the N-tiles of W_k, then those "
                                        "of W_uv [16384, 512] (each XCD keeps one projection's share of the weight in "
                                        "L2 at a time); separate_calls_ms: mla_decompress_k_paged then "
                                        "mla_latent_matmul with W_uv"})


def kv_matmul_row(torch, mp, W):
    kc = W.c4_kv_matmul()
    dc, tt = W.device_kv(kc)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)

    def fn(i=0):
        mp.kv_matmul_paged(tt["hidden"], tt["input_row_offsets"], tt["weight"], cache, kc.layer_idx)
    return Row(fn, "kv_matmul_ring", 2.0 * kc.T * kc.hidden_dim * kc.N,
               kc.T * (kc.hidden_dim * 2 + kc.N * 2) + kc.weight.nbytes, "mfma", PEAK_BF16_TFLOPS,
               info={"tokens": kc.T, "kernel": "kv_matmul_ring"})


def latent_write_row(torch, mp, W, fp8):
    lc = W.c5_latent_write_fp8() if fp8 else W.c5_latent_write()
    ldc, lt = W.device_latent_write(lc)
    lcache = mp.PagedKVCache(ldc.pool, ldc.page_table, ldc.cache_lengths, scales=ldc.scales)
    call = mp.mla_write_latent_paged_fp8 if fp8 else mp.mla_write_latent_paged

    def fn(i=0):
        call(lt["x"], lt["input_row_offsets"], lt["gamma"], lc.eps, lt["freqs"], lc.K, lcache, lc.layer_idx)
    D = lc.x.shape[1]
    if fp8:
        b = lc.T * (D * 2 + (D - lc.K) * 4 + D + -(-D // 128) * 4) + lc.K * 4
        note = ("per token: read the 1152-byte row and its 256-byte rope table row, write 576 e4m3 codes and "
                "5 fp32 scales")
    else:
        b = lc.T * (D * 2 * 2 + (D - lc.K) * 4) + lc.K * 4
        note = "per token: read the 1152-byte row and its 256-byte rope table row, write the 1152-byte cache row"
    return Row(fn, "latent_write_kernel", 0.0, b, "hbm", PEAK_HBM_GBS,
               info={"tokens": lc.T, "kernel": "latent_write_kernel<true>" if fp8 else "latent_write_kernel",
                     "note": note})


def tp8_row(torch, mp, W):
    c = W.c2_prefill()
    ct = dataclasses.replace(c, name="c2_tp8_share", N=2048, weight=np.ascontiguousarray(c.weight[:2048]))
    r = decompress_row(torch, mp, W, ct)
    r.info["note"] = ("the prefill batch against the first 16 heads of W_k (N = 2048), one GPU's share at 8-way "
                      "tensor parallelism over heads")
    return r


def copy_row(torch):
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def fn(i=0):
        dst.copy_(src)
    return Row(fn, "__amd_rocclr_copyBuffer", 0.0, 2.0 * COPY_BYTES, "hbm", PEAK_HBM_GBS)


def build_row(name, torch, mp, W):
    """The named row (the names the JSON line and the profile records use)."""
    if name in ("c1_decode", "c1_product", "c1_gather"):
        case = W.c1_decode()
        if name == "c1_decode":
            return decompress_row(torch, mp, W, case)
        product, gather = product_row(torch, mp, W, case)
        return product if name == "c1_product" else gather
    if name == "c2_prefill":
        return decompress_row(torch, mp, W, W.c2_prefill())
    if name == "c3_fp8":
        return decompress_row(torch, mp, W, W.c3_fp8())
    if name in ("c6_fp8_cache", "c6_fused_kv_fp8_cache"):
        one, two = fp8_cache_rows(torch, mp, W)
        return one if name == "c6_fp8_cache" else two
    if name == "c2_fused_kv":
        return fused_kv_row(torch, mp, W)
    if name == "c2_tp8_share":
        return tp8_row(torch, mp, W)
    if name == "c4_kv_matmul":
        return kv_matmul_row(torch, mp, W)
    if name in ("c5_latent_write", "c5_latent_write_fp8"):
        return latent_write_row(torch, mp, W, name.endswith("fp8"))
    if name in ("c7_absorb", "c7_absorb_fp8"):
        return absorb_row(torch, mp, W, name.endswith("fp8"))
    if name in ("p64", "p256"):
        return probe_row(torch, mp, W, probe_case(W, W.c1_decode(), 1 if name == "p64" else 4))
    if name == "p64_fp8":
        return probe_row_fp8(torch, mp, W, fp8_probe_case(W))
    if name == "p64_fp8_cache":
        return probe_row_fp8_cache(torch, mp, W, fp8_cache_probe_case(W))
    if name == "copy":
        return copy_row(torch)
    raise SystemExit(f"unknown row {name}")


OTHER_ROWS = ("p64", "p256", "p64_fp8", "p64_fp8_cache", "c2_prefill", "c3_fp8", "c6_fp8_cache",
              "c6_fused_kv_fp8_cache", "c2_fused_kv", "c2_tp8_share", "c4_kv_matmul", "c5_latent_write", "c5_latent_write_fp8", "c7_absorb", "c7_absorb_fp8")
PROFILE_ROWS = ("c1_decode", "c1_product", "c1_gather") + OTHER_ROWS + ("copy",)


def time_row(torch, name, row, steps, warmup):
    """One entry of the JSON `rows` object."""
    if row.copies:
        ms = graph_time(torch, row.fn, row.copies, 20, warmup, row.check)
        entry = {"us_per_call": round(ms * 1e3, 3),
                 "timing": f"HIP graph of {row.copies} launches on {row.copies} weight copies, replayed 20 times"}
    else:
        t = Timed(torch, row.fn, steps, warmup)
        ms = t.median_launch_ms
        entry = {"ms": round(ms, 4), "launch_ms": t.summary()}
        if row.separate is not None:
            entry["separate_calls_ms"] = round(Timed(torch, row.separate, steps, warmup).median_launch_ms, 4)
    entry.update(row.info)
    s = ms * 1e-3
    if row.flops:
        entry["tflops"] = round(row.flops / s / 1e12, 2)
    entry["hbm_gbs_algorithmic"] = round(row.bytes / s / 1e9, 1)
    achieved = row.flops / s / 1e12 if row.bound == "mfma" else row.bytes / s / 1e9
    entry["roofline"] = roofline(row.bound, achieved, row.peak, "TFLOP/s" if row.bound == "mfma" else "GB/s",
                                 traffic_from_profile(row.kernel, name))
    if row.kernel == "gemm_fp8_ring":
        entry["fp8_mfma_frac"] = round(row.flops / s / 1e12 / PEAK_FP8_TFLOPS, 4)
    cnt = counters_from_profile(row.kernel, name)
    if cnt:
        entry["counters"] = cnt
    return entry


# ---------------------------------------------------------------------------
# measured ceilings
# ---------------------------------------------------------------------------
def measure_peaks(torch):
    """Ceilings of this GPU, measured in this run with the kernels of
    csrc/peaks/peaks.hip (see there)."""
    import ctypes
    from mla_paged_latent_page_amd import build as B
    if not os.path.exists(B.PEAKS_PATH):
        return None
    lib = ctypes.CDLL(B.PEAKS_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.peaks_mfma_bf16.argtypes = [vp, vp, i32, i32, vp]
    lib.peaks_read.argtypes = [vp, vp, i64, i32, vp]
    lib.peaks_write.argtypes = [vp, i64, i32, vp]
    lib.peaks_empty.argtypes = [vp]
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    src = torch.randn(32768, device="cuda").to(torch.bfloat16)
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    steps = 16384
    t = Timed(torch, lambda: lib.peaks_mfma_bf16(src.data_ptr(), sink.data_ptr(), cus, steps, st()), 5, 2)
    flop = 2.0 * 32 * 32 * 16 * 8 * 8 * steps * cus
    out["mfma_bf16_tflops"] = round(flop / (t.median_launch_ms * 1e-3) / 1e12, 1)
    big = 4 << 30
    buf = torch.empty(big // 4, dtype=torch.int32, device="cuda")
    words = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    grid = 4 * cus
    t = Timed(torch, lambda: lib.peaks_write(buf.data_ptr(), big, grid, st()), 5, 2)
    out["hbm_write_gbs"] = round(big / (t.median_launch_ms * 1e-3) / 1e9, 1)
    t = Timed(torch, lambda: lib.peaks_read(buf.data_ptr(), words.data_ptr(), big, grid, st()), 5, 2)
    out["hbm_read_gbs"] = round(big / (t.median_launch_ms * 1e-3) / 1e9, 1)
    del buf
    small = 16 << 20
    bufs = [torch.ones(small // 4, dtype=torch.int32, device="cuda") for _ in range(32)]
    ms = graph_time(torch, lambda i: lib.peaks_read(bufs[i].data_ptr(), words.data_ptr(), small, cus, st()), 32, 20, 2)
    out["read_16mib_us"] = round(ms * 1e3, 2)
    out["read_16mib_gbs"] = round(small / (ms * 1e-3) / 1e9, 1)
    ms = graph_time(torch, lambda i: lib.peaks_empty(st()), 32, 20, 2)
    out["empty_launch_us"] = round(ms * 1e3, 2)
    del bufs
    torch.cuda.empty_cache()
    out["note"] = ("mfma: 8 waves per CU of back-to-back 32x32x16 bf16 MFMAs on LDS-fed random data; "
                   "hbm_read/hbm_write: 4 GiB non-temporal streams; read_16mib: one 16 MiB read per launch "
                   "(HIP graph over 32 copies, launch included); empty_launch: a launch doing nothing, same replay")
    return out


def cold_product(torch, row, steps):
    """The product launch alone with a 512 MB scratch write (twice the
    last-level cache) before each launch: median over `steps` launches."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ms = []
    for i in range(steps):
        scratch.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        row.fn()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(ms))


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


# ---------------------------------------------------------------------------
# counter records
# ---------------------------------------------------------------------------
def _dispatches(path, kernel):
    """Counter values per dispatch of the kernels whose name holds `kernel`:
    {counter: [value per dispatch]}."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                out.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def _kernel_of(row_name):
    return {"c1_decode": "gemm_bf16_ring", "c1_product": "gemm_bf16_ring", "c1_gather": "gather_rows_kernel",
            "c2_prefill": "gemm_bf16_ring", "c2_fused_kv": "gemm_bf16_ring", "c2_tp8_share": "gemm_bf16_ring",
            "c3_fp8": "gemm_fp8_ring", "c6_fp8_cache": "gemm_fp8_ring", "c6_fused_kv_fp8_cache": "gemm_fp8_ring",
            "c4_kv_matmul": "kv_matmul_ring", "c5_latent_write": "latent_write_kernel",
            "c5_latent_write_fp8": "latent_write_kernel", "c7_absorb": "absorb_bf16", "c7_absorb_fp8": "absorb_fp8",
            "p64": "decompress_small_bf16", "p256": "decompress_small_bf16", "p64_fp8": "decompress_small_fp8_gq", "p64_fp8_cache": "decompress_small_fp8_gc",
            "copy": "__amd_rocclr_copyBuffer"}[row_name]


def write_traffic_record(row_name, fetch_csv, write_csv, commands, alg_bytes):
    kernel = _kernel_of(row_name)
    f = _dispatches(fetch_csv, kernel).get("FETCH_SIZE", [])
    w = _dispatches(write_csv, kernel).get("WRITE_SIZE", [])
    if not f or not w:
        raise SystemExit(f"no FETCH_SIZE / WRITE_SIZE dispatches of {kernel} in the CSVs")
    fk, wk = float(np.mean(f)), float(np.mean(w))
    prof = os.path.join(ROOT, "profiles")
    if row_name == "copy":
        rec = {"kernel": kernel, "workload": f"a {COPY_BYTES >> 30} GiB device-to-device copy (bench.py --profile copy)",
               "fetch_size_kib_per_dispatch": round(fk, 1), "write_size_kib_per_dispatch": round(wk, 1),
               "dispatches_averaged": [len(f), len(w)],
               "fetch_scale": round(COPY_BYTES / (fk * 1024), 4), "write_scale": round(COPY_BYTES / (wk * 1024), 4),
               "commands": commands}
        path = os.path.join(prof, "copy_probe_hbm_calibration.json")
    else:
        with open(os.path.join(prof, "copy_probe_hbm_calibration.json")) as cf:
            cal = json.load(cf)
        rd, wr = int(round(fk * 1024 * cal["fetch_scale"])), int(round(wk * 1024 * cal["write_scale"]))
        rec = {"kernel": kernel, "workload": row_name, "source_hash": source_hash(kernel),
               "fetch_size_kib_per_dispatch": round(fk, 1), "write_size_kib_per_dispatch": round(wk, 1),
               "dispatches_averaged": [len(f), len(w)],
               "scale": {"fetch": cal["fetch_scale"], "write": cal["write_scale"],
                         "from": "profiles/copy_probe_hbm_calibration.json (a 1 GiB device-to-device copy)"},
               "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
               "algorithmic_bytes_per_launch": int(alg_bytes), "commands": commands}
        path = os.path.join(prof, f"{kernel}_{row_name}_hbm_traffic.json")
    rec["setup"] = "MI355X, ROCm 7.2; cd /tmp && export TMPDIR=/tmp, then the commands from the repository root"
    with open(path, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps({"record": os.path.relpath(path, ROOT), **{k: rec[k] for k in rec if k.endswith("launch")}}))


def _durations_ns(path, kernel):
    """Duration of each dispatch of the kernel in a counter CSV (its start and
    end timestamps, ns)."""
    d = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                d[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return list(d.values())


def write_counter_record(row_name, csvs, commands):
    kernel = _kernel_of(row_name)
    vals = {}
    durs = []
    for p in csvs:
        for c, v in _dispatches(p, kernel).items():
            vals[c] = float(np.mean(v))
        durs += _durations_ns(p, kernel)
    rec = {"kernel": kernel, "workload": row_name, "source_hash": source_hash(kernel),
           "counters_mean_per_dispatch": {c: v for c, v in sorted(vals.items())}, "commands": commands,
           "setup": "MI355X, ROCm 7.2; cd /tmp && export TMPDIR=/tmp, then the commands from the repository root"}
    # GRBM_GUI_ACTIVE counts GPU-busy cycles on each of the 8 XCDs (summed);
    # the MFMA busy count is summed over every SIMD (4 per CU), the TA busy
    # count over the 256 TA instances (one per CU).
    gui = vals.get("GRBM_GUI_ACTIVE")
    if gui:
        cycles = gui / 8
        rec["cycles_per_xcd"] = round(cycles)
        simds = 4 * 256
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            rec["mfma_busy_frac"] = round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cycles, 4)
        if "TA_TA_BUSY_sum" in vals:
            rec["ta_busy_frac"] = round(vals["TA_TA_BUSY_sum"] / 256 / cycles, 4)
        if "SQ_BUSY_CU_CYCLES" in vals:
            rec["cu_busy_frac"] = round(vals["SQ_BUSY_CU_CYCLES"] / 256 / cycles, 4)
        # LDS: cycles it serves indexed accesses (over every CU), and the share
        # of those cycles stalled by bank conflicts
        if "SQ_LDS_IDX_ACTIVE" in vals:
            rec["lds_busy_frac"] = round(vals["SQ_LDS_IDX_ACTIVE"] / 256 / cycles, 4)
            if "SQ_LDS_BANK_CONFLICT" in vals and vals["SQ_LDS_IDX_ACTIVE"] > 0:
                rec["lds_bank_conflict_frac"] = round(vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"], 4)
        if durs:
            rec["dispatch_ns_mean"] = round(float(np.mean(durs)))
            # the busy-cycle count over the dispatch time: meaningful for long
            # dispatches only (counter set-up cycles swamp a few microseconds)
            if np.mean(durs) > 1e5:
                rec["clock_ghz"] = round(cycles / float(np.mean(durs)), 3)
    path = os.path.join(ROOT, "profiles", f"{kernel}_{row_name}_counters.json")
    with open(path, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps({"record": os.path.relpath(path, ROOT),
                      **{k: rec[k] for k in ("mfma_busy_frac", "ta_busy_frac", "lds_busy_frac", "lds_bank_conflict_frac",
                                             "clock_ghz", "cycles_per_xcd") if k in rec}}))


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
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured ceilings")
    ap.add_argument("--profile", metavar="ROW", choices=PROFILE_ROWS,
                    help="run only ROW's call, --warmup then --steps times, for rocprofv3")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="with --row: write ROW's HBM traffic record from two counter CSVs")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="with --row: write ROW's counter summary record")
    ap.add_argument("--row", choices=PROFILE_ROWS)
    ap.add_argument("--commands", nargs="*", default=[], help="the commands that made the CSVs (for the record)")
    args = ap.parse_args()
    Timed.warm_seconds = args.warm_seconds
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the path is measured on a single MI355X; "
              "multi-GPU sharding is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    if args.traffic_from or args.counters_from:
        if not args.row:
            raise SystemExit("--traffic-from / --counters-from need --row")
        if args.traffic_from:
            alg = 0
            if args.row != "copy":
                import torch
                import mla_paged_latent_page_amd as mp
                import workloads as W
                alg = _alg_bytes_host(args.row, W)
            write_traffic_record(args.row, args.traffic_from[0], args.traffic_from[1], args.commands, alg)
        if args.counters_from:
            write_counter_record(args.row, args.counters_from, args.commands)
        return

    import torch
    import mla_paged_latent_page_amd as mp
    import workloads as W

    torch.cuda.set_device(0)
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    if args.profile:
        # the same warm-up as a timed row (at least W calls and 0.2 s of GPU
        # work, so the clock has ramped up), then exactly K calls
        row = build_row(args.profile, torch, mp, W)
        n = max(1, row.copies)
        w0, i = time.perf_counter(), 0
        while i < args.warmup or time.perf_counter() - w0 < Timed.warm_seconds:
            row.fn(i % n)
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        for j in range(args.steps):
            row.fn((i + j) % n)
        torch.cuda.synchronize()
        print(f"[bench] profiled {args.profile}: {i} warm-up + {args.steps} calls of {row.kernel}",
              file=sys.stderr, flush=True)
        return

    # ---- main workload: bf16 decode-sized batch
    case = W.c1_decode()
    main_row = decompress_row(torch, mp, W, case)
    tm = Timed(torch, main_row.fn, args.steps, args.warmup)
    call_tf = main_row.flops / (tm.median_launch_ms * 1e-3) / 1e12
    print(f"[bench] c1_decode M={case.M}: {tm.median_launch_ms:.3f} ms/call (median), {call_tf:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    product, gather = product_row(torch, mp, W, case)
    tg = Timed(torch, gather.fn, args.steps, args.warmup)
    tp = Timed(torch, product.fn, args.steps, args.warmup)
    prod_tf = product.flops / (tp.avg_launch_ms * 1e-3) / 1e12
    cold_ms = cold_product(torch, product, max(5, args.steps // 2))
    print(f"[bench] gather {tg.median_launch_ms:.3f} ms ({gather.bytes / tg.median_launch_ms / 1e6:.0f} GB/s), "
          f"product {tp.avg_launch_ms:.3f} ms avg ({prod_tf:.1f} TFLOP/s), cold {cold_ms:.3f} ms",
          file=sys.stderr, flush=True)
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
        "hbm_gbs_algorithmic": round(main_row.bytes / (tm.median_launch_ms * 1e-3) / 1e9, 1),
        "roofline": roofline("mfma", prod_tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                             traffic_from_profile("gemm_bf16_ring", "c1_product")),
        "kernel": "gemm_bf16_ring<2,4> (the product step; 2*M*N*K flop per launch; achieved over the average "
                  "launch time)",
        "launch_ms": {"call": tm.summary(), "product": tp.summary(), "gather": tg.summary()},
        "cold": {"product_ms": round(cold_ms, 4),
                 "tflops": round(product.flops / (cold_ms * 1e-3) / 1e12, 2),
                 "note": "product launch alone after a 512 MB scratch write before each launch (median)"},
        "gather": {"kernel": "gather_rows_kernel", "bytes_per_launch": int(gather.bytes),
                   "roofline": roofline("hbm", gather.bytes / (tg.median_launch_ms * 1e-3) / 1e9, PEAK_HBM_GBS,
                                        "GB/s", traffic_from_profile("gather_rows_kernel", "c1_gather"))},
        "published_baseline": "none: the pages publish no performance numbers",
    }
    cnt = counters_from_profile("gemm_bf16_ring", "c1_product")
    if cnt:
        result["counters"] = cnt
    del main_row, product, gather
    torch.cuda.empty_cache()

    if not args.no_peaks:
        peaks = measure_peaks(torch)
        if peaks:
            result["peaks"] = peaks
            result["roofline_vs_measured_mfma"] = round(prod_tf / peaks["mfma_bf16_tflops"], 4)
            print(f"[bench] peaks: {peaks}", file=sys.stderr, flush=True)

    # ---- the other rows of the path
    if args.rows == "all":
        rows = {}
        steps = max(3, args.steps // 2)
        for name in OTHER_ROWS:
            row = build_row(name, torch, mp, W)
            rows[name] = time_row(torch, name, row, steps, args.warmup)
            r = rows[name]
            t = f"{r['us_per_call']:.2f} us/call (graph)" if "us_per_call" in r else f"{r['ms']:.4f} ms"
            print(f"[bench] {name}: {t}, {r['roofline']['achieved']:.0f} {r['roofline']['unit']} "
                  f"({r['roofline']['frac']:.3f} of peak)", file=sys.stderr, flush=True)
            del row
            torch.cuda.empty_cache()
        result["rows"] = rows

    if args.cpu_seconds > 0:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _alg_bytes_host(row_name, W):
    """Algorithmic HBM bytes of one launch of a row's dominant kernel alone,
    from the workload's shapes (no GPU): for the products, the activation
    columns they read (K of each row), their outputs and the weight once."""
    def bf16_product(c, n):
        return c.M * (c.K * 2 + n * 2) + n * c.K * 2

    def fp8_product(c, n):
        return c.M * (c.K + (c.K // 128) * 4 + n * 2) + n * c.K + (n // 128) * (c.K // 128) * 4
    if row_name == "c1_product":
        return bf16_product(W.c1_decode(), 16384)
    if row_name == "c1_gather":
        c = W.c1_decode()
        return c.M * c.D_c * 2 * 2
    if row_name == "c2_prefill":
        return bf16_product(W.c2_prefill(), 16384)
    if row_name == "c2_fused_kv":
        return bf16_product(W.c2_prefill(), 2 * 16384)
    if row_name == "c2_tp8_share":
        return bf16_product(W.c2_prefill(), 2048)
    if row_name == "c3_fp8":
        return fp8_product(W.c3_fp8(), 16384)
    if row_name in ("c6_fp8_cache", "c6_fused_kv_fp8_cache"):
        return fp8_product(W.c6_fp8_cache(), 16384 if row_name == "c6_fp8_cache" else 2 * 16384)
    if row_name == "c4_kv_matmul":
        k = W.c4_kv_matmul()
        return k.T * (k.hidden_dim * 2 + k.N * 2) + k.weight.nbytes
    if row_name in ("c5_latent_write", "c5_latent_write_fp8"):
        fp8 = row_name.endswith("fp8")
        lc = W.c5_latent_write_fp8() if fp8 else W.c5_latent_write()
        D = lc.x.shape[1]
        if fp8:
            return lc.T * (D * 2 + (D - lc.K) * 4 + D + -(-D // 128) * 4) + lc.K * 4
        return lc.T * (D * 2 * 2 + (D - lc.K) * 4) + lc.K * 4
    if row_name in ("c7_absorb", "c7_absorb_fp8"):
        fp8 = row_name.endswith("fp8")
        c = W.c7_absorb_fp8() if fp8 else W.c7_absorb()
        T, H, L, Dq = c.T, c.H, c.kv_latent_dim, c.q.shape[2]
        wb = H * L * c.d_nope + c.w_scale.nbytes if fp8 else H * L * c.d_nope * 2
        return wb + T * H * Dq * 2 + T * H * c.out_dim * 2
    if row_name in ("p64", "p256"):
        return decompress_costs(probe_case(W, W.c1_decode(), 1 if row_name == "p64" else 4))[1]
    if row_name == "p64_fp8":
        return fp8_product(fp8_probe_case(W), 16384)
    if row_name == "p64_fp8_cache":
        return fp8_cache_call_bytes(fp8_cache_probe_case(W))
    raise SystemExit(f"no algorithmic bytes for {row_name}")


if __name__ == "__main__":
    main()
