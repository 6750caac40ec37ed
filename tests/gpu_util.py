"""Helpers for the GPU parity tests: run an operation through the binding on
seeded inputs, bring results back as raw bits / float64, pick sampled rows."""
import sys

import numpy as np
import torch

import mla_paged_latent_page_amd as mp
import workloads as W

BF16_TOL = 1e-2   # max|gpu - ref| <= BF16_TOL * max|ref|   (bf16 outputs)
FP8_TOL = 3e-2    # same form, fp8 block-scaled outputs
POISON_OUT = 0x7FC3  # NaN bf16 pattern pre-filled into outputs to catch stray writes


GUARD_BYTES = 4096   # canary bytes before and after every output buffer
GUARD_BYTE = 0xA5


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_guarded = []


def guarded_empty(shape, dtype):
    """A contiguous device tensor with GUARD_BYTES of canary bytes right before
    and after it in the same allocation (its start stays 256-byte aligned).
    check_guards() asserts that every canary of every such tensor made since
    the last check is intact: a write before the start or past the end of an
    output shows even where it lands outside the rows a test compares."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((GUARD_BYTES + nbytes + GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device="cuda")
    t = raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)
    _guarded.append(raw)
    return t


def check_guards(what=""):
    torch.cuda.synchronize()
    raws = list(_guarded)
    _guarded.clear()
    for raw in raws:
        g = torch.cat([raw[:GUARD_BYTES], raw[-GUARD_BYTES:]])
        assert bool((g == GUARD_BYTE).all()), f"{what}: a canary byte next to an output changed"


def to_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    raise ValueError(t.dtype)


def run_decompress(case, extra_rows=0, fp8=None):
    """Run the HIP op on a case.  Outputs are over-allocated by extra_rows rows
    pre-filled with a poison pattern.  Returns a dict of device tensors."""
    fp8 = case.weight_dtype == "e4m3" if fp8 is None else fp8
    dc, t = W.device_decompress(case)
    M, D, N = case.M, case.D_c, case.N
    dt = torch.float32 if case.cache.dtype == "f32" else torch.bfloat16
    lat = guarded_empty((M + extra_rows, D), dt)
    out = guarded_empty((M + extra_rows, N), dt)
    if dt == torch.bfloat16:
        lat.view(torch.int16).fill_(POISON_OUT)
        out.view(torch.int16).fill_(POISON_OUT)
    else:
        lat.fill_(float("nan"))
        out.fill_(float("nan"))
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    say(f"[gpu] {case.name}: M={M} N={N} K={case.K} D={D} fp8={fp8}")
    res = {"lat": lat, "out": out, "pool": dc.pool}
    if fp8:
        ws_bytes = mp.mla_decompress_k_paged_fp8_workspace_size(M, case.K)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        mp.mla_decompress_k_paged_fp8(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                      t["weight_scale"], cache, case.layer_idx, lat, out, ws)
        res["ws"] = ws
    else:
        mp.mla_decompress_k_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], cache,
                                  case.layer_idx, lat, out)
    check_guards(case.name)
    return res


def run_decompress_kv(case, case_v, extra_rows=0):
    """Run the fused K and V op (mla_decompress_kv_paged[_fp8]) on a case and
    its second projection; outputs over-allocated by extra_rows poisoned rows."""
    fp8 = case.weight_dtype == "e4m3"
    dc, t = W.device_decompress(case)
    _, tv = W.device_decompress(case_v)
    M, D = case.M, case.D_c
    dt = torch.float32 if case.cache.dtype == "f32" else torch.bfloat16
    lat = guarded_empty((M + extra_rows, D), dt)
    kout = guarded_empty((M + extra_rows, case.N), dt)
    vout = guarded_empty((M + extra_rows, case_v.N), dt)
    for x in (lat, kout, vout):
        if dt == torch.bfloat16:
            x.view(torch.int16).fill_(POISON_OUT)
        else:
            x.fill_(float("nan"))
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    say(f"[gpu] {case.name} fused K+V: M={M} N_k={case.N} N_v={case_v.N} K={case.K} fp8={fp8}")
    res = {"lat": lat, "k": kout, "v": vout, "pool": dc.pool}
    if fp8:
        ws_bytes = mp.mla_decompress_k_paged_fp8_workspace_size(M, case.K)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        mp.mla_decompress_kv_paged_fp8(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                       t["weight_scale"], tv["weight_q"], tv["weight_scale"], cache,
                                       case.layer_idx, lat, kout, vout, ws)
        res["ws"] = ws
    else:
        mp.mla_decompress_kv_paged(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight"], tv["weight"],
                                   cache, case.layer_idx, lat, kout, vout)
    check_guards(case.name + " fused K+V")
    return res


def workspace_views(ws, M, K):
    """(codes uint8 [M, K], scales float32 [M, K/128]) inside an fp8 workspace."""
    a = ws.cpu().numpy()
    off = (M * K + 255) // 256 * 256
    q = a[:M * K].reshape(M, K)
    s = a[off:off + M * (K // 128) * 4].view(np.float32).reshape(M, K // 128)
    return q, s


def rows_as_f64(t, rows, M):
    """The sampled rows as binary64, after a scan on the GPU that every one of
    the first M rows was written (no poison left, nothing non-finite): a tile
    order that skipped or misplaced a tile shows even where no row was sampled."""
    assert bool(torch.isfinite(t[:M]).all()), "an output row was not written (poison or non-finite values)"
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.device)
    return t.index_select(0, idx).double().cpu().numpy()


def sample_rows(case, n_random=256, seed=0):
    """Every request's first and last row, rows at page boundaries (up to 256),
    and n_random uniform rows."""
    bro = case.buffer_row_offsets.astype(np.int64)
    co = case.cache_offsets.astype(np.int64)
    ps = case.cache.page_size
    rows = set()
    boundary = []
    for b in range(case.batch):
        lo, hi = bro[b], bro[b + 1]
        if hi > lo:
            rows.update([lo, hi - 1])
            first = (-co[b]) % ps
            boundary.extend(range(lo + first, hi, ps))
    rng = np.random.default_rng(seed)
    if boundary:
        rows.update(rng.choice(boundary, size=min(256, len(boundary)), replace=False).tolist())
    if case.M:
        rows.update(rng.integers(0, case.M, size=min(n_random, case.M)).tolist())
    return np.array(sorted(rows), np.int64)


def check_close(got, ref, tol, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    say(f"[gpu] {what}: max|err|={err:.3e} max|ref|={scale:.3e} ratio={err / max(scale, 1e-30):.2e} (tol {tol})")
    assert err <= tol * scale, f"{what}: max|err| {err} > {tol} * {scale}"
    return err, scale


def run_decompress_fp8_cache(case, extra_rows=0):
    """Run mla_decompress_k_paged_fp8_cache on a case with an e4m3 cache.
    Outputs are over-allocated by extra_rows rows of poison (codes 0x7F,
    scales NaN, k_buffer POISON_OUT)."""
    dc, t = W.device_decompress(case)
    M, D, N = case.M, case.D_c, case.N
    nblk = case.cache.scale_blocks
    lat = guarded_empty((M + extra_rows, D), torch.uint8)
    lat.fill_(0x7F)
    lsc = guarded_empty((M + extra_rows, nblk), torch.float32)
    lsc.fill_(float("nan"))
    out = guarded_empty((M + extra_rows, N), torch.bfloat16)
    out.view(torch.int16).fill_(POISON_OUT)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    say(f"[gpu] {case.name} fp8 cache: M={M} N={N} K={case.K} D={D} nblk={nblk}")
    mp.mla_decompress_k_paged_fp8_cache(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                        t["weight_scale"], cache, case.layer_idx, lat, lsc, out)
    check_guards(case.name + " fp8 cache")
    return {"lat": lat, "scales": lsc, "out": out}
