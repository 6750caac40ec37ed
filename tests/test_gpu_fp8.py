"""GPU parity of mla_decompress_k_paged_fp8 against the CPU oracle.

The activation codes and scales the kernel leaves in its workspace are an
integer decision taken in binary32 on both sides (amax, 448/amax, x*inv, e4m3
round-to-nearest-even), so they must match the oracle bit for bit; gathered
rows bit for bit; k_buffer within 3e-2 * max|ref| of the oracle's block-scaled
product.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from caselib import elem_f64
from gpu_util import FP8_TOL, POISON_OUT, check_close, rows_as_f64, run_decompress, sample_rows, say, to_bits, \
    workspace_views

pytestmark = pytest.mark.gpu


def _same_codes(got, ref):
    # +0/-0 codes (0x00/0x80) are the same value; everything else must match exactly
    g = np.where(got == 0x80, 0, got)
    r = np.where(ref == 0x80, 0, ref)
    return np.array_equal(g, r)


def _check(case, rows=None):
    res = run_decompress(case, extra_rows=5)
    M, K = case.M, case.K
    ref_lat = oracle.gather(case)
    lat_bits = to_bits(res["lat"])
    assert np.array_equal(lat_bits[:M], ref_lat)
    assert np.all(lat_bits[M:] == POISON_OUT)
    q_ref, s_ref = oracle.quantize_e4m3_rows(ref_lat, K, 128)
    q_got, s_got = workspace_views(res["ws"], M, K)
    assert np.array_equal(s_got.view(np.uint32), s_ref.view(np.uint32)), "activation scales differ"
    assert _same_codes(q_got, q_ref), "activation codes differ"
    ref = oracle.fp8_matmul_nt(q_ref, s_ref, case.weight_q, case.weight_scale, 128, 128, rows)
    got = res["out"][:M].double().cpu().numpy() if rows is None else rows_as_f64(res["out"], rows, M)
    check_close(got, ref, FP8_TOL, f"{case.name} k_buffer fp8")
    assert np.all(to_bits(res["out"])[M:] == POISON_OUT)
    return res, ref_lat


@pytest.mark.parametrize("seed,ps,N", [(0, 16, 512), (1, 128, 1024), (2, 5, 256)])
def test_small_fp8_full_compare(seed, ps, N):
    case = W.small_decompress(seed, batch=5, max_len=400, page_size=ps, K=512, rope=64, N=N, fp8=True)
    _check(case)


@pytest.mark.parametrize("lens,offs,N", [([1], [0], 256), ([31], [0], 512), ([40, 24], [5, 0], 1024), ([97], [3], 256),
                                         ([100, 60, 30], [0, 10, 2], 512), ([192], [0], 256), ([193], [0], 256)])
def test_few_rows_fp8(lens, offs, N):
    """Decode-sized calls: up to 192 rows go to the few-rows product (1, 31,
    59, 94, 178 and 192 rows); 193 is the first count past it."""
    case = W.decompress_case("fp8_few", seed=41, cache_lengths=lens, cache_offsets=offs, page_size=16,
                             kv_lora_rank=512, rope_dim=64, N=N, fp8=True)
    _check(case)


ONE_LAUNCH_CASES = [
    ([1], [0], None, 16, 128, 64),             # one row, two weight tiles
    ([32], [0], None, 16, 256, 64),            # 32 rows (one row block); every block writes 8 rows' copies
    ([21, 15], [3, 0], None, 1, 512, 64),      # 33 rows (two row blocks), one token per page
    ([5] * 70, [4] * 70, [1] * 64 + [0] * 6, 2, 384, 64),   # 70 requests (two rounds of offsets), 64 rows
    ([20000, 30], [19980, 0], None, 1, 256, 64),            # a 40,000-entry page table (looked up in memory)
    ([40, 9], [0, 2], None, 16, 256, 0),       # rows of exactly the 512 latent columns
    ([40, 9], [0, 2], None, 16, 256, 128),     # 640-column rows
    ([65], [0], None, 16, 256, 64),            # 65 rows: past the one-launch form
]


@pytest.mark.parametrize("lens,offs,rows,ps,N,rope", ONE_LAUNCH_CASES)
def test_one_launch_fp8_decode(lens, offs, rows, ps, N, rope):
    """Up to 64 rows from a bf16 cache are gathered, quantised and multiplied in
    one launch: rows, workspace codes and scales must match the oracle as for
    the two-launch form."""
    case = W.decompress_case("fp8_one_launch", seed=43, cache_lengths=lens, cache_offsets=offs, rows=rows,
                             page_size=ps, kv_lora_rank=512, rope_dim=rope, N=N, fp8=True)
    assert case.M == (sum(rows) if rows else sum(l - o for l, o in zip(lens, offs)))
    # an all-zero latent block (scale 1, zero codes) in the first row
    c = case.cache
    pos = int(case.cache_offsets[0])
    pg = int(c.page_table[0, pos // c.page_size])
    c.pool[pg, case.layer_idx, 0, pos % c.page_size, 0, 256:384] = 0
    _check(case)


def test_fp8_decode_probe_full_width():
    """The newest 16 tokens of each of C3's 4 requests (64 rows) against the
    whole 16384-row e4m3 weight."""
    base = W.c3_fp8()
    lens = base.cache.cache_lengths.astype(np.int64)
    bro = np.zeros(len(lens) + 1, np.uint32)
    bro[1:] = np.cumsum(np.full(len(lens), 16))
    case = dataclasses.replace(base, name="fp8_probe64", buffer_row_offsets=bro,
                               cache_offsets=(lens - 16).astype(np.uint32))
    assert case.M == 64
    _check(case)


def test_fp8_k256_and_zero_rows():
    case = W.decompress_case("fp8_k256", seed=11, cache_lengths=[100, 9, 250], cache_offsets=[1, 9, 0],
                             page_size=16, kv_lora_rank=256, rope_dim=64, N=384, fp8=True)
    # an all-zero latent block must give scale 1 and zero codes
    c = case.cache
    pg = c.page_table[2, 0]
    c.pool[pg, case.layer_idx, 0, 3, 0, 128:256] = 0
    _check(case)


def test_fp8_exactly_representable_blocks_match_unquantised_product():
    """Latent blocks built from e4m3 values times 2^e with the block max at 448*2^e
    quantise losslessly, so the fp8 result equals the plain product of the latent
    with the dequantised weight (to bf16 output rounding)."""
    rng = np.random.default_rng(12)
    case = W.small_decompress(12, batch=3, max_len=120, page_size=16, K=256, rope=0, N=256, fp8=True)
    c = case.cache
    used = c.page_table[c.page_table != W.PAGE_NONE].astype(np.int64)
    codes = rng.integers(0, 0x7E, size=(len(used), c.page_size, 256)).astype(np.uint8)
    vals = elem_f64(codes, "e4m3") * np.where(rng.integers(0, 2, size=codes.shape) == 1, 1.0, -1.0)
    vals[..., 0] = 448.0
    vals[..., 128] = -448.0
    vals[..., :128] *= 2.0 ** -7
    vals[..., 128:] *= 2.0 ** -3
    c.pool[used, case.layer_idx, 0, :, 0, :] = W.to_bf16_bits(vals.astype(np.float32))
    res, ref_lat = _check(case)
    w_deq = elem_f64(case.weight_q, "e4m3") * np.repeat(np.repeat(case.weight_scale.astype(np.float64), 128, 0), 128, 1)
    plain = elem_f64(ref_lat, "bf16")[:, :256] @ w_deq.T
    got = res["out"][:case.M].double().cpu().numpy()
    check_close(got, plain, 2.0 ** -7, "lossless fp8 vs plain product")


@pytest.mark.slow
def test_c3_fp8_full_size_sampled():
    case = W.c3_fp8()
    rows = sample_rows(case)
    say(f"[gpu] c3: {len(rows)} sampled rows")
    _check(case, rows)


def test_fp8_zero_negative_and_far_apart_scales():
    """Weight-scale blocks that are zero, negative or 10^12 apart, and latent
    blocks whose magnitudes differ by 2^40 within a row: each scale block must
    enter the sum with its own factor, and a zero block must add nothing."""
    case = W.small_decompress(13, batch=4, max_len=300, page_size=16, K=512, rope=64, N=512, fp8=True)
    ws = case.weight_scale.astype(np.float64)
    ws[0, 1] = 0.0
    ws[1, :] = 0.0
    ws[2, 0] = -ws[2, 0]
    ws[3, 0] *= 1e6
    ws[3, 3] *= 1e-6
    case.weight_scale = ws.astype(np.float32)
    c = case.cache
    used = c.page_table[c.page_table != W.PAGE_NONE].astype(np.int64)
    blk = elem_f64(c.pool[used, case.layer_idx, 0, :, 0, :512], "bf16")
    blk[..., 128:256] *= 2.0 ** 20
    blk[..., 384:512] *= 2.0 ** -20
    c.pool[used, case.layer_idx, 0, :, 0, :512] = W.to_bf16_bits(blk.astype(np.float32))
    res, _ = _check(case)
    got = res["out"][:case.M].double().cpu().numpy()
    assert np.all(got[:, 128:256] == 0.0), "a weight block with zero scales must give exact zeros"


@pytest.mark.parametrize("K,N,batch,max_len", [(512, 8192, 8, 700), (128, 16384, 6, 500), (384, 8192, 10, 700),
                                               (1024, 16384, 6, 500)])
def test_fp8_several_tiles_per_block(K, N, batch, max_len):
    """More output tiles than compute units, so every block carries one tile's
    results into the next tile's stages; K of 1, 3, 4 and 8 scale blocks covers
    every way a tile's rows are spread over its stages."""
    case = W.small_decompress(20 + K // 128, batch=batch, max_len=max_len, page_size=16, K=K, rope=64, N=N, fp8=True)
    tiles = -(-case.M // 256) * (N // 128)
    say(f"[gpu] fp8 K={K} M={case.M} N={N}: {tiles} tiles")
    assert tiles > 256
    _check(case)
