"""GPU parity of mla_decompress_k_paged_fp8_cache (an e4m3 paged cache with one
fp32 scale per 128 columns of each token row) against the CPU oracle.

The gathered codes and scales are bit copies: they must match the oracle bit
for bit, and rows past M must keep their poison.  k_buffer is the block-scaled
product of exactly those codes and scales with the e4m3 weight: no quantisation
happens, so the only differences from the oracle's binary64 sum are fp32
accumulation and the bf16 rounding of the output; it must be within
1e-2 * max|ref| (the bf16 product bound).
"""
import dataclasses

import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import BF16_TOL, POISON_OUT, check_close, check_guards, guarded_empty, rows_as_f64, run_decompress, \
    run_decompress_fp8_cache, sample_rows, say, to_bits

pytestmark = pytest.mark.gpu


def _fp8_case(seed, **kw):
    return W.small_decompress(seed, dtype="e4m3", fp8=True, **kw)


def _check(case, rows=None, extra=5):
    res = run_decompress_fp8_cache(case, extra_rows=extra)
    M = case.M
    codes, scales, ref = oracle.decompress_k_fp8_cache(case, rows)
    lat = to_bits(res["lat"])
    assert np.array_equal(lat[:M], codes), "gathered codes differ"
    assert np.all(lat[M:] == 0x7F)
    sc = res["scales"].cpu().numpy()
    assert np.array_equal(sc[:M].view(np.uint32), scales.view(np.uint32)), "gathered scales differ"
    assert np.all(np.isnan(sc[M:]))
    got = res["out"][:M].double().cpu().numpy() if rows is None else rows_as_f64(res["out"], rows, M)
    check_close(got, ref, BF16_TOL, f"{case.name} k_buffer (fp8 cache)")
    assert np.all(to_bits(res["out"])[M:] == POISON_OUT)
    return res


@pytest.mark.parametrize("seed,ps,N", [(0, 16, 512), (1, 128, 1024), (2, 5, 256), (3, 1, 128)])
def test_small_full_compare(seed, ps, N):
    _check(_fp8_case(seed, batch=5, max_len=400, page_size=ps, K=512, rope=64, N=N))


def test_k256_narrow_rows_and_empty_requests():
    case = W.decompress_case("fp8c_k256", seed=21, cache_lengths=[100, 9, 250, 40], cache_offsets=[1, 9, 0, 40],
                             page_size=16, kv_lora_rank=256, rope_dim=64, N=384, dtype="e4m3", fp8=True)
    _check(case)


def test_many_tiles_and_ragged_tail():
    # M = 1000 + ... spans four 256-row tiles with a ragged last one; N spans several 128-wide tiles
    case = W.decompress_case("fp8c_tiles", seed=22, cache_lengths=[700, 333, 5], cache_offsets=[0, 30, 2],
                             page_size=64, kv_lora_rank=512, rope_dim=64, N=640, dtype="e4m3", fp8=True)
    _check(case)


def test_zero_rows_is_a_no_op():
    case = W.decompress_case("fp8c_empty", seed=23, cache_lengths=[10, 4], cache_offsets=[10, 4], page_size=8,
                             kv_lora_rank=128, rope_dim=0, N=128, dtype="e4m3", fp8=True)
    assert case.M == 0
    res = run_decompress_fp8_cache(case, extra_rows=3)
    assert np.all(to_bits(res["lat"]) == 0x7F) and np.all(to_bits(res["out"]) == POISON_OUT)


def _quantised_copy(case_bf16):
    c = case_bf16.cache
    rows = c.pool.reshape(-1, c.num_heads * c.head_dim)
    q, s = oracle.quantize_e4m3_rows(rows, rows.shape[1], 128)
    cache = dataclasses.replace(c, pool=q.reshape(c.pool.shape), dtype="e4m3",
                                scales=s.reshape(c.pool.shape[:4] + (s.shape[1],)), scale_gran=128)
    return dataclasses.replace(case_bf16, cache=cache)


def test_quantised_cache_gives_the_fp8_form_bit_for_bit():
    """A cache holding exactly the codes and scales the fp8 form computes on
    the fly from a bf16 cache gives the same k_buffer bits: both calls run the
    same product on the same operands."""
    bf = W.small_decompress(24, batch=4, max_len=300, page_size=16, K=512, rope=64, N=512, fp8=True)
    f8 = _quantised_copy(bf)
    a = run_decompress(bf)
    b = _check(f8)
    assert torch.equal(a["out"].float(), b["out"][:bf.M].float())


@pytest.mark.slow
def test_c6_full_size_sampled():
    """The 64K-row prefill shapes on an e4m3 cache, in the launch the bench
    times: every code and scale compared, k_buffer on sampled rows."""
    case = W.c6_fp8_cache()
    rows = sample_rows(case)
    say(f"[gpu] c6: {len(rows)} sampled rows")
    _check(case, rows=rows, extra=0)


def _run_kv(case, case_v, extra=3):
    dc, t = W.device_decompress(case)
    M, D = case.M, case.D_c
    nblk = case.cache.scale_blocks
    lat = guarded_empty((M + extra, D), torch.uint8)
    lat.fill_(0x7F)
    lsc = guarded_empty((M + extra, nblk), torch.float32)
    lsc.fill_(float("nan"))
    kout = guarded_empty((M + extra, case.N), torch.bfloat16)
    vout = guarded_empty((M + extra, case_v.N), torch.bfloat16)
    kout.view(torch.int16).fill_(POISON_OUT)
    vout.view(torch.int16).fill_(POISON_OUT)
    wv = torch.from_numpy(case_v.weight_q).cuda()
    sv = torch.from_numpy(case_v.weight_scale).cuda()
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    say(f"[gpu] {case.name} fp8 cache, K and V: M={M} N_k={case.N} N_v={case_v.N} K={case.K}")
    mp.mla_decompress_kv_paged_fp8_cache(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                         t["weight_scale"], wv, sv, cache, case.layer_idx, lat, lsc, kout, vout)
    check_guards(case.name + " fp8 cache K and V")
    return lat, lsc, kout, vout


@pytest.mark.parametrize("seed,N,Nv", [(0, 512, 256), (1, 1024, 1024), (2, 256, 384)])
def test_k_and_v_from_the_fp8_cache(seed, N, Nv):
    case = _fp8_case(seed, N=N)
    case_v = W.with_second_projection(case, seed=seed + 100, N=Nv)
    lat, lsc, kout, vout = _run_kv(case, case_v)
    M = case.M
    codes, scales, k, v = oracle.decompress_kv_fp8_cache(case, case_v)
    assert np.array_equal(to_bits(lat)[:M], codes), "gathered codes differ"
    assert np.array_equal(lsc.cpu().numpy()[:M].view(np.uint32), scales.view(np.uint32)), "gathered scales differ"
    check_close(kout[:M].double().cpu().numpy(), k, BF16_TOL, f"{case.name} k_buffer (fp8 cache, fused)")
    check_close(vout[:M].double().cpu().numpy(), v, BF16_TOL, f"{case.name} v_buffer (fp8 cache, fused)")
    assert np.all(to_bits(kout)[M:] == POISON_OUT) and np.all(to_bits(vout)[M:] == POISON_OUT)
    # the K half equals the single-projection call bit for bit
    single = run_decompress_fp8_cache(case)
    assert torch.equal(single["out"][:M].view(torch.int16), kout[:M].view(torch.int16))


def test_k_and_v_from_the_fp8_cache_at_full_size_sampled():
    case = W.c6_fp8_cache()
    case_v = W.with_second_projection(case, seed=606, N=case.N)
    lat, lsc, kout, vout = _run_kv(case, case_v, extra=0)
    rows = sample_rows(case)
    codes, scales, k, v = oracle.decompress_kv_fp8_cache(case, case_v, rows)
    M = case.M
    assert np.array_equal(to_bits(lat)[:M], codes), "gathered codes differ"
    check_close(rows_as_f64(kout, rows, M), k, BF16_TOL, "c6 k_buffer (fused, sampled rows)")
    check_close(rows_as_f64(vout, rows, M), v, BF16_TOL, "c6 v_buffer (fused, sampled rows)")


@pytest.mark.parametrize("lens,offs,N", [([1], [0], 128), ([64, 64], [0, 32], 512), ([150, 42], [0, 0], 1024),
                                         ([193], [0], 256)])
def test_few_rows_fp8_cache(lens, offs, N):
    """Decode-sized calls on the e4m3 cache (1, 96 and 192 rows: the few-rows
    product; 193: the large one)."""
    _check(W.decompress_case("fp8c_few", seed=42, cache_lengths=lens, cache_offsets=offs, page_size=16,
                             kv_lora_rank=512, rope_dim=64, N=N, dtype="e4m3", fp8=True))


@pytest.mark.parametrize("lens,offs,rows,ps,N,rope", [
    ([1], [0], None, 16, 128, 64),
    ([32], [0], None, 16, 256, 64),
    ([21, 15], [3, 0], None, 1, 512, 64),
    ([5] * 70, [4] * 70, [1] * 64 + [0] * 6, 2, 384, 64),
    ([20000, 30], [19980, 0], None, 1, 256, 64),
    ([40, 9], [0, 2], None, 16, 256, 0),
    ([40, 9], [0, 2], None, 16, 256, 128),
    ([65], [0], None, 16, 256, 64),
])
def test_one_launch_fp8_cache_decode(lens, offs, rows, ps, N, rope):
    """Up to 64 rows of the e4m3 cache: codes and scales gathered into the
    product's LDS layout and multiplied in one launch (1, 32, 33 and 64 rows,
    70 requests, a 40,000-entry page table, 512- and 640-column rows); 65 rows
    take the two-launch form."""
    _check(W.decompress_case("fp8c_one_launch", seed=44, cache_lengths=lens, cache_offsets=offs, rows=rows,
                             page_size=ps, kv_lora_rank=512, rope_dim=rope, N=N, dtype="e4m3", fp8=True))


@pytest.mark.parametrize("max_len", [300, 60, 14])
def test_zero_activation_scales(max_len):
    """Scale blocks of 0 in the cache (a writer may store s = 0 for an all-zero
    block): a zero block after a non-zero one, a zero first block, and a row
    whose every block is zero.  The oracle's value for such a block is exactly
    0 * (its code sum); the product must stay finite and within the bound, and
    the all-zero row must come out as zeros.  Long requests take the large
    product, short ones (at most 192 rows) the few-rows one, at most 64 rows
    the one-launch form."""
    case = _fp8_case(31, batch=4, max_len=max_len, page_size=16, K=512, rope=64, N=512)
    assert (case.M > 192) == (max_len == 300) and (case.M <= 64) == (max_len == 14)
    c = case.cache
    rng = np.random.default_rng(31)
    sc = c.scales.copy()
    layer = sc[:, case.layer_idx]
    kb = case.K // 128
    kill = rng.random(layer[..., :kb].shape) < 0.3
    layer[..., :kb][kill] = 0.0
    # the first row of request 0 loses every block
    b0_pos = int(case.cache_offsets[0])
    pg = int(c.page_table[0, b0_pos // c.page_size])
    layer[pg, 0, b0_pos % c.page_size, :kb] = 0.0
    case = dataclasses.replace(case, cache=dataclasses.replace(c, scales=sc))
    res = _check(case)
    out0 = res["out"][0].float().cpu().numpy()
    assert np.all(out0 == 0.0), "a row whose every scale block is zero must give zeros"
