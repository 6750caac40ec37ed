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

import oracle
import workloads as W
from gpu_util import BF16_TOL, POISON_OUT, check_close, rows_as_f64, run_decompress, run_decompress_fp8_cache, \
    sample_rows, say, to_bits

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
    got = res["out"][:M].double().cpu().numpy() if rows is None else rows_as_f64(res["out"], rows)
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
