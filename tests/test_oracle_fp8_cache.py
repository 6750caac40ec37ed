"""Pins for the oracle's fp8 paged cache path (page
"generic_flare_mla_decompress_k_cache_ragged_paged", the collection's
scale_dtype_ and quantization_granularity_; page "mla_prefill_decode_graph_fp8",
Parameters m/n/k_scale_granularity and Args w_k, w_k_scale).

What pins it:
  * a tagged e4m3 cache, whose every scale is the exact float naming its page,
    layer, kv half, slot and block, and whose codes are a known function of
    column, slot and page: the gathered rows and scales name exactly the pages
    and slots the page table gives for each request's positions;
  * a cache made by quantising a bf16 cache's rows with the (separately pinned)
    1x128 quantiser gives the same k_buffer as the bf16 cache's fp8 form, bit
    for bit: the activation codes and scales of the first K columns are the same;
  * the gathered rows, decoded and scaled, are within the e4m3 rounding bound of
    the bf16 values they were made from.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W


def _positions(case):
    bro = case.buffer_row_offsets.astype(np.int64)
    co = case.cache_offsets.astype(np.int64)
    b_of = np.repeat(np.arange(case.batch), np.diff(bro))
    pos = np.concatenate([co[b] + np.arange(bro[b + 1] - bro[b]) for b in range(case.batch)])
    return b_of, pos


def _tagged_case(page_size):
    c = W.small_decompress(11, batch=4, max_len=90, page_size=page_size, N=128, dtype="e4m3", fp8=True)
    rng = np.random.default_rng(0)
    cache = W.make_paged_cache(rng, cache_lengths=c.cache.cache_lengths, page_size=page_size, num_heads=1,
                               head_dim=c.D_c, dtype="e4m3", fill="tag")
    return dataclasses.replace(c, cache=cache)


@pytest.mark.parametrize("ps", [1, 7, 16])
def test_tagged_gather_names_the_right_slots(ps):
    case = _tagged_case(ps)
    codes, scales, _ = oracle.decompress_k_fp8_cache(case)
    b_of, pos = _positions(case)
    pages = case.cache.page_table[b_of, pos // ps].astype(np.int64)
    slots = pos % ps
    tag = scales.astype(np.int64)
    assert np.array_equal(scales, tag.astype(np.float32))
    assert np.array_equal(tag // 65536, np.broadcast_to(pages[:, None], tag.shape))
    assert np.array_equal((tag // 32768) % 2, np.full(tag.shape, case.layer_idx))
    assert np.array_equal((tag // 16384) % 2, np.zeros(tag.shape, np.int64))
    assert np.array_equal((tag // 64) % 256, np.broadcast_to(slots[:, None], tag.shape))
    assert np.array_equal(tag % 64, np.broadcast_to(np.arange(tag.shape[1])[None, :], tag.shape))
    col = np.arange(case.D_c)[None, :]
    assert np.array_equal(codes, ((col + 3 * slots[:, None] + 5 * pages[:, None]) % 126).astype(np.uint8))


def _quantised_copy(case_bf16):
    """The bf16 case's cache with every row of its layer quantised per 128
    columns by the oracle's quantiser (rows of NaN poison stay poison)."""
    c = case_bf16.cache
    rows = c.pool.reshape(-1, c.num_heads * c.head_dim)
    q, s = oracle.quantize_e4m3_rows(rows, rows.shape[1], 128)
    pool = q.reshape(c.pool.shape)
    scales = s.reshape(c.pool.shape[:4] + (s.shape[1],))
    cache = dataclasses.replace(c, pool=pool, dtype="e4m3", scales=scales, scale_gran=128)
    return dataclasses.replace(case_bf16, cache=cache)


@pytest.mark.parametrize("seed", [3, 4])
def test_quantised_cache_matches_the_fp8_form(seed):
    bf = W.small_decompress(seed, batch=4, max_len=120, page_size=16, N=256, fp8=True)
    f8 = _quantised_copy(bf)
    lat, q, s, want = oracle.decompress_k_fp8(bf)
    codes, scales, got = oracle.decompress_k_fp8_cache(f8)
    assert np.array_equal(codes[:, :bf.K], q)
    assert np.array_equal(scales[:, :bf.K // 128], s)
    assert np.array_equal(got, want)


def test_dequantised_rows_within_the_e4m3_bound():
    bf = W.small_decompress(5, batch=3, max_len=100, page_size=8, N=128, fp8=True)
    f8 = _quantised_copy(bf)
    x = oracle.bf16_decode(oracle.gather(bf)).astype(np.float64)
    codes, scales, _ = oracle.decompress_k_fp8_cache(f8)
    y = oracle.e4m3_decode(codes) * np.repeat(scales.astype(np.float64), 128, axis=1)[:, :x.shape[1]]
    # 3 mantissa bits: half an ulp is 2^-4 of the value; below 2^-6 the spacing is
    # the subnormal one, 2^-9, so the absolute part is 2^-10 times the scale.
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * np.repeat(scales.astype(np.float64), 128, axis=1)[:, :x.shape[1]]
    assert np.all(np.abs(y - x) <= bound * (1 + 1e-6))


def test_preconditions():
    bf = W.small_decompress(6, batch=2, max_len=40, page_size=8, N=128, fp8=True)
    with pytest.raises(oracle.OracleError):
        oracle.decompress_k_fp8_cache(bf)            # a bf16 cache has no scales
    f8 = _quantised_copy(bf)
    f8 = dataclasses.replace(f8, cache=dataclasses.replace(f8.cache, scale_gran=64))
    with pytest.raises(oracle.OracleError):
        oracle.decompress_k_fp8_cache(f8)            # scales per 64 columns do not fit 1x128 blocks


# ---- the V leg of the fused K and V form on an fp8 cache (page
# "mla_prefill_decode_graph_fp8", Args w_uv and w_uv_scale: the same latent
# rows projected by a second weight)

def _kv_cases(seed, N=256, Nv=384):
    case = W.small_decompress(seed, batch=4, max_len=120, page_size=16, N=N, dtype="e4m3", fp8=True)
    return case, W.with_second_projection(case, seed=seed + 100, N=Nv)


def check_kv_each_projection_on_its_own_weight(orc, seed=21):
    """K and V each equal the single-projection form run on that projection's
    own weight and scales; V differs from K wherever the weights differ."""
    case, case_v = _kv_cases(seed)
    codes, scales, k, v = orc.decompress_kv_fp8_cache(case, case_v)
    c1, s1, k1 = oracle.decompress_k_fp8_cache(case)
    c2, s2, v1 = oracle.decompress_k_fp8_cache(case_v)
    assert np.array_equal(codes, c1) and np.array_equal(scales, s1)
    assert np.array_equal(k, k1)
    assert v.shape == v1.shape and np.array_equal(v, v1)


def check_kv_selection_w_uv(orc, seed=22):
    """A selection W_uv (row n holds code 1.0 at column pi(n), zeros elsewhere;
    unit block scales) returns the named latent columns, dequantised with the
    cache's own scale of the block each column lies in, exactly: one non-zero
    product per output, so no rounding is involved."""
    case, case_v = _kv_cases(seed, Nv=256)
    K, Nv = case.K, case_v.N
    rng = np.random.default_rng(seed)
    pi = rng.permutation(K)[:Nv]
    wq = np.zeros((Nv, K), np.uint8)
    wq[np.arange(Nv), pi] = 0x38                     # e4m3fn 1.0: exponent 7 (bias 7), mantissa 0
    case_v = dataclasses.replace(case_v, weight_q=wq,
                                 weight_scale=np.ones_like(case_v.weight_scale))
    codes, scales, _, v = orc.decompress_kv_fp8_cache(case, case_v)
    deq = oracle.e4m3_decode(codes[:, :K]).astype(np.float64) * \
        np.repeat(scales[:, :K // 128].astype(np.float64), 128, axis=1)
    assert len({int(p) // 128 for p in pi}) == K // 128    # columns from every scale block
    assert np.array_equal(v, deq[:, pi])


def test_kv_each_projection_on_its_own_weight():
    check_kv_each_projection_on_its_own_weight(oracle)


def test_kv_selection_w_uv_returns_the_named_dequantised_columns():
    check_kv_selection_w_uv(oracle)
