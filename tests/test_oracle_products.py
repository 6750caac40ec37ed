"""Pins for the oracle's up-projection and its fp8 block-scaled form.

Sources: page "generic_flare_mla_decompress_k_cache_ragged_paged" (summary: the
gathered latent rows are multiplied by the weight) and page
"mla_prefill_decode_graph_fp8" (Args w_k [num_heads*qk_nope_head_dim,
kv_latent_dim], w_k_scale; Parameters m/n/k_scale_granularity).

What pins them, none of it a re-typing of the oracle's loops:
  * numpy float64 matmul (a library routine) on random shapes with N != K and
    rope columns present (a transposed operand or a wrong K fails);
  * identity and selection weights reproduce / permute the latent exactly;
  * NaN rope columns never reach the product;
  * the hand-worked example;
  * fp8: blocks built to be exactly representable quantise losslessly and the
    block-scaled product then equals a float64 matmul of the dequantised
    operands; the e4m3 rounding error bound holds for random rows; the block
    maximum maps onto +-448; an all-zero block has scale 1 and zero codes.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from caselib import elem_f64, worked_decompress_case


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matmul_nt_matches_numpy_float64(dtype):
    rng = np.random.default_rng(21)
    M, D, K, N = 37, 80, 64, 48
    a = rng.standard_normal((M, D)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    if dtype == "bf16":
        a_bits, w_bits = W.to_bf16_bits(a), W.to_bf16_bits(w)
    else:
        a_bits, w_bits = a.view(np.uint32), w.view(np.uint32)
    out = oracle.matmul_nt(a_bits, dtype, w_bits, dtype, K)
    ref = elem_f64(a_bits, dtype)[:, :K] @ elem_f64(w_bits, dtype).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # a subset of rows gives the same rows
    rows = np.array([36, 0, 17, 17])
    np.testing.assert_array_equal(oracle.matmul_nt(a_bits, dtype, w_bits, dtype, K, rows), out[rows])


def test_identity_and_selection_weights_are_exact():
    rng = np.random.default_rng(22)
    M, K, D = 19, 32, 40
    a_bits = W.to_bf16_bits(rng.standard_normal((M, D)).astype(np.float32))
    eye = W.to_bf16_bits(np.eye(K, dtype=np.float32))
    out = oracle.matmul_nt(a_bits, "bf16", eye, "bf16", K)
    assert np.array_equal(out, elem_f64(a_bits, "bf16")[:, :K])
    perm = rng.permutation(K)[:24]
    sel = np.zeros((24, K), np.float32)
    sel[np.arange(24), perm] = 1.0
    out = oracle.matmul_nt(a_bits, "bf16", W.to_bf16_bits(sel), "bf16", K)
    assert np.array_equal(out, elem_f64(a_bits, "bf16")[:, perm])


def test_rope_columns_never_enter_the_product():
    rng = np.random.default_rng(23)
    M, K, D, N = 9, 16, 24, 8
    a = rng.standard_normal((M, D)).astype(np.float32)
    a[:, K:] = np.nan
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = oracle.matmul_nt(a.view(np.uint32), "f32", w.view(np.uint32), "f32", K)
    assert np.all(np.isfinite(out))


def test_worked_example_product():
    case, _, k_buffer = worked_decompress_case()
    lat, out = oracle.decompress_k(case)
    assert np.array_equal(out, k_buffer)


# ---------------------------------------------------------------------------
# fp8
# ---------------------------------------------------------------------------
def _exact_blocks(rng, M, K, kg=128):
    """bf16 rows whose every k-block is e4m3 codes times 2^e with the block max at 448*2^e."""
    codes = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8)  # finite non-negative codes
    codes |= (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    vals = elem_f64(codes, "e4m3")
    exps = rng.integers(-8, 4, size=(M, K // kg))
    for kb in range(K // kg):
        j = rng.integers(0, kg, size=M)
        vals[np.arange(M), kb * kg + j] = 448.0 * np.where(rng.integers(0, 2, size=M) == 1, 1, -1)
        vals[:, kb * kg:(kb + 1) * kg] *= np.exp2(exps[:, kb])[:, None]
    bits = W.to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(elem_f64(bits, "bf16"), vals)  # representable exactly
    return bits, vals, exps


def test_lossless_blocks_quantise_exactly_and_product_matches_numpy():
    rng = np.random.default_rng(31)
    M, K, N = 23, 512, 256
    a_bits, vals, exps = _exact_blocks(rng, M, K)
    q, s = oracle.quantize_e4m3_rows(a_bits, K)
    assert np.array_equal(s.astype(np.float64), np.exp2(exps))
    np.testing.assert_array_equal(elem_f64(q, "e4m3") * np.repeat(np.exp2(exps), 128, axis=1), vals)
    qw = W.to_e4m3_bits(rng.standard_normal((N, K)).astype(np.float32))
    sw = rng.uniform(0.015, 0.025, size=(N // 128, K // 128)).astype(np.float32)
    out = oracle.fp8_matmul_nt(q, s, qw, sw)
    w_deq = elem_f64(qw, "e4m3") * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    ref = vals @ w_deq.T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_quantisation_error_bound_and_block_max():
    rng = np.random.default_rng(32)
    M, K, D = 64, 512, 576
    a_bits = W.to_bf16_bits(rng.standard_normal((M, D)).astype(np.float32) * 3)
    q, s = oracle.quantize_e4m3_rows(a_bits, K)
    x = elem_f64(a_bits, "bf16")[:, :K]
    sx = np.repeat(s.astype(np.float64), 128, axis=1)
    y = x / sx                       # the value that was rounded (up to one binary32 rounding)
    d = elem_f64(q, "e4m3")
    # e4m3fn: 3 mantissa bits -> half-spacing 2^-4 relative for normals, 2^-10 absolute below 2^-6
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(y - d) <= bound)
    amax = np.abs(x).reshape(M, 4, 128).max(axis=2)
    np.testing.assert_allclose(s.astype(np.float64), amax / 448.0, rtol=2 ** -23)
    for kb in range(4):
        j = np.argmax(np.abs(x[:, kb * 128:(kb + 1) * 128]), axis=1)
        assert np.all(np.abs(d[np.arange(M), kb * 128 + j]) == 448.0)


def test_all_zero_block_has_unit_scale_and_zero_codes():
    M, K = 3, 256
    a = np.zeros((M, K), np.float32)
    a[1, 128:] = np.linspace(-1, 1, 128)
    q, s = oracle.quantize_e4m3_rows(W.to_bf16_bits(a), K)
    assert s[0].tolist() == [1.0, 1.0] and s[1, 0] == 1.0 and s[2].tolist() == [1.0, 1.0]
    assert np.all(elem_f64(q[0], "e4m3") == 0) and np.all(elem_f64(q[1, :128], "e4m3") == 0)
    assert s[1, 1] == np.float32(1.0) / np.float32(448.0)


def test_fp8_scales_are_indexed_by_row_block_and_column_block():
    # one nonzero weight block at a time: only the matching output columns / k-blocks move
    rng = np.random.default_rng(33)
    M, K, N = 5, 384, 384
    a_bits, vals, exps = _exact_blocks(rng, M, K)
    q, s = oracle.quantize_e4m3_rows(a_bits, K)
    qw = np.zeros((N, K), np.uint8)
    qw[128:256, 256:384] = W.to_e4m3_bits(np.ones((128, 128), np.float32))
    sw = np.ones((3, 3), np.float32)
    sw[1, 2] = 0.5
    out = oracle.fp8_matmul_nt(q, s, qw, sw)
    assert np.all(out[:, :128] == 0) and np.all(out[:, 256:] == 0)
    ref = vals[:, 256:384].sum(axis=1) * 0.5
    np.testing.assert_allclose(out[:, 128:256], np.repeat(ref[:, None], 128, 1), rtol=1e-12)


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_kv_is_the_two_products_of_one_gather(fp8):
    """The V product of the fused form is the same definition with W_uv: a
    selection W_uv picks latent columns exactly (bf16), and each output equals
    the single-projection oracle on its own weight."""
    case = W.small_decompress(7, batch=3, max_len=60, page_size=16, K=256, rope=64, N=128, fp8=fp8)
    case_v = W.with_second_projection(case, seed=8, N=256)
    lat, k, v = oracle.decompress_kv(case, case_v)
    if fp8:
        _, _, _, k1 = oracle.decompress_k_fp8(case)
        _, _, _, v1 = oracle.decompress_k_fp8(case_v)
    else:
        _, k1 = oracle.decompress_k(case)
        _, v1 = oracle.decompress_k(case_v)
        # W_uv row n = e_{(3n) mod K}: v[:, n] is latent column (3n) mod K, exactly
        sel = np.zeros((256, case.K), np.float32)
        sel[np.arange(256), (3 * np.arange(256)) % case.K] = 1.0
        case_s = W.with_second_projection(case, seed=9, N=256)
        case_s.weight = W.to_bf16_bits(sel)
        _, _, vs = oracle.decompress_kv(case, case_s)
        assert np.array_equal(vs, oracle.bf16_decode(lat)[:, (3 * np.arange(256)) % case.K].astype(np.float64))
    assert np.array_equal(k, k1) and np.array_equal(v, v1)
    assert v.shape == (case.M, 256)
