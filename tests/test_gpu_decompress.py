"""GPU parity of mla_decompress_k_paged (bf16 and f32) against the CPU oracle.

Gathered rows (k_latent_buffer) must be bit-identical to the oracle's gather;
k_buffer must satisfy max|gpu - ref| <= 1e-2 * max|ref| (bf16), and, for f32,
also the accumulation bound derived from the arithmetic
|err| <= K * 2^-24 * sum_k |a_k w_k| + 2^-24 |ref|.
Rows past buffer_length must keep the poison written before the call.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from caselib import elem_f64
from gpu_util import (BF16_TOL, POISON_OUT, check_close, rows_as_f64, run_decompress, sample_rows, say,
                      to_bits)

pytestmark = pytest.mark.gpu


def _check_full(case, extra_rows=7):
    res = run_decompress(case, extra_rows=extra_rows)
    M = case.M
    ref_lat, ref = oracle.decompress_k(case)
    lat_bits = to_bits(res["lat"])
    assert np.array_equal(lat_bits[:M], ref_lat), f"{case.name}: gathered rows differ"
    got = res["out"][:M].double().cpu().numpy()
    check_close(got, ref, BF16_TOL, f"{case.name} k_buffer")
    if case.cache.dtype == "bf16":
        assert np.all(lat_bits[M:] == POISON_OUT) and np.all(to_bits(res["out"])[M:] == POISON_OUT)
    else:
        assert np.all(np.isnan(res["lat"][M:].cpu().numpy())) and np.all(np.isnan(res["out"][M:].cpu().numpy()))
    return res, ref_lat, ref


def test_c0_tiny_f32():
    case = W.c0_tiny()
    res, ref_lat, ref = _check_full(case)
    got = res["out"][:case.M].double().cpu().numpy()
    a = np.abs(elem_f64(ref_lat, "f32")[:, :case.K])
    w = np.abs(elem_f64(case.weight, "f32"))
    bound = case.K * 2.0 ** -24 * (a @ w.T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("seed,ps,N", [(0, 16, 512), (1, 128, 1024), (2, 1, 512), (3, 7, 768), (4, 64, 2048)])
def test_small_bf16_full_compare(seed, ps, N):
    case = W.small_decompress(seed, batch=6, max_len=400, page_size=ps, K=512, rope=64, N=N)
    _check_full(case)


@pytest.mark.parametrize("lens,offs,M", [([257], [0], 257), ([300, 256], [44, 0], 512), ([513], [0], 513)])
def test_edges_of_the_gather_and_product_path(lens, offs, M):
    """257 rows (the first count past the few-rows kernel), exactly 512 (two
    whole 256-row tiles) and 513 (one row into a third tile)."""
    case = W.decompress_case("edge_m", seed=31, cache_lengths=lens, cache_offsets=offs, page_size=16,
                             kv_lora_rank=512, rope_dim=64, N=1024)
    assert case.M == M
    _check_full(case)


def test_small_bf16_no_rope_k64_and_empty_requests():
    case = W.decompress_case("k64_empty", seed=9, cache_lengths=[40, 10, 77, 5, 300], cache_offsets=[40, 3, 0, 5, 17],
                             page_size=32, kv_lora_rank=64, rope_dim=0, N=64)
    assert case.M == 7 + 77 + 283
    _check_full(case)


def test_identity_weight_returns_latent_exactly():
    case = W.small_decompress(5, batch=4, max_len=300, page_size=16, K=512, rope=64, N=512)
    case.weight = W.to_bf16_bits(np.eye(512, dtype=np.float32))
    res = run_decompress(case)
    ref_lat = oracle.gather(case)
    assert np.array_equal(to_bits(res["out"]), ref_lat[:, :512])


def test_selection_weight_permutes_columns_exactly():
    rng = np.random.default_rng(6)
    case = W.small_decompress(6, batch=3, max_len=200, page_size=128, K=512, rope=64, N=256)
    perm = rng.permutation(512)[:256]
    sel = np.zeros((256, 512), np.float32)
    sel[np.arange(256), perm] = 1.0
    case.weight = W.to_bf16_bits(sel)
    res = run_decompress(case)
    ref_lat = oracle.gather(case)
    assert np.array_equal(to_bits(res["out"]), ref_lat[:, perm])


def test_nan_rope_columns_stay_out_of_the_product():
    case = W.small_decompress(7, batch=3, max_len=200, page_size=16, K=512, rope=64, N=512)
    case.cache.pool[..., 512:] = W.POISON_BF16
    res, ref_lat, ref = _check_full(case)
    assert np.all(np.isfinite(ref))


def test_repeat_runs_are_bit_identical():
    case = W.small_decompress(8, batch=5, max_len=500, page_size=16, K=512, rope=64, N=1024)
    a = run_decompress(case)
    b = run_decompress(case)
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    assert torch.equal(a["lat"].view(torch.int16), b["lat"].view(torch.int16))


def _check_sampled(case, tol=BF16_TOL):
    res = run_decompress(case, extra_rows=3)
    M = case.M
    ref_lat = oracle.gather(case)
    lat_bits = to_bits(res["lat"])
    assert np.array_equal(lat_bits[:M], ref_lat), f"{case.name}: gathered rows differ"
    assert np.all(lat_bits[M:] == POISON_OUT)
    rows = sample_rows(case)
    say(f"[gpu] {case.name}: comparing {len(rows)} sampled rows")
    ref = oracle.matmul_nt(ref_lat, case.cache.dtype, case.weight, case.weight_dtype, case.K, rows)
    got = rows_as_f64(res["out"], rows, M)
    check_close(got, ref, tol, f"{case.name} k_buffer (sampled)")
    tail = res["out"][M:].view(torch.int16)
    assert bool((tail == POISON_OUT).all())


@pytest.mark.slow
def test_c1_decode_full_size_sampled():
    _check_sampled(W.c1_decode())


@pytest.mark.slow
def test_c2_prefill_full_size_sampled():
    _check_sampled(W.c2_prefill())


@pytest.mark.slow
def test_c2_tensor_parallel_share_sampled():
    """One GPU's share of W_k under 8-way tensor parallelism over heads (the
    first 16 heads: N = 2048) on the full prefill batch, as the bench times it."""
    import dataclasses
    c = W.c2_prefill()
    _check_sampled(dataclasses.replace(c, name="c2_tp8_share", N=2048, weight=np.ascontiguousarray(c.weight[:2048])))
