"""GPU parity of the fused K and V decompression (mla_decompress_kv_paged and its
fp8 form) against the CPU oracle: gathered rows bit-exact, k_buffer and v_buffer
within the tolerance of their dtype, rows past M untouched.  Each output must
also equal, bit for bit, what the single-projection call returns with that
weight alone: the fused launch runs the same per-element arithmetic."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (BF16_TOL, FP8_TOL, POISON_OUT, check_close, rows_as_f64, run_decompress,
                      run_decompress_kv, sample_rows, say, to_bits)

pytestmark = pytest.mark.gpu


def _poisoned(t, M):
    if t.dtype == torch.bfloat16:
        return bool(np.all(to_bits(t)[M:] == POISON_OUT))
    return bool(np.all(np.isnan(t[M:].cpu().numpy())))


def _check(case, case_v, rows=None, single=True):
    res = run_decompress_kv(case, case_v, extra_rows=5)
    M = case.M
    lat, ref_k, ref_v = oracle.decompress_kv(case, case_v, rows)
    assert np.array_equal(to_bits(res["lat"])[:M], lat), "gathered rows differ"
    tol = FP8_TOL if case.weight_dtype == "e4m3" else BF16_TOL
    for name, out, ref in (("k_buffer", res["k"], ref_k), ("v_buffer", res["v"], ref_v)):
        got = out[:M].double().cpu().numpy() if rows is None else rows_as_f64(out, rows, M)
        check_close(got, ref, tol, f"{case.name} fused {name}")
        assert _poisoned(out, M), f"{name}: rows past M were written"
    assert _poisoned(res["lat"], M)
    if single:
        # the same outputs from the single-projection call, bit for bit
        for c, key in ((case, "k"), (case_v, "v")):
            one = run_decompress(c, extra_rows=5)
            assert torch.equal(one["out"][:M].view(torch.int16) if one["out"].dtype == torch.bfloat16
                               else one["out"][:M].view(torch.int32),
                               res[key][:M].view(torch.int16) if res[key].dtype == torch.bfloat16
                               else res[key][:M].view(torch.int32)), f"fused {key} differs from the single call"
    return res


@pytest.mark.parametrize("Nk,Nv,batch,max_len,seed", [
    (1024, 1024, 6, 700, 30),   # one launch over both projections (N_k a whole number of 256-wide tiles)
    (512, 768, 6, 700, 31),     # projections of different widths in one launch
    (320, 512, 6, 700, 32),     # N_k not a multiple of 256: two product launches after one gather
])
def test_fused_bf16_full_compare(Nk, Nv, batch, max_len, seed):
    case = W.small_decompress(seed, batch=batch, max_len=max_len, page_size=16, K=512, rope=64, N=Nk)
    case_v = W.with_second_projection(case, seed=seed + 100, N=Nv)
    assert case.M > 256
    _check(case, case_v)


def test_fused_bf16_several_tiles_per_block():
    """More tiles than compute units, K and V tiles interleaved on every XCD."""
    case = W.small_decompress(40, batch=10, max_len=700, page_size=128, K=512, rope=64, N=8192)
    case_v = W.with_second_projection(case, seed=140, N=8192)
    say(f"[gpu] tiles {-(-case.M // 256) * (8192 // 256) * 2}")
    assert -(-case.M // 256) * 64 > 256
    _check(case, case_v, single=False)


def test_fused_few_rows_and_other_k():
    # few rows: the single-launch few-rows kernel, once per projection
    c = W.small_decompress(41, batch=3, max_len=40, page_size=16, K=512, rope=64, N=1024)
    assert c.M <= 256
    _check(c, W.with_second_projection(c, seed=141, N=512))
    # K % 128 != 0: the register-staged product, once per projection
    c = W.small_decompress(42, batch=4, max_len=300, page_size=16, K=192, rope=64, N=512)
    _check(c, W.with_second_projection(c, seed=142, N=256))


def test_fused_f32():
    c = W.c0_tiny()
    _check(c, W.with_second_projection(c, seed=143, N=64, w_std=0.05))


def test_fused_same_weight_gives_identical_outputs():
    case = W.small_decompress(43, batch=5, max_len=600, page_size=16, K=512, rope=64, N=1024)
    case_v = W.with_second_projection(case, seed=0, N=1024)
    case_v.weight = case.weight.copy()
    res = run_decompress_kv(case, case_v)
    assert torch.equal(res["k"].view(torch.int16), res["v"].view(torch.int16))


@pytest.mark.parametrize("Nk,Nv,batch,max_len,seed", [(1024, 1024, 6, 700, 50), (512, 1536, 8, 700, 51),
                                                      (8192, 8192, 8, 700, 52)])
def test_fused_fp8(Nk, Nv, batch, max_len, seed):
    case = W.small_decompress(seed, batch=batch, max_len=max_len, page_size=16, K=512, rope=64, N=Nk, fp8=True)
    case_v = W.with_second_projection(case, seed=seed + 100, N=Nv)
    _check(case, case_v, single=Nk < 8192)


@pytest.mark.slow
def test_fused_c2_full_size_sampled():
    """The C2 prefill batch with W_uv of the same shape as W_k, in the launch the
    fused bench row times; sampled rows against the oracle."""
    case = W.c2_prefill()
    case_v = W.with_second_projection(case, seed=1002, N=case.N)
    rows = sample_rows(case)
    say(f"[gpu] c2 fused: {len(rows)} sampled rows")
    _check(case, case_v, rows, single=False)
