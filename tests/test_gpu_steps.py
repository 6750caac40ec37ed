"""GPU parity of the two steps of the decompress operation as calls of their own
(mla_gather_latent_paged, mla_latent_matmul) and of the debug index check
(mla_check_indices), against the CPU oracle.

The gather must be bit-identical to the oracle's gather; the product must meet
max|gpu - ref| <= 1e-2 * max|ref| (bf16) and agree bit for bit with the fused
call, which launches the same kernels."""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import BF16_TOL, POISON_OUT, check_close, check_guards, guarded_empty, run_decompress, say, to_bits

pytestmark = pytest.mark.gpu

OK, SHAPE, RANGE = 0, 2, 5


def _gather(case, extra_rows=5):
    dc, t = W.device_decompress(case)
    dt = torch.float32 if case.cache.dtype == "f32" else torch.bfloat16
    lat = guarded_empty((case.M + extra_rows, case.D_c), dt)
    lat.view(torch.int16 if dt == torch.bfloat16 else torch.int32).fill_(POISON_OUT)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    say(f"[gpu] gather {case.name}: M={case.M} D={case.D_c} ps={case.cache.page_size}")
    mp.mla_gather_latent_paged(t["buffer_row_offsets"], t["cache_offsets"], case.M, cache, case.layer_idx, lat)
    check_guards("gather " + case.name)
    return lat, dc, t


@pytest.mark.parametrize("seed,ps,dtype", [(11, 16, "bf16"), (12, 1, "bf16"), (13, 5, "f32"), (14, 128, "bf16")])
def test_gather_alone_is_bit_exact(seed, ps, dtype):
    rope = 64 if dtype == "bf16" else 16
    case = W.small_decompress(seed, batch=7, max_len=600, page_size=ps, K=512 if dtype == "bf16" else 64,
                              rope=rope, N=128, dtype=dtype)
    lat, _, _ = _gather(case)
    bits = to_bits(lat)
    assert np.array_equal(bits[:case.M], oracle.gather(case))
    assert np.all(bits[case.M:] == POISON_OUT)


def test_gather_alone_c1_full():
    case = W.c1_decode()
    lat, _, _ = _gather(case, extra_rows=2)
    bits = to_bits(lat)
    assert np.array_equal(bits[:case.M], oracle.gather(case))
    assert np.all(bits[case.M:] == POISON_OUT)


@pytest.mark.parametrize("ld_extra", [0, 64, 8])
def test_latent_matmul_alone(ld_extra):
    """Rows of width K + ld_extra (a padded or rope-carrying row stride); columns
    past K hold NaN and must not reach the product."""
    rng = np.random.default_rng(20 + ld_extra)
    M, N, K = 777, 1024, 512
    a = rng.standard_normal((M, K + ld_extra)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    a_bits, w_bits = W.to_bf16_bits(a), W.to_bf16_bits(w)
    a_bits[:, K:] = W.POISON_BF16
    A = torch.from_numpy(a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    Wt = torch.from_numpy(w_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = guarded_empty((M + 3, N), torch.bfloat16)
    out.view(torch.int16).fill_(POISON_OUT)
    say(f"[gpu] latent_matmul M={M} N={N} K={K} ld={K + ld_extra}")
    mp.mla_latent_matmul(A, M, Wt, out)
    check_guards(f"latent_matmul M={M}")
    ref = oracle.matmul_nt(a_bits, "bf16", w_bits, "bf16", K)
    check_close(out[:M].double().cpu().numpy(), ref, BF16_TOL, f"latent_matmul ld={K + ld_extra}")
    assert np.all(to_bits(out)[M:] == POISON_OUT)


def test_two_steps_equal_the_fused_call():
    case = W.small_decompress(15, batch=6, max_len=900, page_size=64, K=512, rope=64, N=2048)
    fused = run_decompress(case)
    lat, dc, t = _gather(case, extra_rows=0)
    out = torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    mp.mla_latent_matmul(lat, case.M, t["weight"], out)
    torch.cuda.synchronize()
    assert torch.equal(lat.view(torch.int16), fused["lat"].view(torch.int16))
    assert torch.equal(out.view(torch.int16), fused["out"].view(torch.int16))


def test_latent_matmul_f32():
    rng = np.random.default_rng(31)
    M, N, K = 50, 132, 68
    a = rng.standard_normal((M, K + 12)).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    out = torch.full((M, N), float("nan"), device="cuda")
    mp.mla_latent_matmul(torch.from_numpy(a).cuda(), M, torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.matmul_nt(a.view(np.uint32), "f32", w.view(np.uint32), "f32", K)
    check_close(out.double().cpu().numpy(), ref, 1e-5, "latent_matmul f32")


def _u32(x):
    return torch.from_numpy(np.asarray(x, np.uint32).view(np.int32)).cuda()


def test_check_indices_accepts_valid_and_names_the_bad_request():
    case = W.small_decompress(16, batch=5, max_len=300, page_size=16, K=512, rope=64, N=128)
    dc, t = W.device_decompress(case)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    bro, co = case.buffer_row_offsets.copy(), case.cache_offsets.copy()
    assert mp.mla_check_indices(t["buffer_row_offsets"], t["cache_offsets"], case.M, cache) == (OK, -1)
    # wrong total
    assert mp.mla_check_indices(t["buffer_row_offsets"], t["cache_offsets"], case.M + 1, cache)[0] == SHAPE
    # offsets that decrease at request 2
    b2 = bro.copy()
    b2[3] = b2[2] - 1 if b2[2] > 0 else 0
    if b2[3] < b2[2]:
        st, bad = mp.mla_check_indices(_u32(b2), t["cache_offsets"], int(b2[-1]), cache)
        assert (st, bad) == (SHAPE, 2)
    # request 3 reads past its cached length
    c3 = co.copy()
    c3[3] = case.cache.cache_lengths[3]
    rows3 = bro[4] - bro[3]
    st, bad = mp.mla_check_indices(t["buffer_row_offsets"], _u32(c3), case.M, cache)
    assert (st, bad) == ((RANGE, 3) if rows3 > 0 else (OK, -1))
    # a page id past the pool in request 1's first page
    pt = case.cache.page_table.copy()
    pt[1, co[1] // 16] = case.cache.num_pages
    bad_cache = mp.PagedKVCache(dc.pool, _u32(pt), dc.cache_lengths)
    st, bad = mp.mla_check_indices(t["buffer_row_offsets"], t["cache_offsets"], case.M, bad_cache)
    assert (st, bad) == ((RANGE, 1) if bro[2] > bro[1] else (OK, -1))


def test_check_indices_append_mode():
    case = W.small_kv_matmul(17)
    dc, t = W.device_kv(case)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    assert mp.mla_check_indices(t["input_row_offsets"], None, case.T, cache) == (OK, -1)
    lens = case.cache.cache_lengths.copy()
    ps, maxp = case.cache.page_size, case.cache.page_table.shape[1]
    lens[0] = maxp * ps  # no room left in request 0's page-table row
    over = mp.PagedKVCache(dc.pool, dc.page_table, _u32(lens))
    st, bad = mp.mla_check_indices(t["input_row_offsets"], None, case.T, over)
    iro = case.input_row_offsets
    assert (st, bad) == ((RANGE, 0) if iro[1] > iro[0] else (OK, -1))


def test_guard_canaries_catch_a_write_next_to_an_output():
    """The canaries around the tests' outputs: a byte changed right before or
    right after an output buffer (written here from the host) is reported."""
    import gpu_util
    for where in (gpu_util.GUARD_BYTES - 1, -gpu_util.GUARD_BYTES):
        guarded_empty((4, 64), torch.bfloat16).zero_()
        gpu_util._guarded[-1][where] = 0
        with pytest.raises(AssertionError, match="canary"):
            check_guards("planted")
    guarded_empty((4, 64), torch.bfloat16).zero_()
    check_guards("untouched")

