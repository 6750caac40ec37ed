"""GPU parity of the few-rows form of mla_decompress_k_paged (up to 256 rows:
one fused kernel that gathers, writes k_latent_buffer and multiplies) against
the CPU oracle, and of mla_latent_matmul on few rows.

Same bar as the large form: gathered rows bit-identical, k_buffer within
1e-2 * max|ref|, rows past M untouched; selection weights give exact copies."""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import BF16_TOL, POISON_OUT, check_close, check_guards, guarded_empty, run_decompress, say, to_bits

pytestmark = pytest.mark.gpu


def _newest_rows(base, newest):
    """The decode batch with only each request's `newest` last cached rows."""
    lens = base.cache.cache_lengths.astype(np.int64)
    take = np.minimum(lens, newest)
    bro = np.zeros(len(lens) + 1, np.uint32)
    bro[1:] = np.cumsum(take)
    return W.DecompressCase(f"{base.name}_newest{newest}", base.cache, base.layer_idx, bro,
                            (lens - take).astype(np.uint32), base.K, base.N, base.weight, base.weight_dtype)


def _check_full(case, extra_rows=3):
    res = run_decompress(case, extra_rows=extra_rows)
    M = case.M
    ref_lat, ref = oracle.decompress_k(case)
    bits = to_bits(res["lat"])
    assert np.array_equal(bits[:M], ref_lat), f"{case.name}: gathered rows differ"
    assert np.all(bits[M:] == POISON_OUT)
    check_close(res["out"][:M].double().cpu().numpy(), ref, BF16_TOL, f"{case.name} k_buffer")
    assert np.all(to_bits(res["out"])[M:] == POISON_OUT)
    return res, ref_lat


@pytest.mark.parametrize("newest", [1, 4])
def test_decode_probe_batches(newest):
    """64 requests of the decode batch, their newest 1 (64 rows) or 4 (256 rows) tokens."""
    _check_full(_newest_rows(W.c1_decode(), newest))


@pytest.mark.parametrize("lens,offs,ps", [([1], [0], 16), ([40, 1, 3], [9, 0, 2], 1), ([300, 200], [270, 199], 7),
                                          ([100, 90, 80, 70], [37, 30, 28, 11], 32), ([256], [0], 128),
                                          ([100, 90], [5, 0], 16), ([50, 30], [3, 0], 16), ([97], [0], 16),
                                          ([120, 100], [10, 0], 32), ([130, 70], [2, 5], 8)])
def test_ragged_small_batches(lens, offs, ps):
    """Row counts 1 .. 256 over every row-block count (77 rows: 3 blocks of 32;
    97: 4; 185: 6, the weight streamed through the ring slots with the rows;
    210: 7; 193: 7 at its lower edge)."""
    case = W.decompress_case("small_m", seed=21, cache_lengths=lens, cache_offsets=offs, page_size=ps,
                             kv_lora_rank=512, rope_dim=64, N=1024)
    assert case.M <= 256
    _check_full(case)


@pytest.mark.parametrize("lens,offs,rope,N", [([80, 70], [0, 3], 576, 2048), ([60, 50, 40], [5, 0, 9], 64, 16384)])
def test_wide_rows_and_mid_row_counts(lens, offs, rope, N):
    """Rows wider than 2 KB (k_latent_buffer copied without the early register
    copy) and row counts that take the chunk ring (MB = 5: 147 and 136 rows)."""
    case = W.decompress_case("small_wide", seed=25, cache_lengths=lens, cache_offsets=offs, page_size=16,
                             kv_lora_rank=512, rope_dim=rope, N=N)
    assert 128 < case.M <= 160
    _check_full(case)


def test_k1024_and_empty_requests():
    case = W.decompress_case("small_k1024", seed=22, cache_lengths=[50, 10, 0, 77], cache_offsets=[20, 10, 0, 0],
                             page_size=16, kv_lora_rank=1024, rope_dim=64, N=512)
    _check_full(case)


def test_selection_weight_small_exact():
    rng = np.random.default_rng(23)
    case = W.decompress_case("small_sel", seed=23, cache_lengths=[90, 33], cache_offsets=[0, 5], page_size=16,
                             kv_lora_rank=512, rope_dim=64, N=256)
    perm = rng.permutation(512)[:256]
    sel = np.zeros((256, 512), np.float32)
    sel[np.arange(256), perm] = 1.0
    case.weight = W.to_bf16_bits(sel)
    res = run_decompress(case)
    ref_lat = oracle.gather(case)
    assert np.array_equal(to_bits(res["out"]), ref_lat[:, perm])


@pytest.mark.parametrize("M", [1, 33, 64, 96, 97, 128, 150, 160, 161, 185, 192, 193, 200, 224, 256])
def test_latent_matmul_few_rows(M):
    rng = np.random.default_rng(24 + M)
    N, K, ld = 2048, 512, 576
    a = rng.standard_normal((M, ld)).astype(np.float32)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    a_bits, w_bits = W.to_bf16_bits(a), W.to_bf16_bits(w)
    a_bits[:, K:] = W.POISON_BF16
    A = torch.from_numpy(a_bits.view(np.int16)).cuda().view(torch.bfloat16)
    Wt = torch.from_numpy(w_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = guarded_empty((M + 2, N), torch.bfloat16)
    out.view(torch.int16).fill_(POISON_OUT)
    say(f"[gpu] latent_matmul few rows M={M}")
    mp.mla_latent_matmul(A, M, Wt, out)
    check_guards(f"latent_matmul few rows M={M}")
    ref = oracle.matmul_nt(a_bits, "bf16", w_bits, "bf16", K)
    check_close(out[:M].double().cpu().numpy(), ref, BF16_TOL, f"latent_matmul M={M}")
    assert np.all(to_bits(out)[M:] == POISON_OUT)
