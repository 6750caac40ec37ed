"""GPU parity of mla_write_latent_paged_fp8 (the latent write path into an e4m3
cache with one fp32 scale per 128 columns) against the CPU oracle.

The kernel computes the row values in fp32 (the oracle in binary64, rounded to
binary32), so a code may land one e4m3 step away where a value sits within a
few fp32 ulps of a rounding midpoint.  The bar, per element: the decoded value
times its scale is within half an e4m3 step of the oracle's binary64 value
(2^-4 relative in the normal range, 2^-10 of the scale below it) plus 2^-18
relative slack for the fp32 arithmetic; per block, the scale within 2^-20 of
the oracle's; and at least 99.5 % of the codes bit-identical.  Every other byte
of the pool and of the scale pool keeps its bits, and the written rows are read
back by mla_decompress_k_paged_fp8_cache: codes and scales bit for bit, and
through a selection weight as the decoded code times its scale."""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


def run_write(case):
    dc, t = W.device_latent_write(case)
    pool0, sc0 = dc.pool.clone(), dc.scales.clone()
    say(f"[gpu] {case.name}: fp8 write T={case.T} K={case.K} D={case.x.shape[1]}")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    mp.mla_write_latent_paged_fp8(t["x"], t["input_row_offsets"], t["gamma"], case.eps, t["freqs"], case.K,
                                  cache, case.layer_idx)
    torch.cuda.synchronize()
    return dc, pool0, sc0


def _check(case):
    dc, pool0, sc0 = run_write(case)
    q, s, ref, dst, sdst = oracle.latent_write_fp8(case)
    T, D = q.shape
    nb = s.shape[1]
    pool = dc.pool.reshape(-1)
    scl = dc.scales.reshape(-1)
    idx = torch.as_tensor(dst, device=pool.device)[:, None] + torch.arange(D, device=pool.device)[None, :]
    sidx = torch.as_tensor(sdst, device=pool.device)[:, None] + torch.arange(nb, device=pool.device)[None, :]
    got_q = pool[idx.reshape(-1)].reshape(T, D).cpu().numpy().view(np.uint8)
    got_s = scl[sidx.reshape(-1)].reshape(T, nb).cpu().numpy()
    # nothing else changed
    e_pool = pool0.reshape(-1).clone()
    e_pool[idx.reshape(-1)] = pool[idx.reshape(-1)]
    assert torch.equal(e_pool, pool), "pool bytes outside the written rows changed"
    e_sc = sc0.reshape(-1).clone()
    e_sc[sidx.reshape(-1)] = scl[sidx.reshape(-1)]
    assert torch.equal(e_sc.view(torch.int32), scl.view(torch.int32)), "scales outside the written rows changed"
    # scales and values
    assert np.all(np.abs(got_s.astype(np.float64) - s) <= 2.0 ** -20 * np.abs(s)), "block scales"
    scale = np.repeat(got_s.astype(np.float64), 128, axis=1)[:, :D]
    back = oracle.e4m3_decode(got_q).astype(np.float64) * scale
    bound = 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * scale + 2.0 ** -18 * np.abs(ref)
    bad = np.abs(back - ref) > bound
    assert not bad.any(), f"{bad.sum()} values outside the e4m3 bound, first at {np.argwhere(bad)[:3].tolist()}"
    same = (got_q == q).mean()
    assert same >= 0.995, f"only {same:.4f} of the codes match the oracle's"
    return dc, got_q, got_s


@pytest.mark.parametrize("seq_lens,starts,ps", [([3, 0, 5, 2], [2, 7, 0, 9], 4), ([1], [0], 1),
                                                 ([130, 7, 64], [0, 300, 17], 16)])
def test_small_fp8_writes(seq_lens, starts, ps):
    _check(W.latent_write_case("fp8w", seed=31, seq_lens=seq_lens, start_lengths=starts, page_size=ps,
                               dtype="e4m3"))


def test_zero_rows_and_odd_token_counts():
    c = W.latent_write_case("fp8w0", seed=32, seq_lens=[5, 0, 3], start_lengths=[1, 2, 3], page_size=8, dtype="e4m3")
    c.x[2] = 0          # an all-zero token: every block is zero -> scale 1, codes of +-0
    dc, got_q, got_s = _check(c)
    assert np.all(oracle.e4m3_decode(got_q[2]) == 0.0) and np.all(got_s[2] == 1.0)


def test_write_then_read_back_through_the_fp8_cache_decompress():
    c = W.latent_write_case("fp8rt", seed=33, seq_lens=[40, 17, 64], start_lengths=[5, 0, 100], page_size=16,
                            dtype="e4m3")
    dc, got_q, got_s = _check(c)
    # gather exactly the new tokens: cache_offsets = old lengths, rows = new tokens
    lens = np.asarray([40, 17, 64])
    bro = np.zeros(4, np.uint32)
    bro[1:] = np.cumsum(lens)
    t = {"bro": torch.as_tensor(bro.astype(np.int32)).cuda(), "co": dc.cache_lengths.clone()}
    M, D = int(bro[-1]), got_q.shape[1]
    # cache lengths after the write
    dc.cache_lengths += torch.as_tensor(lens.astype(np.int32), device="cuda").view(dc.cache_lengths.dtype)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths, scales=dc.scales)
    N, K = 256, c.K
    wq = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    wq[torch.arange(N), torch.arange(N)] = 0x38          # e4m3 code of 1.0: column n selects latent column n
    ws = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    lat = torch.empty((M, D), dtype=torch.uint8, device="cuda")
    lsc = torch.empty((M, -(-D // 128)), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mp.mla_decompress_k_paged_fp8_cache(t["bro"], t["co"], M, wq, ws, cache, c.layer_idx, lat, lsc, out)
    torch.cuda.synchronize()
    assert np.array_equal(lat.cpu().numpy(), got_q), "gathered codes differ from the written ones"
    assert np.array_equal(lsc.cpu().numpy().view(np.uint32), got_s.view(np.uint32)), "gathered scales differ"
    # column n < 128 is block 0's code times its scale, 128 <= n < 256 block 1's (the product
    # rescales its accumulators between blocks in fp32, so allow two bf16 steps)
    expect = oracle.e4m3_decode(got_q[:, :N]).astype(np.float64)
    expect[:, :128] *= got_s[:, :1]
    expect[:, 128:] *= got_s[:, 1:2]
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - expect) <= 2.0 ** -7 * np.abs(expect)), "selection through the fp8 product"


def test_c5_fp8_write_batch():
    _check(W.c5_latent_write_fp8())
