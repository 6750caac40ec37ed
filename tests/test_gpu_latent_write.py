"""GPU parity of mla_write_latent_paged (the latent write path) against the CPU
oracle: every new token's cache row must be within one bf16 rounding of the
oracle's binary64 values (the kernel computes in fp32 and rounds to nearest
even: |gpu - ref| <= 2^-8 |ref| + 2^-24), at the slot the oracle names; every
other element of the pool (other layer, cached tokens, spare pages, slack
slots) must keep its bits."""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


def run_write(case, times=1):
    dc, t = W.device_latent_write(case)
    before = dc.pool.clone()
    say(f"[gpu] {case.name}: T={case.T} K={case.K} D={case.x.shape[1]}")
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    for _ in range(times):
        mp.mla_write_latent_paged(t["x"], t["input_row_offsets"], t["gamma"], case.eps, t["freqs"], case.K,
                                  cache, case.layer_idx)
    torch.cuda.synchronize()
    return before, dc.pool


def _check(case, times=1):
    before, after = run_write(case, times)
    ref, dst = oracle.latent_write(case)
    D = ref.shape[1]
    flat = after.reshape(-1)
    idx = torch.as_tensor(dst, device=after.device)[:, None] + torch.arange(D, device=after.device)[None, :]
    got_rows = flat[idx.reshape(-1)].reshape(case.T, D)
    expect = before.clone().reshape(-1)
    expect[idx.reshape(-1)] = got_rows.reshape(-1)
    assert torch.equal(expect.view(torch.int16), flat.view(torch.int16)), "bytes outside the written rows changed"
    got = got_rows.double().cpu().numpy()
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -24
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    assert np.all(err <= bound), f"{case.name}: worst element {worst}: got {got[worst]}, ref {ref[worst]}"
    return got


@pytest.mark.parametrize("ps,starts,lens", [(16, [2, 7, 0, 30], [5, 0, 40, 17]), (1, [0, 3], [9, 4]),
                                            (128, [120, 0, 300], [20, 129, 1])])
def test_small_full_compare(ps, starts, lens):
    case = W.latent_write_case(f"lw_ps{ps}", seed=ps, seq_lens=lens, start_lengths=starts, page_size=ps)
    _check(case)


def test_other_widths_and_no_rope():
    _check(W.latent_write_case("lw_k64", seed=3, seq_lens=[7, 33], start_lengths=[1, 60], page_size=8, K=64, R=16))
    _check(W.latent_write_case("lw_norope", seed=4, seq_lens=[12, 5], start_lengths=[0, 9], page_size=4, K=256, R=0))


def test_writing_twice_gives_the_same_rows():
    case = W.latent_write_case("lw_twice", seed=6, seq_lens=[50, 20], start_lengths=[3, 0], page_size=16)
    a = _check(case, times=1)
    b = _check(case, times=2)
    assert np.array_equal(a, b)


def test_written_rows_decompress_back():
    """The decompress path reads what the write path wrote: gathering the new
    positions returns the rows just written, bit for bit."""
    case = W.latent_write_case("lw_roundtrip", seed=7, seq_lens=[30, 0, 45], start_lengths=[4, 2, 0], page_size=16)
    dc, t = W.device_latent_write(case)
    cache = mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths)
    mp.mla_write_latent_paged(t["x"], t["input_row_offsets"], t["gamma"], case.eps, t["freqs"], case.K, cache,
                              case.layer_idx)
    torch.cuda.synchronize()
    _, dst = oracle.latent_write(case)
    D = case.x.shape[1]
    M = case.T
    lat = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, case.K), dtype=torch.bfloat16, device="cuda")
    co = torch.as_tensor(case.cache.cache_lengths.astype(np.int64), dtype=torch.int64).to(torch.int32).cuda()
    mp.mla_decompress_k_paged(t["input_row_offsets"], co, M, w, cache, case.layer_idx, lat, out)
    torch.cuda.synchronize()
    flat = dc.pool.reshape(-1)
    idx = torch.as_tensor(dst, device="cuda")[:, None] + torch.arange(D, device="cuda")[None, :]
    assert torch.equal(lat.view(torch.int16), flat[idx.reshape(-1)].reshape(M, D).view(torch.int16))


@pytest.mark.slow
def test_c5_full_size():
    case = W.c5_latent_write()
    _check(case)


def test_tokens_without_a_slot_are_not_written():
    """The last request's page-table entries name pages past the pool, and the
    second-to-last request's last tokens lie past its page table: those tokens
    are skipped, the others are written as the oracle says, and no other byte
    of the pool changes."""
    import dataclasses
    case = W.latent_write_case("lw_noslot", seed=9, seq_lens=[20, 35, 9], start_lengths=[3, 0, 5], page_size=16)
    c = case.cache
    pt = c.page_table.copy()
    pt[2, :] = c.num_pages + 7
    bad = dataclasses.replace(case, cache=dataclasses.replace(c, page_table=pt))
    # request 1: shrink its table so its tokens from position 16 on have no page
    keep = 16
    before, after = run_write(dataclasses.replace(bad, cache=dataclasses.replace(
        bad.cache, page_table=np.where(np.arange(pt.shape[1])[None, :] >= keep // 16,
                                       np.where(np.arange(pt.shape[0])[:, None] == 1, np.uint32(0xFFFFFFFF), pt),
                                       pt).astype(np.uint32))))
    # valid tokens: all of request 0, the first 16 positions of request 1
    iro = case.input_row_offsets.astype(np.int64)
    valid = np.concatenate([np.arange(iro[0], iro[1]), np.arange(iro[1], iro[1] + keep)])
    ref, dst = oracle.latent_write(case)
    ref, dst = ref[valid], dst[valid]
    D = ref.shape[1]
    flat = after.reshape(-1)
    idx = torch.as_tensor(dst, device=after.device)[:, None] + torch.arange(D, device=after.device)[None, :]
    got_rows = flat[idx.reshape(-1)].reshape(len(valid), D)
    expect = before.clone().reshape(-1)
    expect[idx.reshape(-1)] = got_rows.reshape(-1)
    assert torch.equal(expect.view(torch.int16), flat.view(torch.int16)), "bytes outside the valid rows changed"
    got = got_rows.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -24)
