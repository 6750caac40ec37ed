"""GPU parity of kv_matmul_paged against the CPU oracle.

Written K/V rows must be within 1e-2 * max|ref| of the oracle's product at the
slots the oracle's destinations name; every other element of the pool (other
layer, other kv half, cached tokens, spare pages, slack slots) must be
bit-identical to its value before the call.  A selection weight turns the
product into a copy, so placement is checked bit-exactly.
"""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import BF16_TOL, check_close, say

pytestmark = pytest.mark.gpu


def run_kv(case):
    dc, t = W.device_kv(case)
    before = dc.pool.clone()
    say(f"[gpu] {case.name}: T={case.T} hidden={case.hidden_dim} N={case.N}")
    mp.kv_matmul_paged(t["hidden"], t["input_row_offsets"], t["weight"],
                       mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths), case.layer_idx)
    torch.cuda.synchronize()
    return before, dc.pool


def _written_rows(pool, dst, HD):
    """[T, 2*HD] of the rows the oracle names, gathered from a device pool."""
    flat = pool.reshape(-1)
    idx = torch.as_tensor(dst.reshape(-1), device=pool.device)[:, None] + torch.arange(HD, device=pool.device)[None, :]
    return flat[idx.reshape(-1)].reshape(dst.shape[0], 2 * HD)


def _check(case, rows=None):
    before, after = run_kv(case)
    dst = oracle.kv_destinations(case)
    HD = case.cache.num_heads * case.cache.head_dim
    got_rows = _written_rows(after, dst, HD)
    # nothing else changed
    expect = before.clone().reshape(-1)
    idx = torch.as_tensor(dst.reshape(-1), device=after.device)[:, None] + torch.arange(HD, device=after.device)[None, :]
    expect[idx.reshape(-1)] = got_rows.reshape(-1)
    assert torch.equal(expect.view(torch.int16), after.reshape(-1).view(torch.int16)), "bytes outside the written slots changed"
    assert bool(torch.isfinite(got_rows).all()), "a token's K/V row was not written"
    sel = np.arange(case.T) if rows is None else rows
    ref = oracle.matmul_nn(case.hidden, case.weight, sel)
    got = got_rows[torch.as_tensor(sel, device=after.device)].double().cpu().numpy()
    check_close(got, ref, BF16_TOL, f"{case.name} written K/V rows")
    return got_rows, dst


@pytest.mark.parametrize("seed,ps,start", [(0, 16, "random"), (1, 128, "zero"), (2, 3, "random")])
def test_small_kv_full_compare(seed, ps, start):
    case = W.small_kv_matmul(seed, batch=6, max_len=300, hidden_dim=256, num_kv_heads=2, head_dim=128,
                             page_size=ps, start=start)
    _check(case)


def test_selection_weight_places_hidden_columns_exactly():
    rng = np.random.default_rng(3)
    Kd, H, D = 512, 2, 128
    N = 2 * H * D
    perm = rng.permutation(Kd)[:N]
    sel = np.zeros((Kd, N), np.float32)
    sel[perm, np.arange(N)] = 1.0
    base = W.small_kv_matmul(4, batch=5, max_len=200, hidden_dim=Kd, num_kv_heads=H, head_dim=D, page_size=16)
    case = W.KvMatmulCase(base.name, base.cache, base.layer_idx, base.hidden, base.input_row_offsets,
                          W.to_bf16_bits(sel))
    got_rows, dst = _check(case)
    bits = got_rows.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits, case.hidden[:, perm])


@pytest.mark.slow
def test_c4_full_size_sampled():
    case = W.c4_kv_matmul()
    rng = np.random.default_rng(0)
    iro = case.input_row_offsets.astype(np.int64)
    rows = set(iro[:-1].tolist()) | set((iro[1:] - 1).tolist()) | set(rng.integers(0, case.T, 512).tolist())
    _check(case, np.array(sorted(rows), np.int64))


@pytest.mark.slow
def test_c4_with_cached_prefix_sampled():
    case = W.c4_kv_matmul(start="random")
    rng = np.random.default_rng(1)
    _check(case, np.sort(rng.choice(case.T, 400, replace=False)))


@pytest.mark.parametrize("hidden,heads,dim", [(192, 1, 128), (384, 4, 64), (1024, 2, 256)])
def test_kv_other_shapes(hidden, heads, dim):
    """Shapes off the 256-column / 128-deep tiling (hidden 192, HD 128) take the
    general kernel; HD 256 and 512 with hidden 384 / 1024 the pipelined one."""
    case = W.small_kv_matmul(7, batch=5, max_len=350, hidden_dim=hidden, num_kv_heads=heads, head_dim=dim,
                             page_size=32, start="random")
    _check(case)


def _check_subset(case, before, after, T1):
    """The first T1 tokens were written as the oracle says; nothing else changed."""
    import dataclasses
    c = case.cache
    B1 = int(np.searchsorted(case.input_row_offsets, T1, side="left"))
    trunc = dataclasses.replace(case, hidden=case.hidden[:T1], input_row_offsets=case.input_row_offsets[:B1 + 1],
                                cache=dataclasses.replace(c, page_table=np.ascontiguousarray(c.page_table[:B1]),
                                                          cache_lengths=np.ascontiguousarray(c.cache_lengths[:B1])))
    dst = oracle.kv_destinations(trunc)
    HD = c.num_heads * c.head_dim
    got_rows = _written_rows(after, dst, HD)
    expect = before.clone().reshape(-1)
    idx = torch.as_tensor(dst.reshape(-1), device=after.device)[:, None] + torch.arange(HD, device=after.device)[None, :]
    expect[idx.reshape(-1)] = got_rows.reshape(-1)
    assert torch.equal(expect.view(torch.int16), after.reshape(-1).view(torch.int16)), \
        "bytes outside the valid tokens' slots changed"
    ref = oracle.matmul_nn(case.hidden, case.weight, np.arange(T1))
    check_close(got_rows.double().cpu().numpy(), ref, BF16_TOL, f"{case.name} valid tokens")


@pytest.mark.parametrize("how", ["past_page_table", "page_past_pool"])
@pytest.mark.parametrize("ring", [True, False])
def test_tokens_without_a_slot_are_not_written(how, ring):
    """The last request's tokens have no slot: their positions lie past its page
    table, or its page-table entries name pages past the pool.  They are
    skipped; the other requests' tokens land as usual and no other byte of the
    pool changes (the ring kernel at hidden 256, the general one at hidden 192)."""
    import dataclasses
    hidden = 256 if ring else 192
    case = W.small_kv_matmul(8, batch=4, max_len=120, hidden_dim=hidden, num_kv_heads=2, head_dim=128,
                             page_size=16)
    c = case.cache
    B = len(case.input_row_offsets) - 1
    pt, cl = c.page_table.copy(), c.cache_lengths.copy()
    if how == "past_page_table":
        cl[B - 1] = c.max_pages_per_seq * c.page_size
    else:
        pt[B - 1, :] = c.num_pages + 3
    bad = dataclasses.replace(case, cache=dataclasses.replace(c, page_table=pt, cache_lengths=cl))
    before, after = run_kv(bad)
    _check_subset(bad, before, after, int(case.input_row_offsets[B - 1]))


def test_written_k_rows_decompress_back():
    """kv_matmul_paged, then mla_decompress_k_paged over the K half of the cache
    (viewed as one 1024-wide latent head per token) at the written positions
    with an identity weight: both the gathered rows and k_buffer equal the K
    rows the write path stored, bit for bit."""
    case = W.small_kv_matmul(9, batch=5, max_len=150, hidden_dim=512, num_kv_heads=8, head_dim=128,
                             page_size=16)
    dc, t = W.device_kv(case)
    say(f"[gpu] kv round trip: T={case.T}")
    mp.kv_matmul_paged(t["hidden"], t["input_row_offsets"], t["weight"],
                       mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths), case.layer_idx)
    torch.cuda.synchronize()
    P, Ly, _, ps, H, D = dc.pool.shape
    HD = H * D
    khalf = dc.pool[:, :, 0:1].view(P, Ly, 1, ps, 1, HD)
    M = case.T
    lat = torch.empty((M, HD), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, HD), dtype=torch.bfloat16, device="cuda")
    eye = torch.eye(HD, dtype=torch.float32).to(torch.bfloat16).cuda()
    co = dc.cache_lengths.clone()
    mp.mla_decompress_k_paged(t["input_row_offsets"], co, M, eye, mp.PagedKVCache(khalf, dc.page_table, None),
                              case.layer_idx, lat, out)
    torch.cuda.synchronize()
    dst = oracle.kv_destinations(case)
    krows = _written_rows(dc.pool, dst, HD)[:, :HD]
    assert torch.equal(lat.view(torch.int16), krows.contiguous().view(torch.int16)), "gathered rows differ"
    assert torch.equal(out.view(torch.int16), krows.contiguous().view(torch.int16)), "k_buffer differs"
    ref = oracle.matmul_nn(case.hidden, case.weight, np.arange(M))[:, :HD]
    check_close(out.double().cpu().numpy(), ref, BF16_TOL, "round trip K rows")
