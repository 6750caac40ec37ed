"""Pins for the oracle's paged gather (page "generic_flare_mla_decompress_k_cache_ragged_paged",
summary and Args buffer_row_offsets_1d / cache_offsets_1d / buffer_length / k_latent_buffer).

None of these re-types the oracle's forward page walk:
  * tagged pools: every element carries (page, layer, kv, slot, col) in its bits;
    the test inverts the page table to recover the logical position and checks
    it equals cache_offset + i (an inverse lookup, not the forward formula);
  * an identity page table over a contiguous pool equals a plain slice;
  * page_size 1 equals torch.index_select over the page ids;
  * the hand-worked example in tests/golden/worked_examples.json;
  * precondition violations are refused.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from caselib import decode_tag, explicit_decompress_case, worked_decompress_case


def _inverse_table(table, num_pages):
    inv = {}
    for b in range(table.shape[0]):
        for lp in range(table.shape[1]):
            pg = int(table[b, lp])
            if pg != W.PAGE_NONE:
                assert pg not in inv, "a physical page is shared"
                inv[pg] = (b, lp)
    return inv


@pytest.mark.parametrize("seed,ps", [(0, 16), (1, 4), (2, 1), (3, 128), (4, 7)])
def test_tagged_gather_recovers_logical_positions(seed, ps):
    rng = np.random.default_rng(seed)
    B = 6
    lens = rng.integers(1, 90, size=B)
    offs = np.array([rng.integers(0, l) for l in lens])
    case = W.decompress_case("tag", seed=seed, cache_lengths=lens, cache_offsets=offs, page_size=ps,
                             kv_lora_rank=24, rope_dim=8, N=16, dtype="f32", fill="tag")
    lat = oracle.gather(case)
    page, layer, kv, slot, col = decode_tag(lat)
    inv = _inverse_table(case.cache.page_table, case.cache.num_pages)
    bro = case.buffer_row_offsets
    assert lat.shape == (case.M, 32)
    assert np.all(layer == case.layer_idx) and np.all(kv == 0)
    assert np.all(col == np.arange(32)[None, :])
    for b in range(B):
        for i in range(bro[b + 1] - bro[b]):
            r = bro[b] + i
            assert len(set(page[r].tolist())) == 1 and len(set(slot[r].tolist())) == 1
            owner, lp = inv[int(page[r, 0])]
            assert owner == b
            assert lp * ps + slot[r, 0] == offs[b] + i


def test_identity_page_table_is_a_contiguous_slice():
    rng = np.random.default_rng(11)
    ps, npg, D, M = 8, 5, 12, 29
    pool = rng.standard_normal((npg, 2, 1, ps, 1, D)).astype(np.float32).view(np.uint32)
    case = explicit_decompress_case(pool, "f32", [list(range(npg))], [npg * ps], [0], [M], 1, D, None, "f32")
    lat = oracle.gather(case)
    flat = pool[:, 1, 0, :, 0, :].reshape(npg * ps, D)
    assert np.array_equal(lat, flat[:M])


def test_page_size_one_is_index_select():
    rng = np.random.default_rng(12)
    npg, D = 40, 10
    pool = rng.standard_normal((npg, 2, 1, 1, 1, D)).astype(np.float32).view(np.uint32)
    perm = rng.permutation(npg)
    lens, offs = [15, 9, 16], [3, 0, 15]
    table = np.full((3, 16), W.PAGE_NONE, np.uint32)
    table[0, :15], table[1, :9], table[2, :16] = perm[:15], perm[15:24], perm[24:40]
    rows = [l - o for l, o in zip(lens, offs)]
    case = explicit_decompress_case(pool, "f32", table, lens, offs, rows, 0, D, None, "f32")
    lat = oracle.gather(case)
    idx = np.concatenate([table[b, offs[b]:lens[b]] for b in range(3)]).astype(np.int64)
    ref = torch.index_select(torch.from_numpy(pool[:, 0, 0, 0, 0, :].view(np.float32)), 0,
                             torch.from_numpy(idx)).numpy()
    assert np.array_equal(lat.view(np.float32), ref)


def test_worked_example_gather():
    case, k_latent, _ = worked_decompress_case()
    lat = oracle.gather(case)
    assert np.array_equal(lat.view(np.float32), k_latent)


def test_bf16_gather_is_bit_copy_with_nan_payloads():
    # rows carrying NaN payloads and signed zeros must come through bit for bit
    rng = np.random.default_rng(13)
    ps, npg, D = 4, 6, 8
    pool = rng.integers(0, 65536, size=(npg, 1, 1, ps, 1, D), dtype=np.uint16)
    pool[0, 0, 0, 0, 0, :4] = [0x7FC1, 0xFFFF, 0x8000, 0x7F80]
    table = [[0, 3, 5]]
    case = explicit_decompress_case(pool, "bf16", table, [12], [0], [12], 0, D, None, "bf16")
    lat = oracle.gather(case)
    ref = pool[[0, 3, 5], 0, 0, :, 0, :].reshape(12, D)
    assert np.array_equal(lat, ref)


def test_empty_requests_and_empty_batch():
    case = W.decompress_case("z", seed=0, cache_lengths=[5, 7, 3], cache_offsets=[5, 0, 3],
                             page_size=4, kv_lora_rank=8, rope_dim=0, N=8, dtype="f32")
    assert case.M == 7
    lat = oracle.gather(case)
    direct = oracle.gather(W.decompress_case("z1", seed=0, cache_lengths=[5, 7, 3], cache_offsets=[5, 0, 3],
                                             page_size=4, kv_lora_rank=8, rope_dim=0, N=8, dtype="f32"))
    assert np.array_equal(lat, direct)
    none = W.decompress_case("z2", seed=0, cache_lengths=[5], cache_offsets=[5], page_size=4,
                             kv_lora_rank=8, rope_dim=0, N=8, dtype="f32")
    assert oracle.gather(none).shape == (0, 8)


def test_preconditions_are_refused():
    case = W.decompress_case("p", seed=0, cache_lengths=[10, 10], cache_offsets=[0, 2], page_size=4,
                             kv_lora_rank=8, rope_dim=0, N=8, dtype="f32")
    bad = case.buffer_row_offsets.copy()
    bad[1] = 12  # decreasing
    case_bad = W.DecompressCase(**{**case.__dict__, "buffer_row_offsets": bad})
    with pytest.raises(oracle.OracleError):
        oracle.gather(case_bad)
    # reading past the cached length
    longer = case.buffer_row_offsets.copy()
    longer[2] += 1
    with pytest.raises(oracle.OracleError):
        oracle.gather(W.DecompressCase(**{**case.__dict__, "buffer_row_offsets": longer}))
    # a page id outside the pool
    cache = case.cache
    table = cache.page_table.copy()
    table[0, 0] = cache.num_pages
    bad_cache = W.PagedCache(cache.pool, cache.dtype, table, cache.cache_lengths, cache.used_pages)
    with pytest.raises(oracle.OracleError):
        oracle.gather(W.DecompressCase(**{**case.__dict__, "cache": bad_cache}))
    # layer out of range
    with pytest.raises(oracle.OracleError):
        oracle.gather(W.DecompressCase(**{**case.__dict__, "layer_idx": 2}))
