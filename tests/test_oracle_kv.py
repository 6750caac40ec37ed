"""Pins for the oracle's write path (page "kv_matmul_ragged_paged", summary and
Args hidden_state, input_row_offsets, weight, kv_collection, layer_idx).

  * the product against numpy float64 matmul;
  * the hand-worked example (tests/golden/worked_examples.json);
  * destinations checked by inverse page lookup: each token lands in a page
    its own request owns, at logical position cache_length + i, in the right
    layer, with K and V one kv stride apart; all destinations distinct;
  * a selection weight makes the emulated cache write reproduce hidden
    columns [0, N/2) in the K rows and [N/2, N) in the V rows.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from caselib import elem_f64, worked_kv_case


def test_matmul_nn_matches_numpy_float64():
    rng = np.random.default_rng(41)
    T, Kd, N = 29, 96, 64
    h = W.to_bf16_bits(rng.standard_normal((T, Kd)).astype(np.float32))
    w = W.to_bf16_bits(rng.standard_normal((Kd, N)).astype(np.float32))
    out = oracle.matmul_nn(h, w)
    ref = elem_f64(h, "bf16") @ elem_f64(w, "bf16")
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_worked_example_write_path():
    case, written = worked_kv_case()
    out, dst = oracle.kv_matmul(case)
    c = case.cache
    sp, sl, skv, st = c.strides()
    for w in written:
        t = w["token"]
        assert out[t].tolist() == [w["K"], w["V"]]
        base = w["page"] * sp + case.layer_idx * sl + w["slot"] * st
        assert dst[t].tolist() == [base, base + skv]


def _inverse(table):
    inv = {}
    for b in range(table.shape[0]):
        for lp in range(table.shape[1]):
            if table[b, lp] != W.PAGE_NONE:
                inv[int(table[b, lp])] = (b, lp)
    return inv


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_destinations_by_inverse_lookup(seed):
    case = W.small_kv_matmul(seed, batch=7, max_len=70, hidden_dim=32, num_kv_heads=2, head_dim=16,
                             page_size=8)
    dst = oracle.kv_destinations(case)
    c = case.cache
    sp, sl, skv, st = c.strides()
    inv = _inverse(c.page_table)
    assert len(set(dst.reshape(-1).tolist())) == dst.size
    assert np.all(dst[:, 1] - dst[:, 0] == skv)
    iro = case.input_row_offsets
    for b in range(len(iro) - 1):
        for i, t in enumerate(range(iro[b], iro[b + 1])):
            o = int(dst[t, 0])
            page, rem = divmod(o, sp)
            layer, rem = divmod(rem, sl)
            kv, rem = divmod(rem, skv)
            slot, col = divmod(rem, st)
            assert (layer, kv, col) == (case.layer_idx, 0, 0)
            owner, lp = inv[page]
            assert owner == b and lp * c.page_size + slot == c.cache_lengths[b] + i


def test_selection_weight_write_reproduces_hidden_columns():
    rng = np.random.default_rng(42)
    Kd, H, D = 64, 2, 16
    N = 2 * H * D
    sel = np.zeros((Kd, N), np.float32)
    perm = rng.permutation(Kd)[:N]
    sel[perm, np.arange(N)] = 1.0
    case = W.small_kv_matmul(5, batch=4, max_len=40, hidden_dim=Kd, num_kv_heads=H, head_dim=D, page_size=8)
    case = W.KvMatmulCase(case.name, case.cache, case.layer_idx, case.hidden, case.input_row_offsets,
                          W.to_bf16_bits(sel))
    out, dst = oracle.kv_matmul(case)
    pool = case.cache.pool.reshape(-1).copy()
    before = pool.copy()
    written = W.to_bf16_bits(out.astype(np.float32))  # exact: out holds bf16 values
    for t in range(case.T):
        pool[dst[t, 0]:dst[t, 0] + H * D] = written[t, :H * D]
        pool[dst[t, 1]:dst[t, 1] + H * D] = written[t, H * D:]
    for t in range(case.T):
        assert np.array_equal(pool[dst[t, 0]:dst[t, 0] + H * D], case.hidden[t, perm[:H * D]])
        assert np.array_equal(pool[dst[t, 1]:dst[t, 1] + H * D], case.hidden[t, perm[H * D:]])
    # every written slot was poison before (appended after the cached tokens)
    for t in range(case.T):
        assert np.all(before[dst[t, 0]:dst[t, 0] + H * D] == W.POISON_BF16)


def test_missing_page_is_refused():
    case = W.small_kv_matmul(3, batch=3, max_len=30, hidden_dim=32, num_kv_heads=1, head_dim=16, page_size=8)
    c = case.cache
    table = c.page_table.copy()
    b = int(np.argmax((table != W.PAGE_NONE).sum(1)))
    last = int((table[b] != W.PAGE_NONE).sum()) - 1
    table[b, last] = W.PAGE_NONE
    bad = W.PagedCache(c.pool, c.dtype, table, c.cache_lengths, c.used_pages)
    with pytest.raises(oracle.OracleError):
        oracle.kv_destinations(W.KvMatmulCase(case.name, bad, case.layer_idx, case.hidden,
                                              case.input_row_offsets, case.weight))
