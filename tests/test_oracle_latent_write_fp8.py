"""Pins for the oracle's latent write into an e4m3 cache (page
"mla_prefill_decode_graph_fp8", Args kv_input_fn, kv_norm_gamma, epsilon,
freqs_cis; the collection's scale_dtype_ fp32 and quantization_granularity_ 128
of page "generic_flare_mla_decompress_k_cache_ragged_paged"): the binary32 row
values quantised per 128-column block, and where codes and scales go.

What pins it, none of it a re-typing of the oracle's loops:
  * exactness: a block of e4m3 grid values times 2^e whose largest magnitude is
    448 * 2^e quantises losslessly, with scale 2^e;
  * an all-zero block has scale 1 and codes 0; a block's largest magnitude maps
    onto the code of +-448; a short last block is quantised on its own;
  * the e4m3 error bound: every decoded value is within half a step of its
    input (2^-4 relative in the normal range, 2^-10 * scale below it);
  * placement: on a tagged e4m3 cache, every token's scale offsets hold the tag
    of (page_table[b][p / page_size], layer, slot p % page_size, block), worked
    out here from the page table, not from the oracle's offsets.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _grid_block(rng, n, e):
    """n values from the e4m3 grid (normal and subnormal), times 2^e, with +-448 * 2^e among them."""
    codes = rng.integers(0, 256, size=n).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00          # no NaN codes
    vals = oracle.e4m3_decode(codes).astype(np.float64)
    vals[rng.integers(0, n)] = 448.0 if rng.integers(0, 2) else -448.0
    return (vals * 2.0 ** e).astype(np.float32)


@pytest.mark.parametrize("D,exps", [(256, (-3, 2)), (192, (0, -7)), (576, (1, -2, 0, -5, 3))])
def test_grid_rows_quantise_losslessly(D, exps):
    rng = np.random.default_rng(D)
    nb = -(-D // 128)
    assert len(exps) == nb
    Y = np.concatenate([_grid_block(rng, min(128, D - 128 * j), exps[j]) for j in range(nb)])[None, :]
    q, s = oracle.quantize_f32_rows(Y)
    np.testing.assert_array_equal(s[0], np.float32(2.0) ** np.array(exps, np.float32))
    back = oracle.e4m3_decode(q[0]).astype(np.float64) * np.repeat(s[0].astype(np.float64), 128)[:D]
    np.testing.assert_array_equal(back, Y[0].astype(np.float64))


def test_zero_block_and_short_last_block():
    Y = np.zeros((2, 192), np.float32)
    Y[1, 128:] = np.linspace(-3.0, 5.0, 64, dtype=np.float32)
    q, s = oracle.quantize_f32_rows(Y)
    assert s.shape == (2, 2)
    np.testing.assert_array_equal(s[0], [1.0, 1.0])
    assert not q[0].any() and not q[1, :128].any() and s[1, 0] == 1.0
    # the short block's largest magnitude (5) is the code of +448
    assert q[1, 191] == 0x7E and oracle.e4m3_decode(q[1, 191:192])[0] * s[1, 1] == pytest.approx(5.0, rel=1e-6)


def test_error_bound_on_random_rows():
    rng = np.random.default_rng(3)
    Y = (rng.standard_normal((64, 576)) * np.exp(rng.uniform(-6, 6, size=(64, 1)))).astype(np.float32)
    Y[:, 5] *= 1e-4   # values far below the block's amax, into the subnormal codes
    q, s = oracle.quantize_f32_rows(Y)
    scale = np.repeat(s.astype(np.float64), 128, axis=1)[:, :576]
    back = oracle.e4m3_decode(q).astype(np.float64) * scale
    err = np.abs(back - Y.astype(np.float64))
    assert np.all(err <= 2.0 ** -4 * np.abs(Y) + 2.0 ** -10 * scale + 1e-12 * scale)
    # every block's largest magnitude lands on +-448
    for j in range(5):
        blk = np.abs(Y[:, 128 * j:128 * (j + 1)])
        i = blk.argmax(axis=1)
        assert np.all((q[np.arange(64), 128 * j + i] & 0x7F) == 0x7E)


def test_fp8_write_values_and_placement_on_a_tagged_cache():
    c = W.latent_write_case("pin8", seed=4, seq_lens=[3, 0, 5, 2], start_lengths=[2, 7, 0, 9], page_size=4,
                            K=256, R=64, dtype="e4m3", fill="tag")
    q, s, ref, dst, sdst = oracle.latent_write_fp8(c)
    assert q.shape == (c.T, 320) and s.shape == (c.T, 3)
    # values: within the e4m3 bound of the binary64 write-path values
    scale = np.repeat(s.astype(np.float64), 128, axis=1)[:, :320]
    back = oracle.e4m3_decode(q).astype(np.float64) * scale
    assert np.all(np.abs(back - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * scale + 1e-6 * np.abs(ref))
    # placement from the page table: scales of (page, layer, slot) carry tag page*65536 + layer*32768 + slot*64 + j
    iro = c.input_row_offsets.astype(np.int64)
    flat = c.cache.scales.reshape(-1)
    for b in range(len(iro) - 1):
        for i in range(iro[b + 1] - iro[b]):
            t, p = iro[b] + i, int(c.cache.cache_lengths[b]) + i
            page, slot = int(c.cache.page_table[b, p // 4]), p % 4
            tags = page * 65536 + c.layer_idx * 32768 + slot * 64 + np.arange(3)
            np.testing.assert_array_equal(flat[sdst[t] + np.arange(3)], tags.astype(np.float32))
    assert len(set(sdst.tolist())) == c.T
