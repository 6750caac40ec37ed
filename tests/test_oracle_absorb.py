"""Pins for the oracle's query absorption (page "mla_prefill_decode_graph_fp8",
Args q and w_uk): latent[t, h, c] = sum_d q[t, h, d] * w_uk[h, c, d] over the
d_nope non-rope columns of each head, the rope columns carried over.

What pins it:
  * selection weights (w_uk[h, c, d] = 1 where d = (c + 3h) % d_nope) return the
    named query columns exactly, so a transposed operand, a wrong head or a
    column taken from the rope part fails;
  * numpy's float64 einsum over the same decoded operands (a library routine
    for the same contraction);
  * swapping two heads' weights swaps exactly those heads' outputs;
  * the rope part is the query's own bits.
"""
import numpy as np

import oracle
import workloads as W


def _dec(bits):
    return oracle.bf16_decode(bits).astype(np.float64)


def test_selection_weights_pick_named_columns():
    c = W.absorb_case("pin", seed=1, T=9, H=5, d_nope=32, d_rope=16, kv_latent_dim=64)
    H, NL, DN = c.H, c.kv_latent_dim, c.d_nope
    w = np.zeros((H, NL, DN), np.float32)
    for h in range(H):
        for col in range(NL):
            w[h, col, (col + 3 * h) % DN] = 1.0
    c.w_uk = W.to_bf16_bits(w)
    lat, rope = oracle.absorb_q(c)
    q = _dec(c.q)
    for h in range(H):
        idx = (np.arange(NL) + 3 * h) % DN
        assert np.array_equal(lat[:, h, :], q[:, h, idx])
    assert np.array_equal(rope, c.q[:, :, DN:])


def test_matches_float64_einsum():
    c = W.absorb_case("pin2", seed=2, T=17, H=6, d_nope=64, d_rope=8, kv_latent_dim=96)
    lat, _ = oracle.absorb_q(c)
    want = np.einsum("thd,hcd->thc", _dec(c.q)[:, :, :c.d_nope], _dec(c.w_uk))
    assert np.allclose(lat, want, rtol=1e-12, atol=1e-12)


def test_heads_are_independent():
    c = W.absorb_case("pin3", seed=3, T=5, H=4, d_nope=32, d_rope=0, kv_latent_dim=32, copy_rope=False)
    a, r = oracle.absorb_q(c)
    assert r is None
    c.w_uk = c.w_uk[[2, 1, 0, 3]].copy()
    b, _ = oracle.absorb_q(c)
    q = _dec(c.q)
    assert np.array_equal(b[:, 1], a[:, 1]) and np.array_equal(b[:, 3], a[:, 3])
    assert not np.array_equal(b[:, 0], a[:, 0])
    # head 0 now uses head 2's weight on head 0's query
    want = q[:, 0, :32] @ _dec(c.w_uk[0]).T
    assert np.allclose(b[:, 0], want, rtol=1e-12, atol=1e-12)


def test_fp8_lossless_queries_match_the_dequantised_product():
    """Query blocks built from e4m3 values with the block maximum at 448 * 2^e
    quantise losslessly; the fp8 form then equals the plain product of the
    queries with the dequantised weight (decoded codes times block scales)."""
    c = W.absorb_case("pin4", seed=4, T=11, H=3, d_nope=128, d_rope=0, kv_latent_dim=256, fp8=True)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7E, size=(c.T, c.H, 128)).astype(np.uint8)
    vals = oracle.e4m3_decode(codes) * np.where(rng.integers(0, 2, size=codes.shape) == 1, 1.0, -1.0)
    vals[..., 7] = 448.0
    vals *= 2.0 ** rng.integers(-8, 2, size=(c.T, c.H, 1))
    c.q = W.to_bf16_bits(vals.astype(np.float32))
    lat, _, qc, qs = oracle.absorb_q_fp8(c)
    assert np.array_equal(oracle.e4m3_decode(qc) * qs.astype(np.float64)[:, :, None], vals)
    w = oracle.e4m3_decode(c.w_q) * np.repeat(c.w_scale.astype(np.float64), 128, axis=1)[:, :, :1]
    want = np.einsum("thd,hcd->thc", vals, w)
    assert np.allclose(lat, want, rtol=1e-12, atol=1e-12)


def test_fp8_selection_weight_returns_the_quantised_queries():
    c = W.absorb_case("pin5", seed=6, T=7, H=4, d_nope=128, d_rope=64, kv_latent_dim=128, fp8=True)
    one = W.to_e4m3_bits(np.ones(1, np.float32))[0]
    c.w_q[:] = 0
    for h in range(c.H):
        c.w_q[h, np.arange(128), (np.arange(128) + 5 * h) % 128] = one
    c.w_scale[:] = 1.0
    lat, rope, qc, qs = oracle.absorb_q_fp8(c)
    deq = oracle.e4m3_decode(qc) * qs.astype(np.float64)[:, :, None]
    for h in range(c.H):
        assert np.array_equal(lat[:, h, :], deq[:, h, (np.arange(128) + 5 * h) % 128])
    assert np.array_equal(rope, c.q[:, :, 128:])
