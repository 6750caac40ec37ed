"""Pins for the oracle's latent write path (page "mla_prefill_decode_graph_fp8",
Args kv_input_fn, kv_norm_gamma, epsilon, freqs_cis, input_row_offsets,
kv_collection): RMSNorm of the latent part, rotation of the rope part, and the
token's destination row.

What pins it, none of it a re-typing of the oracle's loops:
  * closed forms of RMSNorm: a constant row normalises to gamma * sign (eps = 0)
    and to gamma * c / sqrt(c^2 + eps) otherwise; with gamma = 1 and eps = 0
    every output row has a sum of squares of exactly K;
  * rotations: (1, 0) leaves a pair unchanged, (0, 1) maps (x0, x1) to
    (-x1, x0), any angle keeps the pair's length and adds its angle;
  * the position of each token (cached length + index within the request)
    selects the rope row: with angle = position * a, the rotation seen on
    token t is pos(t) * a;
  * the destination is the write path's K-half row of that position (pinned by
    the kv write-path tests) and differs for every token.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _case(seq_lens=(3, 0, 5, 2), starts=(2, 7, 0, 9), ps=4, K=64, R=16, eps=1e-6, seed=1):
    return W.latent_write_case("pin", seed=seed, seq_lens=list(seq_lens), start_lengths=list(starts), page_size=ps,
                               K=K, R=R, eps=eps)


def _positions(c):
    iro = c.input_row_offsets.astype(np.int64)
    cl = c.cache.cache_lengths.astype(np.int64)
    return np.concatenate([cl[b] + np.arange(iro[b + 1] - iro[b]) for b in range(len(iro) - 1)])


@pytest.mark.parametrize("cval", [1.5, -0.375, 3.0])
def test_constant_rows_normalise_to_gamma_times_sign(cval):
    c = _case(eps=0.0)
    c.x[:, :c.K] = W.to_bf16_bits(np.full((c.T, c.K), cval, np.float32))
    v, _ = oracle.latent_write(c)
    assert np.array_equal(v[:, :c.K], np.broadcast_to(c.gamma.astype(np.float64) * np.sign(cval), (c.T, c.K)))
    c.eps = 0.25
    v, _ = oracle.latent_write(c)
    want = c.gamma.astype(np.float64) * cval / np.sqrt(cval * cval + 0.25)
    assert np.allclose(v[:, :c.K], want[None, :], rtol=1e-15, atol=0)


def test_unit_gamma_rows_have_sum_of_squares_k():
    c = _case(eps=0.0)
    c.gamma[:] = 1.0
    v, _ = oracle.latent_write(c)
    assert np.allclose((v[:, :c.K] ** 2).sum(1), c.K, rtol=1e-13, atol=0)


def test_rotations():
    c = _case()
    x = oracle.bf16_decode(c.x).astype(np.float64)
    R = c.freqs.shape[1]
    c.freqs[:, 0::2], c.freqs[:, 1::2] = 1.0, 0.0
    v, _ = oracle.latent_write(c)
    assert np.array_equal(v[:, c.K:], x[:, c.K:])
    c.freqs[:, 0::2], c.freqs[:, 1::2] = 0.0, 1.0
    v, _ = oracle.latent_write(c)
    assert np.array_equal(v[:, c.K::2], -x[:, c.K + 1::2]) and np.array_equal(v[:, c.K + 1::2], x[:, c.K::2])
    # angle = position * a (one rate for every pair): each pair turns by pos(t) * a, length kept
    a = 0.0625
    n = c.freqs.shape[0]
    ang = np.arange(n, dtype=np.float64) * a
    c.freqs[:, 0::2] = np.cos(ang)[:, None]
    c.freqs[:, 1::2] = np.sin(ang)[:, None]
    v, _ = oracle.latent_write(c)
    pos = _positions(c)
    x0, x1 = x[:, c.K::2], x[:, c.K + 1::2]
    y0, y1 = v[:, c.K::2], v[:, c.K + 1::2]
    assert np.allclose(np.hypot(y0, y1), np.hypot(x0, x1), rtol=1e-7)
    turn = np.angle((y0 + 1j * y1) / (x0 + 1j * x1))
    want = np.angle(np.exp(1j * (pos * a)))[:, None].astype(np.float32).astype(np.float64)
    assert np.allclose(turn, np.broadcast_to(want, turn.shape), atol=1e-6)
    assert R == 16


def test_destinations_are_the_write_path_rows():
    c = _case(ps=1)
    _, dst = oracle.latent_write(c)
    assert len(set(dst.tolist())) == c.T
    cc = c.cache
    sp, sl, skv, st = cc.strides()
    pos = _positions(c)
    b_of = np.repeat(np.arange(len(c.input_row_offsets) - 1), np.diff(c.input_row_offsets.astype(np.int64)))
    for t in range(c.T):
        pg = cc.page_table[b_of[t], pos[t] // cc.page_size]
        assert dst[t] == pg * sp + c.layer_idx * sl + (pos[t] % cc.page_size) * st


def test_position_past_the_rope_table_is_refused():
    c = _case()
    c.freqs = c.freqs[:3]
    with pytest.raises(oracle.OracleError):
        oracle.latent_write(c)
