"""GPU parity of mla_absorb_q (per-head product of the non-rope query columns
with w_uk, the rope columns carried over) against the CPU oracle.

The latent part is a bf16 product with fp32 accumulation over 128 terms: within
1e-2 * max|ref| of the oracle's binary64 sum (the bf16 product bound); the rope
part is a bit copy.  Outputs are over-allocated by poisoned tokens that must
keep their bits.
"""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import BF16_TOL, POISON_OUT, check_close, check_guards, guarded_empty, say, to_bits

pytestmark = pytest.mark.gpu


def _run(case, extra=3):
    t = W.device_absorb(case)
    T, H = case.T, case.H
    buf = guarded_empty((T + extra, H, case.out_dim), torch.bfloat16)
    buf.view(torch.int16).fill_(POISON_OUT)
    say(f"[gpu] {case.name}: T={T} H={H} L={case.kv_latent_dim} rope={case.d_rope} copy={case.copy_rope}")
    mp.mla_absorb_q(t["q"], t["w_uk"], buf[:T], d_nope=case.d_nope, copy_rope=case.copy_rope)
    check_guards(case.name)
    return buf


def _check(case, extra=3):
    buf = _run(case, extra)
    T, NL = case.T, case.kv_latent_dim
    lat, rope = oracle.absorb_q(case)
    got = buf[:T, :, :NL].double().cpu().numpy()
    check_close(got.reshape(T, -1), lat.reshape(T, -1), BF16_TOL, f"{case.name} q_latent")
    bits = to_bits(buf)
    if case.copy_rope:
        assert np.array_equal(bits[:T, :, NL:], rope)
    assert np.all(bits[T:] == POISON_OUT)
    return buf


@pytest.mark.parametrize("T,H,L,dr", [(1, 8, 512, 64), (128, 16, 512, 64), (129, 3, 256, 64), (300, 9, 128, 32),
                                      (64, 128, 512, 64)])
def test_full_compare(T, H, L, dr):
    _check(W.absorb_case(f"ab_{T}_{H}_{L}_{dr}", seed=T + H, T=T, H=H, kv_latent_dim=L, d_rope=dr))


def test_without_rope_copy_and_without_rope():
    _check(W.absorb_case("ab_nocopy", seed=40, T=77, H=5, copy_rope=False))
    _check(W.absorb_case("ab_norope", seed=41, T=33, H=4, d_rope=0))


def test_many_chunks():
    """Prefill-sized T: several 128-row chunks per block, with a ragged last one."""
    _check(W.absorb_case("ab_long", seed=42, T=1000, H=12, kv_latent_dim=512), extra=0)


def test_selection_weight_is_exact():
    """w_uk[h, c, d] = 1 where d = (c + 3h) % 128: every latent output is a query
    value, exactly (one nonzero term)."""
    c = W.absorb_case("ab_sel", seed=43, T=50, H=10, kv_latent_dim=256)
    w = np.zeros((c.H, c.kv_latent_dim, 128), np.float32)
    for h in range(c.H):
        w[h, np.arange(c.kv_latent_dim), (np.arange(c.kv_latent_dim) + 3 * h) % 128] = 1.0
    c.w_uk = W.to_bf16_bits(w)
    buf = _check(c)
    lat, _ = oracle.absorb_q(c)
    assert np.array_equal(buf[:c.T, :, :c.kv_latent_dim].double().cpu().numpy(), lat)


def test_c7_decode_batch():
    _check(W.c7_absorb(), extra=0)


def _check_fp8(case, extra=3):
    t = W.device_absorb(case)
    T, H, NL = case.T, case.H, case.kv_latent_dim
    buf = guarded_empty((T + extra, H, case.out_dim), torch.bfloat16)
    buf.view(torch.int16).fill_(POISON_OUT)
    say(f"[gpu] {case.name} fp8: T={T} H={H} L={NL} rope={case.d_rope} copy={case.copy_rope}")
    mp.mla_absorb_q_fp8(t["q"], t["w_uk_e4m3"], t["w_uk_scale"], buf[:T], d_nope=case.d_nope,
                        copy_rope=case.copy_rope)
    check_guards(case.name + " fp8")
    lat, rope, _, _ = oracle.absorb_q_fp8(case)
    got = buf[:T, :, :NL].double().cpu().numpy()
    check_close(got.reshape(T, -1), lat.reshape(T, -1), BF16_TOL, f"{case.name} q_latent fp8")
    bits = to_bits(buf)
    if case.copy_rope:
        assert np.array_equal(bits[:T, :, NL:], rope)
    assert np.all(bits[T:] == POISON_OUT)
    return buf


@pytest.mark.parametrize("T,H,L,dr", [(1, 8, 512, 64), (128, 16, 512, 64), (129, 3, 256, 64), (300, 9, 128, 32)])
def test_fp8_full_compare(T, H, L, dr):
    _check_fp8(W.absorb_case(f"abf_{T}_{H}_{L}_{dr}", seed=100 + T + H, T=T, H=H, kv_latent_dim=L, d_rope=dr,
                             fp8=True))


def test_fp8_zero_query_blocks_and_no_rope_copy():
    c = W.absorb_case("abf_zero", seed=130, T=40, H=5, kv_latent_dim=256, copy_rope=False, fp8=True)
    c.q[3, 2, :128] = 0          # an all-zero block: scale 1, codes 0, output 0
    c.q[7, :, :128] = 0
    buf = _check_fp8(c)
    assert torch.all(buf[3, 2, :256].float() == 0) and torch.all(buf[7, :, :256].float() == 0)


def test_fp8_lossless_queries_match_the_dequantised_bf16_form():
    """Query blocks that quantise losslessly (e4m3 values with the block maximum
    at 448 * 2^e) give the product of the queries with the dequantised weight."""
    c = W.absorb_case("abf_lossless", seed=131, T=70, H=6, kv_latent_dim=384, fp8=True)
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 0x7E, size=(c.T, c.H, 128)).astype(np.uint8)
    vals = oracle.e4m3_decode(codes) * np.where(rng.integers(0, 2, size=codes.shape) == 1, 1.0, -1.0)
    vals[..., 0] = 448.0
    vals *= 2.0 ** rng.integers(-8, 2, size=(c.T, c.H, 1))
    c.q[:, :, :128] = W.to_bf16_bits(vals.astype(np.float32))
    buf = _check_fp8(c)
    w = oracle.e4m3_decode(c.w_q) * np.repeat(c.w_scale.astype(np.float64), 128, axis=1)[:, :, :1]
    plain = np.einsum("thd,hcd->thc", vals, w)
    check_close(buf[:c.T, :, :384].double().cpu().numpy().reshape(c.T, -1), plain.reshape(c.T, -1), BF16_TOL,
                "lossless fp8 queries vs dequantised product")


def test_fp8_many_chunks_and_c7_shape():
    _check_fp8(W.absorb_case("abf_long", seed=132, T=700, H=10, fp8=True), extra=0)
    _check_fp8(W.c7_absorb_fp8(), extra=0)
