"""Pins for the oracle's number formats (bf16 decode, e4m3fn decode and encode).

Each is checked against something other than the oracle: torch's own casts
(exhaustively where the domain is small) and hand-worked points of the OCP
OFP8 E4M3 definition (tests/golden/e4m3_points.txt).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from caselib import GOLDEN


def test_bf16_decode_all_65536_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_decode(bits).view(np.uint32)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def _golden_points():
    pts = []
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, code, kind = line.split()[:3]
            pts.append((float(v), int(code, 16), kind))
    return pts


def test_e4m3_hand_worked_points():
    pts = _golden_points()
    vals = np.array([p[0] for p in pts], np.float32)
    codes = np.array([p[1] for p in pts], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    exact = np.array([p[2] == "exact" for p in pts])
    dec = oracle.e4m3_decode(codes[exact])
    assert np.array_equal(dec, vals[exact].astype(np.float64))


def test_e4m3_encode_matches_torch_on_every_midpoint_and_random_values():
    # every finite non-negative value, every midpoint between neighbours (ties),
    # points a hair either side of each midpoint, and random values, both signs,
    # inside the non-saturating range where torch's cast is round-to-nearest-even
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    eps = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(0, 2 ** -5, 20000),
                          rng.uniform(0, 460, 20000)])
    x = np.concatenate([vals, mids, eps, rnd]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < 464]
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_nan():
    x = np.array([448.0, 449.0, 463.9, 464.0, 465.0, 1e6, np.inf, -np.inf, np.nan], np.float32)
    out = oracle.e4m3_encode(x)
    assert out.tolist()[:6] == [0x7E] * 6
    assert out[6] == 0x7E and out[7] == 0xFE and out[8] == 0x7F


def test_e4m3_roundtrip_of_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
