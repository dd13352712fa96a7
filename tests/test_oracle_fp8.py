"""Pins for the oracle's OCP E4M3FN codec (CPU only).

The codec is pinned to torch's float8_e4m3fn conversion (a library routine,
round-to-nearest-even but non-saturating: it is compared only where the two
formats agree, |x| <= 464), to the OCP table points in
tests/golden/ocp_e4m3fn_points.json, and to exhaustive round trips.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3fn_points.json")


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_all_256_codes():
    ours = fp8_e4m3.decode(np.arange(256, dtype=np.uint8))
    ref = torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # sign of zero too
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_ocp_table_points():
    pts = json.load(open(GOLDEN))["points"]
    for p in pts:
        c = int(p["code"], 16)
        v = fp8_e4m3.decode_code(c)
        if p["value"] == "nan":
            assert np.isnan(v)
        else:
            assert v == p["value"] and np.signbit(v) == np.signbit(p["value"])


def test_roundtrip_every_finite_code():
    for c in range(256):
        v = fp8_e4m3.decode_code(c)
        if np.isnan(v):
            continue
        assert int(fp8_e4m3.encode(np.array([v]))[0]) == c, hex(c)


def test_encode_matches_torch_rne_within_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-464, 464, 200000).astype(np.float32),
        (rng.standard_normal(100000) * 1e-2).astype(np.float32),
        np.float32([464.0, -464.0, 463.99997, 0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11]),
    ]).astype(np.float32)
    ours = fp8_e4m3.encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_every_midpoint_ties_to_even():
    vals = fp8_e4m3.DECODE_TABLE[:0x7F]
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2.0          # exact in fp64
        want = c if c % 2 == 0 else c + 1
        assert int(fp8_e4m3.encode(np.array([mid]))[0]) == want
        assert int(fp8_e4m3.encode(np.array([-mid]))[0]) == want | 0x80
        # one fp64 ulp either side of the midpoint decides by distance
        lo, hi = np.nextafter(mid, -np.inf), np.nextafter(mid, np.inf)
        assert int(fp8_e4m3.encode(np.array([lo]))[0]) == c
        assert int(fp8_e4m3.encode(np.array([hi]))[0]) == c + 1


def test_saturation_and_nan():
    big = np.array([448.0, 449.0, 464.0, 465.0, 1e6, np.inf, -np.inf, -1e30])
    codes = fp8_e4m3.encode(big)
    assert codes.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert fp8_e4m3.encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_quantize_divides_in_fp32():
    # x / scale in fp32 rounds before the fp8 rounding; choose a case where the
    # fp64 quotient and the fp32 quotient land on different sides of a midpoint
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32)
    s = np.float32(0.0123)
    ours = fp8_e4m3.quantize(x, s)
    q32 = (x / s).astype(np.float32)
    ref = torch.from_numpy(q32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inrange = np.abs(q32) <= 464
    assert np.array_equal(ours[inrange], ref[inrange])
    assert np.all(ours[~inrange] & 0x7F == 0x7E)
