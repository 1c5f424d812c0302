"""Pins for the oracle's OCP E4M3FN codec.

The codec is pinned to things other than itself:
  * the code/value pairs the OCP OFP8 specification fixes (golden file);
  * torch's float8_e4m3fn type, an independent implementation: its decode of
    all 256 codes, and its round-to-nearest-even cast of every bfloat16 value
    and of every tie point between neighbouring codes (torch's cast overflows
    to NaN rather than saturating, so inputs are clamped to +-448 first);
  * the defining property of round-to-nearest: no other code is closer.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.txt")


def _torch_decode(codes):
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(vals_f32):
    t = torch.from_numpy(np.asarray(vals_f32, np.float32))
    return torch.clamp(t, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_golden_points(orc):
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, val_s = line.split()
        code, val = int(code_s, 16), float(val_s)
        got = orc.e4m3_decode(code)
        if math.isnan(val):
            assert math.isnan(got)
            continue
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code_s, got)
        assert orc.e4m3_encode(val) == code
        n += 1
    assert n >= 10


def test_decode_all_codes_vs_torch(orc):
    codes = list(range(256))
    ref = _torch_decode(codes)
    for c in codes:
        got = orc.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    nan_codes = [c for c in codes if math.isnan(orc.e4m3_decode(c))]
    assert nan_codes == [0x7F, 0xFF]


def test_round_trip_all_finite_codes(orc):
    for c in range(256):
        v = orc.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert orc.e4m3_encode(v) == c


def test_encode_every_bf16_vs_torch(orc):
    bits = np.arange(65536, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    got = orc.e4m3_encode_array(vals)
    ref = _torch_encode(vals)
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN keeps its sign bit; the payload is the single NaN code.
    sign = (bits[nan] >> 31).astype(np.uint8)
    assert np.array_equal(got[nan], (sign << 7) | 0x7F)


def test_encode_ties_and_neighbours_vs_torch(orc):
    mags = sorted({orc.e4m3_decode(c) for c in range(0x7F)})
    pts = []
    for a, b in zip(mags[:-1], mags[1:]):
        mid = np.float32((a + b) / 2)          # exact: a, b have 4 significant bits
        assert float(mid) == (a + b) / 2
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    top = np.float32(464.0)                    # tie between 448 and the missing 480
    pts += [top, np.nextafter(top, np.float32(0)), np.nextafter(top, np.float32(1e9)),
            np.float32(1e30), np.float32(np.inf)]
    pts = np.array(pts, np.float32)
    pts = np.concatenate([pts, -pts])
    got = orc.e4m3_encode_array(pts)
    # saturating: everything at or above 448 in magnitude maps to +-448
    sat = np.abs(pts) >= 448
    assert np.all(got[sat] == np.where(pts[sat] > 0, 0x7E, 0xFE))
    ref = _torch_encode(pts)
    assert np.array_equal(got, ref)


def test_encode_random_f32_is_nearest(orc):
    rng = np.random.default_rng(7)
    vals = (rng.standard_normal(20000) * np.exp2(rng.uniform(-14, 10, 20000))).astype(np.float32)
    got = orc.e4m3_encode_array(vals)
    assert np.array_equal(got, _torch_encode(vals))
    table = np.array([orc.e4m3_decode(c) for c in range(256)])
    finite = ~np.isnan(table)
    for v, c in zip(vals[:3000], got[:3000]):
        x = float(np.clip(v, -448, 448))
        err = abs(table[c] - x)
        assert err <= np.min(np.abs(table[finite] - x)) + 0.0


def test_signed_zero_and_underflow(orc):
    assert orc.e4m3_encode(0.0) == 0x00
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(-1e-5) == 0x80        # rounds to -0
    assert orc.e4m3_encode(2.0 ** -10) == 0x00   # tie at half the smallest subnormal -> even (0)
    assert orc.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


@pytest.mark.parametrize("amax", [0.0, float("nan"), float("inf"), 448.0, 3.5, 1e-30])
def test_scales(orc, amax):
    s, inv = orc.scales_from_amax(amax)
    if amax > 0 and math.isfinite(amax):
        assert s == float(np.float32(amax) / np.float32(448.0))
        assert inv == float(np.float32(448.0) / np.float32(amax))
    else:
        assert s == 1.0 and inv == 1.0
