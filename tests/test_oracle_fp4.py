"""Pins for the oracle's 4-bit store: the OCP MX FP4 (E2M1) codec, the
nibble layout, the scales and attention over a 4-bit store.

  * the 16 code/value pairs of the E2M1 element type (golden file, from the
    OCP Microscaling Formats specification);
  * round-to-nearest-even by brute force: every grid point and random value
    gets the code whose value is nearest, ties to the code with an even
    mantissa bit (an independent search, not the oracle's binade arithmetic);
  * saturation (magnitudes past 6, infinities) and the NaN reading;
  * the packed row: element d in the low nibble of byte d/2 for even d;
  * attention over a FP4 store equals torch's SDPA (float64) on values
    dequantised with the brute-force encoder.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_points.txt")
MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _brute_code(y: float) -> int:
    """Nearest E2M1 code by exhaustive search (ties to the even code)."""
    sign = 8 if math.copysign(1.0, y) < 0 else 0
    if math.isnan(y):
        return sign | 7
    a = abs(y)
    if math.isinf(a):
        return sign | 7
    dist = np.abs(MAGS - a)
    best = np.flatnonzero(dist == dist.min())
    c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return sign | c


def test_golden_points(orc):
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code_s, val_s = line.split()
        code, val = int(code_s, 16), float(val_s)
        got = orc.e2m1_decode(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code_s, got)
        assert orc.e2m1_encode(val) == code
        n += 1
    assert n == 16


def test_round_to_nearest_even_by_search(orc):
    grid = np.arange(-8.0, 8.0 + 1e-9, 1.0 / 64)           # every tie point is on it
    rnd = np.random.default_rng(5).normal(0.0, 3.0, 4000).astype(np.float32)
    tiny = np.array([1e-30, -1e-30, 1e-45, 0.2499999, 0.2500001, 5.999, 6.0001], np.float32)
    for y in np.concatenate([grid.astype(np.float32), rnd, tiny]):
        y = float(np.float32(y))
        assert orc.e2m1_encode(y) == _brute_code(y), y


def test_ties_saturation_and_specials(orc):
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, c in ties.items():
        assert orc.e2m1_encode(y) == c and orc.e2m1_encode(-y) == 8 | c, y
    for y in (6.0, 6.5, 7.0, 1e30, float("inf")):
        assert orc.e2m1_encode(y) == 7 and orc.e2m1_encode(-y) == 15, y
    assert orc.e2m1_encode(float("nan")) == 7
    assert orc.e2m1_encode(-float("nan")) == 15
    assert orc.e2m1_encode(0.0) == 0 and orc.e2m1_encode(-0.0) == 8


def test_scales(orc):
    s, inv = orc.fp4_scales_from_amax(3.0)
    assert s == np.float32(3.0) / np.float32(6.0) and inv == np.float32(6.0) / np.float32(3.0)
    for a in (0.0, float("inf"), float("nan")):
        assert orc.fp4_scales_from_amax(a) == (1.0, 1.0)


def test_packed_row_nibble_order(orc):
    # amax 6 gives inv = 1: codes are those of the inputs themselves
    B, Hkv, D, T = 1, 1, 8, 1
    vals = torch.tensor([1.0, 2.0, -0.5, 6.0, 0.0, 3.0, -4.0, 1.5])
    k = vals.to(torch.bfloat16).reshape(B, T, Hkv, D)
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    c = orc.prefill_pack(k, k, keep, T, 1, 0, orc.FP4, amax=(np.full(1, 6.0, np.float32),) * 2)
    codes = [_brute_code(float(x)) for x in vals]
    want = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(D // 2)]
    assert c.k_pool.shape == (1, D // 2)
    assert list(c.k_pool[0]) == want and list(c.v_pool[0]) == want


def _deq_fp4(x_bf16, amax, orc):
    s, inv = orc.fp4_scales_from_amax(float(amax))
    y = (x_bf16.float() * torch.tensor(inv, dtype=torch.float32)).numpy().ravel()
    vals = np.array([orc.e2m1_decode(_brute_code(float(t))) for t in y])
    return torch.from_numpy(vals.reshape(tuple(x_bf16.shape))) * float(np.float32(s))


@pytest.mark.parametrize("keep_rate,W", [(1.0, 0), (0.3, 8)])
def test_attention_over_fp4_store_is_sdpa(orc, keep_rate, W):
    B, Hq, Hkv, D, T = 2, 4, 2, 16, 40
    keep = workload.random_keep((B, Hkv, T), keep_rate, seed=11)
    k = workload.random_bf16((B, T, Hkv, D), seed=12)
    v = workload.random_bf16((B, T, Hkv, D), seed=13, scale=2.0)
    q = workload.random_bf16((B, Hq, D), seed=14)
    ka, va = orc.prefill_amax(k, v, keep, T, W)
    kd = torch.empty(k.shape, dtype=torch.float64)
    vd = torch.empty(v.shape, dtype=torch.float64)
    for b in range(B):
        for h in range(Hkv):
            kd[b, :, h] = _deq_fp4(k[b, :, h], ka[b * Hkv + h], orc)
            vd[b, :, h] = _deq_fp4(v[b, :, h], va[b * Hkv + h], orc)
    mask = torch.zeros((B, Hkv, T), dtype=torch.bool)
    for b in range(B):
        for h in range(Hkv):
            for p in range(T):
                mask[b, h, p] = p > T - 1 - W or bool(keep[b, h, p])
    sm = 1.0 / math.sqrt(D)
    G = Hq // Hkv
    ref = F.scaled_dot_product_attention(
        q.double()[:, :, None, :], kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3),
        attn_mask=mask.repeat_interleave(G, dim=1)[:, :, None, :], scale=sm,
        enable_gqa=True)[:, :, 0, :]
    out, _ = orc.attention(q, k, v, keep, T - 1, W, orc.FP4, ka, va)
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
