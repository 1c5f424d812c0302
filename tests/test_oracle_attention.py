"""Pins for the oracle's decode attention.

  * keep-all: compact attention is dense attention, checked against torch's
    scaled_dot_product_attention (float64, CPU, enable_gqa) on the stored
    values; the FP8 values are dequantised with torch's own float8 decode;
  * any mask: equal to dense attention with the evicted positions masked out
    (the spec identity), again through torch's SDPA with a mask;
  * closed forms: q = 0 gives the plain mean of the stored values, which pins
    the stored set exactly; a single stored token returns its value; equal
    keys give the mean; an empty set gives zeros and lse = -inf.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workload


def _deq(x_bf16, amax, kv_dtype, orc):
    """Stored value per element, via torch's float8 type (FP8) -- an
    implementation independent of the oracle's codec."""
    x = x_bf16.float()
    if kv_dtype == orc.BF16:
        return x.double()
    s, inv = orc.scales_from_amax(float(amax))
    y = (x * torch.tensor(inv, dtype=torch.float32)).clamp(-448, 448)
    return y.to(torch.float8_e4m3fn).double() * float(np.float32(s))


def _sdpa(q, kd, vd, mask, sm_scale):
    """q [B,Hq,D] f64; kd, vd [B,T,Hkv,D] f64; mask [B,Hkv,T] bool (True=attend)."""
    B, Hq, D = q.shape
    Hkv = kd.shape[2]
    G = Hq // Hkv
    qq = q[:, :, None, :]
    kk = kd.permute(0, 2, 1, 3)
    vv = vd.permute(0, 2, 1, 3)
    m = mask.repeat_interleave(G, dim=1)[:, :, None, :]
    return F.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=sm_scale,
                                          enable_gqa=True)[:, :, 0, :]


def _setup(kv_dtype, keep_rate, W, seed, B=2, Hq=8, Hkv=2, D=32, T=150, orc=None):
    keep = workload.random_keep((B, Hkv, T), keep_rate, seed=seed)
    k = workload.random_bf16((B, T, Hkv, D), seed=seed + 1)
    v = workload.random_bf16((B, T, Hkv, D), seed=seed + 2, scale=2.0)
    q = workload.random_bf16((B, Hq, D), seed=seed + 3)
    ka, va = orc.prefill_amax(k, v, keep, T, W)
    return keep, k, v, q, ka, va


def _dense_values(k, v, ka, va, kv_dtype, orc):
    B, T, Hkv, D = k.shape
    kd = torch.empty(k.shape, dtype=torch.float64)
    vd = torch.empty(v.shape, dtype=torch.float64)
    for b in range(B):
        for h in range(Hkv):
            kd[b, :, h] = _deq(k[b, :, h], ka[b * Hkv + h], kv_dtype, orc)
            vd[b, :, h] = _deq(v[b, :, h], va[b * Hkv + h], kv_dtype, orc)
    return kd, vd


@pytest.mark.parametrize("kv_dtype", [0, 1])
def test_keep_all_is_dense_sdpa(orc, kv_dtype):
    T, W = 150, 16
    keep, k, v, q, ka, va = _setup(kv_dtype, 1.0, W, 100, T=T, orc=orc)
    out, lse = orc.attention(q, k, v, keep, T - 1, W, kv_dtype, ka, va)
    kd, vd = _dense_values(k, v, ka, va, kv_dtype, orc)
    D = q.shape[2]
    B, Hq = q.shape[:2]
    qq = q.double()[:, :, None, :]
    ref = F.scaled_dot_product_attention(qq, kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3),
                                         enable_gqa=True)[:, :, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)
    # lse against a direct logsumexp of the dense logits
    G = Hq // k.shape[2]
    z = torch.einsum("bjd,btjd->bjt", q.double(), kd.repeat_interleave(G, dim=2)) / math.sqrt(D)
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).numpy(), rtol=1e-12)


@pytest.mark.parametrize("kv_dtype,W,rate", [(0, 16, 0.2), (1, 16, 0.2), (0, 0, 0.3), (1, 1, 0.1),
                                             (0, 200, 0.2)])
def test_equals_masked_dense(orc, kv_dtype, W, rate):
    T = 150
    keep, k, v, q, ka, va = _setup(kv_dtype, rate, W, 200 + W, T=T, orc=orc)
    out, _ = orc.attention(q, k, v, keep, T - 1, W, kv_dtype, ka, va, sm_scale=0.3)
    kd, vd = _dense_values(k, v, ka, va, kv_dtype, orc)
    evicted = (keep == 0).clone()
    evicted[:, :, max(0, T - W):] = False
    ref = _sdpa(q.double(), kd, vd, ~evicted, 0.3)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("kv_dtype", [0, 1])
def test_zero_query_gives_mean_of_stored(orc, kv_dtype):
    T, W = 150, 8
    keep, k, v, q, ka, va = _setup(kv_dtype, 0.25, W, 300, T=T, orc=orc)
    q = torch.zeros_like(q)
    out, lse = orc.attention(q, k, v, keep, T - 1, W, kv_dtype, ka, va)
    _, vd = _dense_values(k, v, ka, va, kv_dtype, orc)
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    lay = orc.prefill_layout(keep, T, W, 0)
    for b in range(B):
        for j in range(Hq):
            h = j // (Hq // Hkv)
            idx = np.nonzero(lay["dst"][b, h] >= 0)[0]
            assert len(idx) == W + lay["comp_len"][b * Hkv + h]
            np.testing.assert_allclose(out[b, j], vd[b, idx, h].mean(0).numpy(), rtol=1e-12, atol=1e-13)
            assert abs(lse[b, j] - math.log(len(idx))) < 1e-12


def test_single_stored_token_and_empty_set(orc):
    B, Hq, Hkv, D, T = 1, 4, 1, 16, 20
    k = workload.random_bf16((B, T, Hkv, D), seed=1)
    v = workload.random_bf16((B, T, Hkv, D), seed=2)
    q = workload.random_bf16((B, Hq, D), seed=3)
    none = torch.zeros((B, Hkv, T), dtype=torch.uint8)
    out, lse = orc.attention(q, k, v, none, T - 1, 1, orc.BF16)
    np.testing.assert_array_equal(out[0], np.repeat(v[0, T - 1, 0].double().numpy()[None], Hq, 0))
    z = (q[0].double() @ k[0, T - 1, 0].double()) / math.sqrt(D)
    np.testing.assert_allclose(lse[0], z.numpy(), rtol=1e-13)
    out0, lse0 = orc.attention(q, k, v, none, T - 1, 0, orc.BF16)
    assert np.all(out0 == 0) and np.all(np.isneginf(lse0))


def test_equal_keys_give_mean(orc):
    B, Hq, Hkv, D, T, W = 1, 4, 2, 8, 40, 4
    kr = workload.random_bf16((D,), seed=5)
    k = kr.expand(B, T, Hkv, D).contiguous()
    v = workload.random_bf16((B, T, Hkv, D), seed=6)
    q = workload.random_bf16((B, Hq, D), seed=7)
    keep = workload.random_keep((B, Hkv, T), 0.5, seed=8)
    out, _ = orc.attention(q, k, v, keep, T - 1, W, orc.BF16)
    lay = orc.prefill_layout(keep, T, W, 0)
    for j in range(Hq):
        h = j // 2
        idx = np.nonzero(lay["dst"][0, h] >= 0)[0]
        np.testing.assert_allclose(out[0, j], v[0, idx, h].double().mean(0).numpy(), rtol=1e-12, atol=1e-14)


def test_head_function_matches_layer_function(orc):
    T, W = 150, 16
    keep, k, v, q, ka, va = _setup(1, 0.2, W, 400, T=T, orc=orc)
    out, lse = orc.attention(q, k, v, keep, T - 1, W, orc.FP8, ka, va)
    for b, j in [(0, 0), (1, 5), (1, 7)]:
        o1, l1 = orc.attention_head(q[b, j], k, v, keep, b, j, 4, T - 1, W, orc.FP8, ka, va)
        assert np.array_equal(o1, out[b, j]) and l1 == lse[b, j]
