"""Pins for the oracle's compaction: layout, scales, pack and append.

The layout is pinned by brute force over every keep mask of up to 10 tokens,
checked through invariants that determine it uniquely (not by restating how
it is computed): the rows in use are exactly the ring rows that hold a
position plus a gap-free run of compact rows; every stored position has one
row and no two share one; evicted positions have none; compact rows keep
position order; a ring row holds position p at p mod W.

Pack and append are pinned by reading rows back, by the keep-all / keep-none
special cases, and by the identity "prefill of T tokens followed by S appends
leaves the same segment contents as a prefill of T + S tokens".
"""
import itertools

import numpy as np
import pytest
import torch

import workload


def _check_layout(keep_rows, T, W, reserve, lay, align=1):
    nh = keep_rows.shape[0]
    base = 0
    for i in range(nh):
        row = keep_rows[i]
        dst = lay["dst"].reshape(nh, T)[i]
        cl = int(lay["comp_len"][i])
        assert int(lay["seg_base"][i]) == base
        assert int(lay["seg_cap"][i]) == cl + reserve
        base += -(-(W + cl + reserve) // align) * align
        assert base % align == 0
        recent = set(range(max(0, T - W), T))
        stored = {p for p in range(T) if p in recent or row[p] != 0}
        # stored <-> has a row
        assert {p for p in range(T) if dst[p] >= 0} == stored
        rows = [int(dst[p]) for p in sorted(stored)]
        assert len(set(rows)) == len(rows)
        ring_rows = {int(dst[p]) for p in recent}
        comp_rows = sorted(int(dst[p]) for p in stored - recent)
        assert all(r < W for r in ring_rows)
        for p in recent:
            assert dst[p] == p % W
        # compact rows: a gap-free run W .. W+cl-1, in position order
        assert comp_rows == list(range(W, W + cl))
        older = sorted(stored - recent)
        assert [int(dst[p]) for p in older] == comp_rows
    assert int(lay["seg_base"][nh]) == base


@pytest.mark.parametrize("W,align", [(0, 1), (1, 1), (3, 1), (3, 4), (0, 64)])
def test_layout_brute_force_all_masks(orc, W, align):
    for T in range(0, 11):
        # all masks of this T at once, as heads of one layer (B = #masks, Hkv = 1)
        if T == 0:
            keep = np.zeros((1, 1, 1), np.uint8)
        else:
            masks = np.array(list(itertools.product([0, 1], repeat=T)), np.uint8)
            keep = np.ascontiguousarray(masks.reshape(-1, 1, T))
        lay = orc.prefill_layout(keep, T, W, reserve=2, align=align)
        _check_layout(keep.reshape(-1, keep.shape[2]), T, W, 2, lay, align)


def test_layout_nonbinary_keep_bytes(orc):
    keep = workload.random_keep((3, 4, 300), 0.3, seed=11).numpy()
    assert keep.max() > 1
    lay = orc.prefill_layout(keep, 300, 32, reserve=5)
    _check_layout(keep.reshape(12, 300), 300, 32, 5, lay)
    lay2 = orc.prefill_layout((keep != 0).astype(np.uint8), 300, 32, reserve=5)
    for k in lay:
        assert np.array_equal(lay[k], lay2[k])


def _rows_back(cache, i, rows):
    D, esz = cache.D, 2 if cache.kv_dtype == 0 else 1
    base = int(cache.seg_base[i])
    return cache.k_pool[base + rows], cache.v_pool[base + rows]


def _bf16_bytes(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint8)


@pytest.mark.parametrize("W", [0, 1, 7, 64])
def test_pack_bf16_reads_back(orc, W):
    B, Hkv, D, T = 2, 3, 16, 200
    keep = workload.random_keep((B, Hkv, T), 0.25, seed=3)
    k = workload.random_bf16((B, T, Hkv, D), seed=4)
    v = workload.random_bf16((B, T, Hkv, D), seed=5)
    c = orc.prefill_pack(k, v, keep, T, W, reserve=4, kv_dtype=orc.BF16)
    lay = orc.prefill_layout(keep, T, W, 4)
    for b in range(B):
        assert c.pos[b] == T
        for h in range(Hkv):
            i = b * Hkv + h
            dst = lay["dst"][b, h]
            for p in np.nonzero(dst >= 0)[0]:
                kr, vr = _rows_back(c, i, dst[p])
                assert np.array_equal(kr, _bf16_bytes(k[b, p, h]))
                assert np.array_equal(vr, _bf16_bytes(v[b, p, h]))
                if dst[p] < W:
                    assert c.ring_keep[i * W + dst[p]] == (keep[b, h, p] != 0)


def test_pack_keep_all_is_identity_and_keep_none_is_ring(orc):
    B, Hkv, D, T, W = 1, 2, 8, 50, 5
    k = workload.random_bf16((B, T, Hkv, D), seed=1)
    v = workload.random_bf16((B, T, Hkv, D), seed=2)
    ones = torch.ones((B, Hkv, T), dtype=torch.uint8)
    c = orc.prefill_pack(k, v, ones, T, W, reserve=0, kv_dtype=orc.BF16)
    for h in range(Hkv):
        base = int(c.seg_base[h])
        comp = c.k_pool[base + W: base + W + T - W]
        assert np.array_equal(comp, _bf16_bytes(k[0, : T - W, h]).reshape(T - W, -1))
    zeros = torch.zeros((B, Hkv, T), dtype=torch.uint8)
    c0 = orc.prefill_pack(k, v, zeros, T, W, reserve=0, kv_dtype=orc.BF16)
    assert np.all(c0.comp_len == 0)
    assert int(c0.seg_base[-1]) == B * Hkv * W


def test_amax_special_cases(orc):
    B, Hkv, D, T, W = 2, 2, 32, 100, 10
    k = workload.random_bf16((B, T, Hkv, D), seed=8, scale=3.0)
    v = workload.random_bf16((B, T, Hkv, D), seed=9)
    ones = torch.ones((B, Hkv, T), dtype=torch.uint8)
    ka, va = orc.prefill_amax(k, v, ones, T, W)
    ref_k = k.float().abs().amax(dim=(1, 3)).reshape(-1).numpy()
    ref_v = v.float().abs().amax(dim=(1, 3)).reshape(-1).numpy()
    assert np.array_equal(ka, ref_k) and np.array_equal(va, ref_v)
    zeros = torch.zeros((B, Hkv, T), dtype=torch.uint8)
    ka0, va0 = orc.prefill_amax(k, v, zeros, T, W)
    assert np.array_equal(ka0, k[:, T - W:].float().abs().amax(dim=(1, 3)).reshape(-1).numpy())
    assert np.array_equal(va0, v[:, T - W:].float().abs().amax(dim=(1, 3)).reshape(-1).numpy())


def test_pack_fp8_codes_are_nearest(orc):
    B, Hkv, D, T, W = 1, 2, 16, 120, 8
    keep = workload.random_keep((B, Hkv, T), 0.4, seed=21)
    k = workload.random_bf16((B, T, Hkv, D), seed=22, scale=2.0)
    v = workload.random_bf16((B, T, Hkv, D), seed=23)
    c = orc.prefill_pack(k, v, keep, T, W, reserve=0, kv_dtype=orc.FP8)
    lay = orc.prefill_layout(keep, T, W, 0)
    table = np.array([orc.e4m3_decode(x) for x in range(256)])
    ref = torch.tensor(range(256), dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    for h in range(Hkv):
        _, inv_k = orc.scales_from_amax(c.k_amax[h])
        dst = lay["dst"][0, h]
        for p in np.nonzero(dst >= 0)[0]:
            kr, _ = _rows_back(c, h, dst[p])
            y = (k[0, p, h].float() * np.float32(inv_k)).numpy()
            # torch's RNE cast of the f32 product gives the same codes
            want = torch.from_numpy(y).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(kr, want)
        # the absmax element maps to +-448 exactly
        assert np.max(np.abs(table[c.k_pool[int(c.seg_base[h]):int(c.seg_base[h]) + W + int(c.comp_len[h])]])) == 448.0


@pytest.mark.parametrize("kv_dtype,W", [(0, 16), (1, 16), (0, 0), (1, 1), (0, 40)])
def test_append_equals_longer_prefill(orc, kv_dtype, W):
    B, Hkv, D, T, S = 2, 2, 16, 30, 25
    keep = workload.random_keep((B, Hkv, T + S), 0.3, seed=31)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=32)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=33)
    amax = (np.full(B * Hkv, 2.5, np.float32), np.full(B * Hkv, 3.0, np.float32))
    c = orc.prefill_pack(k, v, keep, T, W, reserve=S, kv_dtype=kv_dtype, amax=amax)
    for s in range(S):
        c.append(k[:, T + s], v[:, T + s], keep[:, :, T + s])
    assert np.all(c.pos == T + S) and c.err[0] == 0
    full = orc.prefill_pack(k, v, keep, T + S, W, reserve=0, kv_dtype=kv_dtype, amax=amax)
    assert np.array_equal(c.comp_len, full.comp_len)
    n = c.stored_rows()
    assert np.array_equal(n, full.stored_rows())
    for i in range(B * Hkv):
        a0, b0 = int(c.seg_base[i]), int(full.seg_base[i])
        assert np.array_equal(c.k_pool[a0:a0 + n[i]], full.k_pool[b0:b0 + n[i]])
        assert np.array_equal(c.v_pool[a0:a0 + n[i]], full.v_pool[b0:b0 + n[i]])
        if W:
            assert np.array_equal(c.ring_keep[i * W:(i + 1) * W], full.ring_keep[i * W:(i + 1) * W])


def test_append_capacity_overflow_sets_error(orc):
    B, Hkv, D, T, W, S = 1, 1, 8, 10, 2, 12
    keep = torch.ones((B, Hkv, T + S), dtype=torch.uint8)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=1)
    c = orc.prefill_pack(k, k, keep, T, W, reserve=3, kv_dtype=orc.BF16)
    cap = int(c.seg_cap[0])
    for s in range(S):
        c.append(k[:, T + s], k[:, T + s], keep[:, :, T + s])
    assert c.err[0] == 1
    assert int(c.comp_len[0]) == cap
