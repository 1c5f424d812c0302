"""Pins for the oracle's byte accounting and stored-row count against the
store the oracle itself builds.

compact_kv_bytes(stored rows, D, format, heads) is the size the FastDMS
page's memory table reports for the compact store (KV bytes per stored
token, plus the per-head scales of the quantised formats).  It is checked
here against what the oracle's store actually holds: every row in use is
located from the definition of the stored set (ring row p mod W for the W
newest positions, compact rows in ascending position order for the kept
older ones), read back from the pool with the pool's own row width, and
unpacked to D values that must equal the element-wise encoding of the
token's K and V.  A wrong bytes-per-row term (FP4's half byte, say)
misaligns the rows and fails this; the scale bytes are the two f32 arrays
the store keeps per head.  orc_stored_count is checked against a brute
count of the same definition and against the prefill layout.
"""
import numpy as np
import pytest
import torch

import workload


def brute_stored(keep_row, P, W):
    """Positions 0..P stored after the token at P: the W newest, plus every
    older one whose keep byte is nonzero."""
    return sum(1 for p in range(P + 1) if p > P - W or keep_row[p] != 0)


def expected_codes(orc, kv, x_bits, amax):
    """The stored codes of one bf16 row: the bits themselves (BF16), or the
    scalar encoder applied to x * inv (FP8, FP4)."""
    if kv == orc.BF16:
        return np.asarray(x_bits, np.uint16)
    import struct
    xs = [struct.unpack("<f", struct.pack("<I", int(u) << 16))[0] for u in x_bits]
    if kv == orc.FP8:
        _, inv = orc.scales_from_amax(float(amax))
        return np.array([orc.e4m3_encode(np.float32(x) * np.float32(inv)) for x in xs], np.uint8)
    _, inv = orc.fp4_scales_from_amax(float(amax))
    return np.array([orc.e2m1_encode(np.float32(x) * np.float32(inv)) for x in xs], np.uint8)


def unpack_row(orc, kv, raw):
    """The values a pool row holds, read with the pool's own row width."""
    if kv == orc.BF16:
        return raw.view(np.uint16)
    if kv == orc.FP8:
        return raw
    return np.stack([raw & 15, raw >> 4], axis=1).reshape(-1)   # low nibble first


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("W", [0, 5, 16])
def test_compact_bytes_are_the_bytes_the_store_holds(orc, kv, W):
    kvd = {"bf16": orc.BF16, "fp8": orc.FP8, "fp4": orc.FP4}[kv]
    B, Hkv, D, T, S = 1, 2, 128, 90, 10
    seed = 700 + 10 * W + kvd
    keep = workload.random_keep((B, Hkv, T + S), 0.3, seed=seed)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 1)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 2)
    kb = k.contiguous().view(torch.int16).numpy().view(np.uint16)
    vb = v.contiguous().view(torch.int16).numpy().view(np.uint16)
    kn = keep.numpy()
    c = orc.prefill_pack(k, v, keep, T, W, S, kvd)
    nh = B * Hkv
    for s in range(S + 1):
        if s > 0:
            c.append(k[:, T + s - 1], v[:, T + s - 1], keep[:, :, T + s - 1].contiguous())
        P = T + s - 1                                   # newest stored position
        n = c.stored_rows()
        for i in range(nh):
            b, h = divmod(i, Hkv)
            assert n[i] == brute_stored(kn[b, h], P, W), (s, i)
        if s not in (0, S):
            continue
        for i in range(nh):
            b, h = divmod(i, Hkv)
            older = [p for p in range(P + 1) if p <= P - W and kn[b, h, p]]
            recent = [p for p in range(max(P - W + 1, 0), P + 1)]
            rows = [(W + r, p) for r, p in enumerate(older)] + [(p % W, p) for p in recent]
            assert len(rows) == n[i]
            for row, p in rows:
                at = int(c.seg_base[i]) + row
                for pool, x, amax in ((c.k_pool, kb, c.k_amax), (c.v_pool, vb, c.v_amax)):
                    got = unpack_row(orc, kvd, pool[at])
                    want = expected_codes(orc, kvd, x[b, p, h], amax[i] if kvd != orc.BF16 else 0)
                    assert got.shape == (D,), (kv, got.shape)
                    assert np.array_equal(got, want), (kv, s, i, row, p)
        held = int(n.sum()) * (c.k_pool.shape[1] + c.v_pool.shape[1])
        if kvd != orc.BF16:
            held += c.k_amax.nbytes + c.v_amax.nbytes
        assert orc.compact_kv_bytes(int(n.sum()), D, kvd, nh) == held, (kv, s)


def test_stored_count_matches_definition_and_layout(orc):
    rng = np.random.default_rng(5)
    for W in (0, 1, 3, 9):
        for rate in (0.0, 0.2, 1.0):
            row = (rng.random(60) < rate).astype(np.uint8) * rng.integers(1, 256, 60).astype(np.uint8)
            for P in range(-1, 60):
                assert orc.stored_count(row, P, W) == brute_stored(row, P, W), (W, rate, P)
            keep = row.reshape(1, 1, 60)
            lay = orc.prefill_layout(keep, 60, W, 0)
            assert orc.stored_count(row, 59, W) == int((lay["dst"] >= 0).sum()), (W, rate)
