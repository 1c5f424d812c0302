"""Helpers shared by the GPU parity tests: run the same seeded inputs through
the HIP path (via the C ABI) and through the CPU oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from compressed_decode_attention_amd import CDA_SEG_ALIGN, CompactKVCache

ATOL, RTOL = 2e-3, 1e-2     # attention tolerance: |gpu - oracle| <= ATOL + RTOL |oracle|


def dev():
    return torch.device("cuda:0")


def odt(kv_dtype: str) -> int:
    return {"bf16": oracle.BF16, "fp8": oracle.FP8, "fp4": oracle.FP4}[kv_dtype]


def log(msg: str):
    print(msg, flush=True)


def gpu_prefill(k, v, keep, T, W, reserve, kv_dtype, amax=None, with_dst=True):
    """COUNT (+dst), allocate, PACK on the GPU.  k, v: bf16 CPU or GPU
    [B, >=T, Hkv, D]; keep [B, Hkv, >=T].  Returns (cache, dst or None)."""
    d = dev()
    B, _, Hkv, D = k.shape
    kd, vd, keepd = k.to(d), v.to(d), keep.to(d)
    c = CompactKVCache(B, Hkv, D, W, kv_dtype, d)
    dst = torch.full((max(B * Hkv * T, 1),), -7, dtype=torch.int32, device=d) if with_dst else None
    c.count(keepd, T, reserve, dst)
    c.allocate()
    # pool bytes not written by the kernels are set to a marker first
    c.k_pool.fill_(0xA5)
    c.v_pool.fill_(0x5A)
    scale_mode = 0
    if amax is not None:
        c.k_amax.copy_(torch.as_tensor(amax[0], dtype=torch.float32))
        c.v_amax.copy_(torch.as_tensor(amax[1], dtype=torch.float32))
        scale_mode = 1
    c.pack(kd, vd, keepd, T, scale_mode)
    return c, dst


def oracle_prefill(k, v, keep, T, W, reserve, kv_dtype, amax=None):
    return oracle.prefill_pack(k, v, keep, T, W, reserve, odt(kv_dtype), amax=amax,
                               align=CDA_SEG_ALIGN)


def compare_state(c: CompactKVCache, o: oracle.OracleCache, what: str = ""):
    """Bit-exact comparison of offsets, lengths, scales and every row in use."""
    torch.cuda.synchronize()
    nh = c.B * c.Hkv
    assert np.array_equal(c.seg_base.cpu().numpy(), o.seg_base), what + " seg_base"
    assert np.array_equal(c.seg_cap.cpu().numpy(), o.seg_cap), what + " seg_cap"
    assert np.array_equal(c.comp_len.cpu().numpy(), o.comp_len), what + " comp_len"
    assert np.array_equal(c.pos[: c.B].cpu().numpy(), o.pos), what + " pos"
    assert c.pool_rows >= int(o.seg_base[-1])
    if c.W:
        assert np.array_equal(c.ring_keep.cpu().numpy()[: nh * c.W], o.ring_keep[: nh * c.W]), \
            what + " ring_keep"
    if c.kv_dtype in ("fp8", "fp4"):
        ga, oa = c.k_amax.cpu().numpy()[:nh], o.k_amax
        assert np.array_equal(np.isnan(ga), np.isnan(oa)) and np.array_equal(ga[~np.isnan(ga)], oa[~np.isnan(oa)]), what + " k_amax"
        ga, oa = c.v_amax.cpu().numpy()[:nh], o.v_amax
        assert np.array_equal(np.isnan(ga), np.isnan(oa)) and np.array_equal(ga[~np.isnan(ga)], oa[~np.isnan(oa)]), what + " v_amax"
    kr = k_rows(c).cpu().numpy()
    vr = v_rows(c).cpu().numpy()
    n = o.stored_rows()
    for i in range(nh):
        a = int(o.seg_base[i])
        if n[i] == 0:
            continue
        if not np.array_equal(kr[a:a + n[i]], o.k_pool[a:a + n[i]]):
            bad = np.nonzero(np.any(kr[a:a + n[i]] != o.k_pool[a:a + n[i]], axis=1))[0]
            raise AssertionError(f"{what} K rows differ in segment {i}: rows {bad[:8]}")
        if not np.array_equal(vr[a:a + n[i]], o.v_pool[a:a + n[i]]):
            bad = np.nonzero(np.any(vr[a:a + n[i]] != o.v_pool[a:a + n[i]], axis=1))[0]
            raise AssertionError(f"{what} V rows differ in segment {i}: rows {bad[:8]}")


def check_close(got, ref, what="", atol=ATOL, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    same = got == ref                       # equal infinities (lse of an empty set)
    with np.errstate(invalid="ignore"):
        err = np.where(same, 0.0, np.abs(got - ref))
    bound = atol + rtol * np.abs(ref)
    bad = ~(same | (err <= bound))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                             f"max abs err {err.max():.3e}; first {idx.tolist()} "
                             f"got {got[bad][:5]} want {ref[bad][:5]}")
    return float(err.max()) if err.size else 0.0


# ---- reading a store back (host-side inspection; synchronises)

def stored_rows(c) -> torch.Tensor:
    """Rows holding data per segment: min(W, pos) + comp_len."""
    ring = torch.clamp(c.pos[: c.B].to(torch.int64), max=c.W)
    return ring.repeat_interleave(c.Hkv) + c.comp_len.to(torch.int64)


def v_rows(c) -> torch.Tensor:
    """The V pool as [pool_rows, row_bytes] bytes in row order (a gather of
    the tiles: four column-major blocks of 16 rows, two rows per byte for
    FP4; FP4 rows hold element d in the low nibble of byte d / 2 for even
    d)."""
    D, rows = c.D, c.pool_rows
    if c.kv_dtype == "fp4":
        t = c.v_pool[: rows * D // 2].view(-1, CDA_SEG_ALIGN // 16, D, 8)   # [tile, blk, d, byte]
        codes = torch.stack([t & 15, t >> 4], dim=-1).reshape(-1, CDA_SEG_ALIGN // 16, D, 16)
        codes = codes.permute(0, 1, 3, 2).reshape(-1, CDA_SEG_ALIGN, D)   # [tile, r, d]
        return (codes[..., 0::2] | (codes[..., 1::2] << 4)).reshape(rows, D // 2)
    e = c.row_bytes // D
    t = c.v_pool[: rows * D * e].view(-1, CDA_SEG_ALIGN // 16, D, 16, e)   # [tile, blk, d, r, byte]
    return t.permute(0, 1, 3, 2, 4).reshape(rows, D * e)


def k_rows(c) -> torch.Tensor:
    """The K pool as [pool_rows, row_bytes] bytes in row order (undoes the
    in-tile chunk permutation described in include/cda.h)."""
    rb = c.row_bytes
    kl = rb // 64
    t = c.k_pool[: c.pool_rows * rb].view(-1, 4, kl, 4, 4, 4, 16)
    # [tile, m, j, kg, gh, gl, byte] -> [tile, gh, m, gl, j, kg, byte]
    return t.permute(0, 4, 1, 5, 2, 3, 6).reshape(c.pool_rows, rb)


def segment_rows(c, i: int, rows: int):
    """Paged store: rows [0, rows) of segment i as (K bytes, V bytes), each
    [rows, row_bytes], gathered through its page table."""
    pt = c.pages()[i]
    idx = torch.arange(rows)
    pool_row = (pt[idx // CDA_SEG_ALIGN].to(torch.int64) * CDA_SEG_ALIGN +
                idx % CDA_SEG_ALIGN).to(c.device)
    return k_rows(c)[pool_row], v_rows(c)[pool_row]
