"""Compact (DMS-style) decode attention for MI355X (gfx950).

Python face of libcda_hip.so.  The calls of the C ABI are exposed under
their own names (:func:`kv_compact`, :func:`decode_attn_compact`,
:func:`decode_step_compact`); the class
:class:`CompactKVCache` holds one layer's device buffers (torch tensors) and
forwards to them.  All arithmetic runs in the library's HIP kernels; this
module only checks shapes and passes pointers.  There is no CPU path: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import (CDA_DEVERR_CAPACITY, CDA_DEVERR_MERGE, CDA_DEVERR_PAGES, CDA_DEVERR_PLAN,
                   CDA_DEVERR_POOL, CDA_KV_BF16, CDA_KV_FP4_E2M1, CDA_KV_FP8_E4M3, CDA_OP_APPEND, CDA_OP_COUNT,
                   CDA_OP_PACK, CDA_OP_PAGE_INIT, CDA_OP_REFILL, CDA_OP_RELEASE, CDA_OUT_BF16,
                   CDA_OUT_F32, CDA_SEG_ALIGN, CdaCompactArgs, CdaError, CdaKvCache)

__all__ = ["CompactKVCache", "PagedKVCache", "kv_compact", "decode_attn_compact",
           "decode_step_compact", "decode_step_compact_noalloc", "chunk_attn_compact", "CdaError", "CDA_SEG_ALIGN", "CDA_DEVERR_CAPACITY",
           "CDA_DEVERR_POOL", "CDA_DEVERR_PAGES", "CDA_DEVERR_MERGE", "CDA_DEVERR_PLAN"]

_DTYPES = {"bf16": CDA_KV_BF16, "fp8": CDA_KV_FP8_E4M3, "fp4": CDA_KV_FP4_E2M1}
_ROW_BYTES = {"bf16": lambda D: 2 * D, "fp8": lambda D: D, "fp4": lambda D: D // 2}


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _on(cache, what: str, *tensors) -> None:
    """Every tensor argument must live on the cache's device: a host
    pointer handed to a kernel would be dereferenced on the GPU."""
    for t in tensors:
        if t is not None and t.device != cache.device:
            raise ValueError(f"{what}: tensors must be on {cache.device}, got {t.device}")


def _workspace(cache, ws) -> None:
    _on(cache, "workspace", ws)
    if ws is not None and (ws.dtype != torch.uint8 or not ws.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor (its numel is its byte size)")


def _compact_args(cache: "CompactKVCache", op: int, T: int = 0, reserve: int = 0,
                  scale_mode: int = 0, keep=None, k=None, v=None, dst_out=None,
                  seq_begin: int = 0, seq_count: int = 0) -> CdaCompactArgs:
    _on(cache, "kv_compact", keep, k, v, dst_out)
    a = CdaCompactArgs()
    a.op, a.T, a.reserve, a.scale_mode = op, T, reserve, scale_mode
    a.seq_begin, a.seq_count = seq_begin, seq_count
    nb = seq_count if seq_count > 0 else cache.B     # sequences the inputs hold
    if keep is not None:
        if keep.dtype != torch.uint8:
            raise TypeError("keep must be uint8")
        if op == CDA_OP_APPEND:
            if not keep.is_contiguous() or keep.numel() != cache.B * cache.Hkv:
                raise ValueError("APPEND keep must be a contiguous [B, Hkv] uint8 tensor")
            a.keep_ld = 1
        else:
            if keep.dim() != 3 or keep.shape[0] != nb or keep.shape[1] != cache.Hkv:
                raise ValueError("keep must be [sequences, Hkv, >=T]")
            if keep.shape[2] < T or keep.stride(2) != 1 or keep.stride(0) != cache.Hkv * keep.stride(1):
                raise ValueError("keep rows must be contiguous with a uniform pitch")
            a.keep_ld = keep.stride(1)
        a.keep = _ptr(keep)
    if k is not None:
        for x in (k, v):
            if x.dtype != torch.bfloat16 or x.shape[-1] != cache.D or x.stride(-1) != 1:
                raise ValueError("k, v must be bfloat16 with contiguous rows of D elements")
        if k.stride() != v.stride():
            raise ValueError("k and v must share strides")
        if op == CDA_OP_PACK:      # [sequences, >=T, Hkv, D]
            if k.shape[0] != nb or k.shape[2] != cache.Hkv or v.shape != k.shape:
                raise ValueError("k, v must be [sequences, >=T, Hkv, D]")
            a.stride_b, a.stride_t, a.stride_h = k.stride(0), k.stride(1), k.stride(2)
        else:                      # [B, Hkv, D]
            a.stride_b, a.stride_t, a.stride_h = k.stride(0), 0, k.stride(1)
        a.k, a.v = _ptr(k), _ptr(v)
    if dst_out is not None:
        if dst_out.dtype != torch.int32 or not dst_out.is_contiguous() or dst_out.numel() < nb * cache.Hkv * T:
            raise ValueError("dst_out must be a contiguous int32 tensor of sequences*Hkv*T elements")
        a.dst_out = _ptr(dst_out)
    return a


def kv_compact(cache: "CompactKVCache", op: int, *, T: int = 0, reserve: int = 0,
               scale_mode: int = 0, keep=None, k=None, v=None, dst_out=None,
               seq_begin: int = 0, seq_count: int = 0) -> None:
    """One kv_compact call (COUNT, PACK, APPEND, or PAGE_INIT / REFILL /
    RELEASE of a paged store) on ``cache``'s stream."""
    a = _compact_args(cache, op, T, reserve, scale_mode, keep, k, v, dst_out, seq_begin,
                      seq_count)
    st = _lib.kv_compact(cache.struct, a, _stream(cache.device))
    if st != 0:
        raise CdaError(st, "kv_compact")


def _check_attention(cache: "CompactKVCache", q, out, lse) -> None:
    _on(cache, "attention", q, out, lse)
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 3:
        raise ValueError("q must be a contiguous bfloat16 [B, Hq, D] tensor")
    B, Hq, D = q.shape
    if B != cache.B or D != cache.D:
        raise ValueError("q shape does not match the cache")
    if out.shape != q.shape or not out.is_contiguous() or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be a contiguous [B, Hq, D] bfloat16 or float32 tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * Hq):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")


def decode_attn_compact(cache: "CompactKVCache", q: torch.Tensor, out: torch.Tensor,
                        lse: torch.Tensor | None = None, sm_scale: float = 0.0,
                        split_tokens: int = 0, workspace: torch.Tensor | None = None) -> None:
    """One decode_attn_compact call: q [B, Hq, D] bf16 -> out [B, Hq, D]."""
    _check_attention(cache, q, out, lse)
    Hq = q.shape[1]
    if workspace is None:
        workspace = cache.workspace(Hq, split_tokens)
    _workspace(cache, workspace)
    out_dtype = CDA_OUT_F32 if out.dtype == torch.float32 else CDA_OUT_BF16
    st = _lib.decode_attn_compact(cache.struct, _ptr(q), Hq, sm_scale, _ptr(out), out_dtype,
                                  _ptr(lse), split_tokens, _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0,
                                  _stream(cache.device))
    if st != 0:
        raise CdaError(st, "decode_attn_compact")


def decode_step_compact(cache: "CompactKVCache", k_new: torch.Tensor, v_new: torch.Tensor,
                        keep_new: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                        lse: torch.Tensor | None = None, sm_scale: float = 0.0,
                        split_tokens: int = 0, workspace: torch.Tensor | None = None) -> None:
    """One decode_step_compact call: append (k_new, v_new [B, Hkv, D] bf16,
    keep_new [B, Hkv] uint8), then attention of q [B, Hq, D] -> out, in one
    launch."""
    _check_attention(cache, q, out, lse)
    Hq = q.shape[1]
    a = _compact_args(cache, CDA_OP_APPEND, keep=keep_new, k=k_new, v=v_new)
    if workspace is None:
        workspace = cache.workspace(Hq, split_tokens)
    _workspace(cache, workspace)
    out_dtype = CDA_OUT_F32 if out.dtype == torch.float32 else CDA_OUT_BF16
    st = _lib.decode_step_compact(cache.struct, a, _ptr(q), Hq, sm_scale, _ptr(out), out_dtype,
                                  _ptr(lse), split_tokens, _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0,
                                  _stream(cache.device))
    if st != 0:
        raise CdaError(st, "decode_step_compact")


def decode_step_compact_noalloc(cache: "CompactKVCache", k_new: torch.Tensor,
                                v_new: torch.Tensor, keep_new: torch.Tensor, q: torch.Tensor,
                                out: torch.Tensor, lse: torch.Tensor | None = None,
                                sm_scale: float = 0.0, split_tokens: int = 0) -> None:
    """One decode_step_compact_noalloc call: decode_step_compact without a
    workspace (the library's static per-GPU scratch is used instead; the
    stream must belong to the current device)."""
    _check_attention(cache, q, out, lse)
    Hq = q.shape[1]
    a = _compact_args(cache, CDA_OP_APPEND, keep=keep_new, k=k_new, v=v_new)
    out_dtype = CDA_OUT_F32 if out.dtype == torch.float32 else CDA_OUT_BF16
    st = _lib.decode_step_compact_noalloc(cache.struct, a, _ptr(q), Hq, sm_scale, _ptr(out),
                                          out_dtype, _ptr(lse), split_tokens,
                                          _stream(cache.device))
    if st != 0:
        raise CdaError(st, "decode_step_compact_noalloc")


def chunk_attn_compact(cache: "CompactKVCache", k_new: torch.Tensor, v_new: torch.Tensor,
                       keep_new: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor | None = None, sm_scale: float = 0.0,
                       workspace: torch.Tensor | None = None) -> None:
    """One chunk_attn_compact call: M new tokens per sequence (k_new, v_new
    [B, M, Hkv, D] bf16, keep_new [B, M, Hkv] uint8, q [B, M, Hq, D] bf16):
    query t answered as the decode step at position pos + t, out [B, M, Hq, D],
    then the M tokens appended."""
    _on(cache, "chunk_attn_compact", k_new, v_new, keep_new, q, out, lse)
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous bfloat16 [B, M, Hq, D] tensor")
    B, M, Hq, D = q.shape
    if B != cache.B or D != cache.D:
        raise ValueError("q shape does not match the cache")
    if out.shape != q.shape or not out.is_contiguous() or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be a contiguous [B, M, Hq, D] bfloat16 or float32 tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * M * Hq):
        raise ValueError("lse must be a contiguous float32 [B, M, Hq] tensor")
    for x in (k_new, v_new):
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (B, M, cache.Hkv, D) or x.stride(-1) != 1:
            raise ValueError("k_new, v_new must be bfloat16 [B, M, Hkv, D] with contiguous rows")
    if k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share strides")
    if keep_new.dtype != torch.uint8 or not keep_new.is_contiguous() or keep_new.numel() != B * M * cache.Hkv:
        raise ValueError("keep_new must be a contiguous uint8 [B, M, Hkv] tensor")
    a = CdaCompactArgs()
    a.op = CDA_OP_APPEND
    a.keep, a.keep_ld = _ptr(keep_new), cache.Hkv
    a.k, a.v = _ptr(k_new), _ptr(v_new)
    a.stride_b, a.stride_t, a.stride_h = k_new.stride(0), k_new.stride(1), k_new.stride(2)
    if workspace is None:
        workspace = cache.chunk_workspace(Hq, M)
    _workspace(cache, workspace)
    out_dtype = CDA_OUT_F32 if out.dtype == torch.float32 else CDA_OUT_BF16
    st = _lib.chunk_attn_compact(cache.struct, a, M, _ptr(q), Hq, sm_scale, _ptr(out), out_dtype,
                                 _ptr(lse), _ptr(workspace), workspace.numel(),
                                 _stream(cache.device))
    if st != 0:
        raise CdaError(st, "chunk_attn_compact")


class CompactKVCache:
    """One layer's compact KV store: metadata and pools as device tensors."""

    def __init__(self, B: int, Hkv: int, D: int, W: int, kv_dtype: str = "bf16",
                 device="cuda"):
        if kv_dtype not in _DTYPES:
            raise ValueError("kv_dtype must be 'bf16', 'fp8' or 'fp4'")
        _lib.load()
        self.B, self.Hkv, self.D, self.W = B, Hkv, D, W
        self.kv_dtype = kv_dtype
        self.row_bytes = _ROW_BYTES[kv_dtype](D)   # bytes of one stored row
        self.device = torch.device(device)
        nh = B * Hkv
        dev = self.device
        self.seg_base = torch.zeros(nh + 1, dtype=torch.int64, device=dev)
        self.seg_cap = torch.zeros(nh, dtype=torch.int32, device=dev)
        self.comp_len = torch.zeros(nh, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(max(B, 1), dtype=torch.int32, device=dev)
        self.ring_keep = torch.zeros(max(nh * W, 1), dtype=torch.uint8, device=dev)
        self.k_amax = torch.zeros(max(nh, 1), dtype=torch.float32, device=dev)
        self.v_amax = torch.zeros(max(nh, 1), dtype=torch.float32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        # host copy of seg_base for the host-side work plan (set by allocate)
        self.seg_base_host = None
        # rows at each segment's end expected empty (the COUNT reserve): a read hint
        self.spare_rows = 0
        self.k_pool = None
        self.v_pool = None
        self.pool_rows = 0
        self._ws = {}
        self.struct = CdaKvCache()
        self._refresh()

    paged = False

    def _refresh(self):
        s = self.struct
        s.B, s.Hkv, s.D, s.W = self.B, self.Hkv, self.D, self.W
        s.kv_dtype = _DTYPES[self.kv_dtype]
        s.spare_rows = self.spare_rows
        s.pool_rows = self.pool_rows
        s.k_pool, s.v_pool = _ptr(self.k_pool), _ptr(self.v_pool)
        s.seg_base, s.seg_cap = _ptr(self.seg_base), _ptr(self.seg_cap)
        s.comp_len, s.pos = _ptr(self.comp_len), _ptr(self.pos)
        s.ring_keep = _ptr(self.ring_keep)
        s.k_amax, s.v_amax = _ptr(self.k_amax), _ptr(self.v_amax)
        s.err = _ptr(self.err)
        s.seg_base_host = _ptr(self.seg_base_host)

    # ---- prefill
    def count(self, keep, T: int, reserve: int, dst_out=None) -> None:
        kv_compact(self, CDA_OP_COUNT, T=T, reserve=reserve, keep=keep, dst_out=dst_out)
        self.spare_rows = int(reserve)
        self.struct.spare_rows = self.spare_rows

    def rows_needed(self) -> int:
        """Pool rows the layout needs (reads seg_base[B*Hkv]: synchronises)."""
        return int(self.seg_base[-1].item())

    def allocate(self, rows: int | None = None) -> None:
        """Allocates the pools for the layout COUNT wrote (one host
        synchronisation) and keeps a host copy of seg_base, with which the
        attention calls plan their work on the host.  A later COUNT must
        give the same layout (same keep, T and reserve), or allocate must be
        called again; otherwise the attention calls flag CDA_DEVERR_PLAN."""
        sbh = self.seg_base.cpu()
        need = int(sbh[-1])
        rows = need if rows is None else rows
        rows = -(-rows // CDA_SEG_ALIGN) * CDA_SEG_ALIGN
        # the host plan describes the layout inside the pool only
        self.seg_base_host = sbh if rows >= need else None
        nbytes = max(rows, 1) * self.row_bytes
        self.k_pool = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.v_pool = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.pool_rows = rows
        self._ws.clear()
        self._refresh()

    def pack(self, k, v, keep, T: int, scale_mode: int = 0) -> None:
        kv_compact(self, CDA_OP_PACK, T=T, scale_mode=scale_mode, keep=keep, k=k, v=v)

    def compact(self, k, v, keep, T: int, reserve: int, scale_mode: int = 0,
                dst_out=None) -> None:
        """COUNT, size the pools, PACK (one host synchronisation)."""
        self.count(keep, T, reserve, dst_out)
        self.allocate()
        self.pack(k, v, keep, T, scale_mode)

    # ---- decode
    def append(self, k_new, v_new, keep_new) -> None:
        kv_compact(self, CDA_OP_APPEND, keep=keep_new, k=k_new, v=v_new)

    def workspace(self, Hq: int, split_tokens: int = 0) -> torch.Tensor:
        key = (Hq, split_tokens)
        if key not in self._ws:
            n = _lib.attn_workspace_bytes(self.struct, Hq, split_tokens)
            # zero-filled once; the library keeps its counters at zero
            self._ws[key] = torch.zeros(max(n, 16), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def chunk_workspace(self, Hq: int, M: int) -> torch.Tensor:
        key = ("chunk", Hq, M)
        if key not in self._ws:
            n = _lib.chunk_workspace_bytes(self.struct, Hq, M)
            self._ws[key] = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def chunk(self, k_new, v_new, keep_new, q, out=None, out_dtype=torch.bfloat16, lse=None,
              sm_scale: float = 0.0, workspace=None) -> torch.Tensor:
        """chunk_attn_compact: q [B, M, Hq, D] over the store plus the chunk,
        then the chunk (k_new, v_new [B, M, Hkv, D], keep_new [B, M, Hkv])
        appended."""
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        chunk_attn_compact(self, k_new, v_new, keep_new, q, out, lse, sm_scale, workspace)
        return out

    def attention(self, q, out=None, out_dtype=torch.bfloat16, lse=None, sm_scale: float = 0.0,
                  split_tokens: int = 0, workspace=None) -> torch.Tensor:
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        decode_attn_compact(self, q, out, lse, sm_scale, split_tokens, workspace)
        return out

    def decode_step(self, k_new, v_new, keep_new, q, out=None, out_dtype=torch.bfloat16,
                    lse=None, sm_scale: float = 0.0, split_tokens: int = 0,
                    workspace=None) -> torch.Tensor:
        """append(k_new, v_new, keep_new) then attention(q), in one launch."""
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        decode_step_compact(self, k_new, v_new, keep_new, q, out, lse, sm_scale, split_tokens,
                            workspace)
        return out

    def decode_step_noalloc(self, k_new, v_new, keep_new, q, out=None,
                            out_dtype=torch.bfloat16, lse=None, sm_scale: float = 0.0,
                            split_tokens: int = 0) -> torch.Tensor:
        """decode_step through decode_step_compact_noalloc (no workspace)."""
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=self.device)
        decode_step_compact_noalloc(self, k_new, v_new, keep_new, q, out, lse, sm_scale,
                                    split_tokens)
        return out

    # ---- inspection (synchronise)
    def error_word(self) -> int:
        return int(self.err.item())


class PagedKVCache(CompactKVCache):
    """One layer's paged compact store: a pool of ``n_pages`` 64-row pages
    shared by all B*Hkv segments, a page table of ``max_pages`` entries per
    segment and a device stack of free pages.  Sequences are admitted
    (COUNT + PACK of a range) and released one range at a time; REFILL keeps
    every live segment ``reserve`` compact rows ahead of its data."""

    paged = True

    def __init__(self, B: int, Hkv: int, D: int, W: int, n_pages: int, max_pages: int,
                 kv_dtype: str = "bf16", device="cuda"):
        super().__init__(B, Hkv, D, W, kv_dtype, device)
        if n_pages < 1 or max_pages < 1:
            raise ValueError("n_pages >= 1 and max_pages >= 1 are required")
        dev = self.device
        nh = B * Hkv
        self.n_pages, self.max_pages = n_pages, max_pages
        self.page_table = torch.full((max(nh * max_pages, 1),), -1, dtype=torch.int32, device=dev)
        self.free_pages = torch.zeros(max(n_pages, 1), dtype=torch.int32, device=dev)
        self.free_top = torch.zeros(1, dtype=torch.int32, device=dev)
        self.pool_rows = n_pages * CDA_SEG_ALIGN
        nbytes = max(self.pool_rows, 1) * self.row_bytes
        self.k_pool = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.v_pool = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self._refresh()
        self.init()

    def _refresh(self):
        super()._refresh()
        s = self.struct
        if getattr(self, "page_table", None) is None:   # during the base constructor
            return
        s.seg_base = 0
        s.page_table = _ptr(self.page_table)
        s.max_pages = self.max_pages
        s.reserved1 = 0
        s.free_pages, s.free_top = _ptr(self.free_pages), _ptr(self.free_top)

    def init(self) -> None:
        """Every page free, every sequence idle (PAGE_INIT)."""
        kv_compact(self, CDA_OP_PAGE_INIT)

    def admit(self, b0: int, k, v, keep, T: int, reserve: int = 0, scale_mode: int = 0,
              dst_out=None) -> None:
        """Prefill of sequences [b0, b0 + n) from k, v [n, >=T, Hkv, D] bf16 and
        keep [n, Hkv, >=T]: COUNT (takes the pages) then PACK.  With too few
        free pages the range stays idle and CDA_DEVERR_PAGES is set."""
        n = keep.shape[0]
        kv_compact(self, CDA_OP_COUNT, T=T, reserve=reserve, keep=keep, dst_out=dst_out,
                   seq_begin=b0, seq_count=n)
        kv_compact(self, CDA_OP_PACK, T=T, scale_mode=scale_mode, keep=keep, k=k, v=v,
                   seq_begin=b0, seq_count=n)

    def refill(self, reserve: int = CDA_SEG_ALIGN) -> None:
        """Tops every live segment up to ``reserve`` free compact rows."""
        kv_compact(self, CDA_OP_REFILL, reserve=reserve)

    def release(self, b0: int, n: int = 1) -> None:
        """Returns the pages of sequences [b0, b0 + n) and makes them idle."""
        kv_compact(self, CDA_OP_RELEASE, seq_begin=b0, seq_count=n)

    def count(self, *a, **kw):
        raise TypeError("a paged store admits sequences with admit()")

    def allocate(self, *a, **kw):
        raise TypeError("a paged store's pool is sized by n_pages")

    def compact(self, *a, **kw):
        raise TypeError("a paged store admits sequences with admit()")

    # ---- inspection (synchronise)
    def free_count(self) -> int:
        return int(self.free_top.item())

    def pages(self) -> torch.Tensor:
        """Page tables as [B*Hkv, max_pages] (CPU)."""
        return self.page_table[: self.B * self.Hkv * self.max_pages].view(
            self.B * self.Hkv, self.max_pages).cpu()
