"""ctypes binding of libcda_hip.so (the C ABI in include/cda.h).

Argument marshalling only: every step of compaction and attention runs in
the HIP kernels of the library.  PyTorch tensors are used for device memory
and streams; their data pointers are passed straight through.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcda_hip.so")

CDA_OK, CDA_ERR_INVALID_ARG, CDA_ERR_UNSUPPORTED, CDA_ERR_WORKSPACE, CDA_ERR_HIP = range(5)
CDA_DEVERR_CAPACITY, CDA_DEVERR_POOL, CDA_DEVERR_PAGES = 1, 2, 8
CDA_DEVERR_MERGE, CDA_DEVERR_PLAN = 16, 32
CDA_KV_BF16, CDA_KV_FP8_E4M3, CDA_KV_FP4_E2M1 = 0, 1, 2
CDA_OUT_BF16, CDA_OUT_F32 = 0, 1
CDA_OP_COUNT, CDA_OP_PACK, CDA_OP_APPEND = 0, 1, 2
CDA_OP_PAGE_INIT, CDA_OP_REFILL, CDA_OP_RELEASE = 3, 4, 5
CDA_VERSION = 7       # the struct layouts below are those of this version
CDA_SCRATCH_BYTES = 4 << 20   # device scratch of decode_step_compact_noalloc, per GPU
CDA_SEG_ALIGN = 64
CDA_MAX_GQA = 16
CDA_MAX_CHUNK = 64
CDA_MAX_CHUNK_WINDOW = 4096

# every symbol include/cda.h declares
EXPORTS = ("kv_compact", "decode_attn_compact", "decode_step_compact",
           "decode_step_compact_noalloc", "chunk_attn_compact",
           "cda_attn_workspace_bytes", "cda_chunk_workspace_bytes", "cda_status_string",
           "cda_version")


class CdaKvCache(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("Hkv", C.c_int32), ("D", C.c_int32), ("W", C.c_int32),
        ("kv_dtype", C.c_int32), ("spare_rows", C.c_int32),
        ("pool_rows", C.c_int64),
        ("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
        ("seg_base", C.c_void_p), ("seg_cap", C.c_void_p), ("comp_len", C.c_void_p),
        ("pos", C.c_void_p), ("ring_keep", C.c_void_p),
        ("k_amax", C.c_void_p), ("v_amax", C.c_void_p), ("err", C.c_void_p),
        ("seg_base_host", C.c_void_p),
        ("page_table", C.c_void_p), ("max_pages", C.c_int32), ("reserved1", C.c_int32),
        ("free_pages", C.c_void_p), ("free_top", C.c_void_p),
    ]


class CdaCompactArgs(C.Structure):
    _fields_ = [
        ("op", C.c_int32), ("T", C.c_int32), ("reserve", C.c_int32), ("scale_mode", C.c_int32),
        ("keep", C.c_void_p), ("keep_ld", C.c_int64),
        ("k", C.c_void_p), ("v", C.c_void_p),
        ("stride_b", C.c_int64), ("stride_t", C.c_int64), ("stride_h", C.c_int64),
        ("dst_out", C.c_void_p),
        ("seq_begin", C.c_int32), ("seq_count", C.c_int32),
    ]


class CdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
            f"g.build()'` (there is no fallback path)")
    L = C.CDLL(path)
    L.kv_compact.argtypes = [C.POINTER(CdaKvCache), C.POINTER(CdaCompactArgs), C.c_void_p]
    L.kv_compact.restype = C.c_int32
    L.decode_attn_compact.argtypes = [C.POINTER(CdaKvCache), C.c_void_p, C.c_int32, C.c_float,
                                      C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                      C.c_void_p, C.c_size_t, C.c_void_p]
    L.decode_attn_compact.restype = C.c_int32
    L.decode_step_compact.argtypes = [C.POINTER(CdaKvCache), C.POINTER(CdaCompactArgs), C.c_void_p,
                                      C.c_int32, C.c_float, C.c_void_p, C.c_int32, C.c_void_p,
                                      C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    L.decode_step_compact.restype = C.c_int32
    L.decode_step_compact_noalloc.argtypes = [C.POINTER(CdaKvCache), C.POINTER(CdaCompactArgs),
                                              C.c_void_p, C.c_int32, C.c_float, C.c_void_p,
                                              C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]
    L.decode_step_compact_noalloc.restype = C.c_int32
    L.cda_attn_workspace_bytes.argtypes = [C.POINTER(CdaKvCache), C.c_int32, C.c_int32]
    L.cda_attn_workspace_bytes.restype = C.c_size_t
    L.chunk_attn_compact.argtypes = [C.POINTER(CdaKvCache), C.POINTER(CdaCompactArgs), C.c_int32,
                                     C.c_void_p, C.c_int32, C.c_float, C.c_void_p, C.c_int32,
                                     C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    L.chunk_attn_compact.restype = C.c_int32
    L.cda_chunk_workspace_bytes.argtypes = [C.POINTER(CdaKvCache), C.c_int32, C.c_int32]
    L.cda_chunk_workspace_bytes.restype = C.c_size_t
    L.cda_status_string.argtypes = [C.c_int32]
    L.cda_status_string.restype = C.c_char_p
    L.cda_version.argtypes = []
    L.cda_version.restype = C.c_int32
    if L.cda_version() != CDA_VERSION:
        raise RuntimeError(f"{path} is version {L.cda_version()}, this binding expects "
                           f"{CDA_VERSION}: rebuild it")
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().cda_status_string(int(status)).decode()


def version() -> int:
    return int(load().cda_version())


def kv_compact(cache: CdaKvCache, args: CdaCompactArgs, stream: int | None) -> int:
    return int(load().kv_compact(C.byref(cache), C.byref(args), C.c_void_p(stream or 0)))


def decode_attn_compact(cache: CdaKvCache, q_ptr: int, Hq: int, sm_scale: float, out_ptr: int,
                        out_dtype: int, lse_ptr: int | None, split_tokens: int,
                        ws_ptr: int | None, ws_bytes: int, stream: int | None) -> int:
    return int(load().decode_attn_compact(
        C.byref(cache), C.c_void_p(q_ptr), int(Hq), float(sm_scale), C.c_void_p(out_ptr),
        int(out_dtype), C.c_void_p(lse_ptr or 0), int(split_tokens), C.c_void_p(ws_ptr or 0),
        C.c_size_t(ws_bytes), C.c_void_p(stream or 0)))


def decode_step_compact(cache: CdaKvCache, args: CdaCompactArgs, q_ptr: int, Hq: int,
                        sm_scale: float, out_ptr: int, out_dtype: int, lse_ptr: int | None,
                        split_tokens: int, ws_ptr: int | None, ws_bytes: int,
                        stream: int | None) -> int:
    return int(load().decode_step_compact(
        C.byref(cache), C.byref(args), C.c_void_p(q_ptr), int(Hq), float(sm_scale),
        C.c_void_p(out_ptr), int(out_dtype), C.c_void_p(lse_ptr or 0), int(split_tokens),
        C.c_void_p(ws_ptr or 0), C.c_size_t(ws_bytes), C.c_void_p(stream or 0)))


def decode_step_compact_noalloc(cache: CdaKvCache, args: CdaCompactArgs, q_ptr: int, Hq: int,
                                sm_scale: float, out_ptr: int, out_dtype: int,
                                lse_ptr: int | None, split_tokens: int, stream: int | None) -> int:
    return int(load().decode_step_compact_noalloc(
        C.byref(cache), C.byref(args), C.c_void_p(q_ptr), int(Hq), float(sm_scale),
        C.c_void_p(out_ptr), int(out_dtype), C.c_void_p(lse_ptr or 0), int(split_tokens),
        C.c_void_p(stream or 0)))


def chunk_attn_compact(cache: CdaKvCache, args: CdaCompactArgs, M: int, q_ptr: int, Hq: int,
                       sm_scale: float, out_ptr: int, out_dtype: int, lse_ptr: int,
                       ws_ptr: int, ws_bytes: int, stream: int | None) -> int:
    return int(load().chunk_attn_compact(
        C.byref(cache), C.byref(args), int(M), C.c_void_p(q_ptr), int(Hq), float(sm_scale),
        C.c_void_p(out_ptr), int(out_dtype), C.c_void_p(lse_ptr or 0), C.c_void_p(ws_ptr or 0),
        C.c_size_t(ws_bytes), C.c_void_p(stream or 0)))


def chunk_workspace_bytes(cache: CdaKvCache, Hq: int, M: int) -> int:
    return int(load().cda_chunk_workspace_bytes(C.byref(cache), Hq, M))


def attn_workspace_bytes(cache: CdaKvCache, Hq: int, split_tokens: int) -> int:
    return int(load().cda_attn_workspace_bytes(C.byref(cache), int(Hq), int(split_tokens)))
