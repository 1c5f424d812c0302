"""CPU oracle for compact decode attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does, and this package
imports nothing from it: the two share no code.

The arithmetic lives in ``cda_oracle.c`` (plain C, fp64 attention); this
module compiles it with gcc when needed and wraps it with ctypes, taking and
returning numpy arrays (bfloat16 data is passed as its uint16 bit patterns).
See the C file for what each function computes and which passage of the
FastDMS page it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_cda.so")
_lock = threading.Lock()
_lib = None

BF16, FP8, FP4 = 0, 1, 2
FP8_MAX = 448.0
FP4_MAX = 6.0


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(_LIB)
            P = C.c_void_p
            i32, i64, f32, f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
            L.orc_e4m3_encode.argtypes = [f32]
            L.orc_e4m3_encode.restype = C.c_uint8
            L.orc_e4m3_decode.argtypes = [C.c_uint8]
            L.orc_e4m3_decode.restype = f64
            L.orc_scales_from_amax.argtypes = [f32, P, P]
            L.orc_e2m1_encode.argtypes = [f32]
            L.orc_e2m1_encode.restype = C.c_uint8
            L.orc_e2m1_decode.argtypes = [C.c_uint8]
            L.orc_e2m1_decode.restype = f64
            L.orc_fp4_scales_from_amax.argtypes = [f32, P, P]
            L.orc_set_threads.argtypes = [i32]
            L.orc_max_threads.restype = i32
            L.orc_stored_count.argtypes = [P, i32, i32]
            L.orc_stored_count.restype = i64
            L.orc_prefill_layout.argtypes = [i32, i32, i32, i32, i32, i32, P, i64, P, P, P, P]
            L.orc_prefill_amax.argtypes = [i32, i32, i32, i32, i32, P, P, i64, i64, i64, P, i64, P, P]
            L.orc_prefill_pack.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, i64, i64, i64,
                                           P, i64, i32, P, P, P, P, P, P, P, P, P]
            L.orc_append.argtypes = [i32, i32, i32, i32, i32, P, P, i64, i64, P, P, P, P, P,
                                     P, P, P, P, P, P]
            L.orc_append.restype = i64
            L.orc_attention_head.argtypes = [i32, i32, i32, i32, P, P, i64, P, f32, f32, P, f64, P, P]
            L.orc_attention.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, i64, i64, i64,
                                        P, i64, P, P, P, f64, P, P]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _bits(x) -> np.ndarray:
    """bfloat16 torch tensor or uint16 array -> contiguous uint16 array."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def _u8(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.uint8)
    return x.contiguous().numpy().astype(np.uint8, copy=False)


def set_threads(n: int) -> int:
    """Threads the oracle's loops over independent (sequence, head) units
    use (n < 1: every core); returns the number now in effect."""
    lib().orc_set_threads(int(n))
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- scalars

def e4m3_encode(y: float) -> int:
    return int(lib().orc_e4m3_encode(float(y)))


def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code)))


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    enc = lib().orc_e4m3_encode
    return np.fromiter((enc(float(v)) for v in y), dtype=np.uint8, count=y.size)


def scales_from_amax(amax: float):
    s, inv = C.c_float(), C.c_float()
    lib().orc_scales_from_amax(float(amax), C.byref(s), C.byref(inv))
    return s.value, inv.value


def e2m1_encode(y: float) -> int:
    """4-bit code (0..15) of the OCP MX FP4 E2M1 encoding of y."""
    return int(lib().orc_e2m1_encode(float(y)))


def e2m1_decode(code: int) -> float:
    return float(lib().orc_e2m1_decode(int(code)))


def fp4_scales_from_amax(amax: float):
    s, inv = C.c_float(), C.c_float()
    lib().orc_fp4_scales_from_amax(float(amax), C.byref(s), C.byref(inv))
    return s.value, inv.value


def stored_count(keep_row: np.ndarray, P: int, W: int) -> int:
    k = _u8(keep_row)
    return int(lib().orc_stored_count(_p(k), int(P), int(W)))


# ---------------------------------------------------------------- prefill

def prefill_layout(keep, T: int, W: int, reserve: int, align: int = 1):
    """keep: [B, Hkv, >=T] bytes.  Returns dict of comp_len, seg_cap,
    seg_base, dst (numpy).  align: segment sizes are rounded up to it."""
    k = _u8(keep)
    B, Hkv, ld = k.shape
    nh = B * Hkv
    comp_len = np.zeros(nh, np.int32)
    seg_cap = np.zeros(nh, np.int32)
    seg_base = np.zeros(nh + 1, np.int64)
    dst = np.zeros((B, Hkv, T), np.int32)
    lib().orc_prefill_layout(B, Hkv, T, W, reserve, align, _p(k), ld, _p(comp_len),
                             _p(seg_cap), _p(seg_base), _p(dst))
    return dict(comp_len=comp_len, seg_cap=seg_cap, seg_base=seg_base, dst=dst)


class OracleCache:
    """The oracle's compact store of one layer (numpy arrays).

    Created by :func:`prefill_pack`; advanced by :meth:`append`."""

    def __init__(self, B, Hkv, D, W, kv_dtype, rows):
        self.B, self.Hkv, self.D, self.W, self.kv_dtype = B, Hkv, D, W, kv_dtype
        rb = row_bytes(D, kv_dtype)
        self.k_pool = np.zeros((rows, rb), np.uint8)
        self.v_pool = np.zeros((rows, rb), np.uint8)
        nh = B * Hkv
        self.seg_base = np.zeros(nh + 1, np.int64)
        self.seg_cap = np.zeros(nh, np.int32)
        self.comp_len = np.zeros(nh, np.int32)
        self.pos = np.zeros(B, np.int32)
        self.ring_keep = np.zeros(max(nh * W, 1), np.uint8)
        self.k_amax = np.zeros(nh, np.float32)
        self.v_amax = np.zeros(nh, np.float32)
        self.err = np.zeros(1, np.int32)
        self.saturated = 0

    def append(self, k_new, v_new, keep_new):
        """k_new, v_new: bf16 [B, Hkv, D]; keep_new: [B, Hkv] bytes."""
        kn, vn, kp = _bits(k_new), _bits(v_new), _u8(keep_new)
        B, Hkv, D = self.B, self.Hkv, self.D
        assert kn.shape == (B, Hkv, D) and kp.shape == (B, Hkv)
        self.saturated += int(lib().orc_append(
            B, Hkv, D, self.W, self.kv_dtype, _p(kn), _p(vn), Hkv * D, D, _p(kp),
            _p(self.k_amax), _p(self.v_amax), _p(self.seg_base), _p(self.seg_cap),
            _p(self.comp_len), _p(self.pos), _p(self.ring_keep), _p(self.k_pool),
            _p(self.v_pool), _p(self.err)))

    def stored_rows(self):
        """Number of valid segment rows per head: min(W, pos) + comp_len."""
        ring = np.minimum(self.W, np.repeat(self.pos, self.Hkv))
        return ring + self.comp_len


def prefill_amax(k, v, keep, T: int, W: int):
    """k, v: bf16 [B, >=T, Hkv, D]; returns (k_amax, v_amax) float32 [B*Hkv]."""
    kb, vb, kp = _bits(k), _bits(v), _u8(keep)
    B, Tt, Hkv, D = kb.shape
    ka = np.zeros(B * Hkv, np.float32)
    va = np.zeros(B * Hkv, np.float32)
    lib().orc_prefill_amax(B, Hkv, D, T, W, _p(kb), _p(vb), Tt * Hkv * D, Hkv * D, D,
                           _p(kp), kp.shape[2], _p(ka), _p(va))
    return ka, va


def prefill_pack(k, v, keep, T: int, W: int, reserve: int, kv_dtype: int,
                 amax=None, align: int = 1) -> OracleCache:
    """Prefill compaction of one layer.  k, v: bf16 [B, >=T, Hkv, D] (only the
    first T positions are read); keep: [B, Hkv, >=T].  amax: optional
    (k_amax, v_amax) to use instead of computing them (FP8, FP4)."""
    kb, vb, kp = _bits(k), _bits(v), _u8(keep)
    B, Tt, Hkv, D = kb.shape
    lay = prefill_layout(kp, T, W, reserve, align)
    rows = int(lay["seg_base"][-1])
    c = OracleCache(B, Hkv, D, W, kv_dtype, rows)
    scale_mode = 0
    if amax is not None:
        c.k_amax[:] = amax[0]
        c.v_amax[:] = amax[1]
        scale_mode = 1
    lib().orc_prefill_pack(B, Hkv, D, T, W, reserve, align, kv_dtype, _p(kb), _p(vb),
                           Tt * Hkv * D, Hkv * D, D, _p(kp), kp.shape[2], scale_mode,
                           _p(c.k_amax), _p(c.v_amax), _p(c.k_pool), _p(c.v_pool),
                           _p(c.ring_keep), _p(c.comp_len), _p(c.seg_cap),
                           _p(c.seg_base), _p(c.pos))
    return c


# ---------------------------------------------------------------- attention

def attention(q, k, v, keep, P, W: int, kv_dtype: int, k_amax=None, v_amax=None,
              sm_scale: float = 0.0):
    """Decode attention from the definition over the dense history.

    q: bf16 [B, Hq, D]; k, v: bf16 [B, >=P+1, Hkv, D]; keep: [B, Hkv, >=P+1];
    P: int or [B] newest position.  Returns (out [B, Hq, D] f64, lse [B, Hq])."""
    qb, kb, vb, kp = _bits(q), _bits(k), _bits(v), _u8(keep)
    B, Hq, D = qb.shape
    _, Tt, Hkv, _ = kb.shape
    Pv = np.ascontiguousarray(np.broadcast_to(np.asarray(P, np.int32), (B,)))
    assert int(Pv.max()) < Tt and kp.shape[2] > int(Pv.max())
    ka = np.ascontiguousarray(k_amax if k_amax is not None else np.zeros(B * Hkv), np.float32)
    va = np.ascontiguousarray(v_amax if v_amax is not None else np.zeros(B * Hkv), np.float32)
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    lib().orc_attention(B, Hq, Hkv, D, W, kv_dtype, _p(Pv), _p(kb), _p(vb),
                        Tt * Hkv * D, Hkv * D, D, _p(kp), kp.shape[2], _p(ka), _p(va),
                        _p(qb), float(sm_scale), _p(out), _p(lse))
    return out, lse


def attention_head(q_row, k, v, keep, b: int, j: int, G: int, P: int, W: int,
                   kv_dtype: int, k_amax=None, v_amax=None, sm_scale: float = 0.0):
    """One (sequence b, query head j) output, for sampled checks at full size.
    k, v: bf16 [B, >=P+1, Hkv, D]; keep: [B, Hkv, >=P+1]; q_row: bf16 [D]."""
    kb, vb, kp, qb = _bits(k), _bits(v), _u8(keep), _bits(q_row)
    B, Tt, Hkv, D = kb.shape
    h = j // G
    i = b * Hkv + h
    off = (b * Tt * Hkv + h) * D
    out = np.zeros(D, np.float64)
    lse = np.zeros(1, np.float64)
    kbase = kb.ctypes.data + 2 * off
    vbase = vb.ctypes.data + 2 * off
    krow = kp.ctypes.data + i * kp.shape[2]
    lib().orc_attention_head(D, W, kv_dtype, int(P), C.c_void_p(kbase), C.c_void_p(vbase),
                             Hkv * D, C.c_void_p(krow),
                             float(k_amax[i]) if k_amax is not None else 0.0,
                             float(v_amax[i]) if v_amax is not None else 0.0,
                             _p(qb), float(sm_scale), _p(out), _p(lse))
    return out, float(lse[0])


# ---------------------------------------------------------------- accounting

def bytes_per_elem(kv_dtype: int) -> float:
    return {BF16: 2, FP8: 1, FP4: 0.5}[kv_dtype]


def row_bytes(D: int, kv_dtype: int) -> int:
    """Bytes of one stored row of D elements (FP4: two elements per byte)."""
    return {BF16: 2 * D, FP8: D, FP4: D // 2}[kv_dtype]


def dense_kv_bytes(layers: int, Hkv: int, D: int, tokens: int, elem_bytes: float) -> float:
    """Bytes of a dense KV pool: every token keeps K and V for every layer and
    KV head (the vLLM baselines of the FastDMS page's memory table)."""
    return float(layers) * Hkv * D * 2 * elem_bytes * tokens


def compact_kv_bytes(stored_tokens: int, D: int, kv_dtype: int, heads: int) -> int:
    """Bytes the compact store holds: every stored token keeps K and V rows of
    D elements, plus two f32 scales per head for FP8 and FP4."""
    b = int(stored_tokens) * 2 * row_bytes(D, kv_dtype)
    if kv_dtype != BF16:
        b += 8 * int(heads)
    return b
