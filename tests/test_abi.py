"""The C-ABI library loads and exports every symbol include/cda.h declares;
host-side argument validation returns the documented status codes.  None of
these calls reach a kernel, so they run without a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from compressed_decode_attention_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from compressed_decode_attention_amd import build
        build.build()
    return _lib


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "cda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == set(lib.EXPORTS), declared
    L = lib.load()
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings(lib):
    assert lib.version() == lib.CDA_VERSION == 7
    assert lib.status_string(0) == "ok"
    assert lib.status_string(3) == "workspace too small"
    assert lib.status_string(99) == "unknown status"


def _cache(lib, **kw):
    c = lib.CdaKvCache()
    c.B, c.Hkv, c.D, c.W, c.kv_dtype = 1, 2, 64, 16, 0
    fake = 0x100000   # never dereferenced: validation fails or the call is not made
    c.seg_base = c.seg_cap = c.comp_len = c.err = c.pos = c.ring_keep = fake
    c.k_amax = c.v_amax = fake
    c.pool_rows = 64
    c.k_pool = c.v_pool = fake
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("D", 96, 2), ("D", 256, 2), ("kv_dtype", 7, 2), ("Hkv", 0, 1), ("W", -1, 1),
    ("B", -1, 1), ("spare_rows", -1, 1), ("seg_base", 0, 1), ("err", 0, 1),
])
def test_cache_validation(lib, field, value, status):
    L = lib.load()
    c = _cache(lib, **{field: value})
    a = lib.CdaCompactArgs()
    a.op = lib.CDA_OP_COUNT
    a.T, a.keep_ld, a.keep = 4, 4, 0x100000
    assert L.kv_compact(C.byref(c), C.byref(a), None) == status


def test_fp4_needs_head_dim_128(lib):
    # the 4-bit store needs K rows of 64 bytes: D = 64 is unsupported
    L = lib.load()
    a = lib.CdaCompactArgs()
    a.op = lib.CDA_OP_PACK
    a.T, a.keep_ld, a.keep = 4, 4, 0x100000
    c = _cache(lib, kv_dtype=lib.CDA_KV_FP4_E2M1, D=64)
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 2
    c = _cache(lib, kv_dtype=lib.CDA_KV_FP4_E2M1, D=128, k_amax=0)   # scales needed
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1


def test_compact_args_validation(lib):
    L = lib.load()
    c = _cache(lib)
    a = lib.CdaCompactArgs()
    assert L.kv_compact(C.byref(c), None, None) == 1
    assert L.kv_compact(None, C.byref(a), None) == 1
    a.op = 9
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.op, a.T, a.keep_ld, a.keep = lib.CDA_OP_COUNT, 10, 5, 0x100000   # keep_ld < T
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.keep_ld, a.keep = 10, 0                                          # keep NULL
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.keep, a.reserve = 0x100000, -1
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    # PACK: misaligned k, stride not a multiple of 8, bad scale mode, bad pool_rows
    a.op, a.reserve, a.k, a.v = lib.CDA_OP_PACK, 0, 0x100002, 0x100000
    a.stride_b = a.stride_t = a.stride_h = 64
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.k, a.stride_t = 0x100000, 12
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.stride_t, a.scale_mode = 64, 2
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    c2 = _cache(lib, pool_rows=100)
    a.scale_mode = 0
    assert L.kv_compact(C.byref(c2), C.byref(a), None) == 1
    # APPEND without keep
    a.op, a.keep = lib.CDA_OP_APPEND, 0
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1


def test_attention_validation(lib):
    L = lib.load()
    c = _cache(lib)
    q = out = ws = C.c_void_p(0x100000)
    need = L.cda_attn_workspace_bytes(C.byref(c), 8, 0)
    assert need > 0
    f = L.decode_attn_compact
    assert f(C.byref(c), q, 7, 0.0, out, 0, None, 0, ws, need, None) == 2        # Hq % Hkv
    assert f(C.byref(c), q, 2 * 17, 0.0, out, 0, None, 0, ws, need, None) == 2   # G > 16
    assert f(C.byref(c), q, 8, 0.0, out, 5, None, 0, ws, need, None) == 2        # out dtype
    assert f(C.byref(c), q, 8, 0.0, out, 0, None, 0, ws, need - 1, None) == 3    # workspace
    assert f(C.byref(c), C.c_void_p(0x100001), 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    assert f(C.byref(c), q, 8, 0.0, out, 0, None, -5, ws, need, None) == 1       # split < 0
    assert f(None, q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    # a bigger split never needs more workspace
    assert L.cda_attn_workspace_bytes(C.byref(c), 8, 4096) <= need
    assert L.cda_attn_workspace_bytes(C.byref(c), 7, 0) == 0


def test_decode_step_validation(lib):
    L = lib.load()
    c = _cache(lib)
    q = out = ws = C.c_void_p(0x100000)
    need = L.cda_attn_workspace_bytes(C.byref(c), 8, 0)
    a = lib.CdaCompactArgs()
    a.op, a.keep, a.k, a.v = lib.CDA_OP_APPEND, 0x100000, 0x100000, 0x100000
    a.stride_b, a.stride_h = 128, 64
    f = L.decode_step_compact
    # attention checks come first, as for decode_attn_compact
    assert f(C.byref(c), C.byref(a), q, 7, 0.0, out, 0, None, 0, ws, need, None) == 2
    assert f(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need - 1, None) == 3
    assert f(None, C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    # then the APPEND arguments
    assert f(C.byref(c), None, q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    a.op = lib.CDA_OP_PACK
    assert f(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    a.op, a.keep = lib.CDA_OP_APPEND, 0
    assert f(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    a.keep, a.k = 0x100000, 0x100008                                   # misaligned k
    assert f(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1
    a.k, a.stride_h = 0x100000, 12                                     # stride not a multiple of 8
    assert f(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need, None) == 1


def _default_split_rule(pool_rows, nh):
    """The documented default: smallest unit (in 64-row tiles) whose estimated
    number of units, pool_rows/64/t + nh/2, stays <= 248."""
    fits = lambda t: pool_rows / 64 / t + nh / 2 <= 248
    if pool_rows < 65536 and fits(4):
        return 4
    return next((t for t in (8, 12, 16, 24, 32, 48, 64) if fits(t)), 8)


@pytest.mark.parametrize("B,Hkv,pool_rows", [
    (1, 8, 11776),       # c = 1, ctx 8192: 256-row units
    (8, 8, 98304),       # c = 8, 24 tiles a segment: 512
    (8, 8, 126976),      # c = 8, 31 tiles a segment: 768
    (8, 8, 61440),       # a small pool that does not fit at 4 tiles: 512
    (8, 8, 262144),      # long segments (64 tiles): 1536
    (64, 8, 1 << 22),    # 512 segments: nothing fits, 512
    (1, 1, 64),
])
def test_default_split(lib, B, Hkv, pool_rows):
    # the default shows in the workspace size, which falls with the unit size
    L = lib.load()
    c = _cache(lib, B=B, Hkv=Hkv, pool_rows=pool_rows)
    t = _default_split_rule(pool_rows, B * Hkv)
    assert L.cda_attn_workspace_bytes(C.byref(c), 4 * Hkv, 0) == \
        L.cda_attn_workspace_bytes(C.byref(c), 4 * Hkv, 64 * t)
    if pool_rows // (64 * t) != pool_rows // 512:     # the unit bound differs from 512's
        assert L.cda_attn_workspace_bytes(C.byref(c), 4 * Hkv, 0) != \
            L.cda_attn_workspace_bytes(C.byref(c), 4 * Hkv, 512)
    expect = {11776: 4, 98304: 8, 126976: 12, 61440: 8, 262144: 24, 1 << 22: 8, 64: 4}
    assert t == expect[pool_rows]


def _paged(lib, **kw):
    c = _cache(lib, **kw)
    fake = 0x100000
    c.page_table = c.free_pages = c.free_top = fake
    c.max_pages = 4
    c.seg_base = 0          # not used by a paged store
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value", [("max_pages", 0), ("reserved1", 1), ("free_pages", 0),
                                         ("free_top", 0), ("pos", 0), ("ring_keep", 0)])
def test_paged_cache_validation(lib, field, value):
    L = lib.load()
    c = _paged(lib, **{field: value})
    a = lib.CdaCompactArgs()
    a.op = lib.CDA_OP_REFILL
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1


def test_paged_ranges_and_ops(lib):
    L = lib.load()
    a = lib.CdaCompactArgs()
    # page operations need a paged store; ranges need one too
    c = _cache(lib)
    for op in (lib.CDA_OP_PAGE_INIT, lib.CDA_OP_REFILL, lib.CDA_OP_RELEASE):
        a.op = op
        assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    a.op, a.seq_count = lib.CDA_OP_COUNT, 1
    assert L.kv_compact(C.byref(c), C.byref(a), None) == 1
    # a paged store: ranges inside the batch only
    p = _paged(lib, B=2)
    a.op, a.T, a.keep, a.keep_ld = lib.CDA_OP_COUNT, 0, 0, 0
    for b0, n in ((0, -1), (-1, 1), (2, 1), (1, 2), (1, 0)):
        a.seq_begin, a.seq_count = b0, n
        assert L.kv_compact(C.byref(p), C.byref(a), None) == 1, (b0, n)
    a.op, a.seq_begin, a.seq_count, a.reserve = lib.CDA_OP_REFILL, 0, 0, -1
    assert L.kv_compact(C.byref(p), C.byref(a), None) == 1
    # the append and the decode step always cover the whole batch
    a.op, a.seq_count, a.reserve = lib.CDA_OP_APPEND, 1, 0
    a.keep = a.k = a.v = 0x100000
    assert L.kv_compact(C.byref(p), C.byref(a), None) == 1
    q = out = ws = C.c_void_p(0x100000)
    need = L.cda_attn_workspace_bytes(C.byref(p), 8, 0)
    assert L.decode_step_compact(C.byref(p), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws, need,
                                 None) == 1


def test_chunk_validation(lib):
    L = lib.load()
    c = _cache(lib)
    a = lib.CdaCompactArgs()
    a.op, a.keep, a.k, a.v = lib.CDA_OP_APPEND, 0x100000, 0x100000, 0x100000
    a.stride_b, a.stride_t, a.stride_h = 512, 128, 64
    q = out = ws = C.c_void_p(0x100000)
    f = L.chunk_attn_compact
    need = L.cda_chunk_workspace_bytes(C.byref(c), 8, 4)
    assert need > 0
    assert L.cda_chunk_workspace_bytes(C.byref(c), 8, 0) == 0
    assert L.cda_chunk_workspace_bytes(C.byref(c), 8, lib.CDA_MAX_CHUNK + 1) == 0
    assert f(C.byref(c), C.byref(a), 0, q, 8, 0.0, out, 0, None, ws, need, None) == 1     # M = 0
    assert f(C.byref(c), C.byref(a), 65, q, 8, 0.0, out, 0, None, ws, need, None) == 1    # M > 64
    assert f(C.byref(c), C.byref(a), 4, q, 7, 0.0, out, 0, None, ws, need, None) == 2     # Hq % Hkv
    assert f(C.byref(c), C.byref(a), 4, q, 8, 0.0, out, 3, None, ws, need, None) == 2     # out dtype
    assert f(C.byref(c), C.byref(a), 4, q, 8, 0.0, out, 0, None, ws, need - 1, None) == 3  # workspace
    assert f(C.byref(c), C.byref(a), 4, q, 8, 0.0, out, 0, None, C.c_void_p(0x100010), need,
             None) == 1                                                                   # ws alignment
    a.stride_t = 12
    assert f(C.byref(c), C.byref(a), 4, q, 8, 0.0, out, 0, None, ws, need, None) == 1     # stride
    a.stride_t, a.op = 128, lib.CDA_OP_PACK
    assert f(C.byref(c), C.byref(a), 4, q, 8, 0.0, out, 0, None, ws, need, None) == 1     # not APPEND
    c2 = _cache(lib, W=lib.CDA_MAX_CHUNK_WINDOW + 1)
    assert f(C.byref(c2), C.byref(a), 4, q, 8, 0.0, out, 0, None, ws,
             L.cda_chunk_workspace_bytes(C.byref(c2), 8, 4), None) == 2                 # W too large
    # the workspace grows with the segments: their chunk tiles, and the
    # partial states once segments outnumber the 256 attention workgroups
    # (the partial states do not grow with M: the workgroups stay ~256)
    assert L.cda_chunk_workspace_bytes(C.byref(c), 32, 64) == \
        L.cda_chunk_workspace_bytes(C.byref(c), 32, 16)
    c3 = _cache(lib, B=300)
    tile = 64 * 64 * 2   # one BF16 D = 64 tile
    assert (L.cda_chunk_workspace_bytes(C.byref(c3), 8, 4) - need >
            2 * tile * (300 * 2 - 2))


@pytest.mark.parametrize("table", [
    [64, 64, 128],        # does not start at 0
    [0, 128, 64],         # decreasing
    [0, 100, 192],        # not a multiple of 64
    [0, 64, 4096],        # past the pool (pool_rows 1024)
])
def test_host_seg_base_is_checked(lib, table):
    # the host copy of seg_base steers which pool rows the kernels read, so
    # every call checks it before anything is enqueued
    L = lib.load()
    c = _cache(lib, B=1, Hkv=2, pool_rows=1024)
    host = (C.c_int64 * 3)(*table)
    c.seg_base_host = C.cast(host, C.c_void_p)
    need = L.cda_attn_workspace_bytes(C.byref(c), 8, 0)
    ws, q, out = 0x200000, 0x300000, 0x400000
    st = L.decode_attn_compact(C.byref(c), C.c_void_p(q), 8, 0.0, C.c_void_p(out), 0, None, 0,
                               C.c_void_p(ws), C.c_size_t(need), None)
    assert st == lib.CDA_ERR_INVALID_ARG


def test_noalloc_step_validates_before_any_hip_call(lib):
    """decode_step_compact_noalloc: the scratch the call needs is checked
    against CDA_SCRATCH_BYTES, and every argument, before anything is
    enqueued (fake pointers: no call here reaches a kernel)."""
    L = lib.load()
    a = lib.CdaCompactArgs()
    a.op, a.keep, a.k, a.v = lib.CDA_OP_APPEND, 0x100000, 0x100000, 0x100000
    q = out = C.c_void_p(0x100000)
    big = _cache(lib, pool_rows=64 * 100000)      # 12502 units of 8 x 64 f32 partials
    need = L.cda_attn_workspace_bytes(C.byref(big), 16, 0)
    assert need > lib.CDA_SCRATCH_BYTES
    assert L.decode_step_compact_noalloc(C.byref(big), C.byref(a), q, 16, 0.0, out, 0, None, 0,
                                         None) == 3
    c = _cache(lib)
    assert L.decode_step_compact_noalloc(C.byref(c), C.byref(a), q, 3, 0.0, out, 0, None, 0,
                                         None) == 2          # Hq % Hkv
    assert L.decode_step_compact_noalloc(C.byref(c), C.byref(a), C.c_void_p(0x100001), 8, 0.0,
                                         out, 0, None, 0, None) == 1   # misaligned q
    a.op = lib.CDA_OP_COUNT
    assert L.decode_step_compact_noalloc(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0,
                                         None) == 1


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="needs a host without a GPU: with one, these fake pointers would "
                           "reach a kernel")
def test_failed_hip_call_returns_err_hip(lib):
    """Arguments that pass every host check, on a host where the HIP runtime
    finds no device: each entry point returns CDA_ERR_HIP (the status of a
    failed HIP call or launch) rather than aborting."""
    L = lib.load()
    a = lib.CdaCompactArgs()
    a.op, a.keep, a.k, a.v = lib.CDA_OP_APPEND, 0x100000, 0x100000, 0x100000
    q = out = C.c_void_p(0x100000)
    c = _cache(lib)
    need = L.cda_attn_workspace_bytes(C.byref(c), 8, 0)
    ws = C.c_void_p(0x200000)
    assert L.kv_compact(C.byref(c), C.byref(a), None) == lib.CDA_ERR_HIP
    assert L.decode_attn_compact(C.byref(c), q, 8, 0.0, out, 0, None, 0, ws, C.c_size_t(need),
                                 None) == lib.CDA_ERR_HIP
    assert L.decode_step_compact(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0, ws,
                                 C.c_size_t(need), None) == lib.CDA_ERR_HIP
    assert L.decode_step_compact_noalloc(C.byref(c), C.byref(a), q, 8, 0.0, out, 0, None, 0,
                                         None) == lib.CDA_ERR_HIP
