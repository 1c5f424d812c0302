"""Multi-query chunk attention over the compact store (chunk_attn_compact).

Query t of a chunk of M tokens must equal the oracle's decode attention at
position P + t (fp64, from the definition over the dense history: the rows
stored after the tokens P .. P+t were appended one by one), and afterwards
the store must be bit for bit the oracle's after M appends.  Cases cover a
chunk longer than the window (chunk tokens leave it unkept), a ring not yet
full (P < W), W = 0, one-token chunks, every storage format, GQA 4 and 8,
chunks followed by chunks and by decode steps, the paged store, many
segments, and full-size layers of the c = 8 workloads in chunks of 64."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import (CDA_SEG_ALIGN, check_close, compare_state, dev, gpu_prefill, log, odt,
                          oracle_prefill, segment_rows)
from compressed_decode_attention_amd import PagedKVCache

pytestmark = pytest.mark.gpu


def _chunk_inputs(lay, T, s0, M):
    """Tokens T+s0 .. T+s0+M-1 of a workload layer, shaped for one chunk."""
    k = lay.k[:, T + s0:T + s0 + M].contiguous()                      # [B, M, Hkv, D]
    v = lay.v[:, T + s0:T + s0 + M].contiguous()
    keep = lay.keep[:, :, T + s0:T + s0 + M].permute(0, 2, 1).contiguous()   # [B, M, Hkv]
    q = lay.q[s0:s0 + M].permute(1, 0, 2, 3).contiguous()              # [B, M, Hq, D]
    return k, v, keep, q


def _check_chunk(out, lse, lay, T, s0, M, W, kv, o, what):
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    ka = o.k_amax if kv != "bf16" else None
    va = o.v_amax if kv != "bf16" else None
    for t in range(M):
        ref, rl = oracle.attention(lay.q[s0 + t], lay.k, lay.v, lay.keep, T + s0 + t, W, odt(kv),
                                   ka, va)
        worst = max(worst, check_close(got[:, t], ref, f"{what} query {t}"))
        check_close(gl[:, t], rl, f"{what} query {t} lse", atol=1e-4, rtol=1e-5)
    return worst


def _oracle_append(o, lay, T, s0, M):
    for t in range(M):
        p = T + s0 + t
        o.append(lay.k[:, p], lay.v[:, p], lay.keep[:, :, p])


@pytest.mark.parametrize("kv,D,W,M,T,B,Hkv,G", [
    ("bf16", 64, 32, 8, 300, 2, 2, 4),
    ("fp8", 128, 64, 16, 500, 2, 2, 4),
    ("fp4", 128, 48, 64, 700, 1, 2, 4),       # chunk longer than the window
    ("fp8", 64, 16, 40, 200, 3, 1, 8),        # GQA 8, chunk longer than the window
    ("bf16", 128, 0, 5, 100, 2, 2, 4),        # W = 0: only kept tokens are stored
    ("fp8", 128, 64, 10, 20, 2, 2, 4),        # P < W: the ring is not full yet
    ("bf16", 64, 16, 1, 150, 2, 4, 2),        # a one-token chunk
    ("fp4", 128, 64, 33, 1000, 2, 2, 16),     # GQA 16
    ("bf16", 128, 32, 64, 300, 1, 2, 4),      # BF16 through the wide kernel
    ("bf16", 64, 16, 40, 200, 2, 2, 8),
    ("fp4", 128, 33, 64, 20, 2, 2, 4),        # odd W, P < W: rows 32 and 33 share V bytes
    ("fp4", 128, 33, 50, 400, 2, 2, 4),       # odd W, full ring
])
def test_chunk_matches_sequential_decode(kv, D, W, M, T, B, Hkv, G):
    S = M + 8
    cfg = workload.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype=kv,
                          keep_lo=0.2, keep_hi=0.6, seed=600 + M)
    lay = workload.make_layer(cfg, 0)
    log(f"chunk {kv} D={D} W={W} M={M} T={T} B={B} Hkv={Hkv} G={G}")
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, S, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, S, kv)
    d = dev()
    k, v, keep, q = (x.to(d) for x in _chunk_inputs(lay, T, 0, M))
    lse = torch.empty(B, M, G * Hkv, dtype=torch.float32, device=d)
    out = c.chunk(k, v, keep, q, out_dtype=torch.float32, lse=lse)
    _check_chunk(out, lse, lay, T, 0, M, W, kv, o, "chunk")
    _oracle_append(o, lay, T, 0, M)
    compare_state(c, o, "after the chunk")
    # a BF16 output is the F32 one rounded
    c2, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, S, kv, with_dst=False)
    ob = c2.chunk(k, v, keep, q, out_dtype=torch.bfloat16)
    assert torch.equal(ob, out.to(torch.bfloat16))
    # the next tokens by decode steps continue from the chunk's state
    kd, vd, qd = lay.k.to(d), lay.v.to(d), lay.q.to(d)
    keep_new = lay.keep[:, :, T:].permute(2, 0, 1).contiguous().to(d)
    for s in range(M, S):
        out1 = c.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s], out_dtype=torch.float32)
        o.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s])
    torch.cuda.synchronize()
    ref, _ = oracle.attention(lay.q[S - 1], lay.k, lay.v, lay.keep, T + S - 1, W, odt(kv),
                              o.k_amax if kv != "bf16" else None, o.v_amax if kv != "bf16" else None)
    check_close(out1.cpu().numpy(), ref, "decode after the chunk")
    compare_state(c, o, "after the decode steps")
    assert c.error_word() == 0


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_chunks_in_a_row(kv):
    """A prompt continued in chunks of uneven sizes on a compacted prefix."""
    B, Hkv, G, D, W, T = 2, 2, 4, 128, 32, 256
    sizes = [17, 64, 1, 30, 64]
    S = sum(sizes)
    cfg = workload.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype=kv,
                          keep_lo=0.1, keep_hi=0.4, seed=77)
    lay = workload.make_layer(cfg, 0)
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, S, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, S, kv)
    d = dev()
    s0 = 0
    for M in sizes:
        k, v, keep, q = (x.to(d) for x in _chunk_inputs(lay, T, s0, M))
        lse = torch.empty(B, M, G * Hkv, dtype=torch.float32, device=d)
        out = c.chunk(k, v, keep, q, out_dtype=torch.float32, lse=lse)
        _check_chunk(out, lse, lay, T, s0, M, W, kv, o, f"chunk at {s0}")
        _oracle_append(o, lay, T, s0, M)
        compare_state(c, o, f"after the chunk at {s0}")
        s0 += M
    assert c.error_word() == 0


def test_chunk_on_the_paged_store():
    """Chunks over a paged store with idle slots; a refill first makes room."""
    B, Hkv, G, D, W = 3, 2, 4, 128, 32
    d = dev()
    c = PagedKVCache(B, Hkv, D, W, n_pages=64, max_pages=16, kv_dtype="fp8", device=d)
    reqs = {}
    for slot, (T, seed) in {0: (300, 1), 2: (450, 2)}.items():
        cfg = workload.custom(B=1, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=80, W=W, kv_dtype="fp8",
                              keep_lo=0.2, keep_hi=0.5, seed=seed)
        lay = workload.make_layer(cfg, 0)
        c.admit(slot, lay.k[:, :T].to(d), lay.v[:, :T].to(d),
                lay.keep[:, :, :T].contiguous().to(d), T, 0)
        reqs[slot] = (lay, T, oracle.prefill_pack(lay.k, lay.v, lay.keep, T, W, 80, oracle.FP8,
                                                  align=CDA_SEG_ALIGN))
    s0 = 0
    for M in (40, 24):
        c.refill(64)
        ks = torch.zeros(B, M, Hkv, D, dtype=torch.bfloat16)
        vs, qs = torch.zeros_like(ks), torch.zeros(B, M, G * Hkv, D, dtype=torch.bfloat16)
        keeps = torch.zeros(B, M, Hkv, dtype=torch.uint8)
        for slot, (lay, T, _) in reqs.items():
            k, v, keep, q = _chunk_inputs(lay, T, s0, M)
            ks[slot], vs[slot], keeps[slot], qs[slot] = k[0], v[0], keep[0], q[0]
        lse = torch.empty(B, M, G * Hkv, dtype=torch.float32, device=d)
        out = c.chunk(ks.to(d), vs.to(d), keeps.to(d), qs.to(d), out_dtype=torch.float32, lse=lse)
        torch.cuda.synchronize()
        assert np.all(out[1].cpu().numpy() == 0) and np.all(np.isneginf(lse[1].cpu().numpy()))
        for slot, (lay, T, o) in reqs.items():
            _check_chunk(out[slot:slot + 1], lse[slot:slot + 1], lay, T, s0, M, W, "fp8", o,
                         f"slot {slot} chunk at {s0}")
            _oracle_append(o, lay, T, s0, M)
            n = o.stored_rows()
            for h in range(Hkv):
                kr, vr = segment_rows(c, slot * Hkv + h, int(n[h]))
                a = int(o.seg_base[h])
                assert np.array_equal(kr.cpu().numpy(), o.k_pool[a:a + n[h]])
                assert np.array_equal(vr.cpu().numpy(), o.v_pool[a:a + n[h]])
        assert int(c.pos[1].item()) == -1
        s0 += M
    assert c.error_word() == 0


@pytest.mark.parametrize("kv", ["fp8", "fp4"])
def test_chunk_past_the_capacity(kv):
    """A chunk whose kept tokens overflow the compact region: the surplus is
    dropped with CDA_DEVERR_CAPACITY, as M APPENDs would drop it (the oracle
    drops the same tokens)."""
    B, Hkv, G, D, W, T, M, reserve = 2, 2, 4, 128, 16, 300, 64, 5
    cfg = workload.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=M, W=W, kv_dtype=kv,
                          keep_lo=0.8, keep_hi=0.95, seed=31)
    lay = workload.make_layer(cfg, 0)
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, reserve, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, reserve, kv)
    d = dev()
    k, v, keep, q = (x.to(d) for x in _chunk_inputs(lay, T, 0, M))
    c.chunk(k, v, keep, q, out_dtype=torch.float32)
    _oracle_append(o, lay, T, 0, M)
    compare_state(c, o, "after the chunk")
    from compressed_decode_attention_amd import CDA_DEVERR_CAPACITY
    assert c.error_word() & CDA_DEVERR_CAPACITY
    assert int(o.err[0]) & CDA_DEVERR_CAPACITY


@pytest.mark.parametrize("kv,B,Hkv", [
    ("fp8", 40, 2),      # 80 segments: the wide kernel's plan takes two passes of 64
    ("bf16", 130, 2),    # 260 segments: more than 256 workgroups, one split each
])
def test_chunk_many_segments(kv, B, Hkv):
    """Chunks over more segments than one wave's lanes, and more than the
    workgroups a chunk call starts by default, through the wide kernel."""
    G, D, W, T, M = 4, 64, 16, 90, 16
    cfg = workload.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=M + 1, W=W, kv_dtype=kv,
                          keep_lo=0.05, keep_hi=0.9, seed=900 + B)
    lay = workload.make_layer(cfg, 0)
    log(f"chunk many segments {kv} B={B} Hkv={Hkv}")
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, M + 1, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, M + 1, kv)
    d = dev()
    k, v, keep, q = (x.to(d) for x in _chunk_inputs(lay, T, 0, M))
    lse = torch.empty(B, M, G * Hkv, dtype=torch.float32, device=d)
    out = c.chunk(k, v, keep, q, out_dtype=torch.float32, lse=lse)
    _check_chunk(out, lse, lay, T, 0, M, W, kv, o, "chunk")
    _oracle_append(o, lay, T, 0, M)
    compare_state(c, o, "after the chunk")
    assert c.error_word() == 0


@pytest.mark.parametrize("name,layer,kv", [("qwen_c8", 0, "fp8"), ("qwen_c8", 35, "fp4"),
                                           ("llama_c8", 0, "bf16")])
def test_chunk_config_layer(name, layer, kv):
    """A full-size layer of the c = 8 workloads (ctx 8192, 128 new tokens) in
    chunks of 64, as `bench.py --chunk 64` runs it (reserve = the 128 new
    tokens): queries 0, 31 and 63 of every chunk against the oracle, the
    store bit-exact after every chunk."""
    cfg = workload.CONFIGS[name]
    T, S, W, M = cfg.T, cfg.S, cfg.W, 64
    lay = workload.make_layer(cfg, layer)
    log(f"chunk config {name} layer {layer} {kv}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} T={T}")
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, S, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, S, kv)
    d = dev()
    ka = o.k_amax if kv != "bf16" else None
    va = o.v_amax if kv != "bf16" else None
    for s0 in range(0, S, M):
        k, v, keep, q = (x.to(d) for x in _chunk_inputs(lay, T, s0, M))
        lse = torch.empty(cfg.B, M, cfg.Hq, dtype=torch.float32, device=d)
        out = c.chunk(k, v, keep, q, out_dtype=torch.float32, lse=lse)
        torch.cuda.synchronize()
        got, gl = out.cpu().numpy(), lse.cpu().numpy()
        for t in (0, M // 2 - 1, M - 1):
            ref, rl = oracle.attention(lay.q[s0 + t], lay.k, lay.v, lay.keep, T + s0 + t, W,
                                       odt(kv), ka, va)
            check_close(got[:, t], ref, f"{name} chunk {s0} query {t}")
            check_close(gl[:, t], rl, f"{name} chunk {s0} query {t} lse", atol=1e-4, rtol=1e-5)
        _oracle_append(o, lay, T, s0, M)
        compare_state(c, o, f"after the chunk at {s0}")
    assert c.error_word() == 0
