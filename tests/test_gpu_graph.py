"""Decode steps, prefill compaction and attention captured in a HIP graph
(torch.cuda.CUDAGraph) give, on every replay, exactly the results of the
same calls issued eagerly: the kernels use no memset and allocate nothing,
every replay restarts from the prefill, and the split merge gives the same
bits whichever unit of a segment finishes last.  Replays are interleaved
with eager work and synchronisations."""
import pytest
import torch

import workload
from _cda_testlib import dev, gpu_prefill, k_rows, log, stored_rows, v_rows

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    B, Hq, Hkv, D, T, S, W = 2, 16, 4, 128, 3000, 6, 64
    log("graph capture of prefill + decode steps + attention")
    keep = workload.random_keep((B, Hkv, T + S), 0.25, seed=81)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=82)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=83)
    q = workload.random_bf16((S, B, Hq, D), seed=84)
    kd, vd, keepd, qd = k.to(dev()), v.to(dev()), keep.to(dev()), q.to(dev())
    keep_new = keepd[:, :, T:].permute(2, 0, 1).contiguous()
    split = 256   # several units per head: the split merge runs

    # eager reference
    ce, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    ref = []
    for s in range(S):
        ref.append(ce.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                                  out_dtype=torch.float32, split_tokens=split).clone())
    ref_attn = ce.attention(qd[S - 1], out_dtype=torch.float32, split_tokens=split).clone()
    torch.cuda.synchronize()
    assert ce.error_word() == 0

    # the same calls captured once
    cg, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    cg.workspace(Hq, split)
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev()) for _ in range(S + 1)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cg.count(keepd, T, reserve=S)
        cg.pack(kd, vd, keepd, T)
        for s in range(S):
            cg.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s], out=outs[s],
                           split_tokens=split)
        cg.attention(qd[S - 1], out=outs[S], split_tokens=split)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for s in range(S):
            assert torch.equal(outs[s], ref[s]), f"replay {rep} step {s}"
        assert torch.equal(outs[S], ref_attn), f"replay {rep} attention"
        assert cg.error_word() == 0, f"replay {rep}: error word {cg.error_word()}"
        assert torch.equal(cg.comp_len, ce.comp_len) and torch.equal(cg.pos, ce.pos)
        assert torch.equal(cg.ring_keep, ce.ring_keep)
        # eager work on the other cache between replays
        ce.attention(qd[0], out_dtype=torch.float32, split_tokens=64)
        torch.cuda.synchronize()


def same_stored_rows(a, b):
    """The rows holding data (the full ring, then the compact rows) of every
    segment are the same bytes in both stores (same layout)."""
    assert torch.equal(a.seg_base, b.seg_base) and bool((a.pos >= a.W).all())
    n, sb = stored_rows(a).tolist(), a.seg_base.tolist()
    ka, kb, va, vb = k_rows(a), k_rows(b), v_rows(a), v_rows(b)
    return all(torch.equal(ka[sb[i]:sb[i] + n[i]], kb[sb[i]:sb[i] + n[i]]) and
               torch.equal(va[sb[i]:sb[i] + n[i]], vb[sb[i]:sb[i] + n[i]]) for i in range(len(n)))


def test_graph_replays_of_chunk_calls_match_eager():
    # prefill, two chunk calls and a decode step captured once: every replay
    # gives the eager bits (the chunk launches write their per-call counters
    # themselves and allocate nothing)
    B, Hq, Hkv, D, T, W, M = 2, 16, 4, 128, 2000, 64, 24
    S = 2 * M + 1
    log("graph capture of prefill + chunk calls + a decode step")
    keep = workload.random_keep((B, Hkv, T + S), 0.25, seed=91)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=92)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=93)
    q = workload.random_bf16((S, B, Hq, D), seed=94)
    kd, vd, keepd, qd = k.to(dev()), v.to(dev()), keep.to(dev()), q.to(dev())
    chunks = []
    for c in range(2):
        a, e = T + c * M, T + (c + 1) * M
        chunks.append((kd[:, a:e].contiguous(), vd[:, a:e].contiguous(),
                       keepd[:, :, a:e].permute(0, 2, 1).contiguous(),
                       qd[c * M:(c + 1) * M].permute(1, 0, 2, 3).contiguous()))
    tl = T + 2 * M
    keep_last = keepd[:, :, tl].contiguous()

    ce, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    ref = [ce.chunk(*x, out_dtype=torch.float32).clone() for x in chunks]
    ref.append(ce.decode_step(kd[:, tl], vd[:, tl], keep_last, qd[2 * M],
                              out_dtype=torch.float32).clone())
    torch.cuda.synchronize()
    assert ce.error_word() == 0

    cg, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    cg.chunk_workspace(Hq, M)
    cg.workspace(Hq, 0)
    outs = [torch.empty((B, M, Hq, D), dtype=torch.float32, device=dev()) for _ in range(2)]
    outs.append(torch.empty((B, Hq, D), dtype=torch.float32, device=dev()))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cg.count(keepd, T, reserve=S)
        cg.pack(kd, vd, keepd, T)
        for x, o in zip(chunks, outs):
            cg.chunk(*x, out=o)
        cg.decode_step(kd[:, tl], vd[:, tl], keep_last, qd[2 * M], out=outs[2])
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep} call {j}"
        assert cg.error_word() == 0, f"replay {rep}: error word {cg.error_word()}"
        assert torch.equal(cg.comp_len, ce.comp_len) and torch.equal(cg.pos, ce.pos)
        assert torch.equal(cg.ring_keep, ce.ring_keep)
        assert same_stored_rows(cg, ce), f"replay {rep}: stored rows"
        # eager work on the other cache between replays
        ce.attention(qd[0], out_dtype=torch.float32, split_tokens=64)
        torch.cuda.synchronize()
