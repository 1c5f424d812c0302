"""Decode steps, prefill compaction and attention captured in a HIP graph
(torch.cuda.CUDAGraph) give, on every replay, exactly the results of the
same calls issued eagerly: the kernels use no memset and allocate nothing,
every replay restarts from the prefill, and the XCD-local merge holds under
the workgroup-to-XCD rotation graph replays use.  Replays are interleaved
with eager work and synchronisations."""
import pytest
import torch

import workload
from _cda_testlib import dev, gpu_prefill, log

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
    split = 256   # several units per head: the XCD-local merge runs

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
