"""GPU parity of decode_step_compact (the append and the attention of one
decode step in a single launch).  After every step the cache must be bit for
bit the oracle's (and what kv_compact APPEND leaves on a second cache), and
the output must match the oracle's fp64 attention over the stored set after
the append (F32 output, |gpu - oracle| <= 2e-3 + 1e-2 |oracle|), through the
ring filling up, tokens leaving it kept or not, W = 0, a full compact region,
several GQA widths and work-unit sizes."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import (check_close, compare_state, dev, gpu_prefill, log, odt,
                          oracle_prefill)

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D, T, S, W, rate, kv_dtype, seed, reserve, split
    (2, 16, 4, 128, 700, 40, 64, 0.2, "fp8", 1, 40, 0),
    (2, 16, 4, 64, 700, 40, 64, 0.3, "bf16", 2, 40, 0),
    (2, 16, 4, 128, 500, 40, 256, 0.2, "bf16", 3, 40, 64),   # many units per segment
    (2, 8, 2, 64, 300, 40, 0, 0.3, "fp8", 4, 40, 0),         # W = 0: kept tokens go to the tail
    (1, 8, 8, 128, 30, 60, 64, 0.5, "fp8", 5, 60, 0),        # ring fills, then tokens leave; G = 1
    (2, 24, 8, 64, 400, 30, 1, 0.4, "bf16", 6, 30, 0),       # W = 1, G = 3
    (1, 32, 2, 128, 900, 30, 100, 0.25, "fp8", 7, 30, 128),  # G = 16
    (2, 16, 2, 64, 200, 30, 16, 0.9, "fp8", 8, 3, 0),        # compact region fills: CAPACITY
    (3, 8, 1, 128, 0, 70, 64, 0.5, "bf16", 9, 70, 0),        # empty prefill
    (2, 8, 2, 64, 0, 20, 0, 0.5, "bf16", 10, 8, 0),          # W = 0, empty prefill, region fills
    (2, 16, 4, 128, 700, 40, 64, 0.2, "fp4", 11, 40, 0),     # 4-bit store
    (1, 8, 8, 128, 30, 60, 64, 0.5, "fp4", 12, 60, 0),       # FP4: ring fills, tokens leave
    (2, 24, 8, 128, 400, 30, 1, 0.4, "fp4", 13, 30, 0),      # FP4, W = 1: moved row pairs with the ring row
    (2, 16, 2, 128, 300, 40, 7, 0.6, "fp4", 14, 40, 64),     # FP4, odd W
    (2, 8, 2, 128, 200, 40, 0, 0.5, "fp4", 15, 40, 0),       # FP4, W = 0
]


def _effective_keep(keep, o_before_cl, o, P, W):
    """The keep mask of what the oracle cache really stores after appending
    position P: a kept token the full compact region dropped counts as not
    kept (the definition's stored set with that token evicted)."""
    B, Hkv = keep.shape[:2]
    grew = (o.comp_len - o_before_cl).reshape(B, Hkv)
    p = P - W if W > 0 else P
    if p < 0:
        return
    kp = keep[:, :, p].numpy() != 0
    dropped = kp & (grew == 0)
    for b, h in zip(*np.nonzero(dropped)):
        keep[b, h, p] = 0


@pytest.mark.parametrize("case", CASES, ids=[f"s{i}" for i in range(len(CASES))])
def test_decode_step_matches_oracle(case):
    B, Hq, Hkv, D, T, S, W, rate, kv_dtype, seed, reserve, split = case
    log(f"decode step case B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} S={S} W={W} {kv_dtype} "
        f"reserve={reserve} split={split}")
    keep = workload.random_keep((B, Hkv, T + S), rate, seed=seed)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 1)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 2)
    q = workload.random_bf16((S, B, Hq, D), seed=seed + 3)
    ca, _ = gpu_prefill(k, v, keep, T, W, reserve, kv_dtype, with_dst=False)   # fused step
    cb, _ = gpu_prefill(k, v, keep, T, W, reserve, kv_dtype, with_dst=False)   # APPEND, attention
    o = oracle_prefill(k, v, keep, T, W, reserve, kv_dtype)
    compare_state(ca, o, "prefill")
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    keep_new = keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev())        # [S, B, Hkv]
    ka = ca.k_amax.cpu().numpy() if kv_dtype != "bf16" else None
    va = ca.v_amax.cpu().numpy() if kv_dtype != "bf16" else None
    keep_eff = keep.clone()
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev())
    worst = 0.0
    for s in range(S):
        P = T + s
        out_a = ca.decode_step(kd[:, P], vd[:, P], keep_new[s], qd[s], out_dtype=torch.float32,
                               lse=lse, split_tokens=split)
        cb.append(kd[:, P], vd[:, P], keep_new[s])
        out_b = cb.attention(qd[s], out_dtype=torch.float32, split_tokens=split)
        cl0 = o.comp_len.copy()
        o.append(k[:, P], v[:, P], keep[:, :, P])
        _effective_keep(keep_eff, cl0, o, P, W)
        if s % 7 == 0 or s == S - 1:
            torch.cuda.synchronize()
            compare_state(ca, o, f"step {s} fused")
            compare_state(cb, o, f"step {s} append")
            ref, rlse = oracle.attention(q[s], k, v, keep_eff, P, W, odt(kv_dtype), ka, va)
            worst = max(worst, check_close(out_a.cpu().numpy(), ref, f"step {s} fused"))
            check_close(out_b.cpu().numpy(), ref, f"step {s} append+attention")
            check_close(lse.cpu().numpy(), rlse, f"step {s} lse", atol=1e-4, rtol=1e-5)
    assert ca.error_word() == cb.error_word() == o.err
    log(f"  worst abs err {worst:.2e}; error word {o.err}")


def test_counters_zero_and_workspace_shared_with_attention():
    # one workspace serves decode steps and plain attention calls in any
    # order; every call leaves its counters at zero
    B, Hq, Hkv, D, T, S, W = 2, 16, 4, 128, 1500, 12, 64
    keep = workload.random_keep((B, Hkv, T + S), 0.3, seed=61)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=62)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=63)
    q = workload.random_bf16((S, B, Hq, D), seed=64)
    c, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    ws = torch.zeros(c.workspace(Hq, 64).numel(), dtype=torch.uint8, device=dev())
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    keep_new = keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev())
    ka, va = c.k_amax.cpu().numpy(), c.v_amax.cpu().numpy()
    splits = [64, 0, 320, 100000]
    for s in range(S):
        P = T + s
        split = splits[s % len(splits)]
        out = c.decode_step(kd[:, P], vd[:, P], keep_new[s], qd[s], out_dtype=torch.float32,
                            split_tokens=split, workspace=ws)
        again = c.attention(qd[s], out_dtype=torch.float32, split_tokens=splits[(s + 1) % 4],
                            workspace=ws)
        torch.cuda.synchronize()
        ref, _ = oracle.attention(q[s], k, v, keep, P, W, oracle.FP8, ka, va)
        check_close(out.cpu().numpy(), ref, f"step {s} split {split}")
        check_close(again.cpu().numpy(), ref, f"step {s} attention after the step")
        assert torch.count_nonzero(ws) == 0   # counters and partial slots
    assert c.error_word() == 0


def test_step_bf16_output_is_rounded_f32_output():
    B, Hq, Hkv, D, T, W = 2, 32, 8, 128, 1200, 256
    keep = workload.random_keep((B, Hkv, T + 1), 0.2, seed=71)
    k = workload.random_bf16((B, T + 1, Hkv, D), seed=72)
    v = workload.random_bf16((B, T + 1, Hkv, D), seed=73)
    q = workload.random_bf16((B, Hq, D), seed=74).to(dev())
    c32, _ = gpu_prefill(k, v, keep, T, W, 1, "fp8", with_dst=False)
    c16, _ = gpu_prefill(k, v, keep, T, W, 1, "fp8", with_dst=False)
    kd, vd = k.to(dev()), v.to(dev())
    kn = keep[:, :, T].contiguous().to(dev())
    o32 = c32.decode_step(kd[:, T], vd[:, T], kn, q, out_dtype=torch.float32)
    o16 = c16.decode_step(kd[:, T], vd[:, T], kn, q, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
