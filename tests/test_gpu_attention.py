"""GPU parity of decode_attn_compact against the CPU oracle's fp64 attention
computed from its definition on the dense history (F32 output, tolerance
|gpu - oracle| <= 2e-3 + 1e-2 |oracle|), including the split-K merge, the
log-sum-exp output, the edge cases of the method, and decode loops."""
import math

import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import (check_close, dev, gpu_prefill, log, odt, oracle_prefill)

pytestmark = pytest.mark.gpu


def _run(B, Hq, Hkv, D, T, W, rate, kv_dtype, seed, split=0, sm_scale=0.0, reserve=4,
         kscale=1.0, vscale=1.0):
    keep = workload.random_keep((B, Hkv, T), rate, seed=seed)
    k = workload.random_bf16((B, T, Hkv, D), seed=seed + 1, scale=kscale)
    v = workload.random_bf16((B, T, Hkv, D), seed=seed + 2, scale=vscale)
    q = workload.random_bf16((B, Hq, D), seed=seed + 3)
    c, _ = gpu_prefill(k, v, keep, T, W, reserve, kv_dtype, with_dst=False)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev())
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev())
    c.attention(q.to(dev()), out=out, lse=lse, sm_scale=sm_scale, split_tokens=split)
    torch.cuda.synchronize()
    quant = kv_dtype in ("fp8", "fp4")
    ka = c.k_amax.cpu().numpy() if quant else None
    va = c.v_amax.cpu().numpy() if quant else None
    if quant:   # the scales themselves are pinned bit-exact elsewhere
        oa = oracle.prefill_amax(k, v, keep, T, W)
        assert np.array_equal(ka[: B * Hkv], oa[0]) and np.array_equal(va[: B * Hkv], oa[1])
    ref, rlse = oracle.attention(q, k, v, keep, T - 1, W, odt(kv_dtype), ka, va, sm_scale)
    return c, out.cpu().numpy(), lse.cpu().numpy(), ref, rlse


CASES = [
    # B, Hq, Hkv, D, T, W, rate, kv_dtype, seed
    (1, 8, 2, 64, 512, 64, 1 / 6.4, "bf16", 1),
    (1, 8, 2, 64, 512, 64, 1 / 6.4, "fp8", 1),
    (2, 32, 8, 128, 1500, 256, 0.15, "fp8", 2),
    (2, 32, 8, 128, 1500, 256, 0.15, "bf16", 3),
    (3, 32, 8, 64, 2100, 256, 0.3, "fp8", 4),
    (1, 16, 16, 128, 777, 20, 0.4, "bf16", 5),     # G = 1
    (2, 16, 2, 64, 900, 10, 0.25, "fp8", 6),       # G = 8
    (1, 32, 2, 128, 650, 33, 0.5, "bf16", 7),      # G = 16
    (2, 12, 4, 64, 333, 7, 0.2, "fp8", 8),         # G = 3
    (1, 8, 2, 128, 50, 64, 0.5, "fp8", 9),         # T < W
    (2, 8, 4, 64, 4100, 1, 0.02, "bf16", 10),      # W = 1, very sparse
    (2, 32, 8, 128, 1500, 256, 0.15, "fp4", 31),   # 4-bit store
    (1, 8, 2, 128, 50, 64, 0.5, "fp4", 32),        # FP4, T < W
    (1, 32, 2, 128, 650, 33, 0.5, "fp4", 33),      # FP4, G = 16, odd W
    (1, 16, 16, 128, 777, 20, 0.4, "fp4", 34),     # FP4, G = 1
]


@pytest.mark.parametrize("case", CASES, ids=[f"a{i}" for i in range(len(CASES))])
def test_attention_matches_oracle(case):
    B, Hq, Hkv, D, T, W, rate, kv_dtype, seed = case
    log(f"attention case B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} W={W} {kv_dtype}")
    c, out, lse, ref, rlse = _run(*case)
    err = check_close(out, ref, "out")
    check_close(lse, rlse, "lse", atol=1e-4, rtol=1e-5)
    log(f"  max abs err {err:.2e}")


@pytest.mark.parametrize("split", [64, 128, 192, 256, 1024, 100000])
@pytest.mark.parametrize("kv_dtype", ["fp8", "fp4"])
def test_split_invariance(split, kv_dtype):
    case = (2, 32, 8, 128, 3000, 256, 0.2, kv_dtype, 21)
    c, out, lse, ref, rlse = _run(*case, split=split)
    check_close(out, ref, f"split {split}")
    check_close(lse, rlse, f"split {split} lse", atol=1e-4, rtol=1e-5)


def test_one_workspace_reused_across_splits_and_caches():
    # the counters and partial slots are left at zero by every call, so a single
    # zero-filled workspace serves calls with different splits and caches
    B, Hq, Hkv, D, T, W = 2, 16, 4, 128, 2000, 64
    keep = workload.random_keep((B, Hkv, T), 0.3, seed=91)
    k = workload.random_bf16((B, T, Hkv, D), seed=92)
    v = workload.random_bf16((B, T, Hkv, D), seed=93)
    q = workload.random_bf16((B, Hq, D), seed=94)
    caches = [gpu_prefill(k, v, keep, T, W, 0, dt, with_dst=False)[0] for dt in ("fp8", "bf16")]
    n = max(c.workspace(Hq, 64).numel() for c in caches)
    ws = torch.zeros(n, dtype=torch.uint8, device=dev())
    refs = {}
    for c in caches:
        ka = c.k_amax.cpu().numpy() if c.kv_dtype == "fp8" else None
        va = c.v_amax.cpu().numpy() if c.kv_dtype == "fp8" else None
        refs[c.kv_dtype] = oracle.attention(q, k, v, keep, T - 1, W, odt(c.kv_dtype), ka, va)[0]
    qd = q.to(dev())
    for rep in range(3):
        for split in (64, 320, 128, 100000, 0):
            for c in caches:
                out = c.attention(qd, out_dtype=torch.float32, split_tokens=split, workspace=ws)
                check_close(out.cpu().numpy(), refs[c.kv_dtype], f"{c.kv_dtype} split {split} rep {rep}")
    assert torch.count_nonzero(ws) == 0   # counters and partial slots


def test_outliers_and_custom_scale():
    # large-magnitude K and V (FP8 scales far from 1) and an explicit sm_scale
    case = (2, 16, 4, 128, 1200, 64, 0.2, "fp8", 31)
    c, out, lse, ref, rlse = _run(*case, sm_scale=0.05, kscale=40.0, vscale=0.01)
    check_close(out, ref, "scaled", atol=2e-3 * 0.01, rtol=1e-2)


def test_empty_segments_give_zero_and_neg_inf_lse():
    B, Hq, Hkv, D, T = 2, 8, 2, 64, 200
    keep = torch.zeros((B, Hkv, T), dtype=torch.uint8)
    keep[1, 0, 17] = 1                  # one segment holds one token
    k = workload.random_bf16((B, T, Hkv, D), seed=1)
    v = workload.random_bf16((B, T, Hkv, D), seed=2)
    q = workload.random_bf16((B, Hq, D), seed=3)
    for kv_dtype in ("bf16", "fp8"):
        c, _ = gpu_prefill(k, v, keep, T, 0, 0, kv_dtype, with_dst=False)
        out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device=dev())
        lse = torch.zeros((B, Hq), dtype=torch.float32, device=dev())
        c.attention(q.to(dev()), out=out, lse=lse)
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        ka = c.k_amax.cpu().numpy() if kv_dtype == "fp8" else None
        va = c.v_amax.cpu().numpy() if kv_dtype == "fp8" else None
        ref, rlse = oracle.attention(q, k, v, keep, T - 1, 0, odt(kv_dtype), ka, va)
        empty = np.isneginf(rlse)
        assert empty.sum() == B * Hq - 4
        assert np.all(o[empty] == 0) and np.all(np.isneginf(l[empty]))
        check_close(o, ref, "single token")


def test_bf16_output_is_rounded_f32_output():
    case = (2, 32, 8, 128, 1500, 256, 0.15, "fp8", 41)
    c, out32, _, ref, _ = _run(*case)
    q = workload.random_bf16((2, 32, 128), seed=44).to(dev())
    o32 = c.attention(q, out_dtype=torch.float32)
    o16 = c.attention(q, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("kv_dtype,D,W", [("fp8", 128, 64), ("bf16", 64, 64), ("fp8", 64, 0),
                                          ("fp4", 128, 64), ("fp4", 128, 0)])
def test_decode_loop_matches_oracle(kv_dtype, D, W):
    B, Hq, Hkv, T, S = 2, 16, 4, 700, 80
    log(f"decode loop {kv_dtype} D={D} W={W}")
    keep = workload.random_keep((B, Hkv, T + S), 0.2, seed=51)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=52)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=53)
    q = workload.random_bf16((S, B, Hq, D), seed=54)
    c, _ = gpu_prefill(k, v, keep, T, W, S, kv_dtype, with_dst=False)
    kd, vd, keepd, qd = k.to(dev()), v.to(dev()), keep.to(dev()), q.to(dev())
    ka = c.k_amax.cpu().numpy() if kv_dtype != "bf16" else None
    va = c.v_amax.cpu().numpy() if kv_dtype != "bf16" else None
    worst = 0.0
    for s in range(S):
        c.append(kd[:, T + s], vd[:, T + s], keepd[:, :, T + s].contiguous())
        out = c.attention(qd[s], out_dtype=torch.float32)
        if s % 9 == 0 or s == S - 1:
            torch.cuda.synchronize()
            ref, _ = oracle.attention(q[s], k, v, keep, T + s, W, odt(kv_dtype), ka, va)
            worst = max(worst, check_close(out.cpu().numpy(), ref, f"step {s}"))
    assert c.error_word() == 0
    log(f"  worst abs err {worst:.2e}")


def test_host_plan_and_device_plan_give_the_same_bits():
    # with the host copy of seg_base the launcher plans the work units over
    # the segments' capacities; without it every wave plans on the device
    # (over the rows holding data for attention, over the capacities for a
    # decode step).  The merge folds the units' partials in unit order, so
    # the two plans give bit-identical results whenever they cut the
    # segments the same way (decode steps), and agree within rounding
    # otherwise (attention)
    B, Hq, Hkv, D, T, W, S = 8, 32, 8, 128, 2500, 256, 4
    rates = torch.rand((B, Hkv, 1), generator=torch.Generator().manual_seed(102)) * 0.3
    keep = (torch.rand((B, Hkv, T + S), generator=torch.Generator().manual_seed(103)) < rates)
    keep = keep.to(torch.uint8)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=104)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=105)
    q = workload.random_bf16((S, B, Hq, D), seed=106)
    c1, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    c2, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    assert c1.seg_base_host is not None
    c2.seg_base_host = None
    c2._refresh()                     # device plan
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    kn = keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev())
    ka, va = c1.k_amax.cpu().numpy(), c1.v_amax.cpu().numpy()
    for split in (256, 512, 0):
        o1 = c1.attention(qd[0], out_dtype=torch.float32, split_tokens=split)
        o2 = c2.attention(qd[0], out_dtype=torch.float32, split_tokens=split)
        torch.cuda.synchronize()
        ref, _ = oracle.attention(q[0], k, v, keep, T - 1, W, oracle.FP8, ka, va)
        check_close(o1.cpu().numpy(), ref, f"host plan, split {split}")
        check_close(o2.cpu().numpy(), ref, f"device plan, split {split}")
    for s in range(S):
        o1 = c1.decode_step(kd[:, T + s], vd[:, T + s], kn[s], qd[s], out_dtype=torch.float32)
        o2 = c2.decode_step(kd[:, T + s], vd[:, T + s], kn[s], qd[s], out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"decode step {s}"
    assert torch.equal(c1.comp_len, c2.comp_len) and torch.equal(c1.pos, c2.pos)
    assert torch.equal(c1.k_pool, c2.k_pool) and torch.equal(c1.v_pool, c2.v_pool)
    assert c1.error_word() == 0 and c2.error_word() == 0


def test_stale_host_plan_is_flagged():
    # a COUNT that changes the layout after the host copy was taken: the
    # attention flags CDA_DEVERR_PLAN instead of reading rows of another
    # layout (the rows it would read stay inside the pool)
    from compressed_decode_attention_amd import CDA_DEVERR_PLAN
    B, Hq, Hkv, D, T, W = 2, 8, 2, 128, 900, 64
    keep = workload.random_keep((B, Hkv, T), 0.3, seed=111)
    k = workload.random_bf16((B, T, Hkv, D), seed=112)
    v = workload.random_bf16((B, T, Hkv, D), seed=113)
    q = workload.random_bf16((B, Hq, D), seed=114).to(dev())
    c, _ = gpu_prefill(k, v, keep, T, W, 0, "fp8", with_dst=False)
    out = c.attention(q, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.error_word() == 0 and torch.isfinite(out).all()
    # reserve 64 more rows per segment: every segment after the first moves
    c.count(keep.to(dev()), T, reserve=64)
    c.err.zero_()
    out = c.attention(q, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.error_word() & CDA_DEVERR_PLAN
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_spare_rows_hint_changes_no_bit(kv_dtype):
    # the spare_rows hint (count sets it to the COUNT reserve) makes the host
    # plan read the tiles it puts wholly in the empty end of a span only once
    # the metadata has arrived.  The right hint (a reserve of 300 rows:
    # several empty tiles per span), no hint, a partly wrong hint (tiles
    # holding data deferred) and one that defers every tile give the same
    # bits, in attention and in decode steps, and the oracle's result
    B, Hq, Hkv, D, T, W, S, reserve = 4, 16, 4, 128, 3000, 128, 6, 300
    rates = torch.rand((B, Hkv, 1), generator=torch.Generator().manual_seed(121)) * 0.4
    keep = (torch.rand((B, Hkv, T + S), generator=torch.Generator().manual_seed(122)) < rates)
    keep = keep.to(torch.uint8)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=123)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=124)
    q = workload.random_bf16((S, B, Hq, D), seed=125)
    caches = [gpu_prefill(k, v, keep, T, W, reserve, kv_dtype, with_dst=False)[0]
              for _ in range(4)]
    assert caches[0].spare_rows == reserve and caches[0].seg_base_host is not None
    for c, hint in zip(caches[1:], (0, 500, 100000)):
        c.spare_rows = hint
        c._refresh()
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    kn = keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev())
    quant = kv_dtype != "bf16"
    ka = caches[0].k_amax.cpu().numpy() if quant else None
    va = caches[0].v_amax.cpu().numpy() if quant else None
    o = [c.attention(qd[0], out_dtype=torch.float32) for c in caches]
    torch.cuda.synchronize()
    assert all(torch.equal(o[0], x) for x in o[1:]), "attention"
    ref, _ = oracle.attention(q[0], k, v, keep, T - 1, W, odt(kv_dtype), ka, va)
    check_close(o[0].cpu().numpy(), ref, "attention, hint = reserve")
    for s in range(S):
        o = [c.decode_step(kd[:, T + s], vd[:, T + s], kn[s], qd[s], out_dtype=torch.float32)
             for c in caches]
        torch.cuda.synchronize()
        assert all(torch.equal(o[0], x) for x in o[1:]), f"decode step {s}"
        ref, _ = oracle.attention(q[s], k, v, keep, T + s, W, odt(kv_dtype), ka, va)
        check_close(o[0].cpu().numpy(), ref, f"decode step {s}, hint = reserve")
    for c in caches[1:]:
        assert torch.equal(c.comp_len, caches[0].comp_len) and torch.equal(c.pos, caches[0].pos)
        assert torch.equal(c.k_pool, caches[0].k_pool) and torch.equal(c.v_pool, caches[0].v_pool)
    assert all(c.error_word() == 0 for c in caches)
