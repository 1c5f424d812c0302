"""GPU parity of kv_compact (COUNT, PACK, APPEND) against the CPU oracle:
offsets, lengths, scales, the dst map and every stored row, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import compare_state, dev, gpu_prefill, k_rows, log, oracle_prefill

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hkv, D, T, W, reserve, rate, kv_dtype, seed
    (1, 2, 64, 512, 64, 1, 1 / 6.4, "bf16", 1),
    (2, 3, 128, 700, 64, 5, 0.2, "fp8", 2),
    (2, 2, 64, 300, 0, 3, 0.3, "bf16", 3),       # no window
    (1, 4, 128, 40, 64, 2, 0.5, "fp8", 5),       # T < W: ring partly filled
    (3, 1, 64, 1000, 1, 0, 0.1, "fp8", 7),       # W = 1
    (1, 2, 128, 4096 + 17, 256, 9, 0.15, "bf16", 9),
    (2, 2, 64, 257, 16, 0, 1.0, "bf16", 11),     # keep all
    (2, 2, 128, 257, 16, 0, 0.0, "fp8", 13),     # keep none
    (1, 1, 64, 0, 8, 4, 0.5, "bf16", 15),        # empty prefill
    (2, 3, 128, 700, 64, 5, 0.2, "fp4", 17),     # 4-bit store
    (1, 4, 128, 40, 64, 2, 0.5, "fp4", 19),      # FP4, T < W
    (3, 1, 128, 1000, 1, 0, 0.1, "fp4", 21),     # FP4, W = 1 (ring row pairs with row 1)
    (2, 2, 128, 257, 17, 0, 1.0, "fp4", 23),     # FP4, odd W, keep all
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_prefill_compaction_bit_exact(case):
    B, Hkv, D, T, W, reserve, rate, kv_dtype, seed = case
    log(f"prefill case B={B} Hkv={Hkv} D={D} T={T} W={W} {kv_dtype} seed={seed}")
    keep = workload.random_keep((B, Hkv, T + 3), rate, seed=seed)
    k = workload.random_bf16((B, T + 3, Hkv, D), seed=seed + 100, scale=1.5)
    v = workload.random_bf16((B, T + 3, Hkv, D), seed=seed + 200)
    c, dst = gpu_prefill(k, v, keep, T, W, reserve, kv_dtype)
    o = oracle_prefill(k, v, keep, T, W, reserve, kv_dtype)
    compare_state(c, o, "prefill")
    lay = oracle.prefill_layout(keep, T, W, reserve, align=64)
    if T > 0:
        assert np.array_equal(dst.cpu().numpy()[: B * Hkv * T], lay["dst"].reshape(-1))
    assert c.error_word() == 0


def test_strided_inputs_and_nonbinary_keep():
    B, Hkv, D, T, W = 2, 4, 128, 333, 32
    big = workload.random_bf16((B, T + 10, Hkv + 2, D), seed=41)     # take heads 1..Hkv
    k = big[:, :, 1:Hkv + 1]
    v = workload.random_bf16((B, T + 10, Hkv + 2, D), seed=42)[:, :, 1:Hkv + 1]
    keep = workload.random_keep((B, Hkv, T + 10), 0.3, seed=43)         # bytes 1..255 kept
    assert keep.max() > 1
    for kv_dtype in ("bf16", "fp8", "fp4"):
        c, _ = gpu_prefill(k, v, keep, T, W, 4, kv_dtype)
        o = oracle_prefill(k.contiguous(), v.contiguous(), keep, T, W, 4, kv_dtype)
        compare_state(c, o, kv_dtype)


def test_fp8_encode_every_bf16_value():
    # amax 448 gives inv = 1 exactly, so each code is the encoding of the input itself
    B, Hkv, D, T = 1, 1, 128, 512
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    k = bits.view(torch.bfloat16).reshape(B, T, Hkv, D)
    v = bits.flip(0).view(torch.bfloat16).reshape(B, T, Hkv, D)
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    amax = (np.full(1, 448.0, np.float32), np.full(1, 448.0, np.float32))
    c, _ = gpu_prefill(k, v, keep, T, 0, 0, "fp8", amax=amax)
    o = oracle_prefill(k, v, keep, T, 0, 0, "fp8", amax=amax)
    compare_state(c, o, "fp8 exhaustive")
    # and BF16 storage copies every bit pattern (NaN payloads included) verbatim
    c, _ = gpu_prefill(k, v, keep, T, 0, 0, "bf16")
    o = oracle_prefill(k, v, keep, T, 0, 0, "bf16")
    compare_state(c, o, "bf16 exhaustive")


def test_fp8_encode_every_bf16_value_scaled():
    # given scales far from 1: x * inv runs past +-448 (saturation), through
    # the subnormal codes and into zero, and carries inf and NaN of both signs
    B, Hkv, D, T = 1, 1, 128, 512
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    k = bits.view(torch.bfloat16).reshape(B, T, Hkv, D)
    v = bits.flip(0).view(torch.bfloat16).reshape(B, T, Hkv, D)
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    for ka, va in ((0.37, 3.1e4), (1.0e-3, 0.75)):
        amax = (np.full(1, ka, np.float32), np.full(1, va, np.float32))
        c, _ = gpu_prefill(k, v, keep, T, 0, 0, "fp8", amax=amax)
        o = oracle_prefill(k, v, keep, T, 0, 0, "fp8", amax=amax)
        compare_state(c, o, f"fp8 scaled k_amax {ka} v_amax {va}")


def test_fp4_encode_every_bf16_value():
    # amax 6 gives inv = 1, so each code is the E2M1 encoding of the input;
    # then given scales far from 1 (saturation, zero, inf and NaN of both signs)
    B, Hkv, D, T = 1, 1, 128, 512
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    k = bits.view(torch.bfloat16).reshape(B, T, Hkv, D)
    v = bits.flip(0).view(torch.bfloat16).reshape(B, T, Hkv, D)
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    for ka, va in ((6.0, 6.0), (0.37, 3.1e4)):
        amax = (np.full(1, ka, np.float32), np.full(1, va, np.float32))
        c, _ = gpu_prefill(k, v, keep, T, 0, 0, "fp4", amax=amax)
        o = oracle_prefill(k, v, keep, T, 0, 0, "fp4", amax=amax)
        compare_state(c, o, f"fp4 k_amax {ka} v_amax {va}")


def test_fp8_scale_edge_cases():
    # heads whose stored values are all zero (amax 0 -> scale 1), or hold an inf
    B, Hkv, D, T, W = 1, 3, 64, 100, 8
    k = workload.random_bf16((B, T, Hkv, D), seed=51)
    v = workload.random_bf16((B, T, Hkv, D), seed=52)
    k[:, :, 0] = 0.0
    v[:, :, 0] = 0.0
    k[0, T - 1, 1, 5] = float("inf")
    v[0, 3, 2, 7] = -float("inf")
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    c, _ = gpu_prefill(k, v, keep, T, W, 0, "fp8")
    o = oracle_prefill(k, v, keep, T, W, 0, "fp8")
    compare_state(c, o, "scale edges")


@pytest.mark.parametrize("kv_dtype,D,W,reserve", [("bf16", 64, 16, 40), ("fp8", 128, 16, 40),
                                                  ("fp8", 64, 0, 40), ("bf16", 128, 1, 40),
                                                  ("fp8", 128, 100, 40), ("fp4", 128, 16, 40),
                                                  ("fp4", 128, 0, 40), ("fp4", 128, 7, 40),
                                                  ("fp4", 128, 1, 40)])
def test_append_steps_bit_exact(kv_dtype, D, W, reserve):
    B, Hkv, T, S = 3, 2, 150, 40
    log(f"append {kv_dtype} D={D} W={W}")
    keep = workload.random_keep((B, Hkv, T + S), 0.35, seed=61)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=62)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=63, scale=3.0)   # decode values saturate
    c, _ = gpu_prefill(k, v, keep, T, W, reserve, kv_dtype)
    o = oracle_prefill(k, v, keep, T, W, reserve, kv_dtype)
    kd, vd, keepd = k.to(dev()), v.to(dev()), keep.to(dev())
    for s in range(S):
        c.append(kd[:, T + s], vd[:, T + s], keepd[:, :, T + s].contiguous())
        o.append(k[:, T + s], v[:, T + s], keep[:, :, T + s])
        if s in (0, 1, S // 2, S - 1):
            compare_state(c, o, f"step {s}")
    assert c.error_word() == 0 and o.err[0] == 0


def test_append_capacity_overflow_sets_error_bit():
    B, Hkv, D, T, W, S = 1, 2, 64, 20, 4, 30
    keep = torch.ones((B, Hkv, T + S), dtype=torch.uint8)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=71)
    c, _ = gpu_prefill(k, k, keep, T, W, 3, "bf16")
    o = oracle_prefill(k, k, keep, T, W, 3, "bf16")
    kd, keepd = k.to(dev()), keep.to(dev())
    for s in range(S):
        c.append(kd[:, T + s], kd[:, T + s], keepd[:, :, T + s].contiguous())
        o.append(k[:, T + s], k[:, T + s], keep[:, :, T + s])
    assert c.error_word() & 1 and o.err[0] == 1
    compare_state(c, o, "overflow")


def test_pack_into_too_small_pool_sets_error_bit():
    B, Hkv, D, T, W = 1, 2, 64, 300, 16
    keep = torch.ones((B, Hkv, T), dtype=torch.uint8)
    k = workload.random_bf16((B, T, Hkv, D), seed=81)
    from compressed_decode_attention_amd import CompactKVCache
    c = CompactKVCache(B, Hkv, D, W, "bf16", dev())
    kd, keepd = k.to(dev()), keep.to(dev())
    c.count(keepd, T, 0)
    need = c.rows_needed()
    c.allocate(need - 128)          # last segment does not fit
    c.pack(kd, kd, keepd, T)
    assert c.error_word() & 2
    o = oracle_prefill(k, k, keep, T, W, 0, "bf16")
    # the first segment is complete
    kr = k_rows(c).cpu().numpy()
    n0 = int(o.stored_rows()[0])
    assert np.array_equal(kr[:n0], o.k_pool[:n0])
