"""Parity at the five workload shapes (ctx 8192, gen 128, c = 1 / 8 for the
Llama-3.2-1B and Qwen3-8B attention shapes, plus the tiny case, and the
c = 8 shapes with the per-layer pyramid budget), in the
launch configuration the benchmark times: prefill compaction of a layer
bit-exact, all 128 decode appends bit-exact, and the attention output of
every query head at several decode steps against the oracle.  Each decode
step runs either as one decode_step_compact launch (what the benchmark
times) or as kv_compact APPEND followed by decode_attn_compact."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import check_close, compare_state, dev, gpu_prefill, log, odt, oracle_prefill

pytestmark = pytest.mark.gpu

RESERVE_EXTRA = 0   # the benchmark reserves exactly gen_len rows per segment


@pytest.mark.parametrize("mode", ["step", "append"])
@pytest.mark.parametrize("name,layer", [("tiny", 0), ("llama_c1", 3), ("llama_c8", 0),
                                        ("qwen_c1", 35), ("qwen_c8", 0)])
def test_config_layer(name, layer, mode):
    _run_config(name, layer, mode, workload.CONFIGS[name].kv_dtype)


@pytest.mark.parametrize("name,layer", [("qwen_c1", 7), ("qwen_c8", 0)])
def test_config_layer_fp4(name, layer):
    # the Qwen3-8B shapes with the 4-bit store, as the benchmark's --kv fp4 runs them
    _run_config(name, layer, "step", "fp4")


@pytest.mark.parametrize("name,layer", [("qwen_c8_pyramid", 0), ("qwen_c8_pyramid", 35),
                                        ("llama_c8_pyramid", 15)])
def test_config_layer_pyramid(name, layer):
    # per-layer budget: layer 0 keeps 1.5x the flat rate, the last layer 0.5x
    _run_config(name, layer, "step", workload.CONFIGS[name].kv_dtype)


def _run_config(name, layer, mode, kv_dtype):
    cfg = workload.CONFIGS[name]
    log(f"config {name} layer {layer} ({mode}): B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} "
        f"T={cfg.T} S={cfg.S} W={cfg.W} {kv_dtype}")
    lay = workload.make_layer(cfg, layer)
    T, S, W = cfg.T, cfg.S, cfg.W
    reserve = S + RESERVE_EXTRA
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, reserve, kv_dtype, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, reserve, kv_dtype)
    compare_state(c, o, "prefill")
    kd, vd, keepd, qd = lay.k.to(dev()), lay.v.to(dev()), lay.keep.to(dev()), lay.q.to(dev())
    keep_new = keepd[:, :, T:].permute(2, 0, 1).contiguous()      # [S, B, Hkv]
    ka = c.k_amax.cpu().numpy() if kv_dtype != "bf16" else None
    va = c.v_amax.cpu().numpy() if kv_dtype != "bf16" else None
    check_steps = {0, S // 2, S - 1}
    worst = 0.0
    for s in range(S):
        if mode == "step":
            out = c.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                                out_dtype=torch.float32)
        else:
            c.append(kd[:, T + s], vd[:, T + s], keep_new[s])
            out = c.attention(qd[s], out_dtype=torch.float32)
        o.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s])
        if s in check_steps:
            torch.cuda.synchronize()
            ref, _ = oracle.attention(lay.q[s], lay.k, lay.v, lay.keep, T + s, W,
                                      odt(kv_dtype), ka, va)
            worst = max(worst, check_close(out.cpu().numpy(), ref, f"{name} step {s}"))
    compare_state(c, o, "after decode")
    assert c.error_word() == 0
    n = o.stored_rows()
    log(f"  stored rows per head: mean {n.mean():.0f} min {n.min()} max {n.max()}; "
        f"worst abs err {worst:.2e}; saturated elements {o.saturated}")
