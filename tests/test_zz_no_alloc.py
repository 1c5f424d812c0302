"""decode_step_compact_noalloc (the library's static per-GPU scratch in
place of a workspace) gives, bit for bit, the outputs, lse and cache state
of decode_step_compact (a workspace) on the same inputs: a larger store
first, then a smaller one on the same scratch."""
import pytest
import torch

import workload
from _cda_testlib import dev, gpu_prefill, log

pytestmark = pytest.mark.gpu


def run_pair(B, Hq, Hkv, D, T, W, S, kv, seed, split):
    log(f"noalloc vs workspace: B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} {kv} split={split}")
    keep = workload.random_keep((B, Hkv, T + S), 0.2, seed=seed)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 1)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 2)
    q = workload.random_bf16((S, B, Hq, D), seed=seed + 3)
    kd, vd, qd = k.to(dev()), v.to(dev()), q.to(dev())
    keep_new = keep.to(dev())[:, :, T:].permute(2, 0, 1).contiguous()
    ca, _ = gpu_prefill(k, v, keep, T, W, S, kv, with_dst=False)
    cb, _ = gpu_prefill(k, v, keep, T, W, S, kv, with_dst=False)
    for s in range(S):
        la = torch.empty((B, Hq), dtype=torch.float32, device=dev())
        lb = torch.empty_like(la)
        oa = ca.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                            out_dtype=torch.float32, lse=la, split_tokens=split)
        ob = cb.decode_step_noalloc(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                                    out_dtype=torch.float32, lse=lb, split_tokens=split)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {s}: outputs differ"
        assert torch.equal(la, lb), f"step {s}: lse differs"
    assert ca.error_word() == 0 and cb.error_word() == 0
    for name in ("comp_len", "pos", "ring_keep", "k_pool", "v_pool"):
        assert torch.equal(getattr(ca, name), getattr(cb, name)), name


def test_noalloc_matches_workspace_entry_point_large_then_small():
    run_pair(4, 32, 8, 128, 3000, 256, 3, "fp8", 901, 256)
    run_pair(2, 16, 4, 64, 700, 64, 2, "bf16", 911, 0)
