"""Seeded random shapes through the chunk call and the decode step.

Each case draws a storage format, head size, KV heads, GQA group, batch,
window (0 and odd values included), prefill length and chunk length, then
runs one chunk call (every query against the oracle's decode attention at its
position, the store bit for bit against M oracle appends) and two decode steps
after it (against the oracle again).  The draws reach corners the hand-picked
cases may miss: segment lengths at and around tile edges, chunks longer than
the window, rings not yet full, single-row segments."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import check_close, compare_state, dev, gpu_prefill, log, odt, oracle_prefill

pytestmark = pytest.mark.gpu


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    kv = ["bf16", "fp8", "fp4"][r.integers(3)]
    D = 128 if kv == "fp4" else int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    B = int(r.integers(1, 4))
    W = int(r.choice([0, 16, 33, 64, 128]))
    T = int(r.integers(1, 1500))
    M = int(r.integers(1, 65))
    lo = float(r.uniform(0.02, 0.5))
    hi = float(min(1.0, lo + r.uniform(0.0, 0.5)))
    return kv, D, Hkv, G, B, W, T, M, lo, hi


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_chunk_then_decode(seed):
    kv, D, Hkv, G, B, W, T, M, lo, hi = draw(seed)
    S = M + 2
    log(f"random shape {seed}: {kv} D={D} Hkv={Hkv} G={G} B={B} W={W} T={T} M={M} "
        f"keep {lo:.2f}-{hi:.2f}")
    cfg = workload.custom(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype=kv,
                          keep_lo=lo, keep_hi=hi, seed=2000 + seed)
    lay = workload.make_layer(cfg, 0)
    c, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, S, kv, with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, S, kv)
    d = dev()
    k = lay.k[:, T:T + M].contiguous().to(d)
    v = lay.v[:, T:T + M].contiguous().to(d)
    keep = lay.keep[:, :, T:T + M].permute(0, 2, 1).contiguous().to(d)
    q = lay.q[:M].permute(1, 0, 2, 3).contiguous().to(d)
    lse = torch.empty(B, M, G * Hkv, dtype=torch.float32, device=d)
    out = c.chunk(k, v, keep, q, out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    ka = o.k_amax if kv != "bf16" else None
    va = o.v_amax if kv != "bf16" else None
    for t in range(M):
        ref, rl = oracle.attention(lay.q[t], lay.k, lay.v, lay.keep, T + t, W, odt(kv), ka, va)
        check_close(got[:, t], ref, f"seed {seed} query {t}")
        check_close(gl[:, t], rl, f"seed {seed} query {t} lse", atol=1e-4, rtol=1e-5)
    for t in range(M):
        p = T + t
        o.append(lay.k[:, p], lay.v[:, p], lay.keep[:, :, p])
    compare_state(c, o, f"seed {seed}: after the chunk")
    kd, vd, qd = lay.k.to(d), lay.v.to(d), lay.q.to(d)
    for s in range(M, S):
        kn = lay.keep[:, :, T + s].contiguous().to(d)
        o1 = c.decode_step(kd[:, T + s], vd[:, T + s], kn, qd[s], out_dtype=torch.float32)
        o.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s])
        torch.cuda.synchronize()
        ka = o.k_amax if kv != "bf16" else None
        va = o.v_amax if kv != "bf16" else None
        ref, _ = oracle.attention(lay.q[s], lay.k, lay.v, lay.keep, T + s, W, odt(kv), ka, va)
        check_close(o1.cpu().numpy(), ref, f"seed {seed} decode step {s}")
    compare_state(c, o, f"seed {seed}: after the decode steps")
    assert c.error_word() == 0
