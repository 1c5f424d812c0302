"""A contiguous store whose pools are smaller than the segments COUNT laid
out (pool_rows < seg_base[B*Hkv]): decode attention, the decode step and the
chunk call read no tile outside the pool, raise CDA_DEVERR_POOL, and give
every head whose segment lies inside the pool the bits of the same call on
the full pool.  The short pools are views of the full allocation, so a read
past pool_rows would still be in mapped memory (and show up here as a
missing flag, not a fault).

Also: the binding refuses tensors on another device, and workspaces that
are not contiguous uint8."""
import pytest
import torch

import workload
from _cda_testlib import dev, gpu_prefill, log
from compressed_decode_attention_amd import CDA_DEVERR_POOL

pytestmark = pytest.mark.gpu

B, Hq, Hkv, D, T, W, S, M = 2, 16, 4, 128, 1500, 64, 8, 8
G = Hq // Hkv


def inputs(seed):
    keep = workload.random_keep((B, Hkv, T + S), 0.3, seed=seed)
    k = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 1)
    v = workload.random_bf16((B, T + S, Hkv, D), seed=seed + 2)
    q = workload.random_bf16((S, B, Hq, D), seed=seed + 3)
    return keep, k, v, q


def cut_pool(c, rows):
    """The pools of c seen as their first `rows` rows; no host plan."""
    c.k_pool = c.k_pool[: rows * c.row_bytes]
    c.v_pool = c.v_pool[: rows * c.row_bytes]
    c.pool_rows = rows
    c.seg_base_host = None
    c._ws.clear()
    c._refresh()


def pair(kv, seed):
    keep, k, v, q = inputs(seed)
    full, _ = gpu_prefill(k, v, keep, T, W, S, kv, with_dst=False)
    short, _ = gpu_prefill(k, v, keep, T, W, S, kv, with_dst=False)
    torch.cuda.synchronize()
    nh = B * Hkv
    sb = full.seg_base.cpu()
    # the last segment keeps its first tile only
    rows = int(sb[nh - 1]) + 64
    assert int(sb[nh]) > rows + 64
    full.seg_base_host = None      # both on the device-side plan: the same units
    full._refresh()
    cut_pool(short, rows)
    return full, short, keep, k, v, q


def heads_inside():
    """Query heads (b, j) whose segment is not the last one."""
    return [(b, j) for b in range(B) for j in range(Hq) if b * Hkv + j // G != B * Hkv - 1]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attention_and_decode_step_stay_in_the_pool(kv):
    log(f"pool bounds: attention + decode step, {kv}")
    full, short, keep, k, v, q = pair(kv, 310)
    qd = q.to(dev())
    for split in (128, 256):   # explicit: the default depends on pool_rows
        a = full.attention(qd[0], out_dtype=torch.float32, split_tokens=split)
        b_ = short.attention(qd[0], out_dtype=torch.float32, split_tokens=split)
        torch.cuda.synchronize()
        assert full.error_word() == 0
        assert short.error_word() & CDA_DEVERR_POOL, f"split {split}: no pool flag"
        for b, j in heads_inside():
            assert torch.equal(a[b, j], b_[b, j]), f"split {split}: head {(b, j)}"
        short.err.zero_()
    kd, vd = k.to(dev()), v.to(dev())
    keep_new = keep.to(dev())[:, :, T:].permute(2, 0, 1).contiguous()
    for s in range(3):
        a = full.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                             out_dtype=torch.float32, split_tokens=128)
        b_ = short.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                               out_dtype=torch.float32, split_tokens=128)
        torch.cuda.synchronize()
        assert full.error_word() == 0
        assert short.error_word() & CDA_DEVERR_POOL, f"step {s}: no pool flag"
        for b, j in heads_inside():
            assert torch.equal(a[b, j], b_[b, j]), f"step {s}: head {(b, j)}"
        assert torch.equal(full.comp_len[:-1], short.comp_len[:-1])
        short.err.zero_()


def test_chunk_stays_in_the_pool():
    log("pool bounds: chunk call, fp8")
    full, short, keep, k, v, q = pair("fp8", 320)
    kd, vd = k.to(dev()), v.to(dev())
    kn = kd[:, T:T + M]
    vn = vd[:, T:T + M]
    keep_new = keep.to(dev())[:, :, T:T + M].permute(0, 2, 1).contiguous()
    qc = q.to(dev())[:M].permute(1, 0, 2, 3).contiguous()
    a = full.chunk(kn, vn, keep_new, qc, out_dtype=torch.float32)
    b_ = short.chunk(kn, vn, keep_new, qc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert full.error_word() == 0
    assert short.error_word() & CDA_DEVERR_POOL
    for b, j in heads_inside():
        assert torch.equal(a[b, :, j], b_[b, :, j]), f"head {(b, j)}"
    assert torch.equal(full.comp_len[:-1], short.comp_len[:-1])


def test_binding_refuses_other_devices_and_bad_workspaces():
    log("binding: device and workspace checks")
    keep, k, v, q = inputs(330)
    c, _ = gpu_prefill(k, v, keep, T, W, S, "fp8", with_dst=False)
    qd = q.to(dev())
    keep_new = keep[:, :, T].contiguous()
    with pytest.raises(ValueError):
        c.attention(q[0])                                     # q on the host
    with pytest.raises(ValueError):
        c.attention(qd[0], out=torch.empty((B, Hq, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError):                           # k_new, v_new, keep on the host
        c.decode_step(k[:, T], v[:, T], keep_new, qd[0])
    with pytest.raises(ValueError):
        c.append(k[:, T], v[:, T], keep_new)
    ws = c.workspace(Hq)
    with pytest.raises(ValueError):
        c.attention(qd[0], workspace=ws.cpu())
    with pytest.raises(ValueError):
        c.attention(qd[0], workspace=torch.zeros(ws.numel(), dtype=torch.float32, device=dev()))
    with pytest.raises(ValueError):
        c.chunk(k[:, T:T + 2], v[:, T:T + 2],
                keep[:, :, T:T + 2].permute(0, 2, 1).contiguous(),
                q[:2].permute(1, 0, 2, 3).contiguous())
    # nothing was launched: the store is as the prefill left it
    torch.cuda.synchronize()
    assert c.error_word() == 0 and int(c.pos[0]) == T
