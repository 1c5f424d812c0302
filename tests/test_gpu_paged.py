"""Paged compact store on the GPU (kv_compact PAGE_INIT / COUNT / PACK /
REFILL / RELEASE with a page table, APPEND, decode_attn_compact and
decode_step_compact over pages).

Checked against the oracle: the page tables and the free stack bit for bit
against the bookkeeping model (oracle/paged.py) after every operation that
moves pages; every stored row of every live segment, gathered through its
page table, bit for bit against a per-request oracle store; attention of
every live sequence against the fp64 oracle; idle slots give out = 0 and
lse = -inf.  A first whole-batch admission must equal the contiguous
store byte for byte, and decoding from it must give bit-identical results."""
import numpy as np
import pytest
import torch

import oracle
import workload
from _cda_testlib import (CDA_SEG_ALIGN, check_close, dev, gpu_prefill, log, odt,
                          oracle_prefill, segment_rows)
from compressed_decode_attention_amd import (CDA_DEVERR_CAPACITY, CDA_DEVERR_PAGES, CompactKVCache,
                                             PagedKVCache)
from oracle.paged import PagedBook

pytestmark = pytest.mark.gpu


def _check_book(c: PagedKVCache, book: PagedBook, what: str):
    torch.cuda.synchronize()
    got = c.pages().numpy()
    want = np.array(book.table_array(), np.int32).reshape(got.shape)
    assert np.array_equal(got, want), f"{what}: page tables differ"
    top = c.free_count()
    assert top == len(book.free), f"{what}: free_top {top} != {len(book.free)}"
    assert np.array_equal(c.free_pages[:top].cpu().numpy(), np.array(book.free, np.int32)), \
        f"{what}: free stack differs"
    caps = c.seg_cap.cpu().numpy()
    for i in range(c.B * c.Hkv):
        want_cap = book.seg_cap(i) if book.live[i // c.Hkv] else 0
        assert caps[i] == want_cap, f"{what}: seg_cap[{i}] {caps[i]} != {want_cap}"


class Request:
    """One sequence's synthetic inputs and its oracle store (B = 1)."""

    def __init__(self, T, S, Hq, Hkv, D, W, kv, seed, keep_rate=0.3):
        self.cfg = workload.custom(B=1, Hq=Hq, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype=kv,
                                   keep_lo=keep_rate / 2, keep_hi=keep_rate, seed=seed)
        self.lay = workload.make_layer(self.cfg, 0)
        self.T, self.S, self.W, self.kv = T, S, W, kv
        self.s = 0   # decode steps done
        # the oracle's capacity is set past every append: the paged store grows by refill
        self.o = oracle.prefill_pack(self.lay.k, self.lay.v, self.lay.keep, T, W, S + 64,
                                     odt(kv), align=CDA_SEG_ALIGN)

    def comp_len(self):
        return oracle.prefill_layout(self.lay.keep, self.T, self.W, 0)["comp_len"]


def _admit(c, book, slot, req, reserve):
    d = dev()
    T = req.T
    c.admit(slot, req.lay.k[:, :T].to(d), req.lay.v[:, :T].to(d),
            req.lay.keep[:, :, :T].contiguous().to(d), T, reserve)
    return book.admit(slot, 1, req.comp_len(), reserve)


def _compare_rows(c: PagedKVCache, slot: int, req: Request, what: str):
    torch.cuda.synchronize()
    o = req.o
    n = o.stored_rows()
    Hkv = c.Hkv
    assert np.array_equal(c.comp_len.cpu().numpy()[slot * Hkv:(slot + 1) * Hkv], o.comp_len), \
        what + " comp_len"
    assert int(c.pos[slot].item()) == int(o.pos[0]), what + " pos"
    if c.W:
        rk = c.ring_keep.cpu().numpy()[slot * Hkv * c.W:(slot + 1) * Hkv * c.W]
        assert np.array_equal(rk, o.ring_keep[:Hkv * c.W]), what + " ring_keep"
    if c.kv_dtype != "bf16":
        assert np.array_equal(c.k_amax.cpu().numpy()[slot * Hkv:(slot + 1) * Hkv], o.k_amax)
        assert np.array_equal(c.v_amax.cpu().numpy()[slot * Hkv:(slot + 1) * Hkv], o.v_amax)
    for h in range(Hkv):
        if n[h] == 0:
            continue
        kr, vr = segment_rows(c, slot * Hkv + h, int(n[h]))
        a = int(o.seg_base[h])
        assert np.array_equal(kr.cpu().numpy(), o.k_pool[a:a + n[h]]), f"{what} K rows, head {h}"
        assert np.array_equal(vr.cpu().numpy(), o.v_pool[a:a + n[h]]), f"{what} V rows, head {h}"


def _step(c, slots, Hq, mode, kv):
    """One decode step over the batch: live slots take their request's next
    token, idle slots zeros.  Returns (out f32, lse, {slot: position})."""
    d = dev()
    B, Hkv, D = c.B, c.Hkv, c.D
    kn = torch.zeros(B, Hkv, D, dtype=torch.bfloat16)
    vn = torch.zeros_like(kn)
    keep = torch.zeros(B, Hkv, dtype=torch.uint8)
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    for b, r in slots.items():
        p = r.T + r.s
        kn[b] = r.lay.k[0, p]
        vn[b] = r.lay.v[0, p]
        keep[b] = r.lay.keep[0, :, p]
        q[b] = r.lay.q[r.s, 0]
    kd, vd, keepd, qd = kn.to(d), vn.to(d), keep.to(d), q.to(d)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=d)
    if mode == "step":
        out = c.decode_step(kd, vd, keepd, qd, out_dtype=torch.float32, lse=lse)
    else:
        c.append(kd, vd, keepd)
        out = c.attention(qd, out_dtype=torch.float32, lse=lse)
    for b, r in slots.items():
        p = r.T + r.s
        r.o.append(r.lay.k[:, p], r.lay.v[:, p], r.lay.keep[:, :, p])
        r.s += 1
    return out, lse


def _check_attention(out, lse, slots, B, Hq, what):
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for b in range(B):
        if b not in slots:
            assert np.all(o[b] == 0) and np.all(np.isneginf(l[b])), f"{what}: idle slot {b}"
            continue
        r = slots[b]
        P = r.T + r.s - 1                     # the token just appended
        ka = r.o.k_amax if r.kv != "bf16" else None
        va = r.o.v_amax if r.kv != "bf16" else None
        ref, rl = oracle.attention(r.lay.q[r.s - 1], r.lay.k, r.lay.v, r.lay.keep, P, r.W,
                                   odt(r.kv), ka, va)
        worst = max(worst, check_close(o[b:b + 1], ref, f"{what} slot {b}"))
        check_close(l[b:b + 1], rl, f"{what} slot {b} lse", atol=1e-4, rtol=1e-5)
    return worst


@pytest.mark.parametrize("kv,D", [("bf16", 64), ("fp8", 128), ("fp4", 128), ("bf16", 128)])
def test_first_admission_is_the_contiguous_store(kv, D):
    """One admission of the whole batch after PAGE_INIT lays the pages out as
    the contiguous segments; decoding from both gives identical bytes."""
    B, Hkv, Hq, W, T, S, reserve = 3, 2, 8, 48, 333, 40, 40
    cfg = workload.custom(B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype=kv,
                          keep_lo=0.1, keep_hi=0.5, seed=71)
    lay = workload.make_layer(cfg, 0)
    log(f"paged vs contiguous {kv} D={D}")
    cc, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, reserve, kv, with_dst=False)
    rows = cc.pool_rows
    d = dev()
    pc = PagedKVCache(B, Hkv, D, W, n_pages=rows // CDA_SEG_ALIGN + 3, max_pages=32,
                      kv_dtype=kv, device=d)
    pc.k_pool.fill_(0xA5)
    pc.v_pool.fill_(0x5A)
    pc.admit(0, lay.k.to(d), lay.v.to(d), lay.keep.to(d), T, reserve)
    book = PagedBook(pc.n_pages, B, Hkv, W, 32)
    assert book.admit(0, B, oracle.prefill_layout(lay.keep, T, W, 0)["comp_len"], reserve)
    _check_book(pc, book, "admission")
    nb = rows * pc.row_bytes
    assert torch.equal(pc.k_pool[:nb], cc.k_pool[:nb]) and torch.equal(pc.v_pool[:nb], cc.v_pool[:nb])
    kd, vd, qd = lay.k.to(d), lay.v.to(d), lay.q.to(d)
    keep_new = lay.keep[:, :, T:].permute(2, 0, 1).contiguous().to(d)
    sp = 128   # the same units for both (the default follows pool_rows, which differ)
    for s in range(S):
        if s % 2:
            a = cc.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                               out_dtype=torch.float32, split_tokens=sp)
            b = pc.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s],
                               out_dtype=torch.float32, split_tokens=sp)
        else:
            cc.append(kd[:, T + s], vd[:, T + s], keep_new[s])
            pc.append(kd[:, T + s], vd[:, T + s], keep_new[s])
            a = cc.attention(qd[s], out_dtype=torch.float32, split_tokens=sp)
            b = pc.attention(qd[s], out_dtype=torch.float32, split_tokens=sp)
        assert torch.equal(a, b), f"step {s}: outputs differ"
    torch.cuda.synchronize()
    assert torch.equal(pc.k_pool[:nb], cc.k_pool[:nb]) and torch.equal(pc.v_pool[:nb], cc.v_pool[:nb])
    assert torch.equal(pc.comp_len, cc.comp_len) and torch.equal(pc.pos, cc.pos)
    assert pc.error_word() == 0 and cc.error_word() == 0


@pytest.mark.parametrize("mode", ["step", "append"])
@pytest.mark.parametrize("kv,D", [("fp8", 128), ("bf16", 64), ("fp4", 128)])
def test_serving_mix(kv, D, mode):
    """Requests of different lengths arrive in free slots, decode together
    with idle slots, finish and hand their pages to the next ones."""
    B, Hkv, Hq, W = 4, 2, 8, 32
    n_pages, max_pages = 96, 24
    c = PagedKVCache(B, Hkv, D, W, n_pages, max_pages, kv, dev())
    book = PagedBook(n_pages, B, Hkv, W, max_pages)
    _check_book(c, book, "init")
    reqs = iter([Request(T, 200, Hq, Hkv, D, W, kv, seed=100 + j)
                 for j, T in enumerate([300, 700, 150, 520, 90, 411])])
    slots = {}
    steps = 0
    log(f"serving mix {kv} D={D} {mode}")

    def admit(slot, reserve=0):
        r = next(reqs)
        assert _admit(c, book, slot, r, reserve)
        slots[slot] = r
        _check_book(c, book, f"admit slot {slot}")
        _compare_rows(c, slot, r, f"prefill slot {slot}")

    def release(slot):
        c.release(slot)
        book.release(slot, 1)
        del slots[slot]
        _check_book(c, book, f"release slot {slot}")

    def run(n, refill_every=16):
        nonlocal steps
        for _ in range(n):
            if steps % refill_every == 0:
                c.refill(64)
                comp = np.zeros(B * Hkv, int)
                for b, r in slots.items():
                    comp[b * Hkv:(b + 1) * Hkv] = r.o.comp_len
                book.refill(comp, 64)
                _check_book(c, book, f"refill at step {steps}")
            out, lse = _step(c, slots, Hq, mode, kv)
            steps += 1
            if steps % 20 == 0:
                _check_attention(out, lse, slots, B, Hq, f"step {steps}")

    admit(0)
    admit(2, reserve=5)
    run(40)
    for b, r in slots.items():
        _compare_rows(c, b, r, f"slot {b} after 40 steps")
    release(0)
    admit(1)
    admit(0)
    run(70)
    release(2)
    admit(3)
    run(50)
    for b, r in slots.items():
        _compare_rows(c, b, r, f"slot {b} at the end")
    assert c.error_word() == 0
    assert book.pages_error is False
    log(f"  pages held at the end: {n_pages - c.free_count()} of {n_pages}")


def test_growth_beyond_the_prefill_reserve():
    """No spare rows at prefill: refills every 64 steps carry a segment past
    any reserve, where the contiguous store reports a full segment."""
    B, Hkv, Hq, D, W, T, S = 2, 2, 8, 128, 64, 400, 200
    cfg = workload.custom(B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, S=S, W=W, kv_dtype="fp8",
                          keep_lo=0.6, keep_hi=0.9, seed=5)
    lay = workload.make_layer(cfg, 0)
    d = dev()
    pc = PagedKVCache(B, Hkv, D, W, n_pages=64, max_pages=16, kv_dtype="fp8", device=d)
    pc.admit(0, lay.k.to(d), lay.v.to(d), lay.keep.to(d), T, reserve=0)
    cc, _ = gpu_prefill(lay.k, lay.v, lay.keep, T, W, 0, "fp8", with_dst=False)
    o = oracle_prefill(lay.k, lay.v, lay.keep, T, W, S, "fp8")
    kd, vd, qd = lay.k.to(d), lay.v.to(d), lay.q.to(d)
    keep_new = lay.keep[:, :, T:].permute(2, 0, 1).contiguous().to(d)
    for s in range(S):
        if s % 64 == 0:
            pc.refill(64)
        out = pc.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s], out_dtype=torch.float32)
        cc.decode_step(kd[:, T + s], vd[:, T + s], keep_new[s], qd[s], out_dtype=torch.float32)
        o.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s])
    torch.cuda.synchronize()
    ref, _ = oracle.attention(lay.q[S - 1], lay.k, lay.v, lay.keep, T + S - 1, W, oracle.FP8,
                              o.k_amax, o.v_amax)
    check_close(out.cpu().numpy(), ref, "last step")
    assert pc.error_word() == 0
    assert cc.error_word() & CDA_DEVERR_CAPACITY       # the contiguous store ran out
    for i in range(B * Hkv):
        n = int(o.stored_rows()[i])
        kr, vr = segment_rows(pc, i, n)
        a = int(o.seg_base[i])
        assert np.array_equal(kr.cpu().numpy(), o.k_pool[a:a + n])
        assert np.array_equal(vr.cpu().numpy(), o.v_pool[a:a + n])


def test_short_stack():
    """Admission that does not fit takes nothing; a refill that does not fit
    serves the earlier segments first; both set CDA_DEVERR_PAGES."""
    B, Hkv, Hq, D, W = 3, 2, 4, 64, 16
    c = PagedKVCache(B, Hkv, D, W, n_pages=12, max_pages=8, kv_dtype="bf16", device=dev())
    book = PagedBook(12, B, Hkv, W, 8)
    r0 = Request(300, 10, Hq, Hkv, D, W, "bf16", seed=1, keep_rate=0.9)
    r1 = Request(900, 10, Hq, Hkv, D, W, "bf16", seed=2, keep_rate=0.9)
    assert _admit(c, book, 0, r0, 0) is True
    _check_book(c, book, "first admission")
    assert _admit(c, book, 1, r1, 0) is False          # too long for what is left
    _check_book(c, book, "refused admission")
    assert c.error_word() & CDA_DEVERR_PAGES
    assert int(c.pos[1].item()) == -1
    c.refill(400)
    comp = np.zeros(B * Hkv, int)
    comp[:Hkv] = r0.o.comp_len
    book.refill(comp, 400)
    _check_book(c, book, "short refill")
    assert book.pages_error and c.free_count() == 0
    c.release(0)
    book.release(0, 1)
    _check_book(c, book, "release")
    assert c.free_count() == 12
