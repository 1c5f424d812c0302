"""Benchmark of compact decode attention on one MI355X.

Workload: the Qwen3-8B attention shape at c = 8 (36 layers, 32 query / 8 KV
heads, head_dim 128, batch 8, ctx 8192, gen 128), FP8-E4M3 compact KV with
per-(sequence, head) scales, keep rates U[0.04, 0.25] per head, 1% outlier
channels x8, always-kept window 256 -- the FastDMS page's Qwen3-8B c = 8
memory-table row, on synthetic inputs (no weights, no dataset).

One step = one pass of the whole path over the batch, everything already
resident in HBM:
  prefill compaction of every layer (kv_compact COUNT + PACK), then
  128 decode steps x 36 layers of decode_step_compact (the append of the
  new token and the attention over the compact store, one launch each),
all enqueued on one stream with no host synchronisation inside the step.
The prefill and the decode launches are captured once into two HIP graphs
(no memset or allocation inside; every replay starts from COUNT, so it
redoes the same work) and replayed each step; --eager issues every call
from Python instead, --unfused uses kv_compact APPEND + decode_attn_compact.

Workloads that fit in the 256 MB last-level cache (--config llama_c1,
qwen_c1, llama_c8) rotate R replicas of every layer's store (--replicas,
default: enough for 1 GB), so that no launch finds its layer in that cache;
decode step s then runs on replica s mod R, at that replica's own position.

Reported: value = decode-attention KV bytes moved per second over the whole
step (algorithmic bytes: every stored row's K and V read once per decode
step and layer, divided by the step's wall time), with the median and
10th/90th percentiles of the step and launch times; the roofline of the
decode-step kernel, its per-launch duration measured with HIP events on its
stream around the decode part of each timed step, beside the measured read
ceiling of the same access pattern (a plain streaming kernel over 2 GiB and
over exactly one layer's tiles); the realised compression ratio of the
store; the CPU oracle timed on one thread and on every core on a bounded
sample, the FP8 saturations and byte accounting of that sample, and the
parity of the GPU output there.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compact decode-attn HBM GB/s (% of peak) + attn tokens/s, Qwen3-8B ctx8192"
HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "compressed_decode_attention_amd", "csrc", "attn.hip")
STREAM_LIB = os.path.join(ROOT, "compressed_decode_attention_amd", "libcda_stream.so")
MALL_BYTES = 256 << 20           # last-level (Infinity) cache of the device
CEILING_BYTES = 2 << 30          # buffer of the read-ceiling measurement

REFILL = 64   # --paged: rows of headroom a refill leaves, and steps between refills
ORACLE_STEPS = 4                 # decode steps of the timed oracle sample


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stored_rows_host(keep_np, T, W, S):
    """n[s, b, h]: stored rows of every segment after the append of step s
    (W most recent positions + kept older ones) -- byte accounting only."""
    B, Hkv, _ = keep_np.shape
    kept = (keep_np != 0).astype(np.int64)
    csum = np.concatenate([np.zeros((B, Hkv, 1), np.int64), np.cumsum(kept, axis=2)], axis=2)
    out = np.zeros((S, B, Hkv), np.int64)
    for s in range(S):
        P = T + s
        older = max(P - W + 1, 0)           # positions 0 .. P-W are "older"
        out[s] = min(W, P + 1) + csum[:, :, older]
    return out


def rows_before_host(keep_np, T, W, s0):
    """n[b, h]: stored rows of every segment before the token at T + s0 is
    appended (after prefill when s0 = 0) -- byte accounting only."""
    kept = (keep_np != 0).astype(np.int64)
    P = T + s0 - 1                          # newest stored position
    older = max(P - W + 1, 0)
    return min(W, P + 1) + kept[:, :, :older].sum(axis=2)


ROW_BYTES = {"bf16": lambda D: 2 * D, "fp8": lambda D: D, "fp4": lambda D: D // 2}
ELEM_BYTES = {"bf16": 2.0, "fp8": 1.0, "fp4": 0.5}


def compression_ratio(stored_rows, layers, B, Hkv, D, tokens, kv):
    """The store's bytes (stored rows x K and V rows, plus two f32 scales per
    head for FP8 / FP4) against dense BF16 and dense same-format pools that
    keep K and V of every position 0 .. tokens - 1 for every layer, sequence
    and KV head."""
    compact = stored_rows * 2 * ROW_BYTES[kv](D) + (0 if kv == "bf16" else 8 * B * Hkv * layers)
    dense_bf16 = layers * B * Hkv * tokens * 2 * D * 2
    dense_same = layers * B * Hkv * tokens * 2 * D * ELEM_BYTES[kv]
    return {"vs_dense_bf16": round(dense_bf16 / compact, 3),
            "vs_dense_same_dtype": round(dense_same / compact, 3),
            "compact_kv_bytes": int(compact), "dense_bf16_bytes": int(dense_bf16),
            "stored_rows_per_head_mean": round(stored_rows / (layers * B * Hkv), 1),
            "positions_per_head": tokens}
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / f16 MFMA of the MI355X


def pct(x, q):
    return round(float(np.percentile(np.asarray(x, np.float64), q)), 3)


def traffic_from_profile():
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current attention kernel source."""
    path = os.path.join(ROOT, "profiles", "attn_qwen_c8_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if rec.get("attn_src_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def chunk_traffic_from_profile():
    """HBM bytes per chunk call (M = 64, its two launches) from the committed
    counter summary, if it was taken on the current chunk kernel source."""
    path = os.path.join(ROOT, "profiles", "chunk_qwen_c8_chunk64_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "compressed_decode_attention_amd", "csrc", "chunk.hip")
    if rec.get("chunk_src_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return rec.get("hbm_bytes_per_call")


def stream_lib():
    if not os.path.exists(STREAM_LIB):
        raise RuntimeError(f"{STREAM_LIB} is missing: build it with `python -c 'import "
                           f"__graft_entry__ as g; g.build()'`")
    L = C.CDLL(STREAM_LIB)
    L.cda_stream_tiles.argtypes = [C.c_void_p] * 3 + [C.c_int32] * 4 + [C.c_void_p] * 2
    L.cda_stream_tiles.restype = C.c_int32
    return L


def graph_us(torch, fn, calls, reps=5):
    """Median time of one call of fn, from a HIP graph of `calls` calls."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t = []
    for _ in range(reps):
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3 / calls)
    return float(np.median(t))


STREAM_SHAPES = [(w, sp) for sp in (0, 1) for w in (1, 2, 4, 8)]   # (waves per group, split)


def read_ceiling(torch, dev, tile_bytes, layer_tiles):
    """The plain streaming read of 64-row tiles (the attention's access
    pattern, no arithmetic), in each launch shape: GB/s over 2 GiB, and the
    time of reading exactly the tiles of one layer's launch -- 200 launches
    in a graph, each on its own copy of the layer's K and V regions (as many
    copies as fit in 2 GiB, in turn), so that no launch finds its tiles in
    the last-level cache.  The best shape of each is the ceiling and the
    load-only floor."""
    L = stream_lib()
    stream = lambda: C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    buf = torch.empty(CEILING_BYTES, dtype=torch.uint8, device=dev)
    base = buf.data_ptr()
    half = CEILING_BYTES // 2
    n_big = half // tile_bytes
    n_layer = len(layer_tiles)
    region = (int(np.max(layer_tiles)) + 1) * tile_bytes     # one pool of the layer
    copies = CEILING_BYTES // (2 * region)
    assert copies >= 1
    sink = torch.empty(2 * max(n_big, n_layer), dtype=torch.int32, device=dev)
    tiles = torch.as_tensor(np.asarray(layer_tiles, np.int32), device=dev)

    def call(k, v, listed, n, waves, split):
        def f():
            st = L.cda_stream_tiles(C.c_void_p(k), C.c_void_p(v),
                                    C.c_void_p(tiles.data_ptr()) if listed else None, n,
                                    tile_bytes, waves, split, C.c_void_p(sink.data_ptr()),
                                    stream())
            assert st == 0, st
        return f

    def layer_calls(waves, split):
        fns = [call(base + (j % copies) * 2 * region, base + (j % copies) * 2 * region + region,
                    True, n_layer, waves, split) for j in range(200)]
        return lambda: [f() for f in fns]
    big, lay = {}, {}
    for w, sp in STREAM_SHAPES:
        us = graph_us(torch, call(base, base + half, False, n_big, w, sp), 10)
        big[f"w{w}s{sp}"] = round(2 * n_big * tile_bytes / (us * 1e-6) / 1e9, 1)
        lay[f"w{w}s{sp}"] = round(graph_us(torch, layer_calls(w, sp), 1) / 200, 3)
    del buf
    best_big = max(big, key=big.get)
    best_lay = min(lay, key=lay.get)
    return {"stream_gbs": big[best_big], "stream_shape": best_big, "stream_bytes": CEILING_BYTES,
            "layer_tiles_us": lay[best_lay], "layer_tiles_shape": best_lay,
            "layer_tiles_gbs": round(2 * n_layer * tile_bytes / (lay[best_lay] * 1e-6) / 1e9, 1),
            "layer_tile_bytes": 2 * n_layer * tile_bytes, "layer_copies": copies,
            "stream_gbs_by_shape": big, "layer_tiles_us_by_shape": lay,
            "kernel": "cda_stream_tiles: 16-byte nontemporal loads of whole 64-row tiles, all "
                      "of a wave's loads in flight together; shape wXsY = X waves per "
                      "workgroup, Y = 1: one wave per K or V tile, Y = 0: one wave reads a K "
                      "tile and its V tile"}


def cpu_baseline(cfg, kv, dev_rows_l0, out_f32_l0, budget_note=""):
    """The oracle, as it stands, on a bounded sample of the same workload:
    layer 0 of the full shape, prefill compaction plus the first
    ORACLE_STEPS decode steps (append, then fp64 attention of all B x Hq
    query heads), timed on one thread and on every core.  Then the rest of
    that layer's appends (FP8 saturations, stored rows and byte accounting
    at the end, checked against the device) and its attention at the last
    position (parity of the GPU's F32 output there)."""
    import oracle
    from workload import make_layer
    od = {"bf16": oracle.BF16, "fp8": oracle.FP8, "fp4": oracle.FP4}[kv]
    T, S, W, B, Hkv, D = cfg.T, cfg.S, cfg.W, cfg.B, cfg.Hkv, cfg.D
    lay = make_layer(cfg, 0)
    times, threads, nbytes = {}, {}, 0
    for mode in (1, 0):
        n = oracle.set_threads(mode)
        t0 = time.perf_counter()
        c = oracle.prefill_pack(lay.k, lay.v, lay.keep, T, W, S, od, align=64)
        nbytes = 0
        for s in range(ORACLE_STEPS):
            c.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s].contiguous())
            oracle.attention(lay.q[s], lay.k, lay.v, lay.keep, T + s, W, od, c.k_amax, c.v_amax)
            nbytes += int(c.stored_rows().sum()) * 2 * oracle.row_bytes(D, od)
        times[mode] = time.perf_counter() - t0
        threads[mode] = n
    for s in range(ORACLE_STEPS, S):
        c.append(lay.k[:, T + s], lay.v[:, T + s], lay.keep[:, :, T + s].contiguous())
    rows = c.stored_rows().astype(np.int64)
    if not np.array_equal(rows, dev_rows_l0.reshape(-1)):
        raise AssertionError("layer 0: device stored rows differ from the oracle's store")
    ref, _ = oracle.attention(lay.q[S - 1], lay.k, lay.v, lay.keep, T + S - 1, W, od,
                              c.k_amax, c.v_amax)
    err = np.abs(out_f32_l0 - ref)
    tol = 2e-3 + 1e-2 * np.abs(ref)
    if not np.all(err <= tol):
        raise AssertionError(f"bench parity failed on layer 0: max err {err.max():.3e}")
    compact = oracle.compact_kv_bytes(int(rows.sum()), D, od, B * Hkv)
    rec = {"value": round(nbytes / times[0] / 1e9, 4), "unit": "GB/s", "cores": threads[0],
           "value_1_thread": round(nbytes / times[1] / 1e9, 4), "kind": "oracle",
           "sample": f"layer 0 of {cfg.name}: prefill compaction + the first {ORACLE_STEPS} "
                     f"decode steps (append, then fp64 attention of all {B}x{cfg.Hq} query "
                     f"heads); {nbytes / 1e6:.1f} MB of compact KV attended; "
                     f"{times[0]:.2f} s on {threads[0]} threads, {times[1]:.2f} s on 1",
           "ms_per_decode_step_all_cores": round(times[0] * 1e3 / ORACLE_STEPS, 1)}
    extra = {"fp8_saturated": int(c.saturated) if od != oracle.BF16 else 0,
             "oracle_compact_kv_bytes_layer0": int(compact),
             "oracle_dense_bf16_bytes_layer0": int(oracle.dense_kv_bytes(1, B * Hkv, D, T + S, 2)),
             "max_abs_err_f32_layer0": float(err.max()),
             "max_rel_err_f32_layer0": float((err / np.maximum(np.abs(ref), 1e-30)).max())}
    return rec, extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="qwen_c8")
    ap.add_argument("--kv", choices=["bf16", "fp8", "fp4"], default=None,
                    help="stored format (default: the config's; fp4 is the 4-bit variant)")
    ap.add_argument("--layers", type=int, default=0, help="0 = all layers of the config")
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=0,
                    help="replicas of every layer's store, rotated per decode step; 0 = as "
                         "many as make the stores at least 1 GB (1 for the c = 8 Qwen shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--eager", action="store_true", help="issue every call from Python (no graphs)")
    ap.add_argument("--paged", action="store_true",
                    help="paged store: 64-row pages, no prefill reserve, a refill every 64 "
                         "steps (inside the timed step)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="M > 0: the gen_len tokens of each layer arrive as chunks of M "
                         "(chunk_attn_compact: multi-query attention, then the append) "
                         "instead of one decode step each")
    ap.add_argument("--unfused", action="store_true",
                    help="decode steps as kv_compact APPEND + decode_attn_compact")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 64 MiB device copy 3 times (the reference for "
                         "scaling WRITE_SIZE), then exit")
    ap.add_argument("--stream-calibration", action="store_true",
                    help="only read 2 GiB with the tile-streaming kernel 3 times (the "
                         "reference for scaling FETCH_SIZE), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the compact decode-attention path runs on a "
              "single device; there is no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workload
    from compressed_decode_attention_amd import CompactKVCache, PagedKVCache

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 64 MiB three times")
        return
    if args.stream_calibration:
        L_ = stream_lib()
        buf = torch.zeros(CEILING_BYTES, dtype=torch.uint8, device=dev)
        sink = torch.empty(1 << 20, dtype=torch.int32, device=dev)
        half, tb = CEILING_BYTES // 2, 8192
        for _ in range(3):
            assert L_.cda_stream_tiles(C.c_void_p(buf.data_ptr()),
                                       C.c_void_p(buf.data_ptr() + half), None, half // tb, tb,
                                       8, 0, C.c_void_p(sink.data_ptr()),
                                       C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)) == 0
        torch.cuda.synchronize()
        log(f"streamed {CEILING_BYTES >> 20} MiB three times ({half // tb} tiles of 2 x {tb} B)")
        return
    cfg = workload.CONFIGS[args.config]
    kv = args.kv or cfg.kv_dtype
    L = args.layers or cfg.L
    B, Hq, Hkv, D, T, S, W = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.T, cfg.S, cfg.W
    row_bytes = ROW_BYTES[kv](D)
    log(f"config {cfg.name}: L={L} B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} S={S} W={W} "
        f"{kv}; generating inputs")

    t0 = time.perf_counter()
    kd, vd, keepd, keep_new, qd, nrows = [], [], [], [], [], []
    for l in range(L):
        lay = workload.make_layer(cfg, l)
        kd.append(lay.k.to(dev))
        vd.append(lay.v.to(dev))
        keepd.append(lay.keep.to(dev))
        keep_new.append(lay.keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev))
        qd.append(lay.q.to(dev))
        nrows.append(stored_rows_host(lay.keep.numpy(), T, W, S))
    # bytes of the stores: one replica unless they fit in the last-level cache
    est = sum(int(nrows[l][S - 1].sum() + B * Hkv * S) * 2 * row_bytes for l in range(L))
    R = args.replicas or (1 if est >= 3 * MALL_BYTES else -(-(1 << 30) // est))
    if args.chunk > 0 or args.paged:
        R = 1
    S_r = [len(range(r, S, R)) for r in range(R)]      # decode steps of each replica

    def new_cache(l):
        if args.paged:
            # pages for each segment's last rows plus one refill's headroom
            pages = -(-(nrows[l][S - 1].astype(np.int64) + REFILL) // 64)
            c = PagedKVCache(B, Hkv, D, W, int(pages.sum()), int(pages.max()), kv, dev)
        else:
            c = CompactKVCache(B, Hkv, D, W, kv, dev)
            c.count(keepd[l], T, reserve=S_r[0])
            c.allocate()
        c.workspace(Hq, args.split)
        return c
    caches = [[new_cache(l) for l in range(L)] for _ in range(R)]     # [replica][layer]
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    # --chunk: per layer and chunk, (start, tokens, keep [B, m, Hkv], q [B, m, Hq, D], out)
    chunks = []
    if args.chunk > 0:
        for l in range(L):
            lc = []
            for s0 in range(0, S, args.chunk):
                m = min(args.chunk, S - s0)
                lc.append((s0, m, keepd[l][:, :, T + s0:T + s0 + m].permute(0, 2, 1).contiguous(),
                           qd[l][s0:s0 + m].permute(1, 0, 2, 3).contiguous(),
                           torch.empty((B, m, Hq, D), dtype=torch.bfloat16, device=dev)))
            chunks.append(lc)
    torch.cuda.synchronize()
    log(f"inputs resident in {time.perf_counter() - t0:.1f} s; {R} replica(s) of the stores")

    # algorithmic bytes of every attention call: stored rows x 2 x D x e;
    # decode step s runs on replica s mod R at that replica's step s // R
    attn_bytes = np.array([[int(nrows[l][s // R].sum()) * 2 * row_bytes for l in range(L)]
                           for s in range(S)], np.float64)          # [S, L]
    step_attn_bytes = float(attn_bytes.sum())

    def prefill_all():
        for reps in caches:
            for l in range(L):
                c = reps[l]
                if args.paged:
                    c.init()
                    c.admit(0, kd[l], vd[l], keepd[l], T, reserve=0)
                else:
                    c.count(keepd[l], T, reserve=S_r[0])
                    c.pack(kd[l], vd[l], keepd[l], T)

    def decode_all():
        if args.chunk > 0:
            for j in range(len(chunks[0])):
                for l in range(L):
                    s0, m, kp, qc, oc = chunks[l][j]
                    c = caches[0][l]
                    if args.paged:
                        c.refill(max(REFILL, m))
                    c.chunk(kd[l][:, T + s0:T + s0 + m], vd[l][:, T + s0:T + s0 + m], kp, qc,
                            out=oc)
            return
        for s in range(S):
            k = s // R                        # the replica's own step
            for l in range(L):
                c = caches[s % R][l]
                if args.paged and s % REFILL == 0:
                    c.refill(REFILL)
                if args.unfused:
                    c.append(kd[l][:, T + k], vd[l][:, T + k], keep_new[l][k])
                    c.attention(qd[l][k], out=outs[l], split_tokens=args.split)
                else:
                    c.decode_step(kd[l][:, T + k], vd[l][:, T + k], keep_new[l][k], qd[l][k],
                                  out=outs[l], split_tokens=args.split)

    # one eager pass first: loads the library, sizes the workspaces
    prefill_all()
    decode_all()
    torch.cuda.synchronize()
    graphs = None
    if not args.eager:
        g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pre):
            prefill_all()
        with torch.cuda.graph(g_dec):
            decode_all()
        torch.cuda.synchronize()
        graphs = (g_pre, g_dec)
        log(f"captured {2 * L * R} prefill and {S * L * (2 if args.unfused else 1)} decode "
            f"launches in two graphs")

    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def run_step():
        ev[0].record(stream)
        if graphs:
            graphs[0].replay()
        else:
            prefill_all()
        ev[1].record(stream)
        if graphs:
            graphs[1].replay()
        else:
            decode_all()
        ev[2].record(stream)

    all_caches = [c for reps in caches for c in reps]
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    words = [c.error_word() for c in all_caches]
    if any(words):
        raise RuntimeError(f"device error words set during warm-up: {words} "
                           f"(1 capacity, 2 pool, 16 merge wait, 32 stale host plan)")
    log(f"warm-up done ({args.warmup} steps); timing {args.steps} steps")

    step_ms, prefill_ms_l, decode_ms_l = [], [], []
    for k in range(args.steps):
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        run_step()
        torch.cuda.synchronize()
        step_ms.append((time.perf_counter() - t_start) * 1e3)
        prefill_ms_l.append(ev[0].elapsed_time(ev[1]))
        decode_ms_l.append(ev[1].elapsed_time(ev[2]))
        log(f"step {k}: {step_ms[-1]:.2f} ms (prefill {prefill_ms_l[-1]:.2f} ms, "
            f"decode {decode_ms_l[-1]:.2f} ms)")

    # the device state after the last step must match the host accounting
    dev_rows = []
    for r in range(R):
        dev_rows.append([])
        for l in range(L):
            c = caches[r][l]
            ring = np.minimum(c.pos[:B].cpu().numpy().astype(np.int64), W)
            got = ring[:, None] + c.comp_len.cpu().numpy().astype(np.int64).reshape(B, Hkv)
            if args.chunk <= 0 and not np.array_equal(got, nrows[l][S_r[r] - 1]):
                raise RuntimeError(f"replica {r} layer {l}: device stored-row counts differ "
                                   f"from the keep mask")
            if c.error_word() != 0:
                raise RuntimeError(f"replica {r} layer {l}: device error word set")
            dev_rows[r].append(got)

    # Per-launch duration of the decode-step kernel: the decode part of each
    # timed step (S x L back-to-back launches on this stream, between two HIP
    # events, gaps between launches included) divided by the launches; the
    # algorithmic bytes per launch are the mean over the same launches.  With
    # --unfused this is the time of one layer step (APPEND + attention).
    n_calls = (len(chunks[0]) if args.chunk > 0 else S) * L
    launch_us = [d * 1e3 / n_calls for d in decode_ms_l]
    kernel_us = float(np.mean(launch_us))
    bytes_per_launch = float(attn_bytes.mean())
    flops_per_call = None
    if args.chunk > 0:
        # each chunk call reads the rows stored before it once (algorithmic
        # bytes), and its queries t see those rows plus chunk tokens <= t:
        # 2 x 2 x D flops per (visible row, query row), for QK and PV
        cb, cf = [], []
        for l in range(L):
            keep_np = keepd[l].cpu().numpy()
            for s0, m, *_ in chunks[l]:
                n0 = rows_before_host(keep_np, T, W, s0).astype(np.float64)
                cb.append(float(n0.sum()) * 2 * row_bytes)
                cf.append(4.0 * D * (Hq // Hkv) * float((m * n0 + m * (m + 1) / 2).sum()))
        step_attn_bytes = float(np.sum(cb))
        bytes_per_launch = float(np.mean(cb))
        flops_per_call = float(np.mean(cf))
    prefill_ms = float(np.mean(prefill_ms_l))

    ms = float(np.mean(step_ms))
    value = step_attn_bytes / (ms * 1e-3) / 1e9
    tokens_per_s = B * S / (ms * 1e-3)
    achieved = bytes_per_launch / (kernel_us * 1e-6) / 1e9
    if flops_per_call is not None:
        tflops = flops_per_call / (kernel_us * 1e-6) / 1e12
        # the committed counters are those of one M = 64 call of this config (FP8)
        traffic = (chunk_traffic_from_profile() if (args.config, kv, R, args.chunk) ==
                   ("qwen_c8", "fp8", 1, 64) and not args.paged else None)
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                    "traffic": traffic}
    else:
        # the committed counters are those of the default run (this config, FP8)
        traffic = (traffic_from_profile() if (args.config, kv, R) == ("qwen_c8", "fp8", 1) and
                   not args.paged and not args.unfused else None)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}

    # the realised compression of the store after the last decode step
    # (replica 0): stored rows x K and V rows (+ two f32 scales per head for
    # FP8 / FP4), against dense pools of every position 0 .. T + S - 1
    stored = sum(int(dev_rows[0][l].sum()) for l in range(L))
    compression = compression_ratio(stored, L, B, Hkv, D, T + S_r[0], kv)

    ceiling = None
    if not args.no_ceiling and not args.paged and args.chunk <= 0:
        log("measuring the read ceiling (tile streaming)")
        c0 = caches[0][0]
        sbh = c0.seg_base_host.numpy()
        rows0 = dev_rows[0][0].reshape(-1)
        tiles = [int(sbh[i]) // 64 + t for i in range(B * Hkv) for t in range(-(-int(rows0[i]) // 64))]
        ceiling = read_ceiling(torch, dev, 64 * row_bytes, tiles)
        ceiling["frac_of_ceiling"] = round(achieved / ceiling["stream_gbs"], 4)
        ceiling["launch_over_layer_tiles_floor"] = round(kernel_us / ceiling["layer_tiles_us"], 3)

    cpu, cpu_extra = None, {}
    if not args.no_cpu_baseline and args.chunk <= 0 and R == 1 and not args.paged:
        log("timing the CPU oracle on a sample")
        # the GPU's F32 answer at the last position of layer 0: attention
        # over the store as the last decode step left it
        out32 = caches[0][0].attention(qd[0][S - 1], out_dtype=torch.float32)
        torch.cuda.synchronize()
        cpu, cpu_extra = cpu_baseline(cfg, kv, dev_rows[0][0], out32.cpu().double().numpy())
        layer0 = compression_ratio(int(dev_rows[0][0].sum()), 1, B, Hkv, D, T + S_r[0], kv)
        if cpu_extra["oracle_compact_kv_bytes_layer0"] != layer0["compact_kv_bytes"]:
            raise AssertionError("compact KV bytes of layer 0 differ from the oracle's accounting")
        if cpu_extra["oracle_dense_bf16_bytes_layer0"] != layer0["dense_bf16_bytes"]:
            raise AssertionError("dense BF16 bytes of layer 0 differ from the oracle's accounting")
        log(f"oracle sample done: {cpu['sample']}")

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.L} layers x (Hq {Hq}, Hkv {Hkv}, D {D}), "
                               f"ctx {T}, gen {S}, c={B}, {kv} compact KV, W={W}" +
                               (", keep rate x1.5 at layer 0 falling linearly to x0.5 "
                                "at the last layer" if cfg.budget == "pyramid" else ""),
                   "layers": L, "global_batch": B, "seq_len": T, "gen_len": S,
                   "kv_storage": kv, "budget": cfg.budget, "replicas": R,
                   "store": (f"paged: 64-row pages, no prefill reserve, refill every {REFILL} steps"
                             if args.paged else f"contiguous segments, reserve {S_r[0]} rows"),
                   "split_tokens": args.split or "library default",
                   "parallelism": "single GPU"},
        "ms_per_step_median": pct(step_ms, 50),
        "ms_per_step_p10": pct(step_ms, 10),
        "ms_per_step_p90": pct(step_ms, 90),
        "attn_tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        ("chunk_call_us" if args.chunk > 0 else "decode_step_kernel_us"): round(kernel_us, 3),
        "launch_us_median": pct(launch_us, 50),
        "launch_us_p10": pct(launch_us, 10),
        "launch_us_p90": pct(launch_us, 90),
        "decode_only_gbs": round(step_attn_bytes / (float(np.mean(decode_ms_l)) * 1e-3) / 1e9, 1),
        "prefill_compaction_ms": round(prefill_ms, 3),
        "decode_ms_per_step": round(float(np.mean(decode_ms_l)), 3),
        "launch": ("eager" if args.eager else "hip graphs") +
                  (f", chunks of {args.chunk} tokens (chunk_attn_compact)" if args.chunk > 0 else
                   ", append + attention" if args.unfused else ", fused decode step"),
        "kv_bytes_per_decode_step": round(float(attn_bytes.sum(axis=1).mean())),
        "kv_pool_mb": round(sum(2 * c.pool_rows * row_bytes for c in all_caches) / 1e6, 1),
        "compression_ratio": compression,
        "roofline": roofline,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    rec.update(cpu_extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
