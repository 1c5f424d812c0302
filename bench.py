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

Reported: value = decode-attention KV bytes moved per second over the whole
step (algorithmic bytes: every stored row's K and V read once per decode
step and layer, divided by the step's wall time); the roofline of the
decode-step kernel, its per-launch duration measured with HIP events on its
stream around the decode part of each timed step; the CPU oracle timed on a
bounded sample; and parity of that sample.
"""
from __future__ import annotations

import argparse
import glob
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


REFILL = 64   # --paged: rows of headroom a refill leaves, and steps between refills


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
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / f16 MFMA of the MI355X


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


def cpu_baseline(cfg, layers, outs, kv_dtype, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample: for layer 0, 1, ...
    (until the budget is spent) the prefill absmax and the attention of all
    B x Hq query heads at the last decode step.  Returns the record and the
    worst parity error of the GPU outputs of those layers."""
    import oracle
    from workload import make_layer
    od = {"bf16": oracle.BF16, "fp8": oracle.FP8, "fp4": oracle.FP4}[kv_dtype]
    T, S, W = cfg.T, cfg.S, cfg.W
    nbytes, t_used, worst, done = 0, 0.0, 0.0, 0
    for l in layers:
        lay = make_layer(cfg, l)
        t0 = time.perf_counter()
        ka, va = oracle.prefill_amax(lay.k, lay.v, lay.keep, T, W)
        ref, _ = oracle.attention(lay.q[S - 1], lay.k, lay.v, lay.keep, T + S - 1, W, od,
                                  ka, va)
        t_used += time.perf_counter() - t0
        n = stored_rows_host(lay.keep.numpy(), T, W, S)[S - 1]
        nbytes += int(n.sum()) * 2 * ROW_BYTES[kv_dtype](cfg.D)
        got = outs[l].float().cpu().numpy()
        err = np.abs(got - ref)
        tol = 2e-3 + 1e-2 * np.abs(ref) + np.abs(ref) * 2.0 ** -8   # bf16 output rounding
        if not np.all(err <= tol):
            raise AssertionError(f"bench parity failed on layer {l}: max err {err.max():.3e}")
        worst = max(worst, float(err.max()))
        done += 1
        if t_used >= budget_s:
            break
    rec = {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"layers 0..{done - 1}: prefill absmax + fp64 attention of all "
                     f"{cfg.B}x{cfg.Hq} query heads at the last decode step "
                     f"({nbytes / 1e6:.1f} MB of compact KV, {t_used:.1f} s)"}
    return rec, worst, done


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
                    help="only run a plain 64 MiB device copy 3 times (the reference kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the compact decode-attention path runs on a "
              "single device; there is no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workload
    from compressed_decode_attention_amd import CompactKVCache, PagedKVCache, _lib

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 64 MiB three times")
        return
    cfg = workload.CONFIGS[args.config]
    kv = args.kv or cfg.kv_dtype
    L = args.layers or cfg.L
    B, Hq, Hkv, D, T, S, W = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.T, cfg.S, cfg.W
    row_bytes = ROW_BYTES[kv](D)
    log(f"config {cfg.name}: L={L} B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} S={S} W={W} "
        f"{kv}; generating inputs")

    t0 = time.perf_counter()
    kd, vd, keepd, keep_new, qd, caches, nrows = [], [], [], [], [], [], []
    for l in range(L):
        lay = workload.make_layer(cfg, l)
        kd.append(lay.k.to(dev))
        vd.append(lay.v.to(dev))
        keepd.append(lay.keep.to(dev))
        keep_new.append(lay.keep[:, :, T:].permute(2, 0, 1).contiguous().to(dev))
        qd.append(lay.q.to(dev))
        nrows.append(stored_rows_host(lay.keep.numpy(), T, W, S))
        if args.paged:
            # pages for each segment's last rows plus one refill's headroom
            pages = -(-(nrows[l][S - 1].astype(np.int64) + REFILL) // 64)
            c = PagedKVCache(B, Hkv, D, W, int(pages.sum()), int(pages.max()), kv, dev)
        else:
            c = CompactKVCache(B, Hkv, D, W, kv, dev)
            c.count(keepd[l], T, reserve=S)
            c.allocate()
        c.workspace(Hq, args.split)
        caches.append(c)
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
    log(f"inputs resident in {time.perf_counter() - t0:.1f} s")

    # algorithmic bytes of every attention call: stored rows x 2 x D x e
    attn_bytes = np.array([[int(nrows[l][s].sum()) * 2 * row_bytes for l in range(L)]
                           for s in range(S)], np.float64)          # [S, L]
    step_attn_bytes = float(attn_bytes.sum())

    def prefill_all():
        for l in range(L):
            c = caches[l]
            if args.paged:
                c.init()
                c.admit(0, kd[l], vd[l], keepd[l], T, reserve=0)
            else:
                c.count(keepd[l], T, reserve=S)
                c.pack(kd[l], vd[l], keepd[l], T)

    def decode_all():
        if args.chunk > 0:
            for j in range(len(chunks[0])):
                for l in range(L):
                    s0, m, kp, qc, oc = chunks[l][j]
                    c = caches[l]
                    if args.paged:
                        c.refill(max(REFILL, m))
                    c.chunk(kd[l][:, T + s0:T + s0 + m], vd[l][:, T + s0:T + s0 + m], kp, qc,
                            out=oc)
            return
        for s in range(S):
            for l in range(L):
                c = caches[l]
                if args.paged and s % REFILL == 0:
                    c.refill(REFILL)
                if args.unfused:
                    c.append(kd[l][:, T + s], vd[l][:, T + s], keep_new[l][s])
                    c.attention(qd[l][s], out=outs[l], split_tokens=args.split)
                else:
                    c.decode_step(kd[l][:, T + s], vd[l][:, T + s], keep_new[l][s], qd[l][s],
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
        log(f"captured {2 * L} prefill and {S * L * (2 if args.unfused else 1)} decode launches "
            f"in two graphs")

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

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    words = [c.error_word() for c in caches]
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
    for l in range(L):
        c = caches[l]
        ring = np.minimum(c.pos[:B].cpu().numpy().astype(np.int64), W)
        got = ring[:, None] + c.comp_len.cpu().numpy().astype(np.int64).reshape(B, Hkv)
        if not np.array_equal(got, nrows[l][S - 1]):
            raise RuntimeError(f"layer {l}: device stored-row counts differ from the keep mask")
        if caches[l].error_word() != 0:
            raise RuntimeError(f"layer {l}: device error word set")

    # Per-launch duration of the decode-step kernel: the decode part of each
    # timed step (S x L back-to-back launches on this stream, between two HIP
    # events, gaps between launches included) divided by the launches; the
    # algorithmic bytes per launch are the mean over the same launches.  With
    # --unfused this is the time of one layer step (APPEND + attention).
    n_calls = (len(chunks[0]) if args.chunk > 0 else S) * L
    kernel_us = float(np.mean(decode_ms_l)) * 1e3 / n_calls
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
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                    "traffic": None}
    else:
        roofline = None
    # the committed counters are those of the default run (this config, FP8)
    traffic = (traffic_from_profile() if (args.config, kv) == ("qwen_c8", "fp8") and
               not args.paged else None)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        # the answers at the last position: the decode step's output, or the
        # last query of the last chunk
        last = outs if args.chunk <= 0 else [chunks[l][-1][4][:, -1] for l in range(L)]
        cpu, worst, nl = cpu_baseline(cfg, list(range(L)), last, kv)
        log(f"oracle sample: {nl} layers, GPU max abs err {worst:.2e}")

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
                   "kv_storage": kv, "budget": cfg.budget,
                   "store": (f"paged: 64-row pages, no prefill reserve, refill every {REFILL} steps"
                             if args.paged else f"contiguous segments, reserve {S} rows"),
                   "split_tokens": args.split or "library default",
                   "parallelism": "single GPU"},
        "attn_tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        ("chunk_call_us" if args.chunk > 0 else "decode_step_kernel_us"): round(kernel_us, 3),
        "prefill_compaction_ms": round(prefill_ms, 3),
        "decode_ms_per_step": round(float(np.mean(decode_ms_l)), 3),
        "launch": ("eager" if args.eager else "hip graphs") +
                  (f", chunks of {args.chunk} tokens (chunk_attn_compact)" if args.chunk > 0 else
                   ", append + attention" if args.unfused else ", fused decode step"),
        "kv_bytes_per_decode_step": round(float(attn_bytes.sum(axis=1).mean())),
        "kv_pool_mb": round(sum(2 * c.pool_rows * row_bytes for c in caches) / 1e6, 1),
        "roofline": roofline or {"bound": "hbm", "achieved": round(achieved, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
