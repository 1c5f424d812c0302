// Single-token GQA decode attention over the compact KV store, for gfx950,
// alone or fused with the decode-time append of the new token.
//
// What is computed (FastDMS page, release and benchmark paragraphs: decode
// over the compact store; PackKV abstract: decompression fused into the
// matrix-vector products): for every sequence b and query head j, softmax
// attention of q[b, j] over the n_i stored rows of its KV head's segment.
//
// Work split.  Each segment's rows are cut into 64-row tiles, and tiles into
// work units of `tpu` tiles; one workgroup (4 or 8 waves) takes one unit and
// each wave one tile at a time.  The unit of workgroup w comes from one of
// two plans:
//   - host plan: the caller gave a host copy of seg_base, so the launcher
//     lists the units of every segment's capacity (its seg_base span) in the
//     kernel arguments, two words per unit.  A workgroup reads its entry
//     with its other arguments and issues the loads of its first tiles
//     before it has read any of the segment's metadata; tiles past the rows
//     holding data are read too and masked out (they lie inside the
//     segment's span, hence inside the pool) -- except the tiles the
//     caller's spare_rows hint puts wholly in the end of the span that is
//     expected empty (the unfilled decode reserve, less one tile of margin
//     for its growth): their waves read them only once the metadata shows
//     data in them.
//   - device plan: every wave derives the unit -> (segment, tiles) map from
//     pos / comp_len / seg_cap (lane l looks at one segment, a wave-wide scan
//     of unit counts finds the segment holding unit w), one round trip of
//     metadata loads before the first tile load.  Used for the paged store,
//     without the host copy, or when the plan does not fit.
// A segment with one unit writes its output directly.  Otherwise every unit
// stores an unnormalised partial (m, l, o) and counts itself in with an
// atomic; the last unit of the segment to do so merges all partials with a
// log-sum-exp merge and resets the counter and the partial slots.
//
// Partials and their merge.  Partial words are stored as the bitwise NOT of
// their f32 bit patterns (0xFFFFFFFF, a NaN, is first replaced by another
// NaN), with device-coherent 8-byte stores, so a word of zero means "not yet
// written" -- the workspace is zero between calls.  A unit does not wait
// for its stores to complete before it counts itself in: the merging unit
// polls each word until it is non-zero (every store it waits for has been
// issued by a running wave, so the wait is short; the number of polls is
// bounded, CDA_DEVERR_MERGE past it), then writes zeros back.  Nothing
// depends on which XCD or CU a workgroup runs on.  The merge folds the
// partials in unit order, its own read back as stored like the others, so
// the result does not depend on which unit merges.
//
// Inside a wave, the G query rows of the KV head (G <= 16) are the N = 16
// columns of two MFMA products per tile:
//   S^T[token][g] = K_tile[token][:] . Q^T[:][g]     v_mfma_f32_16x16x32_bf16
//   O^T[d][g]    += V^T[d][token] . P^T[token][g]    v_mfma_f32_16x16x32_{f16,bf16}
// K is stored in 64-row tiles permuted so that each 64-lane load of the S
// operand is 1 KB of consecutive bytes; V is stored in 64-row tiles of four
// column-major 16-row blocks (FP4: column-major tiles), so the O operand is
// 16-byte loads of 8 or 16 consecutive tokens of one column.  Tokens are assigned to MFMA rows so that the S accumulator of
// each lane holds exactly the 16 tokens that lane needs for its P operand,
// so P never moves between lanes.  FP8 codes are converted to bf16 (K) or
// f16 (V) in registers, exactly; the K scale is folded into the logit scale
// and the V scale into the output.  With FP8 values P enters the product as
// f16 (relative rounding <= 2^-11 per weight; V codes and the products are
// exact in the f16 x f16 -> f32 MFMA).  With BF16 values P is split into a
// high and a low bf16 part (p = hi + lo to ~2^-17), since one bf16 would
// round each weight by up to 2^-9.  All K/V loads of a tile are
// unconditional (a tile never leaves its 64-row-padded segment); rows past
// the end of the segment are masked out of the logits and the values.
//
// Decode step (append fused in; FastDMS memory-table paragraph, "cache +
// staging": the token leaving the W-row ring moves to the compact tail if
// kept, the new token takes its ring row).  The result equals an append
// followed by attention, computed from the state before the append:
//   - the rows before the step are attended as they are, except that the
//     ring row of the token leaving the window is masked when that token is
//     not kept (it is the same row either way: if it moves, its values are
//     the ones now in the ring row);
//   - the new token is one more (logit, value) pair, formed from the BF16
//     input with the frozen scales by wave 0 of the unit that holds the
//     tile of its row, during that wave's first tile; the workgroup's
//     combine folds it in with the waves' partial states;
//   - the same wave then copies the leaving token's row to the compact tail
//     (if it moves) and writes the new token's row; every load of the tile
//     has completed by then.  No other workgroup reads those rows as data
//     (the compact tail is past the attended rows of its segment);
//   - the work units of a decode step are planned from the segment
//     capacities W + seg_cap, which do not change during decode, so no
//     plan depends on another segment's length; rows past the data are
//     masked like any segment end;
//   - comp_len and ring_keep of a segment are written by its last unit to
//     finish (the one that merges, or the only one), after every unit of
//     the segment has read them; that unit then counts the segment in on a
//     per-sequence counter, and the last of the Hkv segments of sequence b
//     writes pos[b] (read by the units of all of them).
//   - every counter sits on a 128-byte line of its own: atomics on one line
//     are performed one after another.
#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

constexpr int kMergeBatch = 8;        // partials loaded per round trip in the merge (2, 4 or 6
                                      // for up to that many units, x2 past 8)
constexpr int kCounterStride = 32;    // ints between counters: one 128-byte line each
constexpr int kMergePolls = 1 << 20;  // polls of one batch of partials before giving up
constexpr int kMaxPlanUnits = 512;    // units a host plan carries in the kernel arguments (4 KB)

struct AttnParams {
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t pool_rows;
  const int64_t* seg_base;     // contiguous segments
  const int32_t* seg_cap;
  int32_t* comp_len;
  int32_t* pos;
  const float* k_amax;
  const float* v_amax;
  const uint16_t* q;
  void* out;
  float* lse;
  int32_t* err;
  uint32_t* part_o;    // [slots][G][D] partial o, each word stored as ~bits
  uint32_t* part_ml;   // [slots][G][2] partial (m, l), likewise
  int32_t* sem;        // [nh] (stride kCounterStride): units of the segment finished so
                       // far (0 between calls)
  // decode step only
  int32_t* seqcnt;     // [B] (stride kCounterStride): segments of the sequence done
  uint8_t* ring_keep;
  const uint16_t* k_new;   // BF16 (b, h, d) at b * new_sb + h * new_sh + d
  const uint16_t* v_new;
  int64_t new_sb, new_sh;
  const uint8_t* keep_new; // [nh]
  int Hkv, G, Hq, W, nh, tpu, out_f32;
  float sm_scale;
  // paged store only
  const int32_t* page_table;   // [nh][max_pages]
  int max_pages, n_pages;
};

// Host plan: unit w of the launch is the unit of workgroup w.
//   u[2w]      pool tile of the unit's first tile (0 for a unit without tiles;
//              bits 0-25) | the first wave of the unit whose tile is read
//              only after the metadata, at most 63 (26-31)
//   u[2w + 1]  segment (bits 0-15) | index of the unit in its segment (16-20)
//              | units of the segment - 1 (21-25) | tiles of the unit (26-31)
struct HostPlan {
  uint32_t u[2 * kMaxPlanUnits];
};
struct NoPlan {
  int unused;
};
template <bool HP>
using PlanArg = typename std::conditional<HP, HostPlan, NoPlan>::type;

__device__ __forceinline__ int units_of(int n, int tpu) {
  const int tiles = (n + kTile - 1) / kTile;
  return max(1, (tiles + tpu - 1) / tpu);
}

// Final output of 4 consecutive d of query row gg of segment (b, h).
__device__ __forceinline__ void write_final4(const AttnParams& p, int b, int h, int gg, int d4,
                                             int D, float M, float L, f32x4 O, float sv) {
  const int64_t row = (int64_t)b * p.Hq + h * p.G + gg;
  const f32x4 v = L > 0.0f ? O * (sv / L) : f32x4{0, 0, 0, 0};
  if (p.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + row * D + 4 * d4) = v;
  } else {
    const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * D + 4 * d4) = u32x2{lo, hi};
  }
  if (d4 == 0 && p.lse) p.lse[row] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Partial words: the bitwise NOT of the f32 bit pattern, so that zero means
// "not written" (the one pattern that would store as zero, 0xFFFFFFFF, is a
// NaN and is stored as the NaN 0x7FFFFFFF instead).
__device__ __forceinline__ uint32_t enc_word(float x) {
  const uint32_t u = __float_as_uint(x);
  return ~(u == 0xFFFFFFFFu ? 0x7FFFFFFFu : u);
}
__device__ __forceinline__ float dec_word(uint32_t w) { return __uint_as_float(~w); }
__device__ __forceinline__ uint64_t enc2(float x, float y) {
  return (uint64_t)enc_word(x) | ((uint64_t)enc_word(y) << 32);
}
__device__ __forceinline__ bool written2(uint64_t w) {
  return (uint32_t)w != 0u && (uint32_t)(w >> 32) != 0u;
}
// Device-coherent 8-byte (and 1-byte) store and 8-byte load (relaxed, agent
// scope).
__device__ __forceinline__ void st_dev64(uint32_t* a, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev8(uint8_t* a, uint8_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(uint32_t* a) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-uniform copies of lane `src`'s value.
__device__ __forceinline__ int lane_i(int x, int src) { return __builtin_amdgcn_readlane(x, src); }
__device__ __forceinline__ float lane_f(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}
__device__ __forceinline__ long long lane_l(long long x, int src) {
  const int lo = __builtin_amdgcn_readlane((int)(x & 0xFFFFFFFF), src);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), src);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Workgroup barrier that orders LDS accesses only (no wait for outstanding
// global memory operations).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rows of a segment in a decode step, from its state before the append
// (P = pos >= 0, 0 <= cl <= cap, kn = keep byte of the new token != 0).
struct StepRows {
  int n_pre;     // rows holding data before the append
  int new_row;   // segment row that receives the new token (< W + cap), -1 if dropped
};
// ring_slot = P mod W (W > 0).
__device__ __forceinline__ StepRows step_rows(int W, int P, int ring_slot, int cl, int cap, int kn) {
  StepRows s;
  s.n_pre = min(W, P) + cl;
  s.new_row = W > 0 ? ring_slot : ((kn && cl < cap) ? cl : -1);
  return s;
}

// The unit a workgroup works on: its segment and that segment's metadata.
struct Unit {
  int i, first, U, n;      // first: index of the segment's first unit; n: rows planned
  long long sb;
  float ka, va;            // absmax of K and V (FP8, FP4)
  int P, cl, cap, kn;      // state before the append (P, cl also for attention)
};

// Device plan: unit k of the launch -- the segments in index order, each
// with units_of(rows) units (rows = n_i, or W + seg_cap with APP).
// Wave-level: every wave of a workgroup calls it with the same arguments
// and gets the same answer.
// Paged store (PG): no seg_base; P keeps its sign (an idle sequence, pos <
// 0, plans no rows in a decode step).
template <bool Q, bool APP, bool PG>
__device__ __forceinline__ bool find_unit(const AttnParams& p, int k, int lane, Unit& un) {
  int carry = 0;
  bool found = false;
  for (int base = 0; base < p.nh; base += 64) {
    const int hi = base + lane;
    int Ui = 0, ni = 0, Pi = 0, cli = 0, capi = 0, kni = 0;
    long long sbi = 0;
    float ka = 0.0f, va = 0.0f;
    if (hi < p.nh) {
      Pi = PG ? p.pos[hi / p.Hkv] : max(p.pos[hi / p.Hkv], 0);
      capi = max(p.seg_cap[hi], 0);
      cli = min(max(p.comp_len[hi], 0), capi);
      if (!PG) sbi = p.seg_base[hi];
      if (Q) {
        ka = p.k_amax[hi];
        va = p.v_amax[hi];
      }
      if (APP) kni = p.keep_new[hi] != 0;
      ni = APP ? ((PG && Pi < 0) ? 0 : p.W + capi) : min(p.W, max(Pi, 0)) + cli;
      Ui = units_of(ni, p.tpu);
    }
    int x = Ui;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const int ex = carry + x - Ui;
    const unsigned long long mine = __ballot(!found && hi < p.nh && k >= ex && k < ex + Ui);
    if (mine) {
      const int src = __ffsll((long long)mine) - 1;
      un.i = base + src;
      un.first = lane_i(ex, src);
      // units past the grid do not exist: a store whose segments need more
      // units than its pool allows (inconsistent pool_rows or seg_cap) has
      // its last segment cut short here, and the kernel flags it
      un.U = min(lane_i(Ui, src), (int)gridDim.x - un.first);
      un.n = lane_i(ni, src);
      un.sb = lane_l(sbi, src);
      un.ka = lane_f(ka, src);
      un.va = lane_f(va, src);
      un.P = lane_i(Pi, src);
      un.cl = lane_i(cli, src);
      un.cap = lane_i(capi, src);
      un.kn = lane_i(kni, src);
      found = true;
    }
    carry += lane_i(x, 63);
  }
  return found;
}

// Decode step: the metadata of segment i after the append, from its state
// before it (the unit's P, cl, cap, kn and the keep bit rk of the ring row
// the new token takes), with the error bits the append raises -- the rules
// of the APPEND operation of kv_compact.  Written by the last unit of the
// segment.
// Paged store (PG): rows are checked against their pages where they are
// written, not here.
template <bool PG>
__device__ __forceinline__ void commit_segment(const AttnParams& p, int i, const Unit& un, int rk) {
  const int W = p.W;
  const int64_t sb = un.sb;
  int cl_new = un.cl, errbits = 0;
  if (W > 0) {
    const int slot = un.P % W;
    if (un.P >= W && rk) {
      if (un.cl < un.cap) {
        if (!PG && (sb + slot >= p.pool_rows || sb + W + un.cl >= p.pool_rows))
          errbits |= CDA_DEVERR_POOL;
        cl_new = un.cl + 1;
      } else {
        errbits |= CDA_DEVERR_CAPACITY;
      }
    }
    if (!PG && sb + slot >= p.pool_rows) errbits |= CDA_DEVERR_POOL;
    p.ring_keep[(int64_t)i * W + slot] = (uint8_t)un.kn;
  } else if (un.kn) {
    if (un.cl < un.cap) {
      if (!PG && sb + un.cl >= p.pool_rows) errbits |= CDA_DEVERR_POOL;
      cl_new = un.cl + 1;
    } else {
      errbits |= CDA_DEVERR_CAPACITY;
    }
  }
  p.comp_len[i] = cl_new;
  if (errbits) atomicOr(p.err, errbits);
}


// Paged store: page of tile t of segment i (the index is clamped into the
// segment's page-table row, so the load never leaves the table; -1 past it).
__device__ __forceinline__ int page_of(const AttnParams& p, int i, int t) {
  const int pg = p.page_table[(int64_t)i * p.max_pages + min(max(t, 0), p.max_pages - 1)];
  return t < p.max_pages ? pg : -1;
}
__device__ __forceinline__ bool page_ok(const AttnParams& p, int pg) {
  return (unsigned)pg < (unsigned)p.n_pages;
}

// PG: the paged store (tiles through the page table; idle sequences).
// HP: the host plan (contiguous segments only).
template <int KV, int D, int NW, bool APP, bool PG, bool HP>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnParams p, PlanArg<HP> plan) {
  constexpr bool FP8 = KV == kKvFP8, FP4 = KV == kKvFP4, Q = KV != kKvBF16;
  constexpr int NTH = 64 * NW;              // threads of the workgroup
  constexpr int E = FP8 ? 1 : 2;            // bytes per element (FP8, BF16)
  constexpr int RB = kv_row_bytes(KV, D);   // bytes per row
  constexpr int NK = D / 32;                // MFMA k-steps of q.K
  constexpr int NT = D / 16;                // 16-wide d tiles of the output
  constexpr int KL = RB / 64;               // 16-byte K loads per (lane, token group)
  constexpr int VL = FP8 ? 1 : 2;           // 16-byte V loads per (lane, d tile); FP4: one 8-byte
  constexpr int EPL = D / 64;               // new-token elements per lane
  static_assert(!FP4 || D == 128, "the 4-bit store needs 64-byte K rows");
  static_assert(!(HP && PG), "a host plan describes contiguous segments");

  __shared__ int s_last;
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ f32x4 s_o[NW][16][D / 4];
  __shared__ f32x4 s_new[APP ? D / 2 : 1];  // decoded new token: K values, then V values
  __shared__ float s_zn[APP ? 16 : 1];        // its logit per query row (log2 units)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15, kg = lane >> 4;
  const int w = blockIdx.x;

  // ---- the unit: its segment, its tiles [t_begin, t_end) and its place
  // among the units of the segment
  Unit un;
  int t_begin, t_end;
  int64_t pre_row = 0;   // host plan: pool row of this wave's first tile
  int64_t sb_dev = 0;    // host plan: seg_base[i] as the device holds it
  int raw_pos = 0, raw_cl = 0, raw_cap = 0, raw_kn = 0;
  bool deferred = false;  // host plan: this wave's first tile is read after the metadata
  if constexpr (HP) {
    const uint32_t tile0 = plan.u[2 * w] & 0x3FFFFFFu, inf = plan.u[2 * w + 1];
    const int wdef = (int)(plan.u[2 * w] >> 26);
    const int ui = (int)((inf >> 16) & 31u), nt = (int)(inf >> 26);
    un.i = (int)(inf & 0xFFFFu);
    un.U = (int)((inf >> 21) & 31u) + 1;
    un.first = w - ui;
    t_begin = ui * p.tpu;
    t_end = t_begin + nt;
    un.sb = ((int64_t)tile0 - t_begin) * kTile;
    // a wave with no tile of its own reads the unit's first again (unused);
    // a unit without tiles reads pool tile 0 (unused)
    // a tile expected empty waits for the metadata: its wave reads the
    // unit's first tile now instead (unused)
    deferred = wave >= wdef;
    pre_row = nt > 0 ? ((int64_t)tile0 + (deferred ? 0 : min(wave, nt - 1))) * kTile : 0;
    // the segment's metadata: loaded now, consumed after the first tile's
    // loads have gone out
    const int bb = un.i / p.Hkv;
    raw_pos = p.pos[bb];
    raw_cl = p.comp_len[un.i];
    raw_cap = p.seg_cap[un.i];
    sb_dev = p.seg_base[un.i];
    if (Q) {
      un.ka = p.k_amax[un.i];
      un.va = p.v_amax[un.i];
    }
    if (APP) raw_kn = p.keep_new[un.i];
  } else {
    if (!find_unit<Q, APP, PG>(p, w, lane, un)) return;
    if (w == un.first && tid == 0 && un.U < units_of(un.n, p.tpu))
      atomicOr(p.err, CDA_DEVERR_POOL);
    // every load of the plan has been used: say so, so that no later write to
    // a register it used waits for the loads issued after this point
    __builtin_amdgcn_s_waitcnt(0);
    t_begin = (w - un.first) * p.tpu;
    t_end = min(t_begin + p.tpu, (un.n + kTile - 1) / kTile);
  }
  const int i = un.i, U = un.U;
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  const int G = p.G;
  const int uidx = w - un.first;   // this unit's place among its segment's units

  // ---- Q^T operand: lane (g, kg) holds 8 d-values of query row g per
  // k-step.  Columns g >= G repeat row 0: their results land in rows of the
  // product nobody reads, and the loads stay free of any condition (nothing
  // waits for them before the first MFMA).
  bf16x8 qop[NK];
  {
    const uint16_t* qrow = p.q + (int64_t)(b * p.Hq + h * G + (g < G ? g : 0)) * D;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      qop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + q_d0<KV>(s, kg)));
    }
  }

  // ---- one tile's loads: K rows for the 4 token groups (each instruction
  // 1 KB of the permuted K tile), V columns for the NT d tiles
  u32x4 kr[4][KL];
  u32x4 vr[NT][VL];
  u32x2 vq[FP4 ? NT : 1];   // FP4: tokens 16 kg .. 16 kg + 15 of column 16 nt + g
  auto load_tile = [&](int64_t trow) {
    const uint8_t* ktile = p.k_pool + trow * (int64_t)RB;
    const uint8_t* vtile = p.v_pool + trow * (int64_t)RB;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < KL; ++j)
        kr[m][j] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(ktile + ((m * KL + j) << 10) + lane * 16));
    if (FP4) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        vq[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
            vtile + v_nib_off(16 * kg, 16 * nt + g, D)));
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < VL; ++j)
          vr[nt][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              vtile + v_tile_off(16 * kg + 8 * j, 16 * nt + g, D, E)));
    }
  };
  if (HP) load_tile(pre_row);

  // host plan: the metadata, now that the first tile is in flight; a plan
  // that does not match the device's seg_base reads nothing and flags it
  bool plan_ok = true;
  if (HP) {
    __asm__ volatile("" : "+v"(raw_pos), "+v"(raw_cl), "+v"(raw_cap), "+v"(raw_kn));
    plan_ok = sb_dev == un.sb;
    un.P = max(raw_pos, 0);
    un.cap = max(raw_cap, 0);
    un.cl = min(max(raw_cl, 0), un.cap);
    un.kn = raw_kn != 0;
    un.n = plan_ok ? (APP ? p.W + un.cap : min(p.W, un.P) + un.cl) : 0;
    if (!plan_ok && tid == 0) atomicOr(p.err, CDA_DEVERR_PLAN);
  }
  const int64_t sb = un.sb;
  // rows of the segment inside the pool, in whole tiles (paged: every page is
  // checked); tiles past them are not read, and flagged (CDA_DEVERR_POOL)
  const int64_t in_pool =
      PG ? INT64_MAX
         : (plan_ok && sb >= 0 && (sb & (kTile - 1)) == 0 ? max(p.pool_rows - sb, (int64_t)0) : 0);
  const float ks = kv_scale<KV>(un.ka);
  const float vs = kv_scale<KV>(un.va);
  // paged store: the page of this wave's first tile, loaded before anything
  // else so that one round trip covers it
  int pg_next = PG ? page_of(p, i, t_begin + wave) : 0;
  const bool idle = PG && APP && un.P < 0;   // paged: a sequence not in use
  const int P = (PG ? max(un.P, 0) : un.P);   // contiguous: already >= 0

  // ---- rows with data (decode step: before the append), the new token's
  // row and its tile
  int n = HP ? (plan_ok ? min(p.W, P) + un.cl : 0) : un.n, new_row = -1, t_own = -1;
  const int ring_slot = (APP && p.W > 0) ? P % p.W : 0;   // ring row of P
  if (APP) {
    const StepRows st = step_rows(p.W, P, ring_slot, un.cl, un.cap, un.kn);
    n = (idle || !plan_ok) ? 0 : st.n_pre;
    if (!idle && plan_ok && st.new_row >= 0 && st.new_row < in_pool) {
      new_row = st.new_row;
      t_own = new_row / kTile;
    }
  }
  // the unit that holds the new token's tile adds it to the segment, and
  // the wave that reads that tile (the row wave) forms the new token and
  // writes the segment's new and moved rows once the tile is consumed
  const bool owner_unit = APP && t_own >= t_begin && t_own < t_end;
  const bool row_wave = owner_unit && wave == (t_own - t_begin) % NW;
  // decode step: where the keep bit of the token leaving the ring (ring
  // row P mod W) is; W = 0: a valid dummy address.  It is read where it is
  // needed, and tested only after the loads that must not wait for it.
  const bool leaving = APP && !idle && p.W > 0 && P >= p.W;
  // paged store, wave 0 of the owner unit: pages of the new token's row and
  // of the compact row the leaving token may move to (same round trip as
  // the tile's page)
  int pg_own = -1, pg_dst = -1;
  if (PG && row_wave) {
    pg_own = page_of(p, i, t_own);
    pg_dst = page_of(p, i, (p.W + un.cl) / kTile);
  }
  const uint8_t* rkp = APP ? (p.W > 0 ? p.ring_keep + (int64_t)i * p.W + ring_slot : p.keep_new + i)
                           : nullptr;
  // decode step: the keep bit for the segment's metadata, loaded now and
  // used at the end (commit)
  const int rkc = APP ? *rkp : 0;
  const float c1 = p.sm_scale * kLog2e * ks;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

  // row wave: its slice of the new token (issued after the accumulators are
  // set up, so that nothing before the tile loads waits for it).  It also
  // reads the ring row the new token replaces (the leaving token's row:
  // 16-byte K chunk `lane`, V elements EPL*lane..), in case it moves to the
  // compact tail.
  uint32_t nk = 0, nv = 0;
  uint32_t ox[EPL];   // kept apart: combining them would wait for the loads here
#pragma unroll
  for (int e = 0; e < EPL; ++e) ox[e] = 0;
  u32x4 okx = u32x4{0, 0, 0, 0};
  if (row_wave) {
    const int64_t off = (int64_t)b * p.new_sb + (int64_t)h * p.new_sh + EPL * lane;
    if (EPL == 2) {
      nk = *reinterpret_cast<const uint32_t*>(p.k_new + off);
      nv = *reinterpret_cast<const uint32_t*>(p.v_new + off);
    } else {
      nk = p.k_new[off];
      nv = p.v_new[off];
    }
    const int rs = new_row & (kTile - 1);
    // paged: a missing page reads tile 0 (unused: nothing is written then)
    const int64_t trow = PG ? (page_ok(p, pg_own) ? (int64_t)pg_own * kTile : 0)
                            : sb + (new_row - rs);
    const uint8_t* kt = p.k_pool + trow * (int64_t)RB;
    const uint8_t* vt = p.v_pool + trow * (int64_t)RB;
    okx = *reinterpret_cast<const u32x4*>(kt + k_chunk_offset(rs, min(lane, RB / 16 - 1), RB));
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      ox[e] = FP4 ? ((uint32_t)vt[v_nib_off(rs, EPL * lane + e, D)] >> (4 * (rs & 1))) & 15u
            : FP8 ? (uint32_t)vt[v_tile_off(rs, EPL * lane + e, D, 1)]
                  : (uint32_t)*reinterpret_cast<const uint16_t*>(
                        vt + v_tile_off(rs, EPL * lane + e, D, 2));
  }

  bool first_tile = true;
  // decode step, the row wave: forms the new token from its BF16 input with
  // the frozen scales -- its values and one logit per query row (from the q
  // operand) into LDS, for the combine -- and returns its stored bytes.  It
  // runs during the new token's tile, while that tile's V is in flight.
  auto new_token = [&](uint32_t& kc, uint32_t& vc) {
    __asm__ volatile("" : "+v"(nk), "+v"(nv));   // keeps this work below the tile loads
    const int d0n = EPL * lane;
    float ka = un.ka, va = un.va;
    __asm__ volatile("" : "+v"(ka), "+v"(va));   // the divisions stay here too
    const float kinv = kv_inv_scale<KV>(ka);
    const float vinv = kv_inv_scale<KV>(va);
    kc = 0;
    vc = 0;
    float* sn = reinterpret_cast<float*>(s_new);
    if (FP4) {   // the lane's two elements: one K byte, two V codes (low: d0n)
      kc = e2m1x2_from_f32(__fmul_rn(__uint_as_float(nk << 16), kinv),
                           __fmul_rn(__uint_as_float(nk & 0xFFFF0000u), kinv));
      vc = e2m1x2_from_f32(__fmul_rn(__uint_as_float(nv << 16), vinv),
                           __fmul_rn(__uint_as_float(nv & 0xFFFF0000u), vinv));
      const auto kf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(kc, 1.0f, 0);
      const auto vf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc, 1.0f, 0);
      sn[d0n] = kf[0];
      sn[d0n + 1] = kf[1];
      sn[D + d0n] = vf[0];
      sn[D + d0n + 1] = vf[1];
    }
#pragma unroll
    for (int e = 0; e < (FP4 ? 0 : EPL); ++e) {
      const uint32_t kb = (nk >> (16 * e)) & 0xFFFFu, vb = (nv >> (16 * e)) & 0xFFFFu;
      if (FP8) {
        const uint32_t kq = e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(kb), kinv));
        const uint32_t vq = e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(vb), vinv));
        sn[d0n + e] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(kq, 1.0f, false)[0];
        sn[D + d0n + e] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vq, 1.0f, false)[0];
        kc |= kq << (8 * e);
        vc |= vq << (8 * e);
      } else {
        sn[d0n + e] = bf16_bits_to_f32(kb);
        sn[D + d0n + e] = bf16_bits_to_f32(vb);
        kc |= kb << (16 * e);
        vc |= vb << (16 * e);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float dot = 0.0f;   // lane (g, kg): its quarter of q[g] . k^
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int d0 = q_d0<KV>(s, kg);
      const f32x4 a = s_new[d0 / 4], c = s_new[d0 / 4 + 1];
      // an opaque copy: converted here, not hoisted above the tile loads
      // (where converting it would wait for the q loads)
      bf16x8 qs = qop[s];
      __asm__ volatile("" : "+v"(qs));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = fmaf((float)qs[e], a[e], dot);
        dot = fmaf((float)qs[4 + e], c[e], dot);
      }
    }
    dot = sum_xor32(sum_xor16(dot));
    if (kg == 0) s_zn[g] = dot * c1;
  };
  uint32_t kc = 0, vc = 0;   // row wave: the new row's stored bytes
  bool nt_done = false;

  // decode step, the row wave once the new token's tile is consumed:
  // copies the leaving token's row to the compact tail if it moves
  // (wants_move: it is kept and the compact region has room) and writes the
  // new row over its ring row.  No other workgroup reads the new token's
  // tile, and the compact tail lies past the rows attended in this launch.
  // The moved K chunks, 4-byte K slices and FP8 V bytes go out through
  // agent-scope stores, which write through the L2: the end of the launch
  // then has none of their lines left to write back (measured faster).
  auto write_rows = [&](bool wants_move) {
    const int d0n = EPL * lane;
    // the leaving token's row (ring row P mod W) moves to compact row
    // W + cl if it is kept; read back from the pool (this wave's reads
    // finish before the new row is written over it)
    const int rs = new_row & (kTile - 1);
    // paged: rows whose page is missing are not written (CDA_DEVERR_POOL)
    const bool own_ok = !PG || page_ok(p, pg_own);
    const bool dst_ok = !PG || page_ok(p, pg_dst);
    const int64_t trow = PG ? (int64_t)pg_own * kTile : sb + (new_row - rs);
    uint8_t* kt = p.k_pool + trow * (int64_t)RB;
    uint8_t* vt = p.v_pool + trow * (int64_t)RB;
    const bool moved = wants_move && own_ok && dst_ok &&
                       (PG || sb + p.W + un.cl < p.pool_rows);
    if (PG && lane == 0 && ((wants_move && !moved) || !own_ok)) atomicOr(p.err, CDA_DEVERR_POOL);
    if (moved) {   // from the copy read at the start of the unit
      const int to = p.W + un.cl, rt = to & (kTile - 1);
      const int64_t drow = PG ? (int64_t)pg_dst * kTile : sb + (to - rt);
      uint8_t* kd = p.k_pool + drow * (int64_t)RB;
      uint8_t* vd = p.v_pool + drow * (int64_t)RB;
      constexpr int KC = RB / 16;   // 16-byte chunks per K row
      if (lane < KC) {
        uint32_t* kq = reinterpret_cast<uint32_t*>(kd + k_chunk_offset(rt, lane, RB));
        st_dev64(kq, (uint64_t)okx[0] | ((uint64_t)okx[1] << 32));
        st_dev64(kq + 2, (uint64_t)okx[2] | ((uint64_t)okx[3] << 32));
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (FP4)
          nib_store(vd + v_nib_off(rt, d0n + e, D), rt & 1, ox[e]);
        else if (FP8)
          st_dev8(vd + v_tile_off(rt, d0n + e, D, 1), (uint8_t)ox[e]);
        else
          *reinterpret_cast<uint16_t*>(vd + v_tile_off(rt, d0n + e, D, 2)) = (uint16_t)ox[e];
      }
    }
    // the new row goes over the ring row: this wave has consumed the tile's
    // old bytes, and the copy above used the ones read at the start of the
    // unit (unused, and harmless, if it did not move).  Byte of this lane's
    // first element in the row, and the lane's bytes:
    constexpr int LB = FP4 ? EPL / 2 : EPL * E;
    const int kb0 = FP4 ? d0n / 2 : d0n * E;
    if (own_ok) {
      uint8_t* kdst = kt + k_chunk_offset(rs, kb0 >> 4, RB) + (kb0 & 15);
      if (LB == 4)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(kdst), kc, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else if (LB == 2)
        *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)kc;
      else
        *kdst = (uint8_t)kc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (FP4)   // after the moved row's write, which may share the byte
          nib_store(vt + v_nib_off(rs, d0n + e, D), rs & 1, (vc >> (4 * e)) & 15u);
        else if (FP8)
          st_dev8(vt + v_tile_off(rs, d0n + e, D, 1), (uint8_t)(vc >> (8 * e)));
        else
          *reinterpret_cast<uint16_t*>(vt + v_tile_off(rs, d0n + e, D, 2)) =
              (uint16_t)(vc >> (16 * e));
      }
    }
  };

  // ---- one tile: S = K Q^T, online softmax, O += V^T P^T.  valid: rows of
  // the tile holding data (<= 0: all masked); own: the tile of the new
  // token's row; rko: keep bit of the token leaving the ring.
  auto tile_body = [&](int valid, bool own, int rko) {
    const bool full = valid == kTile;
    // -- S^T = K . Q^T, 16 tokens per MFMA row block
    f32x4 s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[m] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < NK; ++st) {
        bf16x8 a;
        if (FP4) {
          a = fp4x8_to_bf16x8(kr[m][0][st]);
        } else if (FP8) {
          const u32x4 v = kr[m][st >> 1];
          a = (st & 1) ? fp8x8_to_bf16x8(v[2], v[3]) : fp8x8_to_bf16x8(v[0], v[1]);
        } else {
          a = as_bf16x8(kr[m][st]);
        }
        s[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[st], s[m], 0, 0, 0);
      }
    }

    if (own) {   // while V is still in flight
      new_token(kc, vc);
      nt_done = true;
    }

    // -- decode step: the leaving token's row is masked unless it moves
    //    to the compact tail; tested after QK, so that nothing before the
    //    tile loads waits for the keep bit
    __asm__ volatile("" : "+v"(rko));   // keeps the test from moving up
    const bool moved_t = own && leaving && rko != 0 && un.cl < un.cap &&
                         (PG || sb + p.W + un.cl < p.pool_rows);
    const int mrow = (own && leaving && !moved_t) ? (new_row & (kTile - 1)) : -1;

    // -- online softmax over this tile; lane (g, kg) owns tokens 16kg + 4m + r
    float z[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) z[m][r] = s[m][r] * c1;
    if (!full || mrow >= 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * kg + 4 * m + r;
          if (tok >= valid || tok == mrow) z[m][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, z[m][r]);
    tmax = max_xor32(max_xor16(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // every logit masked so far
    if (!first_tile) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
    }
    float psum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[m][r] = __builtin_amdgcn_exp2f(z[m][r] - m_use);
        psum += z[m][r];
      }
    l_run += psum;
    m_run = m_new;

    // -- rows past the segment end: zero their V bytes (P is 0 there, but
    //    the bytes may not be finite values; every FP4 code is finite)
    if (!FP4 && !full) {
#pragma unroll
      for (int j = 0; j < VL; ++j) {
        const int lim = min(max(valid - 16 * kg - 8 * j, 0), 16 / VL) * E;  // valid bytes
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t msk = bytes_below(lim, q);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) vr[nt][j][q] &= msk;
        }
      }
    }

    // -- O^T += V^T . P^T, per d tile one MFMA (FP8, FP4) or two (BF16:
    //    hi, lo) per 8 tokens of each lane
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (Q) {
        f16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (_Float16)z[2 * hh + (e >> 2)][e & 3];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f16x8 a;
          if (FP4) {
            a = fp4x8_to_f16x8(vq[nt][hh]);
          } else {
            const u32x4 v = vr[nt][0];
            a = hh ? fp8x8_to_f16x8(v[2], v[3]) : fp8x8_to_f16x8(v[0], v[1]);
          }
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf, acc[nt], 0, 0, 0);
        }
      } else {
        bf16x8 phi, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = z[2 * hh + (e >> 2)][e & 3];
          const __bf16 hi = (__bf16)pv;
          phi[e] = hi;
          plo[e] = (__bf16)(pv - (float)hi);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 a = as_bf16x8(vr[nt][hh]);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, acc[nt], 0, 0, 0);
        }
      }
    }
    // the tile's data is all consumed: the row wave writes the rows now,
    // while the other waves still stream
    if (own) write_rows(own && leaving && rko != 0 && un.cl < un.cap);
    first_tile = false;
  };

  int t = t_begin + wave;
  if (HP && !deferred) {
    // the tile whose loads went out first
    int rko = 0;
    if (APP) rko = *rkp;   // issued after that tile's loads
    const int want = min(kTile, n - t * kTile);
    const int valid = (int)min((int64_t)want, in_pool - (int64_t)t * kTile);
    if (t < t_end && want > 0 && valid < want && lane == 0) atomicOr(p.err, CDA_DEVERR_POOL);
    if (t < t_end && valid > 0) tile_body(valid, APP && t == t_own, rko);
    t += NW;
  }
  for (; t < t_end; t += NW) {
    const int r0 = t * kTile;
    const int want = min(kTile, n - r0);
    const int valid = (int)min((int64_t)want, in_pool - r0);
    if (want > 0 && valid < want && lane == 0) atomicOr(p.err, CDA_DEVERR_POOL);
    if (valid <= 0) break;
    int64_t trow = sb + r0;   // pool row of the tile
    if (PG) {
      const int pg = __builtin_amdgcn_readfirstlane(pg_next);
      if (!page_ok(p, pg)) {   // a tile with data and no page: inconsistent store
        if (lane == 0) atomicOr(p.err, CDA_DEVERR_POOL);
        break;
      }
      trow = (int64_t)pg * kTile;
    }
    // decode step: the leaving token's keep bit, issued ahead of the tile
    int rko = 0;
    if (APP) rko = *rkp;
    load_tile(trow);
    // paged: the page of this wave's next tile, in flight with this one
    if (PG) pg_next = page_of(p, i, t + NW);
    tile_body(valid, APP && t == t_own, rko);
  }

  // the new token's tile held no data (nothing of it was attended, so no
  // token leaves the ring here and nothing moves)
  if (row_wave && !nt_done) {
    new_token(kc, vc);
    write_rows(false);
  }

  // ---- combine the waves of the workgroup
  l_run = sum_xor32(sum_xor16(l_run));
  if (kg == 0) {
    s_m[wave][g] = m_run;
    s_l[wave][g] = l_run;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)   // columns g >= G hold no query row
    if (g < G) s_o[wave][g][(16 * nt + 4 * kg) / 4] = acc[nt];
  lds_barrier();

  // decode step, single-unit segment: every wave of the workgroup has read
  // the segment's metadata (the owner's keep bit included)
  int seq_prev = -1;
  if (APP && !idle && U == 1 && tid == 0) {
    if (plan_ok) commit_segment<PG>(p, i, un, leaving && rkc != 0);
    seq_prev = __hip_atomic_fetch_add(p.seqcnt + (int64_t)b * kCounterStride, 1,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // (m, l, o) of the workgroup for query row gg and d = 4 d4 .. 4 d4 + 3:
  // the waves' states, and the new token's (logit, value) pair in the unit
  // that holds it
  auto combine = [&](int gg, int d4, float& M, float& L, f32x4& O) {
    // every LDS read first, then the arithmetic (a wave without rows has
    // m = -inf and weight exp2(-inf) = 0)
    float mw[NW], lw[NW];
    f32x4 ow[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      mw[ww] = s_m[ww][gg];
      lw[ww] = s_l[ww][gg];
      ow[ww] = s_o[ww][gg][d4];
    }
    M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mw[ww]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    O = f32x4{0, 0, 0, 0};
    L = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = __builtin_amdgcn_exp2f(mw[ww] - Mu);
      O += f * ow[ww];
      L += f * lw[ww];
    }
    if (owner_unit) {   // decode step: the new token's (logit, value) pair
      const float zn = s_zn[gg];
      const float M2 = fmaxf(M, zn);
      const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - M2);
      const float pn = __builtin_amdgcn_exp2f(zn - M2);
      O = O * a + pn * s_new[D / 4 + d4];
      L = L * a + pn;
      M = M2;
    }
  };

  const float sv = vs;
  if (U == 1) {
    for (int e = tid; e < G * (D / 4); e += NTH) {   // (query row, 4 consecutive d)
      const int gg = e / (D / 4), d4 = e - gg * (D / 4);
      float M, L;
      f32x4 O;
      combine(gg, d4, M, L, O);
      write_final4(p, b, h, gg, d4, D, M, L, O, sv);
    }
  } else {
    // ---- split segment: store this unit's partial (not waited for) and
    // count the unit in; the last unit of the segment merges.  The partial
    // is stored by the first threads; the counter, the commit and the merge
    // are done by the second half of the workgroup when the items fit in
    // half of it: a wave's wait for a load or an atomic also waits for the
    // stores it has issued before, and these waves have issued none.
    const int items = G * (D / 4);
    const int moff = items <= NTH / 2 ? NTH / 2 : 0;   // first merging thread
    const int ctid = NTH - 64;                        // counting thread (last wave)
    for (int e = tid; e < items; e += NTH) {
      const int gg = e / (D / 4), d4 = e - gg * (D / 4);
      float M, L;
      f32x4 O;
      combine(gg, d4, M, L, O);
      const int64_t sr = (int64_t)(un.first + uidx) * G + gg;
      st_dev64(p.part_o + sr * D + 4 * d4, enc2(O[0], O[1]));
      st_dev64(p.part_o + sr * D + 4 * d4 + 2, enc2(O[2], O[3]));
      if (d4 == 0) st_dev64(p.part_ml + 2 * sr, enc2(M, L));
    }
    if (tid == ctid) {
      int32_t* cnt = p.sem + (int64_t)i * kCounterStride;
      const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == U - 1;
      if (prev == U - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lds_barrier();
    if (s_last) {
      // decode step: every unit of the segment has read its metadata
      if (APP && !idle && tid == ctid) {
        if (plan_ok) commit_segment<PG>(p, i, un, leaving && rkc != 0);
        seq_prev = __hip_atomic_fetch_add(p.seqcnt + (int64_t)b * kCounterStride, 1,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // each thread merges 4 consecutive outputs of one query row, folding
      // the units' partials in unit order (this unit's own too, as stored,
      // so that the result does not depend on which unit merges); the loads
      // of a batch of units go out together and are repeated until every
      // word has arrived (the whole wave together, so that no lane reads a
      // word another lane has already cleared)
      bool late = false;
      // batches of 2, 4, 6 or 8 units for segments of at most that many,
      // else of 16 (one round trip instead of two; fewer units do not pay
      // for the loads and the folds of a larger batch)
      auto merge = [&](auto mb) __attribute__((always_inline)) {
      constexpr int MB = decltype(mb)::value;
      for (int e = tid - moff; e >= 0 && e < items; e += NTH) {
        const int gg = e / (D / 4), d4 = e - gg * (D / 4);
        float M = -INFINITY, L = 0.0f;
        f32x4 O = f32x4{0, 0, 0, 0};
        for (int k0 = 0; k0 < U; k0 += MB) {
          uint64_t ml[MB], oa[MB], ob[MB];
          for (int polls = 0;; ++polls) {
#pragma unroll
            for (int j = 0; j < MB; ++j) {   // unconditional loads, clamped index
              const int64_t sr = (int64_t)(un.first + min(k0 + j, U - 1)) * G + gg;
              ml[j] = ld_dev64(p.part_ml + 2 * sr);
              oa[j] = ld_dev64(p.part_o + sr * D + 4 * d4);
              ob[j] = ld_dev64(p.part_o + sr * D + 4 * d4 + 2);
            }
            bool ok = true;
#pragma unroll
            for (int j = 0; j < MB; ++j)
              if (k0 + j < U) ok = ok && written2(ml[j]) && written2(oa[j]) && written2(ob[j]);
            if (__all(ok)) break;
            if (polls >= kMergePolls) {
              late = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          float mj[MB];
#pragma unroll
          for (int j = 0; j < MB; ++j)
            mj[j] = k0 + j < U ? dec_word((uint32_t)ml[j]) : -INFINITY;
          float Mb = M;
#pragma unroll
          for (int j = 0; j < MB; ++j) Mb = fmaxf(Mb, mj[j]);
          if (Mb == -INFINITY) continue;
          const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
          O *= a;
          L *= a;
#pragma unroll
          for (int j = 0; j < MB; ++j) {
            const float f = (mj[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mj[j] - Mb);
            const f32x4 oj = f32x4{dec_word((uint32_t)oa[j]), dec_word((uint32_t)(oa[j] >> 32)),
                                   dec_word((uint32_t)ob[j]), dec_word((uint32_t)(ob[j] >> 32))};
            O += f * oj;
            L += f * dec_word((uint32_t)(ml[j] >> 32));
          }
          M = Mb;
        }
        write_final4(p, b, h, gg, d4, D, M, L, O, sv);
        // the slots back to zero for the next call: every word was read
        // non-zero above, so its store has landed before these zeros
        for (int j = 0; j < U; ++j) {
          const int64_t sr = (int64_t)(un.first + j) * G + gg;
          st_dev64(p.part_o + sr * D + 4 * d4, 0);
          st_dev64(p.part_o + sr * D + 4 * d4 + 2, 0);
          if (d4 == 0) st_dev64(p.part_ml + 2 * sr, 0);
        }
      }
      };
      if (U <= 2) merge(std::integral_constant<int, 2>{});
      else if (U <= 4) merge(std::integral_constant<int, 4>{});
      else if (U <= 6) merge(std::integral_constant<int, 6>{});
      else if (U <= kMergeBatch) merge(std::integral_constant<int, kMergeBatch>{});
      else merge(std::integral_constant<int, 2 * kMergeBatch>{});
      if (late) atomicOr(p.err, CDA_DEVERR_MERGE);
    }
  }
  // decode step: the last segment of sequence b to be done writes pos[b]
  if (APP && seq_prev == p.Hkv - 1) {
    p.pos[b] = un.P + 1;
    __hip_atomic_store(p.seqcnt + (int64_t)b * kCounterStride, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <bool APP, bool PG, bool HP>
void launch_variant(int kv, int D, int nw, dim3 grid, hipStream_t s, const AttnParams& p,
                    const PlanArg<HP>& plan) {
#define CDA_LAUNCH_ATTN(F, DD)                                                          \
  (nw == 8 ? attn_kernel<F, DD, 8, APP, PG, HP><<<grid, 512, 0, s>>>(p, plan)           \
           : attn_kernel<F, DD, 4, APP, PG, HP><<<grid, 256, 0, s>>>(p, plan))
  if (kv == kKvFP4) {   // D = 128 only
    CDA_LAUNCH_ATTN(kKvFP4, 128);
  } else if (kv == kKvFP8) {
    if (D == 64) CDA_LAUNCH_ATTN(kKvFP8, 64); else CDA_LAUNCH_ATTN(kKvFP8, 128);
  } else {
    if (D == 64) CDA_LAUNCH_ATTN(kKvBF16, 64); else CDA_LAUNCH_ATTN(kKvBF16, 128);
  }
#undef CDA_LAUNCH_ATTN
}

// The host plan of a contiguous store from the host copy of seg_base (its
// consistency was checked by the caller): every segment's span of W +
// seg_cap rows rounded to tiles, cut into units of tpu tiles (at least one
// unit per segment).  False when it does not fit the encoding or the kernel
// arguments; the device plan is used then.
bool host_plan(const cda_kv_cache& c, int tpu, HostPlan& plan, int& n) {
  // tiles wholly past span - spare_rows + 64 rows of a segment are expected
  // empty and read after the metadata (none without the hint)
  const int64_t spare = c.spare_rows;
  const int64_t nh = (int64_t)c.B * c.Hkv;
  if (nh > 65536 || tpu > 63 || c.pool_rows < kTile || c.pool_rows / kTile > 0x3FFFFFFll)
    return false;
  const int64_t* sbh = c.seg_base_host;
  n = 0;
  for (int64_t i = 0; i < nh; ++i) {
    const int64_t tiles = (sbh[i + 1] - sbh[i]) / kTile;
    const int64_t U = std::max<int64_t>(1, (tiles + tpu - 1) / tpu);
    if (U > 32 || n + U > kMaxPlanUnits) return false;
    for (int64_t u = 0; u < U; ++u) {
      const int64_t nt = std::min<int64_t>(tpu, tiles - u * tpu);
      const int64_t span = sbh[i + 1] - sbh[i];
      const int64_t t_def = spare > kTile ? (span - spare + 2 * kTile - 1) / kTile : tiles;
      const int64_t wdef = std::min<int64_t>(63, std::max<int64_t>(0, t_def - u * tpu));
      plan.u[2 * n] = (uint32_t)(sbh[i] / kTile + u * tpu) | ((uint32_t)wdef << 26);
      plan.u[2 * n + 1] = (uint32_t)i | (uint32_t)(u << 16) | (uint32_t)((U - 1) << 21) |
                          (uint32_t)(nt << 26);
      ++n;
    }
  }
  return true;
}

}  // namespace

int64_t attn_max_units(const cda_kv_cache& c, int tpu) {
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return nh + c.pool_rows / ((int64_t)kTile * tpu);
}

// Workspace: [per-segment counters][per-sequence counters] (one 128-byte
// line each) [partial (m, l) words][partial o words], one partial slot per
// work unit.
size_t attn_workspace_bytes(const cda_kv_cache& c, int G, int tpu) {
  const int64_t slots = attn_max_units(c, tpu);
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return align256((size_t)nh * 4 * kCounterStride) + align256((size_t)c.B * 4 * kCounterStride) +
         align256((size_t)slots * G * 2 * 4) + align256((size_t)slots * G * c.D * 4);
}

hipError_t launch_attn(const cda_kv_cache& c, const void* q, int Hq, float sm_scale, void* out,
                       int out_f32, float* lse, int tpu, void* workspace, hipStream_t s,
                       const cda_compact_args* step) {
  const int nh = c.B * c.Hkv;
  if (nh == 0) return hipGetLastError();
  const int G = Hq / c.Hkv;
  const int64_t units = attn_max_units(c, tpu);
  AttnParams p;
  p.k_pool = static_cast<uint8_t*>(c.k_pool);
  p.v_pool = static_cast<uint8_t*>(c.v_pool);
  p.pool_rows = c.pool_rows;
  p.seg_base = c.seg_base;
  p.page_table = c.page_table;
  p.max_pages = c.max_pages;
  p.n_pages = (int)(c.pool_rows / kTile);
  p.seg_cap = c.seg_cap;
  p.comp_len = c.comp_len;
  p.pos = c.pos;
  p.k_amax = c.k_amax;
  p.v_amax = c.v_amax;
  p.q = static_cast<const uint16_t*>(q);
  p.out = out;
  p.lse = lse;
  p.err = c.err;
  char* ws = static_cast<char*>(workspace);
  p.sem = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)nh * 4 * kCounterStride);
  p.seqcnt = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)c.B * 4 * kCounterStride);
  p.part_ml = reinterpret_cast<uint32_t*>(ws);
  ws += align256((size_t)units * G * 2 * 4);
  p.part_o = reinterpret_cast<uint32_t*>(ws);
  p.ring_keep = c.ring_keep;
  p.k_new = step ? static_cast<const uint16_t*>(step->k) : nullptr;
  p.v_new = step ? static_cast<const uint16_t*>(step->v) : nullptr;
  p.new_sb = step ? step->stride_b : 0;
  p.new_sh = step ? step->stride_h : 0;
  p.keep_new = step ? step->keep : nullptr;
  p.Hkv = c.Hkv;
  p.G = G;
  p.Hq = Hq;
  p.W = c.W;
  p.nh = nh;
  p.tpu = tpu;
  p.out_f32 = out_f32;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c.D);
  const int kv = c.kv_dtype;
  const int nw = tpu >= 8 ? 8 : 4;   // waves per workgroup: one tile each per pass
  const bool pg = c.page_table != nullptr;
  if (!pg && c.seg_base_host) {
    HostPlan plan;
    int n = 0;
    if (host_plan(c, tpu, plan, n)) {
      const dim3 grid((unsigned)n);
      if (step) launch_variant<true, false, true>(kv, c.D, nw, grid, s, p, plan);
      else launch_variant<false, false, true>(kv, c.D, nw, grid, s, p, plan);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)units);
  const NoPlan none{0};
  if (step) {
    if (pg) launch_variant<true, true, false>(kv, c.D, nw, grid, s, p, none);
    else launch_variant<true, false, false>(kv, c.D, nw, grid, s, p, none);
  } else {
    if (pg) launch_variant<false, true, false>(kv, c.D, nw, grid, s, p, none);
    else launch_variant<false, false, false>(kv, c.D, nw, grid, s, p, none);
  }
  return hipGetLastError();
}

}  // namespace cda
