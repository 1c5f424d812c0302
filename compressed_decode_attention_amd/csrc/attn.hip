// Single-token GQA decode attention over the compact KV store, for gfx950,
// alone or fused with the decode-time append of the new token.
//
// What is computed (FastDMS page, release and benchmark paragraphs: decode
// over the compact store; PackKV abstract: decompression fused into the
// matrix-vector products): for every sequence b and query head j, softmax
// attention of q[b, j] over the n_i stored rows of its KV head's segment.
//
// Work split.  Each segment's rows [0, n_i) are cut into 64-row tiles, and
// tiles into work units of `tpu` tiles; one workgroup (4 or 8 waves) takes
// one unit at a time and each wave one tile at a time.  Every wave derives
// the unit -> (segment, tiles) map itself from pos / comp_len / seg_cap
// (lane l looks at one segment, a wave-wide scan of unit counts finds the
// segment holding the unit), so the host needs no copy of the lengths and
// no workgroup barrier delays the K/V loads.  A segment with one unit writes
// its output directly; otherwise each unit writes an unnormalised partial
// (m, l, o) and counts itself in with an atomic, and the last unit of the
// segment to finish combines all of them with a log-sum-exp merge and resets
// the counter (so the counters are zero between calls).
//
// XCD-local mode.  The dispatcher hands consecutive workgroups to the XCDs
// round robin: workgroup w runs on XCD (w + c) mod (number of XCDs), with a
// start c fixed for the dispatch (0 for a direct launch; graph replays have
// shown other values).  When that number divides 8, the workgroups
// w = 8k + r of one residue r share one XCD and so one L2, whatever c is.
// The units of segment i are given only to the workgroups of one residue,
// its group (seg_group[i] when COUNT has written the map, which evens out
// the rows per group, else i mod 8): partials are plain stores and the
// merge reads them from that L2.  An XCD keeps one 8-wave workgroup per CU
// resident (32 at a time), so a group with more units than that finishes
// its last ones a whole unit later; the balanced map keeps groups under it.
// Workgroup w walks units k = w/8, w/8 + P, ... of its group's segments.
// Each partial carries the XCD it was written on; the merging workgroup
// sets CDA_DEVERR_XCD if one differs from its own.  Otherwise (XCD count not
// a divisor of 8) every workgroup takes one unit of the global list and
// partials go through agent-scope (device-coherent) stores and loads.
//
// Inside a wave, the G query rows of the KV head (G <= 16) are the N = 16
// columns of two MFMA products per tile:
//   S^T[token][g] = K_tile[token][:] . Q^T[:][g]     v_mfma_f32_16x16x32_bf16
//   O^T[d][g]    += V^T[d][token] . P^T[token][g]    v_mfma_f32_16x16x32_{f16,bf16}
// K is stored in 64-row tiles permuted so that each 64-lane load of the S
// operand is 1 KB of consecutive bytes; V is stored in 64-row column-major
// tiles, so the O operand is 16-byte loads of 8 or 16 consecutive tokens of
// one column.  Tokens are assigned to MFMA rows so that the S accumulator of
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
//     tile of its row, after that unit's tiles are done; the workgroup's
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
#include "attn_common.h"
#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

constexpr int kMergeBatch = 4;   // partials loaded per round trip in the merge
constexpr int kXcdGroups = 8;    // segment groups of the XCD-local mode
constexpr int kCounterStride = 32;   // ints between counters: one 128-byte line each

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
  float* part_o;       // [slots][G][D]
  float* part_ml;      // [slots][G][4]: m, l, XCD of the writer, unused
  int32_t* sem;        // [nh] (stride kCounterStride): units of the segment finished so
                       // far (0 between calls)
  const uint8_t* seg_group;   // XCD-local mode: group of each segment, or NULL (i mod 8)
  // decode step only
  int32_t* seqcnt;     // [B] (stride kCounterStride): segments of the sequence done
  uint8_t* ring_keep;
  const uint16_t* k_new;   // BF16 (b, h, d) at b * new_sb + h * new_sh + d
  const uint16_t* v_new;
  int64_t new_sb, new_sh;
  const uint8_t* keep_new; // [nh]
  int Hkv, G, Hq, W, nh, tpu, out_f32;
  int per_xcd;         // XCD-local mode: workgroups per segment group
  float sm_scale;
  // paged store only (last, so that the other fields keep their offsets)
  const int32_t* page_table;   // [nh][max_pages]
  int max_pages, n_pages;
};

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

// Partials: XCD-local mode keeps them in the shared L2 of the XCD (plain
// 16-byte stores and loads); otherwise they are device-coherent
// (agent-scope stores and loads, one per dword).
template <bool XL>
__device__ __forceinline__ void store_part4(float* a, f32x4 v) {
  if (XL) {
    *reinterpret_cast<f32x4*>(a) = v;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) __hip_atomic_store(a + c, v[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <bool XL>
__device__ __forceinline__ float load_part1(const float* a) {
  return XL ? __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
            : __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool XL>
__device__ __forceinline__ f32x4 load_part4(const float* a) {
  // XCD-local: one 16-byte load (the merging CU has not read these lines
  // before in this kernel, so its L1 holds no stale copy)
  if (XL) return *reinterpret_cast<const f32x4*>(a);
  return f32x4{load_part1<XL>(a), load_part1<XL>(a + 1), load_part1<XL>(a + 2),
               load_part1<XL>(a + 3)};
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
  int i, first, U, n;      // n: rows planned
  long long sb;
  float ka, va;            // absmax of K and V (FP8, FP4)
  int P, cl, cap, kn;      // decode step: state before the append
};

// Unit k of group grp: its segments in index order, each with
// units_of(rows) units (rows = n_i, or W + seg_cap with APP).  With a group
// map the group's segments are those mapped to it; otherwise they are grp,
// grp + xs, grp + 2xs, ...  Wave-level: every wave of a workgroup calls it
// with the same arguments and gets the same answer.  It scans all of the
// group's segments and returns their unit count in `total`.
// Paged store (PG): no seg_base; P keeps its sign (an idle sequence, pos <
// 0, plans no rows in a decode step).
template <bool Q, bool APP, bool PG>
__device__ __forceinline__ bool find_unit(const AttnParams& p, int grp, int xs, int k, int lane,
                                          Unit& un, int& total) {
  const bool mapped = p.seg_group != nullptr;
  const int x0 = mapped ? 0 : grp, st = mapped ? 1 : xs;
  int carry = 0;
  bool found = false;
  for (int base = 0; x0 + st * base < p.nh; base += 64) {
    const int hi = x0 + st * (base + lane);
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
      // the map byte last, through a valid address either way, so that no
      // load of this round trip waits behind it or behind a branch
      const uint8_t gb = *(mapped ? p.seg_group + hi : reinterpret_cast<const uint8_t*>(p.seg_cap + hi));
      const bool in_group = !mapped || (gb & 7) == grp;
      ni = APP ? ((PG && Pi < 0) ? 0 : p.W + capi) : min(p.W, max(Pi, 0)) + cli;
      Ui = in_group ? units_of(ni, p.tpu) : 0;
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
      un.i = x0 + st * (base + src);
      un.first = lane_i(ex, src);
      un.U = lane_i(Ui, src);
      un.n = lane_i(ni, src);
      un.sb = lane_l(sbi, src);
      un.ka = lane_f(ka, src);
      un.va = lane_f(va, src);
      if (APP) {
        un.P = lane_i(Pi, src);
        un.cl = lane_i(cli, src);
        un.cap = lane_i(capi, src);
        un.kn = lane_i(kni, src);
      }
      found = true;
    }
    carry += lane_i(x, 63);
  }
  total = carry;
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
template <int KV, int D, bool XL, int NW, bool APP, bool PG>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnParams p) {
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

  __shared__ int s_last;
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ f32x4 s_o[NW][16][D / 4];
  __shared__ f32x4 s_new[APP ? D / 2 : 1];  // decoded new token: K values, then V values
  __shared__ float s_zn[APP ? 16 : 1];        // its logit per query row (log2 units)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15, kg = lane >> 4;
  const int w = blockIdx.x;
  const int grp = XL ? (w & (kXcdGroups - 1)) : 0;
  const int xcc = XL ? (__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) : 0;   // HW_REG_XCC_ID

  for (int k = XL ? (w / kXcdGroups) : w;; k += p.per_xcd) {
    Unit un;
    int total = 0;
    if (!find_unit<Q, APP, PG>(p, grp, XL ? kXcdGroups : 1, k, lane, un, total)) break;
    // every load of the plan has been used: say so, so that no later write to
    // a register it used waits for the loads issued after this point
    __builtin_amdgcn_s_waitcnt(0);
    // whether this is the workgroup's last unit (its group has `total`
    // units; workgroups take every per_xcd-th of them)
    const bool last_unit = !XL || k + p.per_xcd >= total;
    const int i = un.i, U = un.U;
    const int b = i / p.Hkv, h = i - b * p.Hkv;
    const int G = p.G;
    const int64_t sb = un.sb;
    // rows of the segment inside the pool (paged: every page is checked)
    const int64_t in_pool = PG ? INT64_MAX : p.pool_rows - sb;
    const int ntiles = (un.n + kTile - 1) / kTile;
    const int t_begin = (k - un.first) * p.tpu;
    const int t_end = min(t_begin + p.tpu, ntiles);
    const int slot = XL ? k * kXcdGroups + grp : k;   // this unit's partial
    const float ks = kv_scale<KV>(un.ka);
    const float vs = kv_scale<KV>(un.va);
    // paged store: the page of this wave's first tile, loaded before anything
    // else so that one round trip covers it
    int pg_next = PG ? page_of(p, i, t_begin + wave) : 0;
    const bool idle = PG && APP && un.P < 0;   // paged: a sequence not in use
    const int P = APP ? (PG ? max(un.P, 0) : un.P) : 0;   // contiguous: already >= 0

    // ---- decode step: rows with data, the new token's row and its tile
    int n = un.n, new_row = -1, t_own = -1;
    const int ring_slot = (APP && p.W > 0) ? P % p.W : 0;   // ring row of P
    if (APP) {
      const StepRows st = step_rows(p.W, P, ring_slot, un.cl, un.cap, un.kn);
      n = idle ? 0 : st.n_pre;
      if (!idle && st.new_row >= 0 && st.new_row < in_pool) {
        new_row = st.new_row;
        t_own = new_row / kTile;
      }
    }
    // the unit that holds the new token's tile adds it to the segment
    const bool owner_unit = APP && t_own >= t_begin && t_own < t_end;
    // decode step: where the keep bit of the token leaving the ring (ring
    // row P mod W) is; W = 0: a valid dummy address.  It is read where it is
    // needed, and tested only after the loads that must not wait for it.
    const bool leaving = APP && !idle && p.W > 0 && P >= p.W;
    // paged store, wave 0 of the owner unit: pages of the new token's row and
    // of the compact row the leaving token may move to (same round trip as
    // the tile's page)
    int pg_own = -1, pg_dst = -1;
    if (PG && owner_unit && wave == 0) {
      pg_own = page_of(p, i, t_own);
      pg_dst = page_of(p, i, (p.W + un.cl) / kTile);
    }
    const uint8_t* rkp = APP ? (p.W > 0 ? p.ring_keep + (int64_t)i * p.W + ring_slot : p.keep_new + i)
                             : nullptr;
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
    const float c1 = p.sm_scale * kLog2e * ks;

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

    // owner unit, wave 0: its slice of the new token (issued after the
    // accumulators are set up, so that nothing before the tile loads waits
    // for it)
    // It also reads the ring row the new token replaces (the leaving
    // token's row: 16-byte K chunk `lane`, V elements EPL*lane..), in case
    // it moves to the compact tail.
    uint32_t nk = 0, nv = 0;
    uint32_t ox[EPL];   // kept apart: combining them would wait for the loads here
#pragma unroll
    for (int e = 0; e < EPL; ++e) ox[e] = 0;
    u32x4 okx = u32x4{0, 0, 0, 0};
    if (owner_unit && wave == 0) {
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
        ox[e] = FP4 ? ((uint32_t)vt[(EPL * lane + e) * (kTile / 2) + rs / 2] >> (4 * (rs & 1))) & 15u
              : FP8 ? (uint32_t)vt[(EPL * lane + e) * kTile + rs]
                    : (uint32_t)reinterpret_cast<const uint16_t*>(vt)[(EPL * lane + e) * kTile + rs];
    }

    bool first_tile = true;
    // decode step, wave 0 of the unit holding the new token's tile: forms
    // the new token from its BF16 input with the frozen scales -- its values
    // and one logit per query row (from the q operand) into LDS, for the
    // combine -- and returns its stored bytes.  It runs during wave 0's
    // first tile, while that tile is in flight.
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
    uint32_t kc = 0, vc = 0;   // wave 0 of the owner unit: the new row's stored bytes
    bool nt_done = false;

    for (int t = t_begin + wave; t < t_end; t += NW) {
      const int r0 = t * kTile;
      const int valid = (int)min((int64_t)min(kTile, n - r0), in_pool - r0);
      const bool own = APP && t == t_own;   // the tile of the leaving token's row
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
      {
        const bool full = valid == kTile;
        // decode step: the leaving token's keep bit, issued ahead of the tile
        int rko = 0;
        if (APP) rko = *rkp;
        const uint8_t* ktile = p.k_pool + trow * (int64_t)RB;
        const uint8_t* vtile = p.v_pool + trow * (int64_t)RB;

        // -- loads: K rows for the 4 token groups (each instruction 1 KB of the
        //    permuted K tile), V columns for the NT d tiles
        u32x4 kr[4][KL];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int j = 0; j < KL; ++j)
            kr[m][j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(ktile + ((m * KL + j) << 10) + lane * 16));
        u32x4 vr[NT][VL];
        u32x2 vq[FP4 ? NT : 1];   // FP4: tokens 16 kg .. 16 kg + 15 of column 16 nt + g
        if (FP4) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            vq[nt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
                vtile + (16 * nt + g) * (kTile / 2) + 8 * kg));
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < VL; ++j)
              vr[nt][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                  vtile + ((16 * nt + g) * kTile + 16 * kg + 8 * j) * E));
        }
        // paged: the page of this wave's next tile, in flight with this one
        if (PG) pg_next = page_of(p, i, t + NW);

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

        if (owner_unit && wave == 0 && first_tile) {   // while V is still in flight
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
        first_tile = false;
      }
    }

    if (owner_unit && wave == 0 && !nt_done) new_token(kc, vc);   // wave 0 had no tile

    // decode step: the keep bit again, for the segment's metadata (back
    // before it is needed, after the combine or the merge)
    const int rkc = APP ? *rkp : 0;

    // ---- combine the waves of the workgroup
    l_run = sum_xor32(sum_xor16(l_run));
    if (kg == 0) {
      s_m[wave][g] = m_run;
      s_l[wave][g] = l_run;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)   // columns g >= G hold no query row
      if (g < G) s_o[wave][g][(16 * nt + 4 * kg) / 4] = acc[nt];
    __syncthreads();

    // ---- decode step, the unit holding the new token's tile: wave 0
    // copies the leaving token's row to the compact tail if it moves and
    // writes the new row; every tile load of the workgroup has completed
    // (barrier above)
    if (owner_unit && wave == 0) {
      {
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
        const bool wants_move = leaving && rkc != 0 && un.cl < un.cap;
        const bool moved = wants_move && own_ok && dst_ok &&
                           (PG || sb + p.W + un.cl < p.pool_rows);
        if (PG && lane == 0 && ((wants_move && !moved) || !own_ok)) atomicOr(p.err, CDA_DEVERR_POOL);
        if (moved) {   // from the copy read at the start of the unit
          const int to = p.W + un.cl, rt = to & (kTile - 1);
          const int64_t drow = PG ? (int64_t)pg_dst * kTile : sb + (to - rt);
          uint8_t* kd = p.k_pool + drow * (int64_t)RB;
          uint8_t* vd = p.v_pool + drow * (int64_t)RB;
          constexpr int KC = RB / 16;   // 16-byte chunks per K row
          if (lane < KC) *reinterpret_cast<u32x4*>(kd + k_chunk_offset(rt, lane, RB)) = okx;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            if (FP4)
              nib_store(vd + (d0n + e) * (kTile / 2) + rt / 2, rt & 1, ox[e]);
            else if (FP8)
              vd[(d0n + e) * kTile + rt] = (uint8_t)ox[e];
            else
              reinterpret_cast<uint16_t*>(vd)[(d0n + e) * kTile + rt] = (uint16_t)ox[e];
          }
        }
        // the new row goes over the ring row: the tiles read its old bytes
        // before the barrier above, and the copy above used the ones read at
        // the start of the unit (unused, and harmless, if it did not move)
        // byte of this lane's first element in the row, and the lane's bytes
        constexpr int LB = FP4 ? EPL / 2 : EPL * E;
        const int kb0 = FP4 ? d0n / 2 : d0n * E;
        if (own_ok) {
          uint8_t* kdst = kt + k_chunk_offset(rs, kb0 >> 4, RB) + (kb0 & 15);
          if (LB == 4)
            *reinterpret_cast<uint32_t*>(kdst) = kc;
          else if (LB == 2)
            *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)kc;
          else
            *kdst = (uint8_t)kc;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            if (FP4)   // after the moved row's write, which may share the byte
              nib_store(vt + (d0n + e) * (kTile / 2) + rs / 2, rs & 1, (vc >> (4 * e)) & 15u);
            else if (FP8)
              vt[(d0n + e) * kTile + rs] = (uint8_t)(vc >> (8 * e));
            else
              reinterpret_cast<uint16_t*>(vt)[(d0n + e) * kTile + rs] = (uint16_t)(vc >> (16 * e));
          }
        }
      }
    }
    // decode step, single-unit segment: every wave of the workgroup has read
    // the segment's metadata (the owner's keep bit included)
    int seq_prev = -1;
    if (APP && !idle && U == 1 && tid == 0) {
      commit_segment<PG>(p, i, un, leaving && rkc != 0);
      seq_prev = __hip_atomic_fetch_add(p.seqcnt + (int64_t)b * kCounterStride, 1,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const float sv = vs;
    for (int e = tid; e < G * (D / 4); e += NTH) {     // (query row, 4 consecutive d)
      const int gg = e / (D / 4), d4 = e - gg * (D / 4);
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][gg]);
      f32x4 O = f32x4{0, 0, 0, 0};
      float L = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float mw = s_m[ww][gg];
          if (mw == -INFINITY) continue;
          const float f = __builtin_amdgcn_exp2f(mw - M);
          O += f * s_o[ww][gg][d4];
          L += f * s_l[ww][gg];
        }
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
      if (U == 1) {
        write_final4(p, b, h, gg, d4, D, M, L, O, sv);
      } else {
        store_part4<XL>(p.part_o + ((int64_t)slot * G + gg) * D + 4 * d4, O);
        if (d4 == 0)   // (m, l, XCD of this workgroup)
          store_part4<XL>(p.part_ml + ((int64_t)slot * G + gg) * 4,
                          f32x4{M, L, __int_as_float(xcc), 0.0f});
      }
    }

    if (U > 1) {
      // ---- split segment: the last of its units to get here merges the
      // partials.  Every wave waits for its partial stores to complete before
      // the workgroup counts itself in.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        int32_t* cnt = p.sem + (int64_t)i * kCounterStride;
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == U - 1;
        if (prev == U - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_last) {
        // decode step: every unit of the segment has read its metadata
        if (APP && !idle && tid == 0) {
          commit_segment<PG>(p, i, un, leaving && rkc != 0);
          seq_prev = __hip_atomic_fetch_add(p.seqcnt + (int64_t)b * kCounterStride, 1,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // each thread merges 4 consecutive outputs of one query row; the
        // (m, l) and o loads of a batch of kMergeBatch units go out together.
        // XCD-local mode: a partial written on another XCD than this one
        // (the workgroups of a residue not sharing an L2) sets CDA_DEVERR_XCD.
        bool xcd_clash = false;
        for (int e = tid; e < G * (D / 4); e += NTH) {
          const int gg = e / (D / 4), d4 = e - gg * (D / 4);
          float M = -INFINITY, L = 0.0f;
          f32x4 O = f32x4{0, 0, 0, 0};
          for (int k0 = 0; k0 < U; k0 += kMergeBatch) {
            f32x4 ml[kMergeBatch];
            f32x4 ov[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {   // unconditional loads, clamped index
              const int ku = un.first + min(k0 + j, U - 1);
              const int64_t sl = (int64_t)(XL ? ku * kXcdGroups + grp : ku) * G + gg;
              ml[j] = load_part4<XL>(p.part_ml + sl * 4);
              ov[j] = load_part4<XL>(p.part_o + sl * D + 4 * d4);
            }

#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
              if (XL && __float_as_int(ml[j][2]) != xcc) xcd_clash = true;
              if (k0 + j >= U) ml[j][0] = -INFINITY;
            }
            float Mb = M;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, ml[j][0]);
            if (Mb == -INFINITY) continue;
            const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
            O *= a;
            L *= a;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
              const float f = (ml[j][0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml[j][0] - Mb);
              O += f * ov[j];
              L += f * ml[j][1];
            }
            M = Mb;
          }
          write_final4(p, b, h, gg, d4, D, M, L, O, sv);
        }
        if (xcd_clash) atomicOr(p.err, CDA_DEVERR_XCD);
      }
    }
    // decode step: the last segment of sequence b to be done writes pos[b]
    if (APP && tid == 0 && seq_prev == p.Hkv - 1) {
      p.pos[b] = un.P + 1;
      __hip_atomic_store(p.seqcnt + (int64_t)b * kCounterStride, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (last_unit) break;
    // the next unit starts with nothing in flight (its first loads then wait
    // for nothing of this one), and reuses this unit's LDS
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// XCD-local mode applies when the XCD count divides the 8 segment groups.
int device_xcds() {
  int dev = 0, nx = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) return 0;
  return nx;
}

template <bool APP, bool PG>
void launch_variant(int kv, int D, bool xl, int nw, dim3 grid, hipStream_t s, const AttnParams& p) {
#define CDA_LAUNCH_ATTN(F, DD, X)                                                      \
  (nw == 8 ? attn_kernel<F, DD, X, 8, APP, PG><<<grid, 512, 0, s>>>(p)                 \
           : attn_kernel<F, DD, X, 4, APP, PG><<<grid, 256, 0, s>>>(p))
  if (kv == kKvFP4) {   // D = 128 only
    if (xl) CDA_LAUNCH_ATTN(kKvFP4, 128, true); else CDA_LAUNCH_ATTN(kKvFP4, 128, false);
  } else if (kv == kKvFP8) {
    if (D == 64) {
      if (xl) CDA_LAUNCH_ATTN(kKvFP8, 64, true); else CDA_LAUNCH_ATTN(kKvFP8, 64, false);
    } else {
      if (xl) CDA_LAUNCH_ATTN(kKvFP8, 128, true); else CDA_LAUNCH_ATTN(kKvFP8, 128, false);
    }
  } else {
    if (D == 64) {
      if (xl) CDA_LAUNCH_ATTN(kKvBF16, 64, true); else CDA_LAUNCH_ATTN(kKvBF16, 64, false);
    } else {
      if (xl) CDA_LAUNCH_ATTN(kKvBF16, 128, true); else CDA_LAUNCH_ATTN(kKvBF16, 128, false);
    }
  }
#undef CDA_LAUNCH_ATTN
}

}  // namespace

int64_t attn_max_units(const cda_kv_cache& c, int tpu) {
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return nh + c.pool_rows / ((int64_t)kTile * tpu);
}

// Workspace: [per-segment counters][per-sequence counters] (one 128-byte
// line each) [partial (m, l, XCD)][partial o].
// Partial slots: an XCD-local slot is 8k + group with k below the units of
// the group (at most all units), so 8 x the unit bound covers both modes.
size_t attn_workspace_bytes(const cda_kv_cache& c, int G, int tpu) {
  const int64_t slots = kXcdGroups * attn_max_units(c, tpu);
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return align256((size_t)nh * 4 * kCounterStride) + align256((size_t)c.B * 4 * kCounterStride) +
         align256((size_t)slots * G * 4 * 4) +
         align256((size_t)slots * G * c.D * 4);
}

hipError_t launch_attn(const cda_kv_cache& c, const void* q, int Hq, float sm_scale, void* out,
                       int out_f32, float* lse, int tpu, void* workspace, hipStream_t s,
                       const cda_compact_args* step) {
  const int nh = c.B * c.Hkv;
  if (nh == 0) return hipGetLastError();
  const int G = Hq / c.Hkv;
  const int64_t units = attn_max_units(c, tpu);
  const int64_t slots = kXcdGroups * units;
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
  p.part_ml = reinterpret_cast<float*>(ws);
  ws += align256((size_t)slots * G * 4 * 4);
  p.part_o = reinterpret_cast<float*>(ws);
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
  const int nx = device_xcds();
  const bool xl = nx > 0 && kXcdGroups % nx == 0;
  // the group map (written by COUNT) is used for up to 512 segments; past
  // that it is the identity i mod 8 and scanning it would only cost time
  p.seg_group = (xl && nh <= 512) ? c.seg_group : nullptr;
  // XCD-local: 8 groups of per_xcd workgroups, a quarter more than an even
  // share of the unit bound; a group with more units loops over them.
  p.per_xcd = xl ? (int)((units * 5 / 4 + kXcdGroups - 1) / kXcdGroups) : 0;
  const dim3 grid((unsigned)(xl ? (int64_t)p.per_xcd * kXcdGroups : units));
  const int kv = c.kv_dtype;
  const int nw = tpu >= 8 ? 8 : 4;   // waves per workgroup: one tile each per pass
  const bool pg = c.page_table != nullptr;
  if (step) {
    if (pg) launch_variant<true, true>(kv, c.D, xl, nw, grid, s, p);
    else launch_variant<true, false>(kv, c.D, xl, nw, grid, s, p);
  } else {
    if (pg) launch_variant<false, true>(kv, c.D, xl, nw, grid, s, p);
    else launch_variant<false, false>(kv, c.D, xl, nw, grid, s, p);
  }
  return hipGetLastError();
}

}  // namespace cda
