// Multi-query attention of a chunk of new tokens over the compact KV store,
// for gfx950: a prefill continued chunk by chunk on top of a compacted
// context, or several draft tokens at once.
//
// What is computed (FastDMS page, memory-table paragraph: the compact cache
// plus the W-token staging window; PyramidInfer page: compressing the cache
// already while the prompt is processed): sequence b receives M <= 64 new
// tokens at positions P .. P+M-1 (P = pos[b]) with queries q[b, t], keys and
// values k[b, t], v[b, t] and keep bytes keep[b, t].  Query t gets exactly
// the decode attention at position P + t, i.e. attention over the rows the
// store would hold after the tokens P .. P+t were appended one at a time:
//   - every compact row of the store (kept tokens older than the window);
//   - the store's ring rows, except a token that has left query t's window
//     (position <= P + t - W) without being kept;
//   - the chunk's tokens t' <= t, except one that has left the window
//     without being kept (only when M > W).
// Chunk tokens take part with the values the store would hold for them
// (BF16, or encoded with the segment's frozen FP8/FP4 scales).  Attending
// first and appending afterwards is what makes this exact: appending the
// chunk first would overwrite ring rows that the chunk's earlier queries
// still see.
//
// Launches: (1) attention: workgroup (split of a segment, group of 16
// blocks of 16 query columns) walks its share of the segment's tiles; the
// columns are (token, query head) pairs, column c = t * G + g; the
// workgroup holding the chunk tile first encodes the chunk into one 64-row
// tile in the store's formats (in the workspace); (2) the commit of every
// segment -- the store becomes what M APPEND operations leave, computed for
// all M tokens at once -- side by side with the merge of the splits'
// partial states per column.
//
// Per 64-row tile and wave of 32 columns (two 32-row blocks mu, four 32-d
// blocks of V):
//   S[row][c]    = K_tile[row][:] . Q^T[:][c]        (32 x 32 x 16 bf16)
//   O^T[d][c]   += V^T[d][row] . P^T[row][c]          (32 x 32 x 16 f16/bf16)
// with K staged so that every lane holds, in its S accumulator, the rows
// of its P operand, and V staged column-major.
#include <algorithm>

#include "attn_common.h"
#include "cda_device.h"
#include "cda_launch.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));   // a 32x32 MFMA accumulator

namespace cda {
namespace {

constexpr int kWideTarget = 256;     // attention workgroups in all: one per CU
// The chunk tile counts as 1 + kChunkExtra tiles in the plan: the workgroup
// that holds it encodes the chunk's rows first (their loads and
// conversions).  (Extras of 1, 2, 3, 4: 40.5, 40.8-41.1, 41.7, 42.0 us per
// call at M = 64 on the Qwen c = 8 layer; 1 is also the best at M = 16.)
constexpr int kChunkExtra = 1;
constexpr int kMaxRingTiles = CDA_MAX_CHUNK_WINDOW / kTile;   // chunk commit: ring tiles
// chunk commit, BF16 / FP8: more rows than this are written a lane per row
// (a column per store), fewer a row per pass and a lane per column
constexpr int kRowsByLane = 8;

struct ChunkParams {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t pool_rows;
  const int64_t* seg_base;     // contiguous segments
  const int32_t* page_table;   // paged store
  int max_pages, n_pages;
  const int32_t* seg_cap;
  const int32_t* comp_len;
  const int32_t* pos;
  const uint8_t* ring_keep;
  const float* k_amax;
  const float* v_amax;
  const uint16_t* q;           // [B, M, Hq, D]
  void* out;                   // [B, M, Hq, D]
  float* lse;                  // [B, M, Hq] or NULL
  const uint16_t* k_new;       // chunk: (b, t, h, d) at b*nsb + t*nst + h*nsh + d
  const uint16_t* v_new;
  int64_t nsb, nst, nsh;
  const uint8_t* keep_new;     // [B, M, Hkv]
  uint8_t* chunk_k;            // workspace: [nh] tiles in the K pool format
  uint8_t* chunk_v;            // workspace: [nh] tiles in the V pool format
  void* part_o;                // workspace: [slots][16][D] f32 (BF16 store) or f16 (FP8/FP4)
  float* part_ml;              // workspace: [slots][16][2]
  // slots: [column group][Gw][16 blocks]
  int32_t* plan;               // workspace: [nh][2] first workgroup, splits of each segment
  int32_t* seqcnt;             // workspace: [B] segments of the sequence committed
  int B, Hkv, Hq, G, M, W, nh, NB, out_f32;
  int Gw;                      // attention workgroups per column group
  float sm_scale;
  int32_t* err;
};

// ---------------------------------------------------------------- attention

// Workgroup (split s of a segment, group of up to 16 blocks of 16 (token,
// query head) columns), 8 waves, with splits
// given out in proportion to the segments' tile counts (segment lengths
// differ with their keep rates: equal splits per segment left workgroups
// between 2 and 10 tiles on the Qwen c = 8 layer, and the longest set the
// kernel's time).  The workgroup walks a contiguous range of its segment's
// tiles from the highest down; the top split takes the chunk tile first
// (encoded here from the new rows, as an APPEND would encode them) and
// fewer stored tiles.  The waves stage each tile in one
// of two LDS buffers while computing on the other -- the tile after it
// already in flight in registers -- converting FP8/FP4 codes once, exactly,
// to the MFMA operand types (K to bf16 operands
// of the 32x32x16 products, its rows in the order that makes each lane's S
// values its own P operand; V to a [d][row] f16 image like a BF16 V tile),
// zeroing V rows past the data, and publishing the rows' keep bits as one
// ballot.  Wave w owns 32 columns (blocks 2w and 2w + 1) over every tile:
// each K and V operand read from LDS serves 32 columns (with 16x16 products
// and 16 waves, 35 us against 32 us on that layer: the 512 KB of operand
// reads per tile bounded it).  Masks: a 64-bit row mask per column (rows
// past the data; ring rows that left the query's window unkept, one
// circular interval; chunk tokens after the query or out of its window
// unkept), of which each lane takes its 32 rows.
constexpr int kWideWaves = 8, kWideBlocks = 2;   // waves, column blocks per wave
constexpr int kWideGroup = kWideWaves * kWideBlocks;

// Sum over the 64 lanes of a wave, in every lane: DPP within rows of 16
// (quad swaps, then rotations by 4 and 8), then the 16- and 32-lane swaps.
__device__ __forceinline__ int wave_sum_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);    // quad_perm [1, 0, 3, 2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);    // quad_perm [2, 3, 0, 1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);   // row_ror:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);   // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)(r[0] + r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)(r[0] + r[1]);
}

// Bits a .. b of a 64-bit row mask (none when a > b), a and b clamped to 0 .. 63.
__device__ __forceinline__ uint64_t rows64(int a, int b) {
  a = max(a, 0);
  b = min(b, 63);
  return a > b ? 0ull : ((~0ull >> (63 - b)) & (~0ull << a));
}

// Bits 2 and 3 of x exchanged (the K row order of the 32x32 S products).
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// RS = 2 (chunks of at most 8 blocks, where most waves would have no
// columns): waves 2c and 2c + 1 share column group c, each taking one
// 32-row half of every tile with its own softmax state; the pair merges
// the two states at the end.
template <int KV, int D, bool PG, int RS>
__global__ __launch_bounds__(64 * kWideWaves) void chunk_attn_wide_kernel(ChunkParams p) {
  constexpr int NW = kWideWaves;
  constexpr bool FP8 = KV == kKvFP8, FP4 = KV == kKvFP4, Q = KV != kKvBF16;
  constexpr int RB = kv_row_bytes(KV, D);
  constexpr int NKS = D / 16, ND = D / 32, KL = RB / 64;   // 32x32x16 k-steps, d blocks
  constexpr int TB = kTile * RB;                  // bytes of a stored K (or V) tile
  constexpr int NCH = 2 * TB / 16;                // 16-byte chunks of a stored K + V tile
  constexpr int CPT = (NCH + 64 * NW - 1) / (64 * NW);   // per thread
  constexpr int SPC = FP4 ? 4 : FP8 ? 2 : 1;      // MFMA k-steps per stored 16-byte K chunk
  constexpr int TX = kTile * D * 2;               // bytes of a staged (16-bit) K tile
  constexpr int VP = kTile * 2 + 16;              // bytes per staged V column (padded)
  constexpr int EV = FP8 ? 1 : 2;                 // bytes per BF16 / FP8 V element
  static_assert(NCH % 64 == 0, "tile copy shape");

  // K as bf16 MFMA operands, operand-major: operand (mu, st) of lane l at
  // ((mu * NKS + st) * 64 + l) * 16 holds row 32 mu + swap23(l % 32), d
  // 16 st + 8 (l / 32) .. + 7; V as [d][row] 16-bit values, VP bytes a column
  // Two buffers: the next tile is staged into one while the waves compute
  // on the other.
  __shared__ __attribute__((aligned(16))) uint8_t s_kb[2][TX];
  __shared__ __attribute__((aligned(16))) uint8_t s_vb[2][D * VP];
  __shared__ uint64_t s_keepb[2];   // keep bits of the staged tiles' rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15, kg = lane >> 4;
  const int NCG = (p.NB + kWideGroup - 1) / kWideGroup;
  const int cgi = blockIdx.x % NCG, w = blockIdx.x / NCG;
  const int W = p.W, G = p.G, M = p.M;

  // ---- the plan.  Segment j has nt_j tiles to attend (its stored tiles and
  // the chunk tile, which counts 1 + kChunkExtra; none when idle) and gets SP_j = ceil(nt_j / t) of the Gw
  // workgroups of each column group, t the least tile count per workgroup
  // for which they fit (ceil(total / (Gw - nh)) always does; the 8 counts
  // from ceil(total / Gw) up, below which none can, are tried together);
  // workgroup w takes split w - PS_j of the segment j with PS_j <= w <
  // PS_j + SP_j.  Every wave computes the same plan on its own, lane l
  // taking segments l, l + 64, ... (cross-lane sums and a scan; no LDS, no
  // barrier), and takes its segment's metadata from the lane that loaded it.
  auto seg_meta = [&](int j, int& P_, int& cl_, int& nt_) {
    P_ = p.pos[j / p.Hkv];
    const int cap_ = max(p.seg_cap[j], 0);
    cl_ = min(max(p.comp_len[j], 0), cap_);
    nt_ = P_ < 0 ? 0 : (min(W, P_) + cl_ + kTile - 1) / kTile + 1 + kChunkExtra;
  };
  const int j0 = min(lane, p.nh - 1);   // segment `lane` (of the first 64): its six
  const int P0 = p.pos[j0 / p.Hkv];      // loads in one round trip
  const int cap0 = p.seg_cap[j0], clr0 = p.comp_len[j0];
  const int64_t sb0 = PG ? 0 : p.seg_base[j0];
  const float ka0 = Q ? p.k_amax[j0] : 1.0f;
  const float va0 = Q ? p.v_amax[j0] : 1.0f;
  const int cl0 = min(max(clr0, 0), max(cap0, 0));
  const int nt0 = (lane >= p.nh || P0 < 0) ? 0 : (min(W, P0) + cl0 + kTile - 1) / kTile + 1 + kChunkExtra;
  auto tiles_of = [&](int j) {
    if (j < 64) return nt0;
    int a, c, e;
    seg_meta(j, a, c, e);
    return e;
  };
  int total = 0;
  for (int j = lane; j < p.nh; j += 64) total += tiles_of(j);
  total = wave_sum_i(total);
  const int room = max(p.Gw - p.nh, 1);
  int tpw = max(1, (total + room - 1) / room);          // fits
  const int t_lo = max(1, (total + p.Gw - 1) / p.Gw);   // smaller cannot
  if (t_lo < tpw) {   // the splits for t_lo .. t_lo + 7 together; the least that fits
    constexpr int NCAND = 8;
    int c[NCAND];
#pragma unroll
    for (int k = 0; k < NCAND; ++k) c[k] = 0;
    for (int j = lane; j < p.nh; j += 64) {
      const int nt = tiles_of(j);
#pragma unroll
      for (int k = 0; k < NCAND; ++k) c[k] += (nt + t_lo + k - 1) / (t_lo + k);
    }
    int best = tpw;
#pragma unroll
    for (int k = NCAND - 1; k >= 0; --k)
      if (t_lo + k < tpw && wave_sum_i(c[k]) <= p.Gw) best = t_lo + k;
    tpw = best;
  }
  int i = -1, s = 0, SPi = 0, Praw = -1, cl = 0;
  int64_t sb = 0;
  float ka = 1.0f, va = 1.0f;
  {
    int base = 0;   // splits of the segments before this chunk of 64
    for (int c0 = 0; c0 < p.nh; c0 += 64) {
      const int j = c0 + lane;
      const int sp = j < p.nh ? (tiles_of(j) + tpw - 1) / tpw : 0;
      int x = sp;   // inclusive scan over the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const int ps = base + x - sp;   // PS_j
      if (j < p.nh && w == 0 && cgi == 0 && wave == 0) {
        p.plan[2 * j] = ps;
        p.plan[2 * j + 1] = sp;
      }
      const uint64_t hit = __ballot(j < p.nh && w >= ps && w < ps + sp);
      if (hit != 0 && i < 0) {
        const int src = __builtin_ctzll(hit);   // wave-uniform
        i = __builtin_amdgcn_readlane(j, src);
        s = w - __builtin_amdgcn_readlane(ps, src);
        SPi = __builtin_amdgcn_readlane(sp, src);
        if (c0 == 0) {
          Praw = __builtin_amdgcn_readlane(P0, src);
          cl = __builtin_amdgcn_readlane(cl0, src);
          sb = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sb0, src) |
               ((int64_t)__builtin_amdgcn_readlane((int)(sb0 >> 32), src) << 32);
          ka = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ka0), src));
          va = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(va0), src));
        } else {
          int nt_;
          seg_meta(i, Praw, cl, nt_);
          sb = PG ? 0 : p.seg_base[i];
          ka = Q ? p.k_amax[i] : 1.0f;
          va = Q ? p.v_amax[i] : 1.0f;
        }
      }
      base += __builtin_amdgcn_readlane(x, 63);
    }
  }
  // the commit's counters, for the launch after this one
  if (w == 0 && cgi == 0)
    for (int j = tid; j < p.B; j += 64 * NW) p.seqcnt[j] = 0;
  if (i < 0) return;                              // the whole workgroup: no split left
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  const bool idle = Praw < 0;
  const int P = max(Praw, 0);
  const int n = idle ? 0 : min(W, P) + cl;
  const int ntiles = (n + kTile - 1) / kTile;
  // this split's tiles: a contiguous range [rlo, rhi) of the segment's tiles,
  // the splits' shares of the plan's nt tiles taken from the top down; the
  // top split holds the chunk tile (tile ntiles, worth 1 + kChunkExtra) and
  // the stored tiles just below it, split 0 the lowest (the ring's)
  int rlo = 0, rhi = 0;
  {
    const int nq = ntiles + 1 + kChunkExtra, qb = nq / SPi, qr = nq - qb * SPi;
    const int ctop = max(qb + (SPi - 1 < qr ? 1 : 0) - 1 - kChunkExtra, 0);
    if (s == SPi - 1) {
      rlo = ntiles - ctop;
      rhi = ntiles;
    } else {   // below the top split and the splits s + 1 .. SPi - 2
      const int above = (SPi - 2 - s) * qb + max(0, min(qr, SPi - 1) - (s + 1));
      rhi = ntiles - ctop - above;
      rlo = s == 0 ? 0 : rhi - (qb + (s < qr ? 1 : 0));
    }
    rlo = max(rlo, 0);
    rhi = max(rhi, rlo);
  }
  const float ks = Q ? kv_scale<KV>(ka) : 1.0f;
  const float vs = Q ? kv_scale<KV>(va) : 1.0f;
  const float c1 = p.sm_scale * kLog2e * ks;
  const int pmw = W > 0 ? P % W : 0;

  // this wave's 32 columns: blocks cb0 and cb0 + 1, column cb0 * 16 + cq
  // -> (token, head); lanes l and l + 32 share column l % 32
  const int hi = lane >> 5, cq = lane & 31;
  const int wc = wave / RS, mh = RS == 2 ? (wave & 1) : 0;   // column group, row half
  const int cb0 = cgi * kWideGroup + wc * kWideBlocks;
  constexpr int NMU = 2 / RS, NKB = 4 / RS;   // 32-row blocks, 16-row blocks of this wave
  const int kb0 = RS == 2 ? 2 * mh : 0;       // its first 16-row block
  const int col = cb0 * 16 + cq, tq = col / G;
  const bool busy = cb0 < p.NB;                              // per wave
  const bool col_ok = cb0 + (cq >> 4) < p.NB && tq < M;      // per lane
  // stored bytes of tile tt (and its keep bytes) -> registers
  auto fetch = [&](int tt, u32x4 (&rg)[CPT], uint32_t& kb, bool& ok) {
    const bool ctile = tt == ntiles;
    const uint8_t* kt;
    const uint8_t* vt;
    ok = true;
    if (ctile) {
      kt = p.chunk_k + (int64_t)i * TB;
      vt = p.chunk_v + (int64_t)i * TB;
    } else {
      int64_t trow = sb + (int64_t)tt * kTile;
      if (PG) {
        const int pg = p.page_table[(int64_t)i * p.max_pages + min(tt, p.max_pages - 1)];
        ok = tt < p.max_pages && pg >= 0 && pg < p.n_pages;
        trow = (int64_t)pg * kTile;
      } else {
        // the whole tile inside the pool (a pool smaller than the segments
        // COUNT laid out, or a seg_base entry that is not one of its rows)
        ok = sb >= 0 && (sb & (kTile - 1)) == 0 && trow + kTile <= p.pool_rows;
      }
      if (!ok) {   // wave-uniform: nothing read; the tile is not computed (CDA_DEVERR_POOL)
#pragma unroll
        for (int c = 0; c < CPT; ++c) rg[c] = u32x4{0, 0, 0, 0};
        kb = 0;
        return;
      }
      kt = p.k_pool + trow * RB;
      vt = p.v_pool + trow * RB;
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = min(c * 64 * NW + tid, NCH - 1);   // chunk of the K+V image
      const uint8_t* src = ch * 16 < TB ? kt + ch * 16 : vt + (ch * 16 - TB);
      rg[c] = *reinterpret_cast<const u32x4*>(src);
    }
    kb = 0;
    if (tid < kTile) {
      const int r0 = tt * kTile;
      if (ctile) kb = p.keep_new[((int64_t)b * M + min(tid, M - 1)) * p.Hkv + h];
      else if (r0 < W) kb = p.ring_keep[(int64_t)i * W + min(r0 + tid, W - 1)];
    }
  };

  // The chunk tile, encoded here from the new rows as an APPEND would encode
  // them (the same conversions of the same products, so the same bytes),
  // into the registers in the stored tile's byte order and into the
  // workspace, where the commit reads it.  Rows M .. 63 are zero.
  auto encode_chunk = [&](u32x4 (&rg)[CPT], uint32_t& kb) {
    const float kinv = Q ? kv_inv_scale<KV>(ka) : 1.0f;
    const float vinv = Q ? kv_inv_scale<KV>(va) : 1.0f;
    const int64_t nb0 = (int64_t)b * p.nsb + (int64_t)h * p.nsh;
    auto f = [](uint32_t bits16, float inv) { return __fmul_rn(__uint_as_float(bits16 << 16), inv); };
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = min(c * 64 * NW + tid, NCH - 1);
      u32x4 x = u32x4{0, 0, 0, 0};
      if (ch * 16 < TB) {   // K: 16 bytes of row r from element d0 (the stored tile interleaves rows)
        const int kl = ch & 63, kj = (ch >> 6) % KL, km = (ch >> 6) / KL;
        const int g = kl & 15, kc = kl >> 4;
        const int r = 16 * (g >> 2) + 4 * km + (g & 3);
        const int d0 = FP8 ? 64 * kj + 16 * kc : FP4 ? 32 * kc : 32 * kj + 8 * kc;
        const uint16_t* src = p.k_new + nb0 + (int64_t)min(r, M - 1) * p.nst + d0;
        if (FP8) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(src);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(src + 8);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4& a = q < 2 ? a0 : a1;
            const uint32_t w0 = a[2 * (q & 1)], w1 = a[2 * (q & 1) + 1];
            x[q] = e4m3x2_from_f32(f(w0 & 0xFFFFu, kinv), f(w0 >> 16, kinv)) |
                   (e4m3x2_from_f32(f(w1 & 0xFFFFu, kinv), f(w1 >> 16, kinv)) << 16);
          }
        } else if (FP4) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(src + 8 * q);
            uint32_t y = 0;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2)
              y |= e2m1x2_from_f32(f(a[w2] & 0xFFFFu, kinv), f(a[w2] >> 16, kinv)) << (8 * w2);
            x[q] = y;
          }
        } else {
          x = *reinterpret_cast<const u32x4*>(src);
        }
        if (r >= M) x = u32x4{0, 0, 0, 0};
      } else {              // V: column d, rows row0 .. (16 FP8, 8 BF16; FP4 16 of 2 columns)
        const int vb = ch * 16 - TB;
        constexpr int NR = FP8 ? 16 : FP4 ? 32 : 8;
        // FP4: rows row0 .. row0 + 15 of columns d and d + 1 (v[16 + e])
        int d = 2 * ((vb % (8 * D)) / 16), row0 = 16 * (vb / (8 * D));
        if (!FP4) v_tile_run(vb, D, EV, d, row0);
        uint32_t v[NR];
#pragma unroll
        for (int e = 0; e < NR; ++e) {
          const int re = FP4 ? row0 + (e & 15) : row0 + e, de = FP4 ? d + (e >> 4) : d;
          const uint32_t raw = p.v_new[nb0 + (int64_t)min(re, M - 1) * p.nst + de];
          v[e] = re < M ? raw : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (FP8) {
            x[q] = e4m3x2_from_f32(f(v[4 * q], vinv), f(v[4 * q + 1], vinv)) |
                   (e4m3x2_from_f32(f(v[4 * q + 2], vinv), f(v[4 * q + 3], vinv)) << 16);
          } else if (FP4) {
            uint32_t y = 0;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2)
              y |= e2m1x2_from_f32(f(v[8 * q + 2 * w2], vinv), f(v[8 * q + 2 * w2 + 1], vinv)) << (8 * w2);
            x[q] = y;
          } else {
            x[q] = v[2 * q] | (v[2 * q + 1] << 16);
          }
        }
      }
      rg[c] = x;
      if (c * 64 * NW + tid < NCH) {
        uint8_t* dst = ch * 16 < TB ? p.chunk_k + (int64_t)i * TB + ch * 16
                                    : p.chunk_v + (int64_t)i * TB + (ch * 16 - TB);
        *reinterpret_cast<u32x4*>(dst) = x;
      }
    }
    kb = 0;
    if (tid < kTile) kb = p.keep_new[((int64_t)b * M + min(tid, M - 1)) * p.Hkv + h];
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 acc[ND];   // O^T: register v of lane l: d 32 dl + 8 (v / 4) + 4 hi + v % 4
#pragma unroll
  for (int dl = 0; dl < ND; ++dl)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dl][v] = 0.0f;
  bool first_tile = true;

  u32x4 rg[CPT];          // the fetched tile's bytes
  uint32_t kbyte = 0;     // its keep bytes
  bool ok = true, ok_cur = true;   // it (the tile being computed) has a page
  // ---- tile tt (its bytes in rg, keep bytes in kbyte) -> LDS buffer buf, converted
  auto stage = [&](int tt, int buf) {
    uint8_t* s_k = s_kb[buf];
    uint8_t* s_v = s_vb[buf];
    const bool ctile = tt == ntiles;
    const int r0 = tt * kTile;
    const int valid = ctile ? M : min(kTile, n - r0);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = c * 64 * NW + tid;
      const u32x4 x = rg[c];
      if (ch >= NCH) continue;                   // wave-uniform (NCH is a multiple of 64)
      if (ch * 16 < TB) {                        // K chunk ch: row r, SPC groups of 8 d from d0
        const int kl = ch & 63, kj = (ch >> 6) % KL, km = (ch >> 6) / KL;
        const int g = kl & 15, kc = kl >> 4;   // the stored tile interleaves rows (k_chunk_offset)
        const int r = 16 * (g >> 2) + 4 * km + (g & 3);
        const int d0 = FP8 ? 64 * kj + 16 * kc : FP4 ? 32 * kc : 32 * kj + 8 * kc;
        uint8_t* rowb = s_k + ((r >> 5) * NKS * 64 + swap23(r & 31)) * 16;
        auto dst = [&](int dd) {   // operand slot of d dd .. dd + 7 of row r
          return reinterpret_cast<bf16x8*>(rowb + ((dd >> 4) * 64 + 32 * ((dd >> 3) & 1)) * 16);
        };
        if (FP4) {
#pragma unroll
          for (int q = 0; q < 4; ++q) *dst(d0 + 8 * q) = fp4x8_to_bf16x8(x[q]);
        } else if (FP8) {
          *dst(d0) = fp8x8_to_bf16x8(x[0], x[1]);
          *dst(d0 + 8) = fp8x8_to_bf16x8(x[2], x[3]);
        } else {
          *reinterpret_cast<u32x4*>(dst(d0)) = x;
        }
      } else {                                   // V: rows row0 .. of column d
        const int vb = ch * 16 - TB;             // byte of the stored V tile
        if (FP4) {                               // 16 rows of columns d and d + 1
          const int d = 2 * ((vb % (8 * D)) / 16), row0 = 16 * (vb / (8 * D));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = row0 + 8 * (q & 1);
            f16x8 y = fp4x8_to_f16x8(x[q]);
            if (r + 8 > valid) {                  // rows past the data
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (r + e >= valid) y[e] = (_Float16)0.0f;
            }
            *reinterpret_cast<f16x8*>(s_v + (d + (q >> 1)) * VP + r * 2) = y;
          }
        } else if (FP8) {                        // 16 rows
          int d, row0;
          v_tile_run(vb, D, 1, d, row0);
          uint8_t* dst = s_v + d * VP + row0 * 2;
          f16x8 y0 = fp8x8_to_f16x8(x[0], x[1]), y1 = fp8x8_to_f16x8(x[2], x[3]);
          if (row0 + 16 > valid) {                // rows past the data
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (row0 + e >= valid) y0[e] = (_Float16)0.0f;
              if (row0 + 8 + e >= valid) y1[e] = (_Float16)0.0f;
            }
          }
          *reinterpret_cast<f16x8*>(dst) = y0;
          *reinterpret_cast<f16x8*>(dst + 16) = y1;
        } else {                                 // 8 rows, as stored
          int d, row0;
          v_tile_run(vb, D, 2, d, row0);
          u32x4 y = x;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = row0 + 2 * q;
            y[q] &= (r >= valid ? 0u : 0xFFFFu) | (r + 1 >= valid ? 0u : 0xFFFF0000u);
          }
          *reinterpret_cast<u32x4*>(s_v + d * VP + row0 * 2) = y;
        }
      }
    }
    if (wave == 0) {   // the tile's keep bits, one per row
      const uint64_t km = __ballot(kbyte != 0);
      if (lane == 0) s_keepb[buf] = km;
    }
    if (!ok && tid == 0) atomicOr(p.err, CDA_DEVERR_POOL);
  };

  // Each tile fetched two tiles ahead into registers and staged one tile
  // ahead into the other buffer, so each tile costs one barrier and its
  // staging overlaps the other waves' products.
  // This split's tiles from the highest down: the top split encodes the
  // chunk tile first, its loads beside the q loads.
  const int t0 = (s == SPi - 1 && !idle) ? ntiles : rhi - 1 >= rlo ? rhi - 1 : -1;
  auto next_t = [&](int tt) {
    const int tn_ = tt == ntiles ? rhi - 1 : tt - 1;
    return tn_ >= rlo ? tn_ : -1;
  };
  int cur = 0;
  if (t0 >= 0) {
    if (t0 == ntiles) encode_chunk(rg, kbyte);
    else fetch(t0, rg, kbyte, ok);
  }
  // the q operands after the first tile's loads (the compiler waits for them
  // where they are first moved, which would otherwise hold the tile back)
  bf16x8 qop[NKS];
  {
    const int64_t qrow = col_ok ? ((int64_t)(b * M + tq) * p.Hq + h * G + (col - tq * G))
                                : ((int64_t)b * M * p.Hq + h * G);
    const uint16_t* qr = p.q + qrow * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < NKS; ++st)
      qop[st] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * st));
  }

  if (t0 >= 0) {
    stage(t0, 0);
    ok_cur = ok;
    const int t1 = next_t(t0);
    if (t1 >= 0) fetch(t1, rg, kbyte, ok);
  }
  __syncthreads();
  for (int tt = t0; tt >= 0;) {
    const int tn = next_t(tt);
    const bool ok_next = ok;
    if (tn >= 0) {
      stage(tn, cur ^ 1);
      const int tnn = next_t(tn);
      if (tnn >= 0) fetch(tnn, rg, kbyte, ok);
    }
    if (busy && ok_cur) {
      const bool ctile = tt == ntiles;
      const int r0 = tt * kTile;
      const int valid = ctile ? M : min(kTile, n - r0);
      const uint8_t* s_k = s_kb[cur];
      const uint8_t* s_v = s_vb[cur];
      const uint64_t s_keep = s_keepb[cur];
      // ---- visible rows of the tile for this lane's query, as a 64-bit mask,
      // then this lane's 32 rows: bit 8 k + e of vl is row 16 k + 8 hi + e
      const uint64_t keep64 = s_keep;
      uint64_t vis = col_ok ? rows64(0, valid - 1) : 0ull;
      if (ctile) {   // chunk tokens rr <= t, in the window or kept
        vis &= rows64(tq - W + 1, tq) | (keep64 & rows64(0, tq));
      } else if (r0 < W) {
        // ring rows whose token left query t's window: P >= W: the t + 1
        // rows from pmw on (circularly); P < W: rows 0 .. P + t - W
        uint64_t hid;
        if (P >= W) {
          const int len = min(tq + 1, W);
          hid = rows64(pmw - r0, min(pmw + len, W) - 1 - r0) | rows64(-r0, pmw + len - W - 1 - r0);
        } else {
          hid = rows64(-r0, min(P + tq - W, W - 1) - r0);
        }
        vis &= ~(hid & ~keep64);
      }
      uint32_t vl = 0;   // bit 8 kk + e: row 16 (kb0 + kk) + 8 hi + e
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
        vl |= (uint32_t)((vis >> (16 * (kb0 + kk) + 8 * hi)) & 0xFFu) << (8 * kk);
      constexpr uint32_t kAll = RS == 2 ? 0xFFFFu : 0xFFFFFFFFu;

      // ---- S = K . Q^T: two 32-row blocks; register v of block mu is row
      // 32 mu + 16 (v / 8) + 8 hi + v % 8 (the K rows were staged in that order)
      f32x16 sc[NMU];
#pragma unroll
      for (int mm = 0; mm < NMU; ++mm)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[mm][v] = 0.0f;
#pragma unroll
      for (int st = 0; st < NKS; ++st)
#pragma unroll
        for (int mm = 0; mm < NMU; ++mm) {
          const int mu = RS == 2 ? mh : mm;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(s_k + ((mu * NKS + st) * 64 + lane) * 16);
          sc[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], sc[mm], 0, 0, 0);
        }

      // ---- online softmax over the column (this lane's 32 rows and lane l ^ 32's);
      // z[k][e] is row 16 k + 8 hi + e.  Masked logits -> -inf (a real
      // branch: most tiles need none); the scale c1 > 0 goes into the max and
      // the exponent.
      float z[NKB][8];   // z[kk]: row block kb0 + kk
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) z[kk][e] = sc[kk >> 1][8 * (kk & 1) + e];
      if (__ballot(vl != kAll) != 0) {   // wave-uniform
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!((vl >> (8 * kk + e)) & 1u)) z[kk][e] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, z[kk][e]);
      tmax = max_xor32(tmax) * c1;
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      if (!first_tile) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
        if (__ballot(alpha != 1.0f)) {   // once the maxima settle, most tiles skip this
#pragma unroll
          for (int dl = 0; dl < ND; ++dl) acc[dl] *= alpha;
        }
      }
      float psum = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z[kk][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[kk][e], c1, -m_use));
          psum += z[kk][e];
        }
      l_run += psum;
      m_run = m_new;

      // ---- O^T += V^T . P^T over the 4 row blocks of 16: this lane's P
      // operand for block k is z[k] (rows 16 k + 8 hi + e), V^T's the d
      // column 32 dl + cq at the same rows
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int k = kb0 + kk;
        f16x8 pf;
        bf16x8 phi, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (Q) {
            pf[e] = (_Float16)z[kk][e];
          } else {
            const __bf16 hb = (__bf16)z[kk][e];
            phi[e] = hb;
            plo[e] = (__bf16)(z[kk][e] - (float)hb);
          }
        }
#pragma unroll
        for (int dl = 0; dl < ND; ++dl) {
          const u32x4 vv = *reinterpret_cast<const u32x4*>(s_v + (32 * dl + cq) * VP + (16 * k + 8 * hi) * 2);
          if (Q) {
            acc[dl] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vv), pf, acc[dl], 0, 0, 0);
          } else {
            acc[dl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), phi, acc[dl], 0, 0, 0);
            acc[dl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vv), plo, acc[dl], 0, 0, 0);
          }
        }
      }
      first_tile = false;
    }
    __syncthreads();   // buffer cur is read by every wave before it is staged again
    ok_cur = ok_next;
    cur ^= 1;
    tt = tn;
  }

  // ---- this lane's partial state (column cq: block cb0 + cq / 16)
  float lsum = sum_xor32(l_run);
  if (RS == 2) {
    // the odd wave of each pair hands its state to the even one, through
    // the staging buffers (free after the loop's last barrier): pairs 0, 1
    // in the K buffers, 2, 3 in the V buffers, ND * 1024 floats each
    __shared__ float s_pm[NW / 2][64], s_pl[NW / 2][64];
    static_assert(2 * TX >= 2 * ND * 4096 && 2 * D * VP >= 2 * ND * 4096, "pair state space");
    float* pacc = wc < 2 ? reinterpret_cast<float*>(&s_kb[0][0]) + wc * ND * 1024
                         : reinterpret_cast<float*>(&s_vb[0][0]) + (wc - 2) * ND * 1024;
    __syncthreads();
    if (mh == 1) {
      s_pm[wc][lane] = m_run;
      s_pl[wc][lane] = lsum;
#pragma unroll
      for (int dl = 0; dl < ND; ++dl)
#pragma unroll
        for (int v = 0; v < 16; ++v) pacc[(dl * 16 + v) * 64 + lane] = acc[dl][v];
    }
    __syncthreads();
    if (mh == 0) {
      const float m1 = s_pm[wc][lane], l1 = s_pl[wc][lane];
      const float mx = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx);
      const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
#pragma unroll
      for (int dl = 0; dl < ND; ++dl)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dl][v] = acc[dl][v] * a0 + pacc[(dl * 16 + v) * 64 + lane] * a1;
      lsum = lsum * a0 + l1 * a1;
      m_run = mx;
    }
  }
  const int cb = cb0 + (cq >> 4);
  if (busy && mh == 0 && cb < p.NB) {
    const int64_t slot = ((int64_t)cgi * p.Gw + w) * kWideGroup + (cb - cgi * kWideGroup);
    const int64_t row = slot * 16 + (cq & 15);
    if (Q) {
      // FP8/FP4: o / l, a weighted mean of codes (|code| <= 448, or 6), in
      // f16; the merge weights it by l and applies the V scale
      const float il = lsum > 0.0f ? 1.0f / lsum : 0.0f;
      _Float16* po = static_cast<_Float16*>(p.part_o) + row * D;
#pragma unroll
      for (int dl = 0; dl < ND; ++dl)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f16x2 y0 = {(_Float16)(acc[dl][4 * a4] * il), (_Float16)(acc[dl][4 * a4 + 1] * il)};
          const f16x2 y1 = {(_Float16)(acc[dl][4 * a4 + 2] * il), (_Float16)(acc[dl][4 * a4 + 3] * il)};
          *reinterpret_cast<u32x2*>(po + 32 * dl + 8 * a4 + 4 * hi) =
              u32x2{__builtin_bit_cast(uint32_t, y0), __builtin_bit_cast(uint32_t, y1)};
        }
    } else {
      float* po = static_cast<float*>(p.part_o) + row * D;
#pragma unroll
      for (int dl = 0; dl < ND; ++dl)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<f32x4*>(po + 32 * dl + 8 * a4 + 4 * hi) =
              f32x4{acc[dl][4 * a4], acc[dl][4 * a4 + 1], acc[dl][4 * a4 + 2], acc[dl][4 * a4 + 3]} * vs;
    }
    if (hi == 0) {
      p.part_ml[row * 2] = m_run;
      p.part_ml[row * 2 + 1] = lsum;
    }
  }
}

// ---------------------------------------------------------------- commit

// Segment i's commit (one workgroup): the chunk's M tokens appended to it, with the result of
// M APPEND operations but without their M sequential round trips.  At step
// t the token at position lp = P + t - W leaves the window (W = 0: the new
// token itself); if it is kept it goes to compact row W + cl0 + (its rank
// among the kept leaving tokens) while there is room (the rest are dropped
// with CDA_DEVERR_CAPACITY).  Its bytes are those of old ring row lp mod W
// (lp < P) or of chunk row lp - P (encoded in the workspace tile).  Ring row
// r then takes the last chunk token that maps to it.  All reads come first,
// issued together: the chunk's encoded tile whole (16-byte copies) and the
// moved rows (a lane per row for V), into LDS, so every old ring row is read
// before any is overwritten.  V rows are written a lane per row (a column
// per store, so a wave's stores fall in one column run), except BF16 and
// FP8 runs of at most kRowsByLane rows: a row per pass of a wave and a lane
// per column there (one row's values lie 16 * e bytes apart in its 16-row
// block, so a store covers 8 lines instead of 8 stores one).  FP4 V elements share
// a byte between two rows: each byte is written by one thread, keeping the
// nibble of a row it does not write; the compact and the ring writes go in
// two rounds because rows W - 1 and W can share a byte.  The last segment of
// a sequence to finish advances pos (a counter per sequence, zeroed by the
// attention launch).
template <int KV, int D, bool PG>
__device__ __forceinline__ void chunk_commit(const ChunkParams& p, int i, uint8_t* k_pool,
                                             uint8_t* v_pool, int32_t* comp_len,
                                             uint8_t* ring_keep, int32_t* pos) {
  constexpr int RB = kv_row_bytes(KV, D);
  constexpr int KC = RB / 16;                  // 16-byte K chunks per row
  constexpr bool FP4 = KV == kKvFP4;
  constexpr int E = KV == kKvBF16 ? 2 : 1;     // bytes per V element (FP4: one code per LDS byte)
  constexpr int NWV = kBlock / 64;             // waves
  constexpr int TCH = kTile * RB / 16;         // 16-byte chunks of one stored tile
  constexpr int TPT = TCH / kBlock;            // chunk tile copy (K, and V), per thread
  static_assert(TCH % kBlock == 0, "tile copy shape");
  constexpr int MPT = (kTile * KC + kBlock - 1) / kBlock;     // moved K chunks, per thread
  constexpr int DPW = D / NWV;                 // V columns per wave
  static_assert(D % NWV == 0, "V columns per wave");
  __shared__ int s_src[kTile];                 // k-th moved token: ring row -1 - r, or chunk row
  __shared__ int s_nmove, s_full;
  __shared__ __attribute__((aligned(16))) uint8_t s_mk[kTile * RB];   // moved rows, K
  __shared__ __attribute__((aligned(16))) uint8_t s_mv[D * kTile * E];   // moved rows, V [d][row]
  __shared__ __attribute__((aligned(16))) uint8_t s_ct[2 * kTile * RB];  // the chunk tile, K then V
  __shared__ uint8_t s_rk[CDA_MAX_CHUNK_WINDOW];   // the ring rows' keep bytes
  constexpr int RKPT = CDA_MAX_CHUNK_WINDOW / kBlock;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  // the u-th V column of this wave, in an order that puts consecutive
  // stores in different cache lines (the 16-row runs of neighbouring
  // columns share a line of the stored tile)
  auto vcol = [&](int u) {
    return wave * DPW + (u % 4) * (DPW / 4) + u / 4;
  };
  const int W = p.W, M = p.M;
  const uint8_t* ck = p.chunk_k + (int64_t)i * kTile * RB;   // the chunk's encoded rows
  const uint8_t* cv = p.chunk_v + (int64_t)i * kTile * RB;
  // Every load that does not depend on the metadata goes out beside it: the
  // ring's keep bytes (the ranking reads those of rows (P + t) mod W), the
  // chunk tokens' keep bytes, the chunk's encoded tile.  (Loads are
  // unconditional, from a valid address, and zeroed after where not wanted:
  // a load under a branch would be waited for at the join.)
  const int P = pos[b];
  const int cap_r = p.seg_cap[i], clr = comp_len[i];
  const int64_t sbase = PG ? 0 : p.seg_base[i];
  u32x4 tck[TPT], tcv[TPT], mk[MPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    tck[u] = *reinterpret_cast<const u32x4*>(ck + 16 * (u * kBlock + tid));
    tcv[u] = *reinterpret_cast<const u32x4*>(cv + 16 * (u * kBlock + tid));
  }
  uint32_t rkb[RKPT];
  const uint8_t* rkrow = ring_keep + (int64_t)i * W;
#pragma unroll
  for (int u = 0; u < RKPT; ++u) rkb[u] = W > 0 ? rkrow[min(u * kBlock + tid, max(W, 1) - 1)] : 0u;
  const int tkn = min(max(tid - W, 0), M - 1);   // chunk token t - W of ranking thread t
  const uint32_t knb = p.keep_new[((int64_t)b * M + tkn) * p.Hkv + h];
  if (P < 0) return;                           // idle (paged store): every segment of b
  const int cap = max(cap_r, 0);
  const int cl0 = min(max(clr, 0), cap);
#pragma unroll
  for (int u = 0; u < RKPT; ++u)
    if (u * kBlock + tid < W) s_rk[u * kBlock + tid] = (uint8_t)rkb[u];
  const uint8_t* s_ck = s_ct;
  const uint8_t* s_cv = s_ct + kTile * RB;
  // The rows this commit touches lie in the ring tiles [0, nrt) and the two
  // tiles from the first compact row written on.  Their pool rows are looked
  // up once here: inside the copy loops a load of the page table (or of
  // seg_base) would be repeated after every byte store, which may alias it.
  const int nrt = (W + kTile - 1) / kTile, dt0 = (W + cl0) / kTile;
  __shared__ int64_t s_tile[kMaxRingTiles + 2];
  for (int t = tid; t < nrt + 2; t += kBlock) {
    const int tt = t < nrt ? t : dt0 + (t - nrt);
    int64_t x = sbase + (int64_t)tt * kTile;
    if (PG) {
      const int pg = p.page_table[(int64_t)i * p.max_pages + min(tt, p.max_pages - 1)];
      x = (tt < p.max_pages && pg >= 0 && pg < p.n_pages) ? (int64_t)pg * kTile : -1;
    }
    s_tile[t] = x;
  }
  // pool row of segment row r: -1 if it has no page or leaves the pool
  auto prow = [&](int r) -> int64_t {
    const int tt = r / kTile;
    const int slot = tt < nrt ? tt : nrt + (tt - dt0);
    const int64_t x0 = (slot >= 0 && slot < nrt + 2) ? s_tile[slot] : -1;
    const int64_t x = x0 < 0 ? -1 : x0 + r % kTile;
    return x >= 0 && x < p.pool_rows ? x : -1;
  };
  auto kaddr = [&](uint8_t* pool, int64_t row, int c) {   // 16-byte K chunk c of a pool row
    return pool + (row - row % kTile) * RB + k_chunk_offset((int)(row % kTile), c, RB);
  };
  auto vaddr = [&](uint8_t* pool, int64_t row, int d) {   // V element (row, d); FP4: its byte
    return FP4 ? pool + (row - row % kTile) * RB + v_nib_off((int)(row % kTile), d, D)
               : pool + (row - row % kTile) * D * E + v_tile_off((int)(row % kTile), d, D, E);
  };
  // V element (row j, column d) of the chunk tile in LDS (FP4: its code)
  auto cvel = [&](int j, int d) -> uint32_t {
    if (FP4) return ((uint32_t)s_cv[v_nib_off(j, d, D)] >> (4 * (j & 1))) & 15u;
    if (E == 2) return *reinterpret_cast<const uint16_t*>(s_cv + v_tile_off(j, d, D, 2));
    return s_cv[v_tile_off(j, d, D, 1)];
  };

  __syncthreads();   // s_rk
  // 1. the tokens that move, ranked (one wave: M <= 64)
  if (tid < 64) {
    const int t = tid;
    bool kept = false;
    int src = 0;
    if (t < M) {
      const int lp = P + t - W;
      if (lp >= 0) {
        if (lp < P) {   // in the ring before the chunk (so W > t)
          const int r = lp % W;
          kept = s_rk[r] != 0;
          src = -1 - r;
        } else {        // chunk token lp - P = t - W
          kept = knb != 0;
          src = lp - P;
        }
      }
    }
    const uint64_t bal = __ballot(kept);
    const int rank = __popcll(bal & ((1ull << t) - 1ull));
    if (kept && cl0 + rank < cap) s_src[rank] = src;
    if (t == 0) {
      const int nk = __popcll(bal);
      s_nmove = min(nk, cap - cl0);
      s_full = nk > cap - cl0;
    }
  }
  __syncthreads();
  const int nmove = s_nmove;
  const int nr = W > 0 ? min(M, W) : 0, j0 = M - nr;   // chunk tokens that end in the ring
  const int rs = W > 0 ? (P + j0) % W : 0;              // ring row of chunk token j0
  int bad = 0;

  // 2. every source into registers, then LDS.  Lane `lane` of each wave owns
  // moved row k = lane for V, over the wave's DPW columns.
  uint32_t mv[DPW];
  const bool vrow = lane < nmove;
  int64_t vfrom = -1;
  int vsrc = 0;
  if (vrow) {
    vsrc = min(s_src[lane], kTile - 1);
    if (vsrc < 0) {
      vfrom = prow(-1 - vsrc);
      if (vfrom < 0) bad = 1;
    }
  }
#pragma unroll
  for (int u = 0; u < MPT; ++u) {
    // s_src holds only nmove entries: the others are not read
    const bool in = u * kBlock + tid < nmove * KC;
    const int e = in ? u * kBlock + tid : 0;
    const int k = e / KC, c = e - k * KC;
    const int src = in ? s_src[k] : 0;
    const int64_t from = src < 0 ? prow(-1 - src) : -1;
    const bool want = in && (src >= 0 || from >= 0);
    const uint8_t* a = (src < 0 && from >= 0) ? kaddr(k_pool, from, c)
                                              : ck + k_chunk_offset(min(max(src, 0), kTile - 1), c, RB);
    mk[u] = *reinterpret_cast<const u32x4*>(a);
    if (!want) mk[u] = u32x4{0, 0, 0, 0};
  }
  if (nmove > 0) {
    // this lane's row vr of a tile at vt: column d at vt + v_tile_off(vr, d)
    // (FP4: the byte vt + v_nib_off(vr, d), the code at bit vsh)
    const bool vok = vrow && (vsrc >= 0 || vfrom >= 0);
    const int vr = vsrc >= 0 ? vsrc : (int)(max(vfrom, (int64_t)0) % kTile);
    const uint8_t* vt = (vrow && vsrc < 0 && vfrom >= 0)
                            ? v_pool + (vfrom - vfrom % kTile) * RB
                            : cv;
    const int vsh = FP4 ? 4 * (vr & 1) : 0;
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int d = vcol(u);
      const uint8_t* a = FP4 ? vt + v_nib_off(vr, d, D) : vt + v_tile_off(vr, d, D, E);
      uint32_t x = E == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(a) : (uint32_t)*a;
      if (FP4) x = (x >> vsh) & 15u;
      mv[u] = vok ? x : 0u;
    }
  }
  if (nr > 0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      *reinterpret_cast<u32x4*>(s_ct + 16 * (u * kBlock + tid)) = tck[u];
      *reinterpret_cast<u32x4*>(s_ct + kTile * RB + 16 * (u * kBlock + tid)) = tcv[u];
    }
  }
#pragma unroll
  for (int u = 0; u < MPT; ++u) {
    const int e = u * kBlock + tid;
    if (e < nmove * KC) *reinterpret_cast<u32x4*>(s_mk + 16 * e) = mk[u];   // row e / KC, chunk e % KC
  }
  if (nmove > 0 && vrow) {
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int d = vcol(u);
      if (E == 2) *reinterpret_cast<uint16_t*>(s_mv + (d * kTile + lane) * 2) = (uint16_t)mv[u];
      else s_mv[d * kTile + lane] = (uint8_t)mv[u];
    }
  }
  __syncthreads();   // every old ring row has been read

  // 3. moved rows -> compact rows [R0, R1)
  const int R0 = W + cl0, R1 = R0 + nmove;
  for (int e = tid; e < nmove * KC; e += kBlock) {
    const int k = e / KC, c = e - k * KC;
    const int64_t to = prow(R0 + k);
    if (to < 0) { bad = 1; continue; }
    *reinterpret_cast<u32x4*>(kaddr(k_pool, to, c)) = *reinterpret_cast<const u32x4*>(s_mk + k * RB + 16 * c);
  }
  if (FP4 && W % 2 == 0 && nmove <= kRowsByLane) {
    // few rows (and no byte shared with a ring row): a byte (rows 2q,
    // 2q + 1) per pass of a wave, a lane per column
    const int q0 = R0 / 2, nq = nmove > 0 ? (R1 - 1) / 2 - q0 + 1 : 0;
    for (int x = wave; x < nq; x += NWV) {
      const int q = q0 + x;
      const int64_t base = prow(2 * q);        // both rows of a byte share a page
      const bool lo_in = 2 * q >= R0, hi_in = 2 * q + 1 < R1;
      if (base < 0) {
        bad = 1;
        continue;
      }
      for (int d = lane; d < D; d += 64) {
        uint8_t* bp = vaddr(v_pool, base, d);
        uint32_t byte = (lo_in && hi_in) ? 0u : (uint32_t)*bp;
        if (lo_in) byte = (byte & 0xF0u) | s_mv[d * kTile + (2 * q - R0)];
        if (hi_in) byte = (byte & 0x0Fu) | ((uint32_t)s_mv[d * kTile + (2 * q + 1 - R0)] << 4);
        *bp = (uint8_t)byte;
      }
    }
  } else if (FP4) {
    // byte q0 + lane (rows 2q, 2q + 1), one per lane
    const int q0 = R0 / 2, nq = nmove > 0 ? (R1 - 1) / 2 - q0 + 1 : 0;
    if (lane < nq) {
      const int q = q0 + lane;
      const int64_t base = prow(2 * q);        // both rows of a byte share a page
      const bool lo_in = 2 * q >= R0, hi_in = 2 * q + 1 < R1;
      if (base < 0) {
        bad = 1;
      } else {
        uint32_t old[DPW];   // the bytes first, all loads together
#pragma unroll
        for (int u = 0; u < DPW; ++u) old[u] = *vaddr(v_pool, base, vcol(u));
#pragma unroll
        for (int u = 0; u < DPW; ++u) {
          const int d = vcol(u);
          uint32_t byte = (lo_in && hi_in) ? 0u : old[u];
          if (lo_in) byte = (byte & 0xF0u) | s_mv[d * kTile + (2 * q - R0)];
          if (hi_in) byte = (byte & 0x0Fu) | ((uint32_t)s_mv[d * kTile + (2 * q + 1 - R0)] << 4);
          *vaddr(v_pool, base, d) = (uint8_t)byte;
        }
      }
    }
  } else if (nmove > kRowsByLane) {
    // BF16 / FP8, many rows: a lane per row, a column per store
    if (vrow) {
      const int64_t to = prow(R0 + lane);
      if (to < 0) {
        bad = 1;
      } else {
        for (int u = 0; u < DPW; ++u) {
          const int d = vcol(u);
          uint8_t* dp = vaddr(v_pool, to, d);
          if (E == 2)
            *reinterpret_cast<uint16_t*>(dp) =
                *reinterpret_cast<const uint16_t*>(s_mv + (d * kTile + lane) * 2);
          else
            *dp = s_mv[d * kTile + lane];
        }
      }
    }
  } else {
    // BF16 / FP8, few rows: a moved row per pass of a wave, a lane per
    // column (one row's values lie 16 * E bytes apart in its 16-row block)
    for (int k = wave; k < nmove; k += NWV) {
      const int64_t to = prow(R0 + k);
      if (to < 0) {
        bad = 1;
        continue;
      }
      for (int d = lane; d < D; d += 64) {
        uint8_t* dp = vaddr(v_pool, to, d);
        if (E == 2)
          *reinterpret_cast<uint16_t*>(dp) =
              *reinterpret_cast<const uint16_t*>(s_mv + (d * kTile + k) * 2);
        else
          *dp = s_mv[d * kTile + k];
      }
    }
  }
  __syncthreads();   // rows W - 1 and W may share an FP4 byte

  // 4. the last nr chunk tokens -> ring rows (P + j) mod W
  if (nr > 0) {
    for (int e = tid; e < nr * KC; e += kBlock) {
      const int j = e / KC, c = e - j * KC;
      const int64_t to = prow((P + j0 + j) % W);
      if (to < 0) { bad = 1; continue; }
      *reinterpret_cast<u32x4*>(kaddr(k_pool, to, c)) =
          *reinterpret_cast<const u32x4*>(s_ck + k_chunk_offset(j0 + j, c, RB));
    }
    if (FP4) {
      // ring row r holds chunk token j0 + off, off = (r - rs) mod W, when
      // off < nr: rows [rs, rs + n1) and [0, nr - n1).  The bytes of the
      // second run come first; the first run's first byte is skipped when the
      // second run already ends in it (odd rs, nr = W).
      const int n1 = min(nr, W - rs), n2 = nr - n1;
      const int nq2 = n2 > 0 ? (n2 - 1) / 2 + 1 : 0;
      int qa = rs / 2;
      if (nq2 > 0 && (n2 - 1) / 2 == qa) ++qa;
      const int nq1 = (rs + n1 - 1) / 2 - qa + 1;
      // few bytes (and none shared with a compact row): a byte per pass of a
      // wave, a lane per column; else a lane per byte, a column per store
      const bool by_col = W % 2 == 0 && nq2 + nq1 <= kRowsByLane / 2;
      for (int x = wave; by_col && x < nq2 + nq1; x += NWV) {
        const int q = x < nq2 ? x : qa + (x - nq2);
        const int off0 = (2 * q - rs + W) % W, off1 = (2 * q + 1 - rs + W) % W;
        const bool lo_in = off0 < nr, hi_in = 2 * q + 1 < W && off1 < nr;
        if (!lo_in && !hi_in) continue;
        const int64_t base = prow(2 * q);
        if (base < 0) { bad = 1; continue; }
        for (int d = lane; d < D; d += 64) {
          uint8_t* bp = vaddr(v_pool, base, d);
          uint32_t byte = (lo_in && hi_in) ? 0u : (uint32_t)*bp;
          if (lo_in) byte = (byte & 0xF0u) | cvel(j0 + off0, d);
          if (hi_in) byte = (byte & 0x0Fu) | (cvel(j0 + off1, d) << 4);
          *bp = (uint8_t)byte;
        }
      }
      for (int x = lane; !by_col && x < nq2 + nq1; x += 64) {
        const int q = x < nq2 ? x : qa + (x - nq2);
        const int off0 = (2 * q - rs + W) % W, off1 = (2 * q + 1 - rs + W) % W;
        const bool lo_in = off0 < nr, hi_in = 2 * q + 1 < W && off1 < nr;
        if (!lo_in && !hi_in) continue;
        const int64_t base = prow(2 * q);
        if (base < 0) { bad = 1; continue; }
        uint32_t old[DPW];   // the bytes first, all loads together
#pragma unroll
        for (int u = 0; u < DPW; ++u) old[u] = *vaddr(v_pool, base, vcol(u));
#pragma unroll
        for (int u = 0; u < DPW; ++u) {
          const int d = vcol(u);
          uint32_t byte = (lo_in && hi_in) ? 0u : old[u];
          if (lo_in) byte = (byte & 0xF0u) | cvel(j0 + off0, d);
          if (hi_in) byte = (byte & 0x0Fu) | (cvel(j0 + off1, d) << 4);
          *vaddr(v_pool, base, d) = (uint8_t)byte;
        }
      }
    } else if (nr > kRowsByLane) {
      // BF16 / FP8, many rows: a lane per row, a column per store
      if (lane < nr) {
        const int64_t to = prow((P + j0 + lane) % W);
        if (to < 0) {
          bad = 1;
        } else {
          for (int u = 0; u < DPW; ++u) {
            const int d = vcol(u);
            uint8_t* dp = vaddr(v_pool, to, d);
            if (E == 2) *reinterpret_cast<uint16_t*>(dp) = (uint16_t)cvel(j0 + lane, d);
            else *dp = (uint8_t)cvel(j0 + lane, d);
          }
        }
      }
    } else {
      // BF16 / FP8, few rows: a ring row per pass of a wave, a lane per column
      for (int j = wave; j < nr; j += NWV) {
        const int64_t to = prow((P + j0 + j) % W);
        if (to < 0) {
          bad = 1;
          continue;
        }
        for (int d = lane; d < D; d += 64) {
          uint8_t* dp = vaddr(v_pool, to, d);
          if (E == 2) *reinterpret_cast<uint16_t*>(dp) = (uint16_t)cvel(j0 + j, d);
          else *dp = (uint8_t)cvel(j0 + j, d);
        }
      }
    }
    for (int j = tid; j < nr; j += kBlock)
      ring_keep[(int64_t)i * W + (P + j0 + j) % W] = p.keep_new[((int64_t)b * M + j0 + j) * p.Hkv + h] != 0;
  }
  if (bad) atomicOr(p.err, CDA_DEVERR_POOL);
  if (tid == 0) {
    comp_len[i] = cl0 + nmove;
    if (s_full) atomicOr(p.err, CDA_DEVERR_CAPACITY);
    // every segment of b has read pos[b] before it counts itself in
    const int prev = atomicAdd(p.seqcnt + b, 1);
    if (prev == p.Hkv - 1) {
      pos[b] = P + M;
      p.seqcnt[b] = 0;
    }
  }
}

// ---------------------------------------------------------------- merge

// Workgroups 0 .. nh - 1 commit segment blockIdx.x; workgroup nh + (segment
// i, column block cb) merges the split states of each of that block's 16
// columns, normalised, into out and lse: BF16 store, o carrying the V
// scale (weight 2^(m - M)); FP8/FP4, o / l in f16 (weight 2^(m - M) l, the
// V scale applied at the end).  The commits read and write none of what the merges use, so the two
// run side by side in one launch, the commits dispatched first.  (The
// workgroups of 4 waves leave about 4 waves per SIMD: the kernel may use
// the registers of that occupancy to keep every load in flight.)
template <int KV, int D, bool PG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4)))
void chunk_merge_commit_kernel(ChunkParams p, uint8_t* k_pool, uint8_t* v_pool,
                               int32_t* comp_len, uint8_t* ring_keep, int32_t* pos) {
  // each thread merges IPT items (4 consecutive outputs of one column); the
  // (m, l) and o loads of kMB splits of every item go out together, merged
  // online (a batch's max, then the running sums rescaled to it)
  constexpr int IPT = 16 * (D / 4) / kBlock, kMB = 8;
  static_assert(16 * (D / 4) % kBlock == 0, "merge items per thread");
  if ((int)blockIdx.x < p.nh) {
    chunk_commit<KV, D, PG>(p, blockIdx.x, k_pool, v_pool, comp_len, ring_keep, pos);
    return;
  }
  const int wm = blockIdx.x - p.nh;
  const int i = wm / p.NB, cb = wm - i * p.NB;
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  // the segment's splits, from its plan (slots of consecutive workgroups)
  const int first = min(max(p.plan[2 * i], 0), p.Gw);   // (within the slots)
  const int nsp = min(max(p.plan[2 * i + 1], 0), p.Gw - first);
  const int64_t slot0 = ((int64_t)(cb / kWideGroup) * p.Gw + first) * kWideGroup + cb % kWideGroup;
  constexpr int64_t sstep = kWideGroup;   // slot stride between splits
  constexpr bool Q = KV != kKvBF16;
  float Mx[IPT], L[IPT];
  f32x4 O[IPT];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    Mx[it] = -INFINITY;
    L[it] = 0.0f;
    O[it] = f32x4{0, 0, 0, 0};
  }
  for (int k0 = 0; k0 < nsp; k0 += kMB) {
    float2 ml[IPT][kMB];
    f32x4 ov[IPT][kMB];
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int e = it * kBlock + threadIdx.x, c = e / (D / 4), d4 = e - c * (D / 4);
#pragma unroll
      for (int j = 0; j < kMB; ++j) {   // unconditional loads, clamped split
        const int64_t sl = (slot0 + min(k0 + j, nsp - 1) * sstep) * 16 + c;
        ml[it][j] = *reinterpret_cast<const float2*>(p.part_ml + sl * 2);
        if (Q) {
          const u32x2 hv = *reinterpret_cast<const u32x2*>(static_cast<const _Float16*>(p.part_o) + sl * D + 4 * d4);
          // (the words through scalars: a bit cast of a vector element reads element 0 here)
          const uint32_t w0 = hv.x, w1 = hv.y;
          const f16x2 y0 = __builtin_bit_cast(f16x2, w0), y1 = __builtin_bit_cast(f16x2, w1);
          ov[it][j] = f32x4{(float)y0[0], (float)y0[1], (float)y1[0], (float)y1[1]};
        } else {
          ov[it][j] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.part_o) + sl * D + 4 * d4);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      float Mb = Mx[it];
#pragma unroll
      for (int j = 0; j < kMB; ++j) {
        if (k0 + j >= nsp) ml[it][j].x = -INFINITY;
        Mb = fmaxf(Mb, ml[it][j].x);
      }
      // branch-free (a branch here would let the compiler sink the loads
      // behind it): with no state yet every weight is 0 and Mx stays -inf
      const float Ms = Mb == -INFINITY ? 0.0f : Mb;
      const float a = Mx[it] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mx[it] - Ms);
      O[it] *= a;
      L[it] *= a;
#pragma unroll
      for (int j = 0; j < kMB; ++j) {
        const float f = ml[it][j].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[it][j].x - Ms);
        const float fl = f * ml[it][j].y;
        O[it] += (Q ? fl : f) * ov[it][j];
        L[it] += fl;
      }
      Mx[it] = Mb;
    }
  }
  const float sv = Q ? kv_scale<KV>(p.v_amax[i]) : 1.0f;
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int e = it * kBlock + threadIdx.x, c = e / (D / 4), d4 = e - c * (D / 4);
    const int col = cb * 16 + c, tq = col / p.G, hq = col - tq * p.G;
    if (tq >= p.M) continue;
    const int64_t row = ((int64_t)b * p.M + tq) * p.Hq + h * p.G + hq;
    const f32x4 v = L[it] > 0.0f ? O[it] * (sv / L[it]) : f32x4{0, 0, 0, 0};
    if (p.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + row * D + 4 * d4) = v;
    } else {
      const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * D + 4 * d4) = u32x2{lo, hi};
    }
    if (d4 == 0 && p.lse) p.lse[row] = L[it] > 0.0f ? (Mx[it] + log2f(L[it])) * kLn2 : -INFINITY;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Column blocks of a chunk call: NB blocks of 16 (token, query head)
// columns; Gw 8-wave attention workgroups per group of 16 blocks (about one
// per CU in all, at least one per segment), shared out among the segments
// by the kernel's own plan.  Slots: the partial states the merge reads, 16
// columns each.
void chunk_shape(int nh, int G, int M, int& NB, int& Gw, int64_t& slots) {
  NB = (G * M + 15) / 16;
  const int ncg = (NB + kWideGroup - 1) / kWideGroup;
  Gw = std::max((kWideTarget + ncg - 1) / ncg, nh);
  slots = (int64_t)ncg * Gw * kWideGroup;
}

template <bool PG>
void launch_chunk_kernels(int kv, int D, int nh, int NB, hipStream_t s, const ChunkParams& p,
                          uint8_t* k_pool, uint8_t* v_pool, int32_t* comp_len,
                          uint8_t* ring_keep, int32_t* pos) {
  const int ncg = (NB + kWideGroup - 1) / kWideGroup;
  const dim3 grid((unsigned)(ncg * p.Gw));
#define CDA_CHUNK(F, DD)                                                        \
  do {                                                                          \
    if (NB <= kWideGroup / 2)                                                   \
      chunk_attn_wide_kernel<F, DD, PG, 2><<<grid, 64 * kWideWaves, 0, s>>>(p); \
    else                                                                        \
      chunk_attn_wide_kernel<F, DD, PG, 1><<<grid, 64 * kWideWaves, 0, s>>>(p); \
    chunk_merge_commit_kernel<F, DD, PG><<<nh * (NB + 1), kBlock, 0, s>>>(      \
        p, k_pool, v_pool, comp_len, ring_keep, pos);                           \
  } while (0)
  if (kv == kKvFP4) {
    CDA_CHUNK(kKvFP4, 128);
  } else if (kv == kKvFP8) {
    if (D == 64) CDA_CHUNK(kKvFP8, 64); else CDA_CHUNK(kKvFP8, 128);
  } else {
    if (D == 64) CDA_CHUNK(kKvBF16, 64); else CDA_CHUNK(kKvBF16, 128);
  }
#undef CDA_CHUNK
}

}  // namespace

// Workspace: [chunk K tiles][chunk V tiles][commit counters][plan]
// [partial (m, l)][partial o].
size_t chunk_workspace_bytes(const cda_kv_cache& c, int G, int M) {
  const int nh = c.B * c.Hkv;
  int NB, Gw;
  int64_t slots;
  chunk_shape(nh, G, M, NB, Gw, slots);
  const size_t tile = (size_t)kTile * kv_row_bytes(c.kv_dtype, c.D);
  const size_t cols = (size_t)slots * 16;
  const size_t ob = c.kv_dtype == kKvBF16 ? 4 : 2;   // partial o: f32, or f16 (FP8/FP4)
  return 2 * align256((size_t)nh * tile) + align256((size_t)c.B * 4) +
         align256((size_t)nh * 2 * 4) + align256(cols * 2 * 4) + align256(cols * c.D * ob);
}

hipError_t launch_chunk(const cda_kv_cache& c, const cda_compact_args& a, int M, const void* q,
                        int Hq, float sm_scale, void* out, int out_f32, float* lse,
                        void* workspace, hipStream_t s) {
  const int nh = c.B * c.Hkv;
  if (nh == 0 || M <= 0) return hipGetLastError();
  const int G = Hq / c.Hkv;
  ChunkParams p;
  p.k_pool = static_cast<const uint8_t*>(c.k_pool);
  p.v_pool = static_cast<const uint8_t*>(c.v_pool);
  p.pool_rows = c.pool_rows;
  p.seg_base = c.seg_base;
  p.page_table = c.page_table;
  p.max_pages = c.max_pages;
  p.n_pages = (int)(c.pool_rows / kTile);
  p.seg_cap = c.seg_cap;
  p.comp_len = c.comp_len;
  p.pos = c.pos;
  p.ring_keep = c.ring_keep;
  p.k_amax = c.k_amax;
  p.v_amax = c.v_amax;
  p.q = static_cast<const uint16_t*>(q);
  p.out = out;
  p.lse = lse;
  p.k_new = static_cast<const uint16_t*>(a.k);
  p.v_new = static_cast<const uint16_t*>(a.v);
  p.nsb = a.stride_b;
  p.nst = a.stride_t;
  p.nsh = a.stride_h;
  p.keep_new = a.keep;
  p.B = c.B;
  p.Hkv = c.Hkv;
  p.Hq = Hq;
  p.G = G;
  p.M = M;
  p.W = c.W;
  p.nh = nh;
  int64_t slots;
  chunk_shape(nh, G, M, p.NB, p.Gw, slots);
  p.out_f32 = out_f32;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c.D);
  p.err = c.err;
  const size_t tile = (size_t)kTile * kv_row_bytes(c.kv_dtype, c.D);
  const size_t cols = (size_t)slots * 16;
  char* ws = static_cast<char*>(workspace);
  p.chunk_k = reinterpret_cast<uint8_t*>(ws);
  ws += align256((size_t)nh * tile);
  p.chunk_v = reinterpret_cast<uint8_t*>(ws);
  ws += align256((size_t)nh * tile);
  p.seqcnt = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)c.B * 4);
  p.plan = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)nh * 2 * 4);
  p.part_ml = reinterpret_cast<float*>(ws);
  ws += align256(cols * 2 * 4);
  p.part_o = ws;
  uint8_t* kp = static_cast<uint8_t*>(c.k_pool);
  uint8_t* vp = static_cast<uint8_t*>(c.v_pool);
  if (c.page_table)
    launch_chunk_kernels<true>(c.kv_dtype, c.D, nh, p.NB, s, p, kp, vp, c.comp_len,
                               c.ring_keep, c.pos);
  else
    launch_chunk_kernels<false>(c.kv_dtype, c.D, nh, p.NB, s, p, kp, vp, c.comp_len,
                                c.ring_keep, c.pos);
  return hipGetLastError();
}

}  // namespace cda
