// Prefill compaction and decode-time append of the compact KV store
// (FastDMS page, release paragraph: a compact store that physically
// reclaims evicted slots; memory-table paragraph: cache + staging window).
//
//   count_kernel     keep mask -> per-segment kept count, optional dst map
//   seg_scan_kernel  aligned segment sizes -> seg_base (exclusive prefix sum)
//   amax_kernel      per-segment absmax of the stored prefill K and V (FP8)
//   pack_kernel      stored prefill rows -> pool tiles (BF16 copy / FP8 encode)
//   append_kernel    one decode step: ring exit -> compact tail, new token -> ring
//   page_init_kernel / page_kernel   the paged store's page bookkeeping
//
// Paged store: the pool's 64-row tiles are pages; a segment's tile t is page
// page_table[i * max_pages + t].  COUNT, PACK and RELEASE then act on a range
// of sequences (their inputs indexed from the range's first sequence), and
// sequences with pos < 0 are idle: the append leaves them alone.
//
// All of these run once per prefill or move at most one row per segment per
// step; the decode hot loop is the attention kernel.
#include <algorithm>
#include <type_traits>

#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

// ---------------------------------------------------------------- COUNT

// Workgroup x: segment i0 + x, whose keep row (and dst_out row) is row x.
__global__ __launch_bounds__(kBlock) void count_kernel(
    const uint8_t* __restrict__ keep, int64_t keep_ld, int T, int W, int reserve, int i0,
    int32_t* __restrict__ comp_len, int32_t* __restrict__ seg_cap,
    int32_t* __restrict__ dst_out) {
  __shared__ int smem[4];
  const int x = blockIdx.x, i = i0 + x, tid = threadIdx.x;
  const uint8_t* row = keep + (int64_t)x * keep_ld;
  const int ncand = T - W > 0 ? T - W : 0;       // positions older than the window
  const int limit = dst_out ? T : ncand;
  int running = 0;
  for (int base = 0; base < limit; base += kBlock * 16) {
    const int p0 = base + tid * 16;
    uint32_t flags = 0;
    int cnt = 0;
    uint8_t kb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) kb[j] = ncand > 0 ? row[min(p0 + j, ncand - 1)] : 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int f = (p0 + j < ncand) && kb[j] != 0;
      flags |= (uint32_t)f << j;
      cnt += f;
    }
    int total;
    int rank = block_exclusive_scan(cnt, &total, smem) + running;
    if (dst_out) {
      int32_t* d = dst_out + (int64_t)x * T;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int p = p0 + j;
        if (p < T) {
          int r = -1;
          if (p >= ncand) r = p % W;                 // ring row (W > 0 here)
          else if ((flags >> j) & 1u) r = W + rank++;
          d[p] = r;
        }
      }
    }
    running += total;
  }
  if (tid == 0) {
    comp_len[i] = running;
    seg_cap[i] = running + reserve;
  }
}

// Exclusive prefix sum (int64) over the 256 threads of a workgroup.
__device__ __forceinline__ long long block_exclusive_scan64(long long v, long long* total,
                                                            long long* smem) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) smem[wid] = x;
  __syncthreads();
  long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) {
    before += (w < wid) ? smem[w] : 0;
    all += smem[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// seg_base by a prefix sum of the aligned segment sizes.
__global__ __launch_bounds__(kBlock) void seg_scan_kernel(
    int nh, int W, const int32_t* __restrict__ seg_cap, int64_t* __restrict__ seg_base,
    int32_t* __restrict__ err) {
  __shared__ long long smem[4];
  long long carry = 0;
  for (int base = 0; base < nh; base += kBlock) {
    const int i = base + threadIdx.x;
    long long size = 0;
    if (i < nh) size = ((long long)W + seg_cap[i] + kTile - 1) / kTile * kTile;
    long long total;
    long long ex = block_exclusive_scan64(size, &total, smem) + carry;
    if (i < nh) seg_base[i] = ex;
    carry += total;
  }
  if (threadIdx.x == 0) {
    seg_base[nh] = carry;
    err[0] = 0;
  }
}

// ---------------------------------------------------------------- PACK

// |x| of a bf16 as the upper half of a binary32 bit pattern; unsigned
// comparison of these orders magnitudes, and any NaN compares largest.
__device__ __forceinline__ uint32_t abs_bits(uint32_t word, int half) {
  return ((word >> (16 * half)) & 0x7FFFu) << 16;
}

__global__ void amax_zero_kernel(int i0, int nh, float* __restrict__ k_amax,
                                 float* __restrict__ v_amax) {
  const int i = i0 + blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nh) {
    k_amax[i] = 0.0f;
    v_amax[i] = 0.0f;
  }
}

// Workgroup (x, chunk c): absmax of K and V of segment i0 + x over the
// stored prefill rows of positions [256c, 256c+256), folded into k_amax /
// v_amax with an unsigned atomic max on the magnitude bit patterns.  Its
// inputs are row x of keep and sequence x / Hkv of k and v.
__global__ __launch_bounds__(kBlock) void amax_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t sb, int64_t st,
    int64_t sh, const uint8_t* __restrict__ keep, int64_t keep_ld, int T, int W, int Hkv,
    int D, int i0, float* __restrict__ k_amax, float* __restrict__ v_amax) {
  __shared__ int smem[4];
  __shared__ int s_pos[kBlock];
  __shared__ uint32_t red[2][kBlock / 64];
  const int x = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int i = i0 + x;
  const int b = x / Hkv, h = x - b * Hkv;
  const uint8_t* krow = keep + (int64_t)x * keep_ld;
  const int pp = c * kBlock + tid;
  const int stored = pp < T && (pp >= T - W || krow[pp] != 0);
  int nst;
  const int slot = block_exclusive_scan(stored, &nst, smem);
  if (stored) s_pos[slot] = pp;
  __syncthreads();
  const int lpr = D / 8;                 // lanes per row, 8 bf16 (16 B) each
  const int rows_per_pass = kBlock / lpr;
  const int lr = tid % lpr;
  uint32_t mk = 0, mv = 0;
  for (int e0 = tid / lpr; e0 < nst; e0 += 4 * rows_per_pass) {
    u32x4 a[4], cc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // rows past the end repeat the last stored row: same maximum
      const int e = min(e0 + j * rows_per_pass, nst - 1);
      const int64_t off = (int64_t)b * sb + (int64_t)s_pos[e] * st + (int64_t)h * sh + lr * 8;
      a[j] = *reinterpret_cast<const u32x4*>(k + off);
      cc[j] = *reinterpret_cast<const u32x4*>(v + off);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          mk = max(mk, abs_bits(a[j][w], hf));
          mv = max(mv, abs_bits(cc[j][w], hf));
        }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mk = max(mk, (uint32_t)__shfl_xor((int)mk, o, 64));
    mv = max(mv, (uint32_t)__shfl_xor((int)mv, o, 64));
  }
  const int wid = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][wid] = mk;
    red[1][wid] = mv;
  }
  __syncthreads();
  if (tid == 0 && nst > 0) {
    uint32_t x = 0, y = 0;
    for (int w = 0; w < kBlock / 64; ++w) {
      x = max(x, red[0][w]);
      y = max(y, red[1][w]);
    }
    atomicMax(reinterpret_cast<unsigned int*>(k_amax + i), x);
    atomicMax(reinterpret_cast<unsigned int*>(v_amax + i), y);
  }
}

struct PackParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, st, sh;
  const uint8_t* keep;
  int64_t keep_ld;
  int T, W, Hkv, D;
  int i0;                    // first segment of the range (paged store)
  const int64_t* seg_base;   // contiguous segments
  const int32_t* page_table; // paged store: [nh][max_pages], or NULL
  const int32_t* seg_cap;
  int max_pages, n_pages;
  const int32_t* comp_len;
  int64_t pool_rows;
  uint8_t* k_pool;
  uint8_t* v_pool;
  uint8_t* ring_keep;
  int32_t* pos;
  const float* k_amax;
  const float* v_amax;
  int32_t* err;
};

// Element offset of (row, d) in a BF16 or FP8 V pool (64-row tiles of four
// column-major 16-row blocks; v_tile_off in elements).
__device__ __forceinline__ int64_t v_elem(int64_t row, int d, int D) {
  return (row / kTile) * kTile * D + v_tile_off((int)(row % kTile), d, D, 1);
}

// Workgroup (segment i, y) writes the 64-row pool tiles j = y, y + gridDim.y,
// ... of segment i that hold ring rows or stored rows, one whole tile at a
// time: it finds the source position of each row of the tile (ring row r:
// the position p of the window with p mod W = r; compact row W + c: the
// c-th kept older position, by a scan of the keep row), loads the BF16 rows
// (each 64-lane load is whole rows), encodes them into LDS images of the
// K tile (chunk-permuted rows) and the V tile (column-major; stored in the
// pool's 16-row blocks, FP4 column-major), and stores
// both with 16-byte writes.  Rows of the tile with no source are zero.
// The V image holds one byte per element (an FP4 code in its low nibble);
// FP4 tiles are packed two rows per byte on the way out.
template <int KV, int D>
__global__ __launch_bounds__(kBlock) void pack_kernel(PackParams p) {
  constexpr bool Q = KV != kKvBF16;         // quantised store
  constexpr int RB = kv_row_bytes(KV, D);   // pool bytes per row
  constexpr int CPR = D / 8;                // 8-element input chunks per row
  constexpr int RPI = 64 / CPR;             // rows per 64-lane load
  constexpr int NI = kTile / (RPI * (kBlock / 64));   // loads per wave and tensor
  constexpr int VS = Q ? 68 : 132;          // LDS bytes per V column: 64 rows + pad
  constexpr int kScan = 32;                 // keep bytes per thread per scan pass
  __shared__ int s_src[kTile];
  __shared__ int smem[4];
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kTile * RB];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[D * VS];
  const int x = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = p.i0 + x;                     // segment; x indexes the inputs
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  const int bx = x / p.Hkv;                   // sequence index in the inputs
  const bool paged = p.page_table != nullptr;
  const int T = p.T, W = p.W;
  const int ncand = T - W > 0 ? T - W : 0;  // positions older than the window
  const int nring = min(W, T);
  const uint8_t* krow = p.keep + (int64_t)x * p.keep_ld;
  // paged: a sequence COUNT left idle (no pages) is skipped (pos stays -1;
  // once admitted it reads 0 or T, never below 0)
  if (paged && p.pos[b] < 0) return;
  const bool row16 = (reinterpret_cast<uintptr_t>(krow) & 15) == 0;   // 16-byte keep loads
  // this thread's keep bytes of the first scan pass of the first tile, read
  // before the segment's metadata (one round trip for both)
  u32x4 pre0 = u32x4{0, 0, 0, 0}, pre1 = u32x4{0, 0, 0, 0};
  const bool pre = row16 && (int)blockIdx.y * kTile + kTile > W && tid * kScan + kScan <= ncand;
  if (pre) {
    pre0 = *reinterpret_cast<const u32x4*>(krow + tid * kScan);
    pre1 = *reinterpret_cast<const u32x4*>(krow + tid * kScan + 16);
  }
  // rows the segment has room for: its pages, or its aligned contiguous size
  const int64_t sb = paged ? 0 : p.seg_base[i];
  const int64_t alloc = paged ? (int64_t)W + max(p.seg_cap[i], 0) : p.seg_base[i + 1] - sb;
  const int cl = min(max(p.comp_len[i], 0), ncand);   // from COUNT
  // tiles holding ring rows or stored rows, inside the segment's rows
  const int64_t rows = min((int64_t)max(nring + cl, W), alloc);
  const int ntiles = (int)((rows + kTile - 1) / kTile);
  float kinv = 1.0f, vinv = 1.0f;
  if (Q) {
    kinv = kv_inv_scale<KV>(p.k_amax[i]);
    vinv = kv_inv_scale<KV>(p.v_amax[i]);
  }
  if (blockIdx.y == 0 && h == 0 && tid == 0) p.pos[b] = T;

  for (int j = blockIdx.y; j < ntiles; j += gridDim.y) {
    const int r0 = j * kTile;
    // ---- source position of each row: ring rows here, compact rows below
    if (tid < kTile) {
      const int r = r0 + tid;
      int src = -1;
      if (r < W) {
        if (T >= W) {
          const int base = T - W;             // window: positions base .. T-1
          src = base + (r - base % W + W) % W;
        } else if (r < T) {
          src = r;
        }
        p.ring_keep[(int64_t)i * W + r] = (uint8_t)(src >= 0 && krow[src] != 0);
      }
      s_src[tid] = src;
    }
    const int c_lo = max(r0 - W, 0), c_hi = r0 + kTile - W;   // compact ranks of the tile
    if (c_hi > 0 && cl > c_lo) {
      // the kept older positions of ranks [c_lo, c_hi), by a running scan of
      // the keep row (its barriers also order the ring entries above)
      int carry = 0;
      for (int q0 = 0; q0 < ncand && carry < c_hi; q0 += kBlock * kScan) {
        const int pp = q0 + tid * kScan;
        uint32_t flags = 0;   // bit e: position pp + e is kept
        if (row16 && pp + kScan <= ncand) {
          const bool use_pre = pre && q0 == 0 && j == (int)blockIdx.y;
          const u32x4 x0 = use_pre ? pre0 : *reinterpret_cast<const u32x4*>(krow + pp);
          const u32x4 x1 = use_pre ? pre1 : *reinterpret_cast<const u32x4*>(krow + pp + 16);
#pragma unroll
          for (int e = 0; e < kScan; ++e) {
            const uint32_t wd = e < 16 ? x0[e >> 2] : x1[(e - 16) >> 2];
            flags |= (uint32_t)(((wd >> (8 * (e & 3))) & 0xFFu) != 0u) << e;
          }
        } else {
          uint8_t kb[kScan];
#pragma unroll
          for (int e = 0; e < kScan; ++e) kb[e] = krow[min(pp + e, ncand - 1)];
#pragma unroll
          for (int e = 0; e < kScan; ++e) flags |= (uint32_t)((pp + e < ncand) && kb[e] != 0) << e;
        }
        const int cnt = __builtin_popcount(flags);
        int total;
        int rank = block_exclusive_scan(cnt, &total, smem) + carry;
        if (rank < c_hi && rank + cnt > c_lo) {
          for (uint32_t f = flags; f != 0u; f &= f - 1u, ++rank)
            if (rank >= c_lo && rank < c_hi) s_src[W + rank - r0] = pp + __builtin_ctz(f);
        }
        carry += total;
      }
    }
    __syncthreads();
    // the rows with a source are a prefix of the tile (ring rows fill from
    // row 0, compact rows follow them in rank order), so row 0 has one if
    // any row does
    const int any = s_src[0];

    // ---- loads: wave w, load k covers rows (w NI + k) RPI .. + RPI - 1,
    // lane = (row, 8-element chunk); rows with no source read the tile's
    // source row `any` (no extra HBM traffic) and are zeroed below
    const int cc = lane % CPR, d0 = 8 * cc;
    u32x4 kin[NI], vin[NI];
    int rr[NI];
    bool has[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      rr[k] = (wave * NI + k) * RPI + lane / CPR;
      const int src = s_src[rr[k]];
      has[k] = src >= 0;
      kin[k] = u32x4{0, 0, 0, 0};
      vin[k] = u32x4{0, 0, 0, 0};
      if (any >= 0) {
        const int64_t off = (int64_t)bx * p.sb + (int64_t)(has[k] ? src : any) * p.st +
                            (int64_t)h * p.sh + d0;
        kin[k] = *reinterpret_cast<const u32x4*>(p.k + off);
        vin[k] = *reinterpret_cast<const u32x4*>(p.v + off);
      }
    }
    // ---- encode into the LDS tile images
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = rr[k];
      const u32x4 kx = has[k] ? kin[k] : u32x4{0, 0, 0, 0};
      const u32x4 vx = has[k] ? vin[k] : u32x4{0, 0, 0, 0};
      if (KV == kKvFP4) {
        uint32_t kc = 0;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {   // elements 2 w2 (low nibble), 2 w2 + 1
          const float k0 = __fmul_rn(__uint_as_float(kx[w2] << 16), kinv);
          const float k1 = __fmul_rn(__uint_as_float(kx[w2] & 0xFFFF0000u), kinv);
          const float v0 = __fmul_rn(__uint_as_float(vx[w2] << 16), vinv);
          const float v1 = __fmul_rn(__uint_as_float(vx[w2] & 0xFFFF0000u), vinv);
          kc |= e2m1x2_from_f32(k0, k1) << (8 * w2);
          const uint32_t vb = e2m1x2_from_f32(v0, v1);
          s_v[(d0 + 2 * w2) * VS + r] = (uint8_t)(vb & 15u);
          s_v[(d0 + 2 * w2 + 1) * VS + r] = (uint8_t)(vb >> 4);
        }
        *reinterpret_cast<uint32_t*>(s_k + k_chunk_offset(r, (d0 / 2) >> 4, RB) + ((d0 / 2) & 15)) = kc;
      } else if (KV == kKvFP8) {
        uint32_t kc[2] = {0, 0}, vc[2] = {0, 0};
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {   // elements 2 w2, 2 w2 + 1
          const float k0 = __fmul_rn(__uint_as_float(kx[w2] << 16), kinv);
          const float k1 = __fmul_rn(__uint_as_float(kx[w2] & 0xFFFF0000u), kinv);
          const float v0 = __fmul_rn(__uint_as_float(vx[w2] << 16), vinv);
          const float v1 = __fmul_rn(__uint_as_float(vx[w2] & 0xFFFF0000u), vinv);
          kc[w2 >> 1] |= e4m3x2_from_f32(k0, k1) << (16 * (w2 & 1));
          vc[w2 >> 1] |= e4m3x2_from_f32(v0, v1) << (16 * (w2 & 1));
        }
        *reinterpret_cast<u32x2*>(s_k + k_chunk_offset(r, d0 >> 4, RB) + (d0 & 15)) = u32x2{kc[0], kc[1]};
#pragma unroll
        for (int e = 0; e < 8; ++e) s_v[(d0 + e) * VS + r] = (uint8_t)(vc[e >> 2] >> (8 * (e & 3)));
      } else {
        *reinterpret_cast<u32x4*>(s_k + k_chunk_offset(r, cc, RB)) = kx;
        uint16_t* v16 = reinterpret_cast<uint16_t*>(s_v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v16[(d0 + e) * (VS / 2) + r] = (uint16_t)((vx[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
    __syncthreads();

    // ---- stores: both tiles as 16-byte chunks.  Tiles and pool_rows are
    // multiples of 64 rows, so a tile is wholly inside the pool or wholly
    // outside it (a pool smaller than seg_base[B*Hkv], or a page-table entry
    // that is not a page); outside, the rows with data are flagged and
    // nothing is written.
    int64_t tr = sb + r0;   // pool row of the tile
    if (paged) {
      const int pg = p.page_table[(int64_t)i * p.max_pages + min(j, p.max_pages - 1)];
      tr = (j < p.max_pages && pg >= 0 && pg < p.n_pages) ? (int64_t)pg * kTile : p.pool_rows;
    }
    if (p.pool_rows - tr >= kTile) {
      uint8_t* kt = p.k_pool + tr * (int64_t)RB;
      uint8_t* vt = p.v_pool + tr * (int64_t)RB;
      for (int ch = tid; ch < kTile * RB / 16; ch += kBlock) {
        *reinterpret_cast<u32x4*>(kt + ch * 16) = *reinterpret_cast<const u32x4*>(s_k + ch * 16);
        u32x4 vv;
        if (KV == kKvFP4) {   // chunk ch: rows r .. r + 15 of columns d and d + 1, two per byte
          const int blk = ch / (D / 2), d = 2 * (ch % (D / 2)), r = 16 * blk;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t* src =
                reinterpret_cast<const uint32_t*>(s_v + (d + (q >> 1)) * VS + r + 8 * (q & 1));
            const uint32_t a = src[0], c = src[1];   // one code per byte
            const uint32_t lo = (a & 0xFu) | ((a >> 4) & 0xF0u) | ((a >> 8) & 0xF00u) | ((a >> 12) & 0xF000u);
            const uint32_t hi = (c & 0xFu) | ((c >> 4) & 0xF0u) | ((c >> 8) & 0xF00u) | ((c >> 12) & 0xF000u);
            vv[q] = lo | (hi << 16);
          }
        } else {              // chunk ch: rows r .. r + 16/E - 1 of column d
          constexpr int E = KV == kKvFP8 ? 1 : 2;
          int d, r;
          v_tile_run(ch * 16, D, E, d, r);
          const uint32_t* src = reinterpret_cast<const uint32_t*>(s_v + d * VS + r * E);
          vv = u32x4{src[0], src[1], src[2], src[3]};
        }
        *reinterpret_cast<u32x4*>(vt + ch * 16) = vv;
      }
    } else if (tid < kTile && s_src[tid] >= 0) {
      atomicOr(p.err, CDA_DEVERR_POOL);
    }
    __syncthreads();   // the next tile reuses s_src and the LDS images
  }
}

// ---------------------------------------------------------------- APPEND

struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, st, sh;        // token t of a chunk at t * st
  const uint8_t* keep;       // [B, M, Hkv]
  int M;                     // tokens appended, one after another
  int W, Hkv, D;
  const int64_t* seg_base;   // contiguous segments
  const int32_t* page_table; // paged store: [nh][max_pages], or NULL
  int max_pages, n_pages;
  const int32_t* seg_cap;
  int32_t* comp_len;
  int32_t* pos;
  uint8_t* ring_keep;
  const float* k_amax;
  const float* v_amax;
  int64_t pool_rows;
  uint8_t* k_pool;
  uint8_t* v_pool;
  int32_t* err;
};

// 8 consecutive K elements of a row: 4 FP4 bytes, 8 FP8 bytes or 8 bf16
// (16 bytes).
template <int KV>
struct Row8 {
  typedef typename std::conditional<KV == kKvFP4, uint32_t,
                                    typename std::conditional<KV == kKvFP8, u32x2, u32x4>::type>::type type;
};

// Workgroup b handles sequence b.  Thread t owns elements [8c, 8c+8) of one
// head's K and V rows (c = t mod D/8).  Straight-line code, two dependent
// round trips: (1) position, segment metadata and its slice of the new
// token; (2) the exiting ring row's keep bit and its slice of that row.
// Then it writes the moved slice (if kept) and the new token's slice into
// the ring row; the old slice was read by the same thread, before.  FP4 V
// elements share bytes with the neighbouring row, so they are written as
// read-modify-writes of their nibble (no other thread writes those bytes:
// a byte's two rows are the moved row or the new row and a row nobody
// writes in this step).  Paged store: the three rows' pages come from the
// page table first (one more round trip); an idle sequence (pos < 0) is
// left as it is.  A chunk of M tokens is appended one token after another,
// with a barrier between them: a later token reads ring rows, ring keep
// bytes and comp_len that an earlier one wrote (same workgroup).
template <int KV>
__global__ __launch_bounds__(kBlock) void append_kernel(AppendParams p) {
  typedef typename std::conditional<KV == kKvBF16, uint16_t, uint8_t>::type elem_t;
  typedef typename Row8<KV>::type krow_t;
  constexpr bool Q = KV != kKvBF16;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int W = p.W, D = p.D;
  const int RB = kv_row_bytes(KV, D);
  const int cpr = D / 8;                       // 8-element chunks per row
  const int P0 = p.pos[b];
  const bool paged = p.page_table != nullptr;
  if (paged && P0 < 0) return;      // idle sequence (uniform over the workgroup)
  elem_t* vp = reinterpret_cast<elem_t*>(p.v_pool);
  for (int tk = 0; tk < p.M; ++tk) {
  const int P = P0 + tk;
  for (int h0 = 0; h0 < p.Hkv; h0 += kBlock / cpr) {
    const int h = h0 + tid / cpr, d0 = (tid % cpr) * 8;
    if (h >= p.Hkv) continue;
    const int64_t i = (int64_t)b * p.Hkv + h;
    const int64_t base = paged ? 0 : p.seg_base[i];
    // pool row of segment row r (paged: through the page table; a missing
    // page gives the out-of-pool row pool_rows)
    const int32_t* pt = paged ? p.page_table + i * p.max_pages : nullptr;
    auto prow = [&](int r) -> int64_t {
      if (!paged) return base + r;
      if (r < 0) return p.pool_rows;
      const int t = r / kTile;
      const int pg = pt[min(t, p.max_pages - 1)];
      return (t < p.max_pages && pg >= 0 && pg < p.n_pages) ? (int64_t)pg * kTile + r % kTile
                                                             : p.pool_rows;
    };
    const int cl0 = p.comp_len[i];
    const int cap = p.seg_cap[i];
    const int kept = p.keep[((int64_t)b * p.M + tk) * p.Hkv + h] != 0;
    const float kinv = Q ? kv_inv_scale<KV>(p.k_amax[i]) : 1.0f;
    const float vinv = Q ? kv_inv_scale<KV>(p.v_amax[i]) : 1.0f;
    const int64_t off = (int64_t)b * p.sb + (int64_t)tk * p.st + (int64_t)h * p.sh + d0;
    const u32x4 kn = *reinterpret_cast<const u32x4*>(p.k + off);
    const u32x4 vn = *reinterpret_cast<const u32x4*>(p.v + off);
    // byte of this thread's K slice in a row
    const int kb0 = KV == kKvFP4 ? d0 / 2 : d0 * (KV == kKvFP8 ? 1 : 2);

    int64_t from = -1, to = -1, nw = -1;
    int cl = cl0, full = 0, bad = 0;
    if (W > 0) {
      const int exit_pos = P - W;
      const int eslot = exit_pos >= 0 ? exit_pos % W : 0;
      const int64_t slot = prow(eslot);
      // the exiting row's keep bit and slice are read whether or not it moves
      // (unconditional loads, clamped into the pool, so they share one trip)
      const bool readable = slot < p.pool_rows;
      const int64_t rslot = readable ? slot : 0;
      const int rk = p.ring_keep[i * W + eslot];
      const krow_t ok = *reinterpret_cast<const krow_t*>(p.k_pool + k_byte(rslot, kb0, RB));
      elem_t ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (KV == kKvFP4)
          ov[j] = (uint8_t)((p.v_pool[v_nib_byte(rslot, d0 + j, D)] >> (4 * (rslot & 1))) & 15u);
        else
          ov[j] = vp[v_elem(rslot, d0 + j, D)];
      }
      if (exit_pos >= 0 && rk) {
        if (cl < cap) {
          from = slot;
          to = prow(W + cl);
          ++cl;
        } else {
          full = 1;
        }
      }
      nw = prow(P % W);
      if (from >= 0 && (!readable || to >= p.pool_rows)) {
        from = -1;
        bad = 1;
      }
      if (from >= 0) {
        *reinterpret_cast<krow_t*>(p.k_pool + k_byte(to, kb0, RB)) = ok;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (KV == kKvFP4)
            nib_store(p.v_pool + v_nib_byte(to, d0 + j, D), (int)(to & 1), ov[j]);
          else
            vp[v_elem(to, d0 + j, D)] = ov[j];
        }
      }
    } else if (kept) {
      if (cl < cap) {
        nw = prow(cl);
        ++cl;
      } else {
        full = 1;
      }
    }
    if (nw >= p.pool_rows) {
      nw = -1;
      bad = 1;
    }
    if (nw >= 0) {
      if (KV == kKvFP4) {
        uint32_t kc = 0;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {   // elements 2 w2 (low nibble), 2 w2 + 1
          kc |= e2m1x2_from_f32(__fmul_rn(__uint_as_float(kn[w2] << 16), kinv),
                                __fmul_rn(__uint_as_float(kn[w2] & 0xFFFF0000u), kinv)) << (8 * w2);
          const uint32_t vb = e2m1x2_from_f32(__fmul_rn(__uint_as_float(vn[w2] << 16), vinv),
                                              __fmul_rn(__uint_as_float(vn[w2] & 0xFFFF0000u), vinv));
          nib_store(p.v_pool + v_nib_byte(nw, d0 + 2 * w2, D), (int)(nw & 1), vb & 15u);
          nib_store(p.v_pool + v_nib_byte(nw, d0 + 2 * w2 + 1, D), (int)(nw & 1), vb >> 4);
        }
        *reinterpret_cast<uint32_t*>(p.k_pool + k_byte(nw, kb0, RB)) = kc;
      } else if (KV == kKvFP8) {
        uint32_t kc[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t kb = (kn[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t vb = (vn[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          kc[j >> 2] |= e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(kb), kinv)) << (8 * (j & 3));
          vp[v_elem(nw, d0 + j, D)] = (elem_t)e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(vb), vinv));
        }
        *reinterpret_cast<u32x2*>(p.k_pool + k_byte(nw, kb0, RB)) = u32x2{kc[0], kc[1]};
      } else {
        *reinterpret_cast<u32x4*>(p.k_pool + k_byte(nw, kb0, RB)) = kn;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          vp[v_elem(nw, d0 + j, D)] = (elem_t)((vn[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
    }
    if (d0 == 0) {
      p.comp_len[i] = cl;
      if (W > 0) p.ring_keep[i * W + P % W] = (uint8_t)kept;
      if (full) atomicOr(p.err, CDA_DEVERR_CAPACITY);
      if (bad) atomicOr(p.err, CDA_DEVERR_POOL);
    }
  }
  __syncthreads();                  // this token's writes before the next token's reads
  }
  if (tid == 0) p.pos[b] = P0 + p.M;   // every thread read pos[b] before the first barrier
}

// ---------------------------------------------------------------- PAGES

// Every page free (stacked so that page 0 is on top), every page-table entry
// -1, every sequence idle with empty segments.  Grid-stride over the largest
// of the arrays.
__global__ __launch_bounds__(kBlock) void page_init_kernel(
    int n_pages, int nh, int max_pages, int B, int W, int32_t* __restrict__ free_pages,
    int32_t* __restrict__ free_top, int32_t* __restrict__ page_table,
    int32_t* __restrict__ comp_len, int32_t* __restrict__ seg_cap, int32_t* __restrict__ pos,
    uint8_t* __restrict__ ring_keep, int32_t* __restrict__ err) {
  const int64_t n_pt = (int64_t)nh * max_pages, n_rk = (int64_t)nh * W;
  const int64_t n = max(max((int64_t)n_pages, n_pt), max(n_rk, (int64_t)max(nh, B)));
  for (int64_t x = (int64_t)blockIdx.x * kBlock + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * kBlock) {
    if (x < n_pages) free_pages[x] = n_pages - 1 - (int32_t)x;
    if (x < n_pt) page_table[x] = -1;
    if (x < n_rk) ring_keep[x] = 0;
    if (x < nh) {
      comp_len[x] = 0;
      seg_cap[x] = 0;
    }
    if (x < B) pos[x] = -1;
    if (x == 0) {
      *free_top = n_pages;
      *err = 0;
    }
  }
}

enum PageOp { kPageAdmit = 0, kPageRefill = 1, kPageRelease = 2 };

struct PageParams {
  int op;
  int nh, Hkv, W, max_pages, n_pages;
  int i0, i1;          // admit, release: segments [i0, i1) (whole sequences)
  int reserve;         // admit, refill: spare compact rows
  int32_t* page_table;
  int32_t* free_pages;
  int32_t* free_top;
  int32_t* seg_cap;
  int32_t* comp_len;
  int32_t* pos;
  uint8_t* ring_keep;
  int32_t* err;
};

__device__ __forceinline__ int pages_for(int64_t rows) { return (int)((rows + kTile - 1) / kTile); }

// Pages held by segment i of a live sequence: seg_cap = 64 * pages - W, and
// a live segment's pages always cover the W ring rows.
__device__ __forceinline__ int pages_held(const PageParams& p, int i) {
  return p.pos[i / p.Hkv] >= 0 ? (p.W + max(p.seg_cap[i], 0)) / kTile : 0;
}

// One workgroup: the page bookkeeping of one operation.  Pages are taken
// from the top of the stack (the k-th taken is free_pages[top - 1 - k]) and returned
// on top of it, in segment order and then row order, by prefix sums over
// the segments: the result does not depend on thread timing.
//   admit   segments [i0, i1) of idle sequences, comp_len from COUNT: each
//           gets pages_for(W + comp_len + reserve) pages, all segments or
//           none (CDA_DEVERR_PAGES: stack short, or a segment over
//           max_pages); its sequences become live with pos = 0.
//   refill  every live segment is topped up to pages_for(W + comp_len +
//           reserve) pages (at most max_pages); a short stack serves the
//           earlier segments first and sets CDA_DEVERR_PAGES.
//   release segments [i0, i1): their pages go back on the stack, the
//           segments are emptied and their sequences become idle (pos = -1).
__global__ __launch_bounds__(kBlock) void page_kernel(PageParams p) {
  __shared__ int smem[4];
  __shared__ int s_top, s_over;
  const int tid = threadIdx.x, mp = p.max_pages, W = p.W;
  if (tid == 0) {
    s_top = min(max(*p.free_top, 0), p.n_pages);   // every stack index stays inside
    s_over = 0;
  }
  __syncthreads();
  const int top = s_top;
  int taken = 0, given = 0;   // pages taken from / returned to the stack (block totals)

  if (p.op == kPageAdmit) {
    // pass 1: the total, and whether a segment needs more than max_pages
    for (int base = p.i0; base < p.i1; base += kBlock) {
      const int i = base + tid;
      int need = 0;
      if (i < p.i1) {
        need = pages_for((int64_t)W + max(p.comp_len[i], 0) + p.reserve);
        if (need > mp) s_over = 1;
      }
      int total;
      block_exclusive_scan(need, &total, smem);
      taken += total;
    }
    __syncthreads();
    const bool ok = s_over == 0 && taken <= top;
    if (!ok) taken = 0;
    // pass 2: the pages, or the idle state
    int k0 = 0;
    for (int base = p.i0; base < p.i1; base += kBlock) {
      const int i = base + tid;
      int need = 0;
      if (i < p.i1) need = pages_for((int64_t)W + max(p.comp_len[i], 0) + p.reserve);
      int total;
      const int ex = block_exclusive_scan(need, &total, smem) + k0;
      k0 += total;
      if (i < p.i1) {
        int32_t* row = p.page_table + (int64_t)i * mp;
        const int got = ok ? need : 0;
        for (int j = 0; j < got; ++j) row[j] = p.free_pages[top - 1 - (ex + j)];
        for (int j = got; j < mp; ++j) row[j] = -1;
        p.seg_cap[i] = ok ? got * kTile - W : 0;
        if (!ok) p.comp_len[i] = 0;
      }
    }
    for (int b = p.i0 / p.Hkv + tid; b < p.i1 / p.Hkv; b += kBlock) p.pos[b] = ok ? 0 : -1;
    if (tid == 0 && !ok) atomicOr(p.err, CDA_DEVERR_PAGES);
  } else if (p.op == kPageRefill) {
    int k0 = 0;
    for (int base = 0; base < p.nh; base += kBlock) {
      const int i = base + tid;
      int cur = 0, add = 0;
      if (i < p.nh && p.pos[i / p.Hkv] >= 0) {
        cur = pages_held(p, i);
        const int want = min(pages_for((int64_t)W + max(p.comp_len[i], 0) + p.reserve), mp);
        add = max(want - cur, 0);
      }
      int total;
      const int ex = block_exclusive_scan(add, &total, smem) + k0;
      k0 += total;
      if (add > 0) {
        const int got = max(0, min(add, top - ex));   // what is left on the stack
        int32_t* row = p.page_table + (int64_t)i * mp;
        for (int j = 0; j < got; ++j) row[cur + j] = p.free_pages[top - 1 - (ex + j)];
        p.seg_cap[i] = (cur + got) * kTile - W;
      }
    }
    taken = min(k0, top);
    if (tid == 0 && k0 > top) atomicOr(p.err, CDA_DEVERR_PAGES);
  } else {   // kPageRelease
    int k0 = 0;
    for (int base = p.i0; base < p.i1; base += kBlock) {
      const int i = base + tid;
      const int cur = i < p.i1 ? min(pages_held(p, i), mp) : 0;
      int total;
      const int ex = block_exclusive_scan(cur, &total, smem) + k0;
      k0 += total;
      if (i < p.i1) {
        int32_t* row = p.page_table + (int64_t)i * mp;
        for (int j = 0; j < cur; ++j) {
          if (top + ex + j < p.n_pages) p.free_pages[top + ex + j] = row[j];
          row[j] = -1;
        }
        p.seg_cap[i] = 0;
        p.comp_len[i] = 0;
        for (int r = 0; r < W; ++r) p.ring_keep[(int64_t)i * W + r] = 0;
      }
    }
    __syncthreads();   // every thread has read pos (pages_held) of the range
    for (int b = p.i0 / p.Hkv + tid; b < p.i1 / p.Hkv; b += kBlock) p.pos[b] = -1;
    given = k0;
  }
  if (tid == 0) *p.free_top = min(top - taken + given, p.n_pages);
}

}  // namespace

namespace {

// The sequences a COUNT / PACK / RELEASE call covers: [b0, b0 + nb).
void seq_range(const cda_kv_cache& c, const cda_compact_args& a, int& b0, int& nb) {
  b0 = a.seq_count > 0 ? a.seq_begin : 0;
  nb = a.seq_count > 0 ? a.seq_count : c.B;
}

PageParams page_params(const cda_kv_cache& c, int op, int b0, int nb, int reserve) {
  PageParams p;
  p.op = op;
  p.nh = c.B * c.Hkv;
  p.Hkv = c.Hkv;
  p.W = c.W;
  p.max_pages = c.max_pages;
  p.n_pages = (int)(c.pool_rows / kTile);
  p.i0 = b0 * c.Hkv;
  p.i1 = (b0 + nb) * c.Hkv;
  p.reserve = reserve;
  p.page_table = c.page_table;
  p.free_pages = c.free_pages;
  p.free_top = c.free_top;
  p.seg_cap = c.seg_cap;
  p.comp_len = c.comp_len;
  p.pos = c.pos;
  p.ring_keep = c.ring_keep;
  p.err = c.err;
  return p;
}

}  // namespace

hipError_t launch_count(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  int b0, nb;
  seq_range(c, a, b0, nb);
  const int nh = c.B * c.Hkv, nr = nb * c.Hkv;
  if (nr > 0) {
    count_kernel<<<nr, kBlock, 0, s>>>(a.keep, a.keep_ld, a.T, c.W, a.reserve, b0 * c.Hkv,
                                       c.comp_len, c.seg_cap, a.dst_out);
  }
  if (c.page_table)
    page_kernel<<<1, kBlock, 0, s>>>(page_params(c, kPageAdmit, b0, nb, a.reserve));
  else
    seg_scan_kernel<<<1, kBlock, 0, s>>>(nh, c.W, c.seg_cap, c.seg_base, c.err);
  return hipGetLastError();
}

hipError_t launch_page_op(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  if (a.op == CDA_OP_PAGE_INIT) {
    const int nh = c.B * c.Hkv;
    const int64_t n = std::max(std::max(c.pool_rows / kTile, (int64_t)nh * c.max_pages),
                               std::max((int64_t)nh * c.W, (int64_t)std::max(nh, c.B)));
    const int grid = (int)std::min<int64_t>(std::max<int64_t>((n + kBlock - 1) / kBlock, 1), 1024);
    page_init_kernel<<<grid, kBlock, 0, s>>>((int)(c.pool_rows / kTile), nh, c.max_pages, c.B,
                                             c.W, c.free_pages, c.free_top, c.page_table,
                                             c.comp_len, c.seg_cap, c.pos, c.ring_keep, c.err);
  } else {
    int b0, nb;
    seq_range(c, a, b0, nb);
    const int op = a.op == CDA_OP_REFILL ? kPageRefill : kPageRelease;
    page_kernel<<<1, kBlock, 0, s>>>(page_params(c, op, b0, nb, a.reserve));
  }
  return hipGetLastError();
}

constexpr int kPackY = 32;   // workgroups per segment of the pack kernel

hipError_t launch_pack(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  int b0, nb;
  seq_range(c, a, b0, nb);
  const int nr = nb * c.Hkv, i0 = b0 * c.Hkv;   // the range's segments
  if (nr == 0) return hipGetLastError();
  const dim3 grid(nr, a.T > 0 ? (a.T + kBlock - 1) / kBlock : 1);
  if (c.kv_dtype != CDA_KV_BF16 && a.scale_mode == 0) {
    amax_zero_kernel<<<(nr + kBlock - 1) / kBlock, kBlock, 0, s>>>(i0, i0 + nr, c.k_amax,
                                                                  c.v_amax);
    amax_kernel<<<grid, kBlock, 0, s>>>(static_cast<const uint16_t*>(a.k),
                                      static_cast<const uint16_t*>(a.v), a.stride_b, a.stride_t,
                                      a.stride_h, a.keep, a.keep_ld, a.T, c.W, c.Hkv, c.D, i0,
                                      c.k_amax, c.v_amax);
  }
  PackParams p;
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.sb = a.stride_b;
  p.st = a.stride_t;
  p.sh = a.stride_h;
  p.keep = a.keep;
  p.keep_ld = a.keep_ld;
  p.T = a.T;
  p.W = c.W;
  p.Hkv = c.Hkv;
  p.D = c.D;
  p.i0 = i0;
  p.seg_base = c.seg_base;
  p.page_table = c.page_table;
  p.seg_cap = c.seg_cap;
  p.max_pages = c.max_pages;
  p.n_pages = (int)(c.pool_rows / kTile);
  p.comp_len = c.comp_len;
  p.pool_rows = c.pool_rows;
  p.k_pool = static_cast<uint8_t*>(c.k_pool);
  p.v_pool = static_cast<uint8_t*>(c.v_pool);
  p.ring_keep = c.ring_keep;
  p.pos = c.pos;
  p.k_amax = c.k_amax;
  p.v_amax = c.v_amax;
  p.err = c.err;
  // tiles of a segment: at most ceil(max(T, W) / 64); workgroups take every
  // kPackY-th of them
  const int max_tiles = (int)((std::max<int64_t>(a.T, c.W) + kTile - 1) / kTile);
  const dim3 pgrid(nr, std::max(1, std::min(max_tiles, kPackY)));
  if (c.kv_dtype == CDA_KV_FP4_E2M1) {
    pack_kernel<kKvFP4, 128><<<pgrid, kBlock, 0, s>>>(p);   // FP4 needs D = 128
  } else if (c.kv_dtype == CDA_KV_FP8_E4M3) {
    if (c.D == 64) pack_kernel<kKvFP8, 64><<<pgrid, kBlock, 0, s>>>(p);
    else pack_kernel<kKvFP8, 128><<<pgrid, kBlock, 0, s>>>(p);
  } else {
    if (c.D == 64) pack_kernel<kKvBF16, 64><<<pgrid, kBlock, 0, s>>>(p);
    else pack_kernel<kKvBF16, 128><<<pgrid, kBlock, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_append(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s, int M) {
  if (c.B * c.Hkv == 0 || M <= 0) return hipGetLastError();
  AppendParams p;
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.sb = a.stride_b;
  p.st = a.stride_t;
  p.sh = a.stride_h;
  p.keep = a.keep;
  p.M = M;
  p.W = c.W;
  p.Hkv = c.Hkv;
  p.D = c.D;
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
  p.pool_rows = c.pool_rows;
  p.k_pool = static_cast<uint8_t*>(c.k_pool);
  p.v_pool = static_cast<uint8_t*>(c.v_pool);
  p.err = c.err;
  if (c.kv_dtype == CDA_KV_FP4_E2M1)
    append_kernel<kKvFP4><<<c.B, kBlock, 0, s>>>(p);
  else if (c.kv_dtype == CDA_KV_FP8_E4M3)
    append_kernel<kKvFP8><<<c.B, kBlock, 0, s>>>(p);
  else
    append_kernel<kKvBF16><<<c.B, kBlock, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace cda
