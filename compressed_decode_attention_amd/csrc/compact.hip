// Prefill compaction and decode-time append of the compact KV store
// (FastDMS page, release paragraph: a compact store that physically
// reclaims evicted slots; memory-table paragraph: cache + staging window).
//
//   count_kernel     keep mask -> per-segment kept count, optional dst map
//   seg_scan_kernel  aligned segment sizes -> seg_base (exclusive prefix sum)
//   amax_kernel      per-segment absmax of the stored prefill K and V (FP8)
//   pack_kernel      stored prefill rows -> pool rows (BF16 copy / FP8 encode)
//   append_kernel    one decode step: ring exit -> compact tail, new token -> ring
//
// All of these run once per prefill or move at most one row per segment per
// step; the decode hot loop is the attention kernel.
#include <type_traits>

#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

// ---------------------------------------------------------------- COUNT

__global__ __launch_bounds__(kBlock) void count_kernel(
    const uint8_t* __restrict__ keep, int64_t keep_ld, int T, int W, int reserve,
    int32_t* __restrict__ comp_len, int32_t* __restrict__ seg_cap,
    int32_t* __restrict__ dst_out) {
  __shared__ int smem[4];
  const int i = blockIdx.x, tid = threadIdx.x;
  const uint8_t* row = keep + (int64_t)i * keep_ld;
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
      int32_t* d = dst_out + (int64_t)i * T;
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

// Segments whose attention work is spread over the 8 XCD groups by size.
constexpr int kBalanceMax = 512;

// seg_base by a prefix sum of the aligned segment sizes; then, if asked, the
// group map: segments ranked by size in 64-row tiles (larger first, ties by
// index) and dealt to the 8 groups in snake order (0..7, 7..0, ...), so
// that every group gets a near-equal share of rows.
__global__ __launch_bounds__(kBlock) void seg_scan_kernel(
    int nh, int W, const int32_t* __restrict__ seg_cap, int64_t* __restrict__ seg_base,
    int32_t* __restrict__ err, uint8_t* __restrict__ seg_group) {
  __shared__ long long smem[4];
  __shared__ int s_tiles[kBalanceMax];
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
  if (seg_group) {
    if (nh <= kBalanceMax) {
      for (int i = threadIdx.x; i < nh; i += kBlock)
        s_tiles[i] = (int)(((long long)W + seg_cap[i] + kTile - 1) / kTile);
      __syncthreads();
      for (int i = threadIdx.x; i < nh; i += kBlock) {
        const int wi = s_tiles[i];
        int rank = 0;
        for (int j = 0; j < nh; ++j) {
          const int wj = s_tiles[j];
          rank += (wj > wi) || (wj == wi && j < i);
        }
        const int round = rank >> 3, slot = rank & 7;
        seg_group[i] = (uint8_t)((round & 1) ? 7 - slot : slot);
      }
    } else {
      for (int i = threadIdx.x; i < nh; i += kBlock) seg_group[i] = (uint8_t)(i & 7);
    }
  }
}

// ---------------------------------------------------------------- PACK

// |x| of a bf16 as the upper half of a binary32 bit pattern; unsigned
// comparison of these orders magnitudes, and any NaN compares largest.
__device__ __forceinline__ uint32_t abs_bits(uint32_t word, int half) {
  return ((word >> (16 * half)) & 0x7FFFu) << 16;
}

__global__ void amax_zero_kernel(int nh, float* __restrict__ k_amax, float* __restrict__ v_amax) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nh) {
    k_amax[i] = 0.0f;
    v_amax[i] = 0.0f;
  }
}

// Workgroup (segment i, chunk c): absmax of K and V over the stored prefill
// rows of positions [256c, 256c+256), folded into k_amax / v_amax with an
// unsigned atomic max on the magnitude bit patterns.
__global__ __launch_bounds__(kBlock) void amax_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t sb, int64_t st,
    int64_t sh, const uint8_t* __restrict__ keep, int64_t keep_ld, int T, int W, int Hkv,
    int D, float* __restrict__ k_amax, float* __restrict__ v_amax) {
  __shared__ int smem[4];
  __shared__ int s_pos[kBlock];
  __shared__ uint32_t red[2][kBlock / 64];
  const int i = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int b = i / Hkv, h = i - b * Hkv;
  const uint8_t* krow = keep + (int64_t)i * keep_ld;
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
  const int64_t* seg_base;
  int64_t pool_rows;
  uint8_t* k_pool;
  uint8_t* v_pool;
  uint8_t* ring_keep;
  int32_t* pos;
  const float* k_amax;
  const float* v_amax;
  int32_t* err;
};

// Byte offset of element (row, d) in a V pool of column-major 64-row tiles.
__device__ __forceinline__ int64_t v_elem(int64_t row, int d, int D) {
  return (row / kTile) * kTile * D + (int64_t)d * kTile + (row % kTile);
}

// Store 8 consecutive elements (d0 .. d0+7) of one row: K row-major, V into
// its column-major tile; FP8 encodes x * inv.
template <bool FP8>
__device__ __forceinline__ void store_row8(uint8_t* k_pool, uint8_t* v_pool, int64_t r, int d0,
                                           int D, u32x4 kin, u32x4 vin, float kinv, float vinv) {
  if (FP8) {
    uint32_t kc[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t kb = (kin[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t vb = (vin[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      kc[j >> 2] |= e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(kb), kinv)) << (8 * (j & 3));
      v_pool[v_elem(r, d0 + j, D)] = (uint8_t)e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(vb), vinv));
    }
    *reinterpret_cast<u32x2*>(k_pool + k_elem8(r, d0, D, 1)) = u32x2{kc[0], kc[1]};
  } else {
    *reinterpret_cast<u32x4*>(k_pool + k_elem8(r, d0, D, 2)) = kin;
    uint16_t* vp = reinterpret_cast<uint16_t*>(v_pool);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vp[v_elem(r, d0 + j, D)] = (uint16_t)((vin[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
  }
}

// Workgroup (segment i, chunk c) handles prefill positions [256c, 256c+256).
template <bool FP8>
__global__ __launch_bounds__(kBlock) void pack_kernel(PackParams p) {
  constexpr int kPre = 32;   // keep bytes per thread of the prefix count
  __shared__ int smem[4];
  __shared__ int s_pos[kBlock], s_dst[kBlock];
  const int i = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  const int T = p.T, W = p.W, D = p.D;
  const uint8_t* row = p.keep + (int64_t)i * p.keep_ld;
  const int ncand = T - W > 0 ? T - W : 0;
  const int pp = c * kBlock + tid;

  // kept older positions before this chunk (up to 8192 bytes per pass, one
  // round trip), and this thread's own keep byte
  const int lim = min(c * kBlock, ncand);
  const int own = (pp < ncand) ? row[pp] : 0;
  int before = 0;
  for (int q0 = tid * kPre; q0 < lim; q0 += kBlock * kPre) {
    uint8_t kb[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) kb[j] = row[min(q0 + j, lim - 1)];
#pragma unroll
    for (int j = 0; j < kPre; ++j) before += (q0 + j < lim) && kb[j] != 0;
  }
  before = block_sum(before, smem);

  const int flag = (pp < ncand) && own != 0;
  int dummy;
  const int rank = block_exclusive_scan(flag, &dummy, smem);
  int stored = 0, dst = -1;
  if (pp < T) {
    if (pp >= ncand) {
      dst = pp % W;
      stored = 1;
    } else if (flag) {
      dst = W + before + rank;
      stored = 1;
    }
  }
  if (stored && dst < W) p.ring_keep[(int64_t)i * W + dst] = row[pp] != 0;
  if (c == 0) {
    for (int r = T + tid; r < W; r += kBlock) p.ring_keep[(int64_t)i * W + r] = 0;
    if (h == 0 && tid == 0) p.pos[b] = T;
  }
  int nst;
  const int slot = block_exclusive_scan(stored, &nst, smem);
  if (stored) {
    s_pos[slot] = pp;
    s_dst[slot] = dst;
  }
  __syncthreads();

  float kinv = 1.0f, vinv = 1.0f;
  if (FP8) {
    kinv = fp8_inv_scale(p.k_amax[i]);
    vinv = fp8_inv_scale(p.v_amax[i]);
  }
  const int64_t base = p.seg_base[i];
  const int lpr = D / 8;
  const int rows_per_pass = kBlock / lpr;
  const int d0 = (tid % lpr) * 8;
  for (int e0 = tid / lpr; e0 < nst; e0 += 4 * rows_per_pass) {
    u32x4 kin[4], vin[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = min(e0 + j * rows_per_pass, nst - 1);
      const int64_t off = (int64_t)b * p.sb + (int64_t)s_pos[e] * p.st + (int64_t)h * p.sh + d0;
      kin[j] = *reinterpret_cast<const u32x4*>(p.k + off);
      vin[j] = *reinterpret_cast<const u32x4*>(p.v + off);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * rows_per_pass;
      if (e >= nst) continue;
      const int64_t r = base + s_dst[e];
      if (r < 0 || r >= p.pool_rows) {
        if (d0 == 0) atomicOr(p.err, CDA_DEVERR_POOL);
        continue;
      }
      store_row8<FP8>(p.k_pool, p.v_pool, r, d0, D, kin[j], vin[j], kinv, vinv);
    }
  }
}

// ---------------------------------------------------------------- APPEND

struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, sh;
  const uint8_t* keep;
  int W, Hkv, D;
  const int64_t* seg_base;
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

// 8 consecutive K elements of a row (8 FP8 bytes or 8 bf16 = 16 bytes).
template <bool FP8>
struct Row8 {
  typedef typename std::conditional<FP8, u32x2, u32x4>::type type;
};

// Workgroup b handles sequence b.  Thread t owns elements [8c, 8c+8) of one
// head's K and V rows (c = t mod D/8).  Straight-line code, two dependent
// round trips: (1) position, segment metadata and its slice of the new
// token; (2) the exiting ring row's keep bit and its slice of that row.
// Then it writes the moved slice (if kept) and the new token's slice into
// the ring row; the old slice was read by the same thread, before.
template <bool FP8>
__global__ __launch_bounds__(kBlock) void append_kernel(AppendParams p) {
  typedef typename std::conditional<FP8, uint8_t, uint16_t>::type elem_t;
  typedef typename Row8<FP8>::type krow_t;
  constexpr int E = FP8 ? 1 : 2;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int W = p.W, D = p.D;
  const int cpr = D / 8;                       // 8-element chunks per row
  const int P = p.pos[b];
  elem_t* vp = reinterpret_cast<elem_t*>(p.v_pool);
  for (int h0 = 0; h0 < p.Hkv; h0 += kBlock / cpr) {
    const int h = h0 + tid / cpr, d0 = (tid % cpr) * 8;
    if (h >= p.Hkv) continue;
    const int64_t i = (int64_t)b * p.Hkv + h;
    const int64_t base = p.seg_base[i];
    const int cl0 = p.comp_len[i];
    const int cap = p.seg_cap[i];
    const int kept = p.keep[i] != 0;
    const float kinv = FP8 ? fp8_inv_scale(p.k_amax[i]) : 1.0f;
    const float vinv = FP8 ? fp8_inv_scale(p.v_amax[i]) : 1.0f;
    const int64_t off = (int64_t)b * p.sb + (int64_t)h * p.sh + d0;
    const u32x4 kn = *reinterpret_cast<const u32x4*>(p.k + off);
    const u32x4 vn = *reinterpret_cast<const u32x4*>(p.v + off);

    int64_t from = -1, to = -1, nw = -1;
    int cl = cl0, full = 0, bad = 0;
    if (W > 0) {
      const int exit_pos = P - W;
      const int eslot = exit_pos >= 0 ? exit_pos % W : 0;
      const int64_t slot = base + eslot;
      // the exiting row's keep bit and slice are read whether or not it moves
      // (unconditional loads, clamped into the pool, so they share one trip)
      const bool readable = slot < p.pool_rows;
      const int64_t rslot = readable ? slot : 0;
      const int rk = p.ring_keep[i * W + eslot];
      const krow_t ok = *reinterpret_cast<const krow_t*>(p.k_pool + k_elem8(rslot, d0, D, E));
      elem_t ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ov[j] = vp[v_elem(rslot, d0 + j, D)];
      if (exit_pos >= 0 && rk) {
        if (cl < cap) {
          from = slot;
          to = base + W + cl;
          ++cl;
        } else {
          full = 1;
        }
      }
      nw = base + P % W;
      if (from >= 0 && (!readable || to >= p.pool_rows)) {
        from = -1;
        bad = 1;
      }
      if (from >= 0) {
        *reinterpret_cast<krow_t*>(p.k_pool + k_elem8(to, d0, D, E)) = ok;
#pragma unroll
        for (int j = 0; j < 8; ++j) vp[v_elem(to, d0 + j, D)] = ov[j];
      }
    } else if (kept) {
      if (cl < cap) {
        nw = base + cl;
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
      if (FP8) {
        uint32_t kc[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t kb = (kn[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t vb = (vn[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          kc[j >> 2] |= e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(kb), kinv)) << (8 * (j & 3));
          vp[v_elem(nw, d0 + j, D)] = (elem_t)e4m3_from_f32(__fmul_rn(bf16_bits_to_f32(vb), vinv));
        }
        *reinterpret_cast<u32x2*>(p.k_pool + k_elem8(nw, d0, D, 1)) = u32x2{kc[0], kc[1]};
      } else {
        *reinterpret_cast<u32x4*>(p.k_pool + k_elem8(nw, d0, D, 2)) = kn;
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
  __syncthreads();                  // every thread has read pos[b]
  if (tid == 0) p.pos[b] = P + 1;
}

}  // namespace

hipError_t launch_count(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  const int nh = c.B * c.Hkv;
  if (nh > 0) {
    count_kernel<<<nh, kBlock, 0, s>>>(a.keep, a.keep_ld, a.T, c.W, a.reserve, c.comp_len,
                                       c.seg_cap, a.dst_out);
  }
  seg_scan_kernel<<<1, kBlock, 0, s>>>(nh, c.W, c.seg_cap, c.seg_base, c.err, c.seg_group);
  return hipGetLastError();
}

hipError_t launch_pack(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  const int nh = c.B * c.Hkv;
  if (nh == 0) return hipGetLastError();
  const bool fp8 = c.kv_dtype == CDA_KV_FP8_E4M3;
  const dim3 grid(nh, a.T > 0 ? (a.T + kBlock - 1) / kBlock : 1);
  if (fp8 && a.scale_mode == 0) {
    amax_zero_kernel<<<(nh + kBlock - 1) / kBlock, kBlock, 0, s>>>(nh, c.k_amax, c.v_amax);
    amax_kernel<<<grid, kBlock, 0, s>>>(static_cast<const uint16_t*>(a.k),
                                      static_cast<const uint16_t*>(a.v), a.stride_b, a.stride_t,
                                      a.stride_h, a.keep, a.keep_ld, a.T, c.W, c.Hkv, c.D,
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
  p.seg_base = c.seg_base;
  p.pool_rows = c.pool_rows;
  p.k_pool = static_cast<uint8_t*>(c.k_pool);
  p.v_pool = static_cast<uint8_t*>(c.v_pool);
  p.ring_keep = c.ring_keep;
  p.pos = c.pos;
  p.k_amax = c.k_amax;
  p.v_amax = c.v_amax;
  p.err = c.err;
  if (fp8)
    pack_kernel<true><<<grid, kBlock, 0, s>>>(p);
  else
    pack_kernel<false><<<grid, kBlock, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_append(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s) {
  if (c.B * c.Hkv == 0) return hipGetLastError();
  AppendParams p;
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.sb = a.stride_b;
  p.sh = a.stride_h;
  p.keep = a.keep;
  p.W = c.W;
  p.Hkv = c.Hkv;
  p.D = c.D;
  p.seg_base = c.seg_base;
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
  if (c.kv_dtype == CDA_KV_FP8_E4M3)
    append_kernel<true><<<c.B, kBlock, 0, s>>>(p);
  else
    append_kernel<false><<<c.B, kBlock, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace cda
