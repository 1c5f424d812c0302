// Single-token GQA decode attention over the compact KV store, for gfx950.
//
// What is computed (FastDMS page, release and benchmark paragraphs: decode
// over the compact store; PackKV abstract: decompression fused into the
// matrix-vector products): for every sequence b and query head j, softmax
// attention of q[b, j] over the n_i stored rows of its KV head's segment.
//
// Work split.  Each segment's rows [0, n_i) are cut into 64-row tiles, and
// tiles into work units of `tpu` tiles; one workgroup (4 waves) takes one
// unit at a time and each wave one tile at a time.  Every wave derives the
// unit -> (segment, tiles) map itself from pos / comp_len / seg_cap (lane l
// looks at one segment, a wave-wide scan of unit counts finds the segment
// holding the unit), so the host needs no copy of the lengths and no
// workgroup barrier delays the K/V loads.  A segment with one unit writes
// its output directly; otherwise each unit writes an unnormalised partial
// (m, l, o) and counts itself in with an atomic, and the last unit of the
// segment to finish combines all of them with a log-sum-exp merge and resets
// the counter (so the counters are zero between calls).
//
// XCD-local mode.  Workgroup w runs on XCD w mod (number of XCDs) on this
// chip.  When that number divides 8, the units of segment i are given only
// to workgroups w = 8k + (i mod 8), so all of them share one L2: partials
// are plain stores and the merge reads them from that L2.  Workgroup w then
// walks units k = w/8, w/8 + P, ... of its group's segments.  Otherwise
// every workgroup takes one unit of the global list and partials go through
// agent-scope (device-coherent) stores and loads.
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
// and the V scale into the output.  P is split into a high and a low 16-bit
// part (p = hi + lo to ~2^-17) so that the 16-bit P operand adds no visible
// rounding.  All K/V loads of a tile are unconditional (a tile never leaves
// its 64-row-padded segment); rows past the end of the segment are masked
// out of the logits and the values.
#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMergeBatch = 8;   // partials loaded per round trip in the merge
constexpr int kMergeElems = 2;   // outputs per thread merged together
constexpr int kXcdGroups = 8;    // segment groups of the XCD-local mode

struct AttnParams {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t pool_rows;
  const int64_t* seg_base;
  const int32_t* seg_cap;
  const int32_t* comp_len;
  const int32_t* pos;
  const float* k_amax;
  const float* v_amax;
  const uint16_t* q;
  void* out;
  float* lse;
  int32_t* err;
  float* part_o;       // [slots][G][D]
  float* part_ml;      // [slots][G][2]
  int32_t* sem;        // [nh]: units of the segment finished so far (0 between calls)
  int Hkv, G, Hq, W, nh, tpu, out_f32;
  int per_xcd;         // XCD-local mode: workgroups per segment group
  int nxcc;            // XCD-local mode: XCDs of the device (divides 8)
  float sm_scale;
};

__device__ __forceinline__ int units_of(int n, int tpu) {
  const int tiles = (n + kTile - 1) / kTile;
  return max(1, (tiles + tpu - 1) / tpu);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store_out(const AttnParams& p, int64_t idx, float v) {
  if (p.out_f32)
    static_cast<float*>(p.out)[idx] = v;
  else
    static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16_rne(v);
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
// stores; loads that skip the CU's L1); otherwise they are device-coherent
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
__device__ __forceinline__ void store_part2(float* a, float x, float y) {
  if (XL) {
    *reinterpret_cast<float2*>(a) = make_float2(x, y);
  } else {
    __hip_atomic_store(a, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a + 1, y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <bool XL>
__device__ __forceinline__ float load_part1(const float* a) {
  return XL ? __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
            : __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool XL>
__device__ __forceinline__ float2 load_part2(const float* a) {
  return make_float2(load_part1<XL>(a), load_part1<XL>(a + 1));
}
template <bool XL>
__device__ __forceinline__ f32x4 load_part4(const float* a) {
  return f32x4{load_part1<XL>(a), load_part1<XL>(a + 1), load_part1<XL>(a + 2),
               load_part1<XL>(a + 3)};
}

// The unit a workgroup works on: its segment and that segment's metadata.
struct Unit {
  int i, first, U, n;
  long long sb;
  float ks, vs;
};

// Unit k among the segments x0, x0 + xs, x0 + 2xs, ... (in that order, each
// with units_of(n_i) units).  Wave-level: every wave of a workgroup calls it
// with the same arguments and gets the same answer.
template <bool FP8>
__device__ __forceinline__ bool find_unit(const AttnParams& p, int x0, int xs, int k, int lane,
                                          Unit& un) {
  int carry = 0;
  for (int base = 0; x0 + xs * base < p.nh; base += 64) {
    const int hi = x0 + xs * (base + lane);
    int Ui = 0, ni = 0;
    long long sbi = 0;
    float ka = 1.0f, va = 1.0f;
    if (hi < p.nh) {
      const int P = p.pos[hi / p.Hkv];
      const int cap = max(p.seg_cap[hi], 0);
      const int cl = p.comp_len[hi];
      sbi = p.seg_base[hi];
      if (FP8) {
        ka = p.k_amax[hi];
        va = p.v_amax[hi];
      }
      ni = min(p.W, max(P, 0)) + min(max(cl, 0), cap);
      Ui = units_of(ni, p.tpu);
    }
    int x = Ui;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const int ex = carry + x - Ui;
    const unsigned long long mine = __ballot(hi < p.nh && k >= ex && k < ex + Ui);
    if (mine) {
      const int src = __ffsll((long long)mine) - 1;
      un.i = x0 + xs * (base + src);
      un.first = __shfl(ex, src, 64);
      un.U = __shfl(Ui, src, 64);
      un.n = __shfl(ni, src, 64);
      un.sb = __shfl(sbi, src, 64);
      un.ks = fp8_scale(__shfl(ka, src, 64));
      un.vs = fp8_scale(__shfl(va, src, 64));
      return true;
    }
    carry += __shfl(x, 63, 64);
  }
  return false;
}

// Mask of the bytes of dword w (bytes 4w .. 4w+3) that lie below `lim`.
__device__ __forceinline__ uint32_t bytes_below(int lim, int w) {
  const int k = lim - 4 * w;
  return k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
}

template <bool FP8, int D, bool XL, int NW>
__global__ __launch_bounds__(64 * NW) void attn_kernel(AttnParams p) {
  constexpr int NTH = 64 * NW;              // threads of the workgroup
  constexpr int E = FP8 ? 1 : 2;            // bytes per stored element
  constexpr int NK = D / 32;                // MFMA k-steps of q.K
  constexpr int NT = D / 16;                // 16-wide d tiles of the output
  constexpr int KL = FP8 ? D / 64 : D / 32; // 16-byte K loads per (lane, token group)
  constexpr int VL = FP8 ? 1 : 2;           // 16-byte V loads per (lane, d tile)

  __shared__ int s_last;
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ f32x4 s_o[NW][16][D / 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15, kg = lane >> 4;
  const int w = blockIdx.x;
  const int grp = XL ? (w & (kXcdGroups - 1)) : 0;
  if (XL && tid == 0) {
    // the XCD-local merge relies on workgroup w running on XCD w mod nxcc
    const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;   // HW_REG_XCC_ID
    if (xcc != w % p.nxcc) atomicOr(p.err, CDA_DEVERR_XCD);
  }

  for (int k = XL ? (w / kXcdGroups) : w;; k += p.per_xcd) {
    Unit un;
    if (!find_unit<FP8>(p, grp, XL ? kXcdGroups : 1, k, lane, un)) return;
    const int i = un.i, U = un.U, n = un.n;
    const int b = i / p.Hkv, h = i - b * p.Hkv;
    const int G = p.G;
    const int64_t sb = un.sb;
    const int64_t in_pool = p.pool_rows - sb;
    const int ntiles = (n + kTile - 1) / kTile;
    const int t_begin = (k - un.first) * p.tpu;
    const int t_end = min(t_begin + p.tpu, ntiles);
    const int slot = XL ? k * kXcdGroups + grp : k;   // this unit's partial

    // ---- Q^T operand: lane (g, kg) holds 8 d-values of query row g per k-step
    bf16x8 qop[NK];
    {
      const bool have = g < G;
      const uint16_t* qrow = p.q + (int64_t)(b * p.Hq + h * G + (have ? g : 0)) * D;
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const int d0 = FP8 ? (64 * (s >> 1) + 16 * kg + 8 * (s & 1)) : (32 * s + 8 * kg);
        u32x4 v = have ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
        qop[s] = as_bf16x8(v);
      }
    }
    const float c1 = p.sm_scale * kLog2e * (FP8 ? un.ks : 1.0f);

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

    bool first_tile = true;
    for (int t = t_begin + wave; t < t_end; t += NW) {
      const int r0 = t * kTile;
      const int valid = (int)min((int64_t)min(kTile, n - r0), in_pool - r0);
      if (valid <= 0) break;
      const bool full = valid == kTile;
      const uint8_t* ktile = p.k_pool + (sb + r0) * (int64_t)(D * E);
      const uint8_t* vtile = p.v_pool + (sb + r0) * (int64_t)(D * E);

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
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < VL; ++j)
          vr[nt][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              vtile + ((16 * nt + g) * kTile + 16 * kg + 8 * j) * E));

      // -- S^T = K . Q^T, 16 tokens per MFMA row block
      f32x4 s[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        s[m] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < NK; ++st) {
          bf16x8 a;
          if (FP8) {
            const u32x4 v = kr[m][st >> 1];
            a = (st & 1) ? fp8x8_to_bf16x8(v[2], v[3]) : fp8x8_to_bf16x8(v[0], v[1]);
          } else {
            a = as_bf16x8(kr[m][st]);
          }
          s[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[st], s[m], 0, 0, 0);
        }
      }

      // -- online softmax over this tile; lane (g, kg) owns tokens 16kg + 4m + r
      float z[4][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[m][r] = s[m][r] * c1;
      if (!full) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kg + 4 * m + r >= valid) z[m][r] = -INFINITY;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, z[m][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      if (!first_tile) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
      }
      float psum = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[m][r] = __builtin_amdgcn_exp2f(z[m][r] - m_new);
          psum += z[m][r];
        }
      l_run += psum;
      m_run = m_new;

      // -- rows past the segment end: zero their V bytes (P is 0 there, but
      //    the bytes may not be finite values)
      if (!full) {
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

      // -- O^T += V^T . P^T, two MFMAs (8 tokens per lane each) per d tile
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if (FP8) {
          f16x8 phi, plo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = z[2 * hh + (e >> 2)][e & 3];
            const _Float16 hi = (_Float16)pv;
            phi[e] = hi;
            plo[e] = (_Float16)(pv - (float)hi);
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const u32x4 v = vr[nt][0];
            const f16x8 a = hh ? fp8x8_to_f16x8(v[2], v[3]) : fp8x8_to_f16x8(v[0], v[1]);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, phi, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, plo, acc[nt], 0, 0, 0);
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

    // ---- combine the 4 waves of the workgroup
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (kg == 0) {
      s_m[wave][g] = m_run;
      s_l[wave][g] = l_run;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s_o[wave][g][(16 * nt + 4 * kg) / 4] = acc[nt];
    __syncthreads();

    const float sv = FP8 ? un.vs : 1.0f;
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
      if (U == 1) {
        write_final4(p, b, h, gg, d4, D, M, L, O, sv);
      } else {
        store_part4<XL>(p.part_o + ((int64_t)slot * G + gg) * D + 4 * d4, O);
        if (d4 == 0) store_part2<XL>(p.part_ml + ((int64_t)slot * G + gg) * 2, M, L);
      }
    }

    if (U > 1) {
      // ---- split segment: the last of its units to get here merges the
      // partials.  Every wave waits for its partial stores to complete before
      // the workgroup counts itself in.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const int prev =
            __hip_atomic_fetch_add(p.sem + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == U - 1;
        if (prev == U - 1)
          __hip_atomic_store(p.sem + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_last) {
        // each thread merges 4 consecutive outputs of one query row; the
        // (m, l) and o loads of a batch of kMergeBatch units go out together
        for (int e = tid; e < G * (D / 4); e += NTH) {
          const int gg = e / (D / 4), d4 = e - gg * (D / 4);
          float M = -INFINITY, L = 0.0f;
          f32x4 O = f32x4{0, 0, 0, 0};
          for (int k0 = 0; k0 < U; k0 += kMergeBatch) {
            float2 ml[kMergeBatch];
            f32x4 ov[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {   // unconditional loads, clamped index
              const int ku = un.first + min(k0 + j, U - 1);
              const int64_t sl = (int64_t)(XL ? ku * kXcdGroups + grp : ku) * G + gg;
              ml[j] = load_part2<XL>(p.part_ml + sl * 2);
              ov[j] = load_part4<XL>(p.part_o + sl * D + 4 * d4);
            }
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j)
              if (k0 + j >= U) ml[j].x = -INFINITY;
            float Mb = M;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, ml[j].x);
            if (Mb == -INFINITY) continue;
            const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
            O *= a;
            L *= a;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
              const float f = (ml[j].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml[j].x - Mb);
              O += f * ov[j];
              L += f * ml[j].y;
            }
            M = Mb;
          }
          write_final4(p, b, h, gg, d4, D, M, L, O, sv);
        }
      }
    }
    if (!XL) return;
    __syncthreads();   // the LDS of this unit is reused by the next one
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

}  // namespace

int64_t attn_max_units(const cda_kv_cache& c, int tpu) {
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return nh + c.pool_rows / ((int64_t)kTile * tpu);
}

// Partial slots: an XCD-local slot is 8k + group with k below the units of
// the group (at most all units), so 8 x the unit bound covers both modes.
size_t attn_workspace_bytes(const cda_kv_cache& c, int G, int tpu) {
  const int64_t slots = kXcdGroups * attn_max_units(c, tpu);
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return align256((size_t)nh * 4) + align256((size_t)slots * G * 2 * 4) +
         align256((size_t)slots * G * c.D * 4);
}

hipError_t launch_attn(const cda_kv_cache& c, const void* q, int Hq, float sm_scale, void* out,
                       int out_f32, float* lse, int tpu, void* workspace, hipStream_t s) {
  const int nh = c.B * c.Hkv;
  if (nh == 0) return hipGetLastError();
  const int G = Hq / c.Hkv;
  const int64_t units = attn_max_units(c, tpu);
  const int64_t slots = kXcdGroups * units;
  AttnParams p;
  p.k_pool = static_cast<const uint8_t*>(c.k_pool);
  p.v_pool = static_cast<const uint8_t*>(c.v_pool);
  p.pool_rows = c.pool_rows;
  p.seg_base = c.seg_base;
  p.seg_cap = c.seg_cap;
  p.comp_len = c.comp_len;
  p.pos = c.pos;
  p.k_amax = c.k_amax;
  p.v_amax = c.v_amax;
  p.q = static_cast<const uint16_t*>(q);
  p.out = out;
  p.lse = lse;
  p.err = c.err;
  // workspace: [sem: nh int32][part_ml: slots*G*2 f32][part_o: slots*G*D f32]
  char* ws = static_cast<char*>(workspace);
  p.sem = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)nh * 4);
  p.part_ml = reinterpret_cast<float*>(ws);
  ws += align256((size_t)slots * G * 2 * 4);
  p.part_o = reinterpret_cast<float*>(ws);
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
  p.nxcc = xl ? nx : 1;
  // XCD-local: 8 groups of per_xcd workgroups, a quarter more than an even
  // share of the unit bound; a group with more units loops over them.
  p.per_xcd = xl ? (int)((units * 5 / 4 + kXcdGroups - 1) / kXcdGroups) : 0;
  const dim3 grid((unsigned)(xl ? (int64_t)p.per_xcd * kXcdGroups : units));
  const bool fp8 = c.kv_dtype == CDA_KV_FP8_E4M3;
  const int nw = tpu >= 8 ? 8 : 4;   // waves per workgroup: one tile each per pass
#define CDA_LAUNCH_ATTN(F, DD, X)                                                   \
  (nw == 8 ? attn_kernel<F, DD, X, 8><<<grid, 512, 0, s>>>(p)                       \
           : attn_kernel<F, DD, X, 4><<<grid, 256, 0, s>>>(p))
  if (fp8) {
    if (c.D == 64) {
      if (xl) CDA_LAUNCH_ATTN(true, 64, true); else CDA_LAUNCH_ATTN(true, 64, false);
    } else {
      if (xl) CDA_LAUNCH_ATTN(true, 128, true); else CDA_LAUNCH_ATTN(true, 128, false);
    }
  } else {
    if (c.D == 64) {
      if (xl) CDA_LAUNCH_ATTN(false, 64, true); else CDA_LAUNCH_ATTN(false, 64, false);
    } else {
      if (xl) CDA_LAUNCH_ATTN(false, 128, true); else CDA_LAUNCH_ATTN(false, 128, false);
    }
  }
#undef CDA_LAUNCH_ATTN
  return hipGetLastError();
}

}  // namespace cda
