// Single-token GQA decode attention over the compact KV store, for gfx950.
//
// What is computed (FastDMS page, release and benchmark paragraphs: decode
// over the compact store; PackKV abstract: decompression fused into the
// matrix-vector products): for every sequence b and query head j, softmax
// attention of q[b, j] over the n_i stored rows of its KV head's segment.
//
// Work split.  Each segment's rows [0, n_i) are cut into 64-row tiles, and
// tiles into work units of `tpu` tiles; one workgroup (4 waves) takes one
// unit and each wave one tile at a time.  Every workgroup derives the unit
// -> (segment, tiles) map itself from pos / comp_len / seg_cap, so the host
// needs no copy of the lengths; all per-segment metadata it needs is read in
// that one pass, so the K/V loads start after a single dependent round trip.
// A segment with one unit writes its output directly; otherwise each unit
// writes an unnormalised partial (m, l, o), counts itself in with a
// device-scope atomic, and the last unit of the segment to finish combines
// all of them with a log-sum-exp merge and resets the counter (so the
// counters are zero between calls).
//
// Inside a wave, the G query rows of the KV head (G <= 16) are the N = 16
// columns of two MFMA products per tile:
//   S^T[token][g] = K_tile[token][:] . Q^T[:][g]     v_mfma_f32_16x16x32_bf16
//   O^T[d][g]    += V^T[d][token] . P^T[token][g]    v_mfma_f32_16x16x32_{f16,bf16}
// K is stored in 64-row tiles permuted so that each 64-lane load of the S
// operand is 1 KB of consecutive bytes; V is stored in 64-row column-major
// tiles, so the O operand is 16-byte loads of 8 or 16 consecutive tokens of
// one column.  Tokens are assigned to MFMA
// rows so that the S accumulator of each lane holds exactly the 16 tokens
// that lane needs for its P operand, so P never moves between lanes.  FP8
// codes are converted to bf16 (K) or f16 (V) in registers, exactly; the K
// scale is folded into the logit scale and the V scale into the output.
// P is split into a high and a low 16-bit part (p = hi + lo to ~2^-17) so
// that the 16-bit P operand adds no visible rounding.
#include "cda_device.h"
#include "cda_launch.h"

namespace cda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMergeBatch = 8;   // partials loaded per round trip in the merge

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
  float* part_o;       // [units][G][D]
  float* part_ml;      // [units][G][2]
  int32_t* sem;        // [nh]: units of the segment finished so far (0 between calls)
  int Hkv, G, Hq, W, nh, tpu, out_f32;
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

// Final output of query row gg of segment (b, h) from its merged state.
__device__ __forceinline__ void write_final(const AttnParams& p, int b, int h, int gg, int d,
                                            int D, float M, float L, float O, float sv) {
  const int64_t row = (int64_t)b * p.Hq + h * p.G + gg;
  store_out(p, row * D + d, L > 0.0f ? O / L * sv : 0.0f);
  if (d == 0 && p.lse) p.lse[row] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <bool FP8, int D>
__global__ __launch_bounds__(kBlock) void attn_kernel(AttnParams p) {
  constexpr int E = FP8 ? 1 : 2;            // bytes per stored element
  constexpr int NK = D / 32;                // MFMA k-steps of q.K
  constexpr int NT = D / 16;                // 16-wide d tiles of the output
  constexpr int KL = FP8 ? D / 64 : D / 32; // 16-byte K loads per (lane, token group)
  constexpr int VL = FP8 ? 1 : 2;           // 16-byte V loads per (lane, d tile)

  __shared__ int s_last;
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ f32x4 s_o[4][16][D / 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;

  // ---- which segment and which tiles this workgroup covers.  Every wave
  //      works this out by itself (lane l looks at segment base + l; a
  //      wave-wide scan of unit counts finds the segment holding unit u), so
  //      no workgroup barrier delays the K/V loads; all the metadata the
  //      kernel needs about the segment is read in this one pass.
  int i = -1, first = 0, U = 1, n = 0;
  long long sb = 0;
  float ks = 1.0f, vs = 1.0f;
  int carry = 0;
  for (int base = 0; base < p.nh && i < 0; base += 64) {
    const int hi = base + lane;
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
    const unsigned long long mine = __ballot(hi < p.nh && u >= ex && u < ex + Ui);
    if (mine) {
      const int src = __ffsll((long long)mine) - 1;
      i = base + src;
      first = __shfl(ex, src, 64);
      U = __shfl(Ui, src, 64);
      n = __shfl(ni, src, 64);
      sb = __shfl(sbi, src, 64);
      ks = fp8_scale(__shfl(ka, src, 64));
      vs = fp8_scale(__shfl(va, src, 64));
    }
    carry += __shfl(x, 63, 64);
  }
  if (i < 0) return;        // the same for every wave of the workgroup
  const int b = i / p.Hkv, h = i - b * p.Hkv;
  const int G = p.G;
  const int64_t in_pool = p.pool_rows - sb;
  const int ntiles = (n + kTile - 1) / kTile;
  const int t_begin = (u - first) * p.tpu;
  const int t_end = min(t_begin + p.tpu, ntiles);

  const int g = lane & 15, kg = lane >> 4;

  // ---- Q^T operand: lane (g, kg) holds 8 d-values of query row g per k-step
  bf16x8 qop[NK];
  {
    const bool have = g < G;
    const uint16_t* qrow = p.q + (int64_t)(b * p.Hq + h * G + (have ? g : 0)) * D;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int d0 = FP8 ? (64 * (s >> 1) + 16 * kg + 8 * (s & 1)) : (32 * s + 8 * kg);
      u32x4 w = have ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
      qop[s] = as_bf16x8(w);
    }
  }
  const float c1 = p.sm_scale * kLog2e * (FP8 ? ks : 1.0f);

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

  for (int t = t_begin + wave; t < t_end; t += 4) {
    const int r0 = t * kTile;
    const int valid = (int)min((int64_t)min(kTile, n - r0), in_pool - r0);
    if (valid <= 0) break;
    const uint8_t* ktile = p.k_pool + (sb + r0) * (int64_t)(D * E);
    const uint8_t* vtile = p.v_pool + (sb + r0) * (int64_t)(D * E);

    // -- loads: K rows for the 4 token groups (each instruction 1 KB of the
    //    permuted K tile), V columns for the NT d tiles
    u32x4 kr[4][KL];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 16 * (g >> 2) + 4 * m + (g & 3);
#pragma unroll
      for (int j = 0; j < KL; ++j)
        kr[m][j] = row < valid
                       ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                             ktile + ((m * KL + j) << 10) + lane * 16))
                       : u32x4{0, 0, 0, 0};
    }
    u32x4 vr[NT][VL];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int d = 16 * nt + g;
#pragma unroll
      for (int j = 0; j < VL; ++j) {
        const int tok0 = 16 * kg + 8 * j;
        vr[nt][j] = tok0 < valid
                        ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                              vtile + (d * kTile + tok0) * E))
                        : u32x4{0, 0, 0, 0};
      }
    }

    // -- S^T = K . Q^T, 16 tokens per MFMA row block
    f32x4 s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[m] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < NK; ++st) {
        bf16x8 a;
        if (FP8) {
          const u32x4 w = kr[m][st >> 1];
          a = (st & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
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
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * kg + 4 * m + r;
        z[m][r] = tok < valid ? s[m][r] * c1 : -INFINITY;
        tmax = fmaxf(tmax, z[m][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[m][r] = exp2f(z[m][r] - m_new);
        psum += z[m][r];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;

    // -- O^T += V^T . P^T, two MFMAs (8 tokens per lane each) per d tile
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int tok0 = 16 * kg + 8 * hh;
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
          const u32x4 w = vr[nt][0];
          f16x8 a = hh ? fp8x8_to_f16x8(w[2], w[3]) : fp8x8_to_f16x8(w[0], w[1]);
          if (valid < kTile) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (tok0 + e >= valid) a[e] = (_Float16)0.0f;
          }
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
          bf16x8 a = as_bf16x8(vr[nt][hh]);
          if (valid < kTile) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (tok0 + e >= valid) a[e] = (__bf16)0.0f;
          }
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, acc[nt], 0, 0, 0);
        }
      }
    }
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

  const float sv = FP8 ? vs : 1.0f;
  for (int w = tid; w < G * D; w += kBlock) {
    const int gg = w / D, d = w - gg * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][gg]);
    float O = 0.0f, L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = s_m[ww][gg];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        O += f * s_o[ww][gg][d >> 2][d & 3];
        L += f * s_l[ww][gg];
      }
    }
    if (U == 1) {
      write_final(p, b, h, gg, d, D, M, L, O, sv);
    } else {
      // agent-scope stores write through to where every XCD reads them
      __hip_atomic_store(p.part_o + ((int64_t)u * G + gg) * D + d, O, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(p.part_ml + ((int64_t)u * G + gg) * 2, M, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.part_ml + ((int64_t)u * G + gg) * 2 + 1, L, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (U == 1) return;

  // ---- split segment: the last of its units to get here merges the partials.
  // Every wave waits for its partial stores to complete before the workgroup
  // counts itself in; no cache-wide fence is needed because both the stores
  // and the merge's loads are agent-scope.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(p.sem + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == U - 1;
    if (prev == U - 1) __hip_atomic_store(p.sem + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  for (int w = tid; w < G * D; w += kBlock) {
    const int gg = w / D, d = w - gg * D;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < U; k0 += kMergeBatch) {
      float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {   // unconditional loads, clamped index
        const int64_t slot = (int64_t)(first + min(k0 + j, U - 1)) * G + gg;
        mv[j] = __hip_atomic_load(p.part_ml + slot * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lv[j] = __hip_atomic_load(p.part_ml + slot * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ov[j] = __hip_atomic_load(p.part_o + slot * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j)
        if (k0 + j >= U) mv[j] = -INFINITY;
      float Mb = M;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) Mb = fmaxf(Mb, mv[j]);
      if (Mb == -INFINITY) continue;
      const float a = (M == -INFINITY) ? 0.0f : exp2f(M - Mb);
      O *= a;
      L *= a;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const float f = (mv[j] == -INFINITY) ? 0.0f : exp2f(mv[j] - Mb);
        O += f * ov[j];
        L += f * lv[j];
      }
      M = Mb;
    }
    write_final(p, b, h, gg, d, D, M, L, O, sv);
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int64_t attn_max_units(const cda_kv_cache& c, int tpu) {
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return nh + c.pool_rows / ((int64_t)kTile * tpu);
}

size_t attn_workspace_bytes(const cda_kv_cache& c, int G, int tpu) {
  const int64_t units = attn_max_units(c, tpu);
  const int64_t nh = (int64_t)c.B * c.Hkv;
  return align256((size_t)nh * 4) + align256((size_t)units * G * 2 * 4) +
         align256((size_t)units * G * c.D * 4);
}

hipError_t launch_attn(const cda_kv_cache& c, const void* q, int Hq, float sm_scale, void* out,
                       int out_f32, float* lse, int tpu, void* workspace, hipStream_t s) {
  const int nh = c.B * c.Hkv;
  if (nh == 0) return hipGetLastError();
  const int G = Hq / c.Hkv;
  const int64_t units = attn_max_units(c, tpu);
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
  // workspace: [sem: nh int32][part_ml: units*G*2 f32][part_o: units*G*D f32]
  char* ws = static_cast<char*>(workspace);
  p.sem = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)nh * 4);
  p.part_ml = reinterpret_cast<float*>(ws);
  ws += align256((size_t)units * G * 2 * 4);
  p.part_o = reinterpret_cast<float*>(ws);
  p.Hkv = c.Hkv;
  p.G = G;
  p.Hq = Hq;
  p.W = c.W;
  p.nh = nh;
  p.tpu = tpu;
  p.out_f32 = out_f32;
  p.sm_scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)c.D);
  const bool fp8 = c.kv_dtype == CDA_KV_FP8_E4M3;
  const dim3 grid((unsigned)units);
  if (fp8) {
    if (c.D == 64)
      attn_kernel<true, 64><<<grid, kBlock, 0, s>>>(p);
    else
      attn_kernel<true, 128><<<grid, kBlock, 0, s>>>(p);
  } else {
    if (c.D == 64)
      attn_kernel<false, 64><<<grid, kBlock, 0, s>>>(p);
    else
      attn_kernel<false, 128><<<grid, kBlock, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace cda
