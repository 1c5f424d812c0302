// C-ABI entry points declared in include/cda.h: argument validation, then
// the launchers.  Nothing here allocates, frees, synchronises or prints.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/cda.h"
#include "cda_launch.h"

// Scratch of decode_step_compact_noalloc: the attention workspace (counters
// and partial slots) as a device array of its own, one per GPU the library
// runs on, held until the process ends.  Host code uses only the address
// hipGetSymbolAddress gives for it on each device, never the array's name.
static __device__ __align__(256) uint8_t scratch[CDA_SCRATCH_BYTES];

namespace {

constexpr int64_t kLargePoolRows = 1 << 16;
constexpr double kResidentUnits = 248;  // 8-wave attention workgroups resident at once
                                        // (one per CU of 256, less a few for unevenness)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_cache(const cda_kv_cache* c) {
  if (!c) return CDA_ERR_INVALID_ARG;
  if (c->B < 0 || c->Hkv < 1 || c->W < 0 || c->spare_rows < 0) return CDA_ERR_INVALID_ARG;
  if (c->W > (1 << 28)) return CDA_ERR_INVALID_ARG;
  if (c->D != 64 && c->D != 128) return CDA_ERR_UNSUPPORTED;
  if (c->kv_dtype != CDA_KV_BF16 && c->kv_dtype != CDA_KV_FP8_E4M3 &&
      c->kv_dtype != CDA_KV_FP4_E2M1)
    return CDA_ERR_UNSUPPORTED;
  if (c->kv_dtype == CDA_KV_FP4_E2M1 && c->D != 128) return CDA_ERR_UNSUPPORTED;
  if ((int64_t)c->B * c->Hkv > (1 << 24)) return CDA_ERR_INVALID_ARG;
  if (!c->seg_cap || !c->comp_len || !c->err || c->reserved1 != 0) return CDA_ERR_INVALID_ARG;
  if (c->page_table) {   // paged store
    if (c->max_pages < 1 || (int64_t)c->B * c->Hkv * c->max_pages > INT32_MAX)
      return CDA_ERR_INVALID_ARG;
    if (!c->free_pages || !c->free_top || !c->pos) return CDA_ERR_INVALID_ARG;
    if (c->W > 0 && !c->ring_keep) return CDA_ERR_INVALID_ARG;
    if (c->pool_rows < CDA_SEG_ALIGN || c->pool_rows / CDA_SEG_ALIGN > INT32_MAX)
      return CDA_ERR_INVALID_ARG;   // at least one page
  } else if (!c->seg_base) {
    return CDA_ERR_INVALID_ARG;
  }
  return CDA_OK;
}

// The sequence range of COUNT, PACK and RELEASE: paged store only (both 0
// for contiguous segments); seq_count 0 = the whole batch.
int32_t check_range(const cda_kv_cache* c, const cda_compact_args* a) {
  if (!c->page_table) return (a->seq_begin == 0 && a->seq_count == 0) ? CDA_OK : CDA_ERR_INVALID_ARG;
  if (a->seq_count == 0) return a->seq_begin == 0 ? CDA_OK : CDA_ERR_INVALID_ARG;
  if (a->seq_count < 0 || a->seq_begin < 0 || a->seq_begin > c->B - a->seq_count)
    return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

// Pools and per-sequence state used by PACK, APPEND and attention.
int32_t check_pools(const cda_kv_cache* c) {
  if (c->pool_rows < 0 || c->pool_rows % CDA_SEG_ALIGN != 0) return CDA_ERR_INVALID_ARG;
  if (c->pool_rows > 0 && (!c->k_pool || !c->v_pool)) return CDA_ERR_INVALID_ARG;
  if (!aligned(c->k_pool, 16) || !aligned(c->v_pool, 16)) return CDA_ERR_INVALID_ARG;
  if (!c->pos || (c->W > 0 && !c->ring_keep)) return CDA_ERR_INVALID_ARG;
  if (c->kv_dtype != CDA_KV_BF16 && (!c->k_amax || !c->v_amax)) return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

int32_t check_bf16_rows(const void* k, const void* v, int64_t sb, int64_t st, int64_t sh) {
  if (!k || !v) return CDA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16)) return CDA_ERR_INVALID_ARG;
  if (sb < 0 || st < 0 || sh < 0 || sb % 8 || st % 8 || sh % 8) return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? CDA_OK : CDA_ERR_HIP; }

// Per device: the device address of `scratch` and whether its zero fill has
// been enqueued.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};

__global__ void zero_words(uint4* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = uint4{0, 0, 0, 0};
}

// The scratch address on the current device (which must be the stream's),
// looked up on the first call on that device; that call also enqueues the
// array's zero fill on the stream, ahead of the kernel that first uses it
// (a kernel, not a memset, so that a captured graph replays it as well).
int32_t device_scratch(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CDA_ERR_HIP;
  if (s) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return CDA_ERR_HIP;
    if (sdev != dev) return CDA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CDA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  if (!g_scratch_zeroed[dev]) {
    const int64_t n = CDA_SCRATCH_BYTES / 16;
    zero_words<<<256, 256, 0, s>>>(static_cast<uint4*>(g_scratch_ptr[dev]), n);
    if (hipGetLastError() != hipSuccess) return CDA_ERR_HIP;
    g_scratch_zeroed[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return CDA_OK;
}

// The optional host copy of seg_base (contiguous store): non-decreasing
// multiples of 64 starting at 0, the last entry inside the pool.
int32_t check_seg_base_host(const cda_kv_cache* c) {
  if (!c->seg_base_host || c->page_table) return CDA_OK;
  const int64_t nh = (int64_t)c->B * c->Hkv;
  const int64_t* s = c->seg_base_host;
  if (s[0] != 0 || s[nh] > c->pool_rows) return CDA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < nh; ++i)
    if (s[i + 1] < s[i] || s[i + 1] % CDA_SEG_ALIGN != 0) return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

// Default work-unit size in 64-row tiles.  One unit is one workgroup; the
// attention kernels keep one 8-wave workgroup per CU resident, so with more
// units than that the last ones start a whole unit late, which costs about
// half again the layer's time.  The estimate of the units is the pool's
// tiles / tpu plus half a unit of rounding per segment (pool_rows counts
// capacity, so it errs high).  Small pools that fit at 4 tiles keep 4-tile
// units (4-wave workgroups, more of them in flight); otherwise the smallest
// 8-wave unit that fits.  When none fits (hundreds of segments) the extra
// rounds are unavoidable and 8-tile units do the least work per round.
int default_tpu(const cda_kv_cache* c) {
  const double tiles = (double)c->pool_rows / CDA_SEG_ALIGN;
  const double nh = (double)c->B * c->Hkv;
  const auto fits = [&](int t) { return tiles / t + nh / 2 <= kResidentUnits; };
  if (c->pool_rows < kLargePoolRows && fits(4)) return 4;
  for (const int t : {8, 12, 16, 24, 32, 48, 64})
    if (fits(t)) return t;
  return 8;
}

int tiles_per_unit(const cda_kv_cache* c, int32_t split_tokens) {
  if (split_tokens <= 0) return default_tpu(c);
  return (split_tokens + CDA_SEG_ALIGN - 1) / CDA_SEG_ALIGN;
}

}  // namespace

extern "C" {

int32_t kv_compact(const cda_kv_cache* c, const cda_compact_args* a, void* stream) {
  int32_t st = check_cache(c);
  if (st != CDA_OK) return st;
  if (!a) return CDA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = check_range(c, a)) != CDA_OK) return st;
  // segments the call covers (the range's, or the batch's)
  const int64_t nh = (int64_t)(a->seq_count > 0 ? a->seq_count : c->B) * c->Hkv;
  switch (a->op) {
    case CDA_OP_PAGE_INIT:
    case CDA_OP_REFILL:
    case CDA_OP_RELEASE:
      if (!c->page_table) return CDA_ERR_INVALID_ARG;
      if (a->op == CDA_OP_REFILL && (a->reserve < 0 || a->reserve > (1 << 28)))
        return CDA_ERR_INVALID_ARG;
      return hip_status(cda::launch_page_op(*c, *a, s));
    case CDA_OP_COUNT:
    case CDA_OP_PACK: {
      if (a->T < 0 || a->T > (1 << 24) || a->keep_ld < a->T) return CDA_ERR_INVALID_ARG;
      if (nh > 0 && a->T > 0 && !a->keep) return CDA_ERR_INVALID_ARG;
      if (a->op == CDA_OP_COUNT) {
        if (a->reserve < 0 || a->reserve > (1 << 28)) return CDA_ERR_INVALID_ARG;
        return hip_status(cda::launch_count(*c, *a, s));
      }
      if ((st = check_pools(c)) != CDA_OK) return st;
      if (a->scale_mode != 0 && a->scale_mode != 1) return CDA_ERR_INVALID_ARG;
      if (nh > 0 && a->T > 0 &&
          (st = check_bf16_rows(a->k, a->v, a->stride_b, a->stride_t, a->stride_h)) != CDA_OK)
        return st;
      return hip_status(cda::launch_pack(*c, *a, s));
    }
    case CDA_OP_APPEND: {
      if ((st = check_pools(c)) != CDA_OK) return st;
      if (a->seq_count != 0) return CDA_ERR_INVALID_ARG;   // always the whole batch
      if (nh > 0) {
        if (!a->keep) return CDA_ERR_INVALID_ARG;
        if ((st = check_bf16_rows(a->k, a->v, a->stride_b, 0, a->stride_h)) != CDA_OK) return st;
      }
      return hip_status(cda::launch_append(*c, *a, s));
    }
    default:
      return CDA_ERR_INVALID_ARG;
  }
}

size_t cda_attn_workspace_bytes(const cda_kv_cache* c, int32_t Hq, int32_t split_tokens) {
  if (check_cache(c) != CDA_OK || Hq <= 0 || Hq % c->Hkv != 0 || split_tokens < 0) return 0;
  return cda::attn_workspace_bytes(*c, Hq / c->Hkv, tiles_per_unit(c, split_tokens));
}

}  // extern "C"

namespace {

// Checks shared by the attention entry points, all but the workspace's; on
// success *tpu is the work-unit size in tiles and *need the workspace bytes.
int32_t check_attention_args(const cda_kv_cache* c, const void* q, int32_t Hq, void* out,
                             int32_t out_dtype, float* lse, int32_t split_tokens, int* tpu,
                             size_t* need) {
  int32_t st = check_cache(c);
  if (st != CDA_OK) return st;
  if ((st = check_pools(c)) != CDA_OK) return st;
  if (Hq <= 0 || split_tokens < 0) return CDA_ERR_INVALID_ARG;
  if (Hq % c->Hkv != 0 || Hq / c->Hkv > CDA_MAX_GQA) return CDA_ERR_UNSUPPORTED;
  if (out_dtype != CDA_OUT_BF16 && out_dtype != CDA_OUT_F32) return CDA_ERR_UNSUPPORTED;
  if (c->B > 0) {
    if (!q || !out || !aligned(q, 16) || !aligned(out, 4)) return CDA_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return CDA_ERR_INVALID_ARG;
  }
  if ((st = check_seg_base_host(c)) != CDA_OK) return st;
  *tpu = tiles_per_unit(c, split_tokens);
  *need = cda::attn_workspace_bytes(*c, Hq / c->Hkv, *tpu);
  if (cda::attn_max_units(*c, *tpu) > 0x7FFFFFFF) return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

// check_attention_args, then the caller's workspace.
int32_t check_attention(const cda_kv_cache* c, const void* q, int32_t Hq, void* out,
                        int32_t out_dtype, float* lse, int32_t split_tokens, void* workspace,
                        size_t workspace_bytes, int* tpu) {
  size_t need = 0;
  const int32_t st = check_attention_args(c, q, Hq, out, out_dtype, lse, split_tokens, tpu, &need);
  if (st != CDA_OK) return st;
  if (workspace_bytes < need) return CDA_ERR_WORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return CDA_ERR_INVALID_ARG;
  return CDA_OK;
}

// The APPEND arguments of a decode step.
int32_t check_step_args(const cda_kv_cache* c, const cda_compact_args* a) {
  if (!a || a->op != CDA_OP_APPEND || a->seq_begin != 0 || a->seq_count != 0)
    return CDA_ERR_INVALID_ARG;
  if (c->B > 0) {
    if (!a->keep) return CDA_ERR_INVALID_ARG;
    return check_bf16_rows(a->k, a->v, a->stride_b, 0, a->stride_h);
  }
  return CDA_OK;
}

}  // namespace

extern "C" {

int32_t decode_attn_compact(const cda_kv_cache* c, const void* q, int32_t Hq, float sm_scale,
                            void* out, int32_t out_dtype, float* lse, int32_t split_tokens,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int tpu = 0;
  const int32_t st = check_attention(c, q, Hq, out, out_dtype, lse, split_tokens, workspace,
                                     workspace_bytes, &tpu);
  if (st != CDA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(cda::launch_attn(*c, q, Hq, sm_scale, out, out_dtype == CDA_OUT_F32, lse,
                                     tpu, workspace, s, nullptr));
}

int32_t decode_step_compact(const cda_kv_cache* c, const cda_compact_args* a, const void* q,
                            int32_t Hq, float sm_scale, void* out, int32_t out_dtype, float* lse,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int tpu = 0;
  int32_t st = check_attention(c, q, Hq, out, out_dtype, lse, split_tokens, workspace,
                               workspace_bytes, &tpu);
  if (st != CDA_OK) return st;
  if ((st = check_step_args(c, a)) != CDA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(cda::launch_attn(*c, q, Hq, sm_scale, out, out_dtype == CDA_OUT_F32, lse,
                                     tpu, workspace, s, a));
}

int32_t decode_step_compact_noalloc(const cda_kv_cache* c, const cda_compact_args* a,
                                    const void* q, int32_t Hq, float sm_scale, void* out,
                                    int32_t out_dtype, float* lse, int32_t split_tokens,
                                    void* stream) {
  // every argument checked, and the scratch the call needs against the
  // array's size, before any HIP call; the array stands in for the workspace
  int tpu = 0;
  size_t need = 0;
  int32_t st = check_attention_args(c, q, Hq, out, out_dtype, lse, split_tokens, &tpu, &need);
  if (st != CDA_OK) return st;
  if (need > CDA_SCRATCH_BYTES) return CDA_ERR_WORKSPACE;
  if ((st = check_step_args(c, a)) != CDA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ptr = nullptr;
  if ((st = device_scratch(s, &ptr)) != CDA_OK) return st;
  return hip_status(cda::launch_attn(*c, q, Hq, sm_scale, out, out_dtype == CDA_OUT_F32, lse,
                                     tpu, ptr, s, a));
}

size_t cda_chunk_workspace_bytes(const cda_kv_cache* c, int32_t Hq, int32_t M) {
  if (check_cache(c) != CDA_OK || Hq <= 0 || Hq % c->Hkv != 0 || M < 1 || M > CDA_MAX_CHUNK)
    return 0;
  return cda::chunk_workspace_bytes(*c, Hq / c->Hkv, M);
}

int32_t chunk_attn_compact(const cda_kv_cache* c, const cda_compact_args* a, int32_t M,
                           const void* q, int32_t Hq, float sm_scale, void* out,
                           int32_t out_dtype, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int32_t st = check_cache(c);
  if (st != CDA_OK) return st;
  if ((st = check_pools(c)) != CDA_OK) return st;
  if (M < 1 || M > CDA_MAX_CHUNK || Hq <= 0) return CDA_ERR_INVALID_ARG;
  if (Hq % c->Hkv != 0 || Hq / c->Hkv > CDA_MAX_GQA) return CDA_ERR_UNSUPPORTED;
  if (c->W > CDA_MAX_CHUNK_WINDOW) return CDA_ERR_UNSUPPORTED;
  if (out_dtype != CDA_OUT_BF16 && out_dtype != CDA_OUT_F32) return CDA_ERR_UNSUPPORTED;
  if (!a || a->op != CDA_OP_APPEND || a->seq_begin != 0 || a->seq_count != 0)
    return CDA_ERR_INVALID_ARG;
  if (c->B > 0) {
    if (!a->keep) return CDA_ERR_INVALID_ARG;
    if ((st = check_bf16_rows(a->k, a->v, a->stride_b, a->stride_t, a->stride_h)) != CDA_OK)
      return st;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return CDA_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return CDA_ERR_INVALID_ARG;
  }
  const size_t need = cda::chunk_workspace_bytes(*c, Hq / c->Hkv, M);
  if (workspace_bytes < need) return CDA_ERR_WORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return CDA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(cda::launch_chunk(*c, *a, M, q, Hq, sm_scale, out, out_dtype == CDA_OUT_F32,
                                      lse, workspace, s));
}

const char* cda_status_string(int32_t status) {
  switch (status) {
    case CDA_OK: return "ok";
    case CDA_ERR_INVALID_ARG: return "invalid argument";
    case CDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case CDA_ERR_WORKSPACE: return "workspace too small";
    case CDA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t cda_version(void) { return CDA_VERSION; }

}  // extern "C"
