// Host-side launchers of the gfx950 kernels (one translation unit each).
// Arguments are validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/cda.h"

namespace cda {

hipError_t launch_count(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s);
hipError_t launch_pack(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s);
// M tokens per sequence, one after another (token t of sequence b at
// b * stride_b + t * stride_t + h * stride_h; keep [B, M, Hkv]).
hipError_t launch_append(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s,
                         int M = 1);
// Paged store: PAGE_INIT, REFILL and RELEASE.
hipError_t launch_page_op(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s);

// Multi-query attention of a chunk of M new tokens per sequence, then their
// append (decode attention of position pos + t for query t).
size_t chunk_workspace_bytes(const cda_kv_cache& c, int G, int M);
hipError_t launch_chunk(const cda_kv_cache& c, const cda_compact_args& a, int M, const void* q,
                        int Hq, float sm_scale, void* out, int out_f32, float* lse,
                        void* workspace, hipStream_t s);

// Work units of the attention kernel: an upper bound on the number of
// workgroups it launches (one per unit) for this cache and split.
int64_t attn_max_units(const cda_kv_cache& c, int tiles_per_unit);
size_t attn_workspace_bytes(const cda_kv_cache& c, int G, int tiles_per_unit);
// step == NULL: attention only; otherwise the APPEND arguments of the new
// token, appended in the same launch (decode step).
hipError_t launch_attn(const cda_kv_cache& c, const void* q, int Hq, float sm_scale,
                       void* out, int out_f32, float* lse, int tiles_per_unit,
                       void* workspace, hipStream_t s, const cda_compact_args* step);

}  // namespace cda
