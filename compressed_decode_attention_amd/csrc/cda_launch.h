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
hipError_t launch_append(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s);
// Paged store: PAGE_INIT, REFILL and RELEASE.
hipError_t launch_page_op(const cda_kv_cache& c, const cda_compact_args& a, hipStream_t s);

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
