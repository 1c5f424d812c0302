// Measurement kernel of the benchmark (libcda_stream.so, not part of the
// C ABI of the attention library): a plain streaming read of 64-row tiles in
// the decode attention's own access pattern -- 64-lane waves, 16-byte
// nontemporal loads of whole tiles -- with no arithmetic beyond folding the
// words read into one value per wave (so that the loads are not dropped).
// A wave reads the K tile and then the V tile of one listed tile, or (split)
// only one of the two; workgroups hold 1 to 8 waves.  Timed over a large
// buffer it gives the read ceiling of this pattern on the device; over the
// tiles of one layer's compact store, in the best of these launch shapes,
// the load-only floor of one attention launch; read by a counter run, it
// calibrates FETCH_SIZE.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxWaves = 8;

// Job j = blockIdx.x * (blockDim.x / 64) + wave.  Without split, job j reads
// tile tiles[j] (or j without a list) of both buffers; with split, job j
// reads tile tiles[j / 2] of k (j even) or of v (j odd).  A tile is KB loads
// of 16 bytes per lane; every load of the job is issued before the first
// result is used.
template <int KB>
__global__ __launch_bounds__(64 * kMaxWaves) void stream_tiles_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ tiles, int n_jobs, int split, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * (blockDim.x >> 6) + wave;
  if (j >= n_jobs) return;
  const int i = split ? j >> 1 : j;
  const int64_t t = tiles ? tiles[i] : i;
  const int64_t off = t * (int64_t)KB * 1024 + lane * 16;
  u32x4 x[2 * KB];
  if (split) {
    const uint8_t* src = (j & 1) ? v + off : k + off;
#pragma unroll
    for (int c = 0; c < KB; ++c)
      x[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c * 1024));
#pragma unroll
    for (int c = KB; c < 2 * KB; ++c) x[c] = u32x4{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int c = 0; c < KB; ++c)
      x[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off + c * 1024));
#pragma unroll
    for (int c = 0; c < KB; ++c)
      x[KB + c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off + c * 1024));
  }
  // every load is in flight before the first result is waited for: no load
  // moves below the first statement, and the results are all taken (with one
  // wait for the last) before any is combined
  __asm__ volatile("" ::: "memory");
#pragma unroll
  for (int c = 0; c < 2 * KB; ++c) __asm__ volatile("" : "+v"(x[c]));
  u32x4 acc = x[0];
#pragma unroll
  for (int c = 1; c < 2 * KB; ++c) acc ^= x[c];
  uint32_t y = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) y ^= __shfl_xor(y, o, 64);
  if (lane == 0) sink[j] = y;
}

}  // namespace

extern "C" {

// Reads n_tiles tiles of tile_bytes (4096, 8192 or 16384) from k and from v:
// tile tiles[j] (or tile j if tiles is NULL) at byte tiles[j] * tile_bytes of
// each buffer, all of which the caller guarantees to be inside them.
// waves: waves per workgroup, 1 to 8.  split = 0: one wave reads a tile of k
// and then the same tile of v, and writes one word to sink[j] (n_tiles
// words); split = 1: one wave per tile of each buffer, sink[2j] for k and
// sink[2j + 1] for v (2 n_tiles words).  Returns 0, 1 for invalid arguments,
// 4 for a launch error.
int32_t cda_stream_tiles(const void* k, const void* v, const int32_t* tiles, int32_t n_tiles,
                         int32_t tile_bytes, int32_t waves, int32_t split, uint32_t* sink,
                         void* stream) {
  if (n_tiles < 0 || n_tiles > (1 << 29) ||
      (tile_bytes != 4096 && tile_bytes != 8192 && tile_bytes != 16384) || waves < 1 ||
      waves > kMaxWaves || (split != 0 && split != 1) || !k || !v || !sink)
    return 1;
  if (n_tiles == 0) return 0;
  const int jobs = split ? 2 * n_tiles : n_tiles;
  const dim3 grid((jobs + waves - 1) / waves), block(64 * waves);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* kb = static_cast<const uint8_t*>(k);
  const uint8_t* vb = static_cast<const uint8_t*>(v);
  if (tile_bytes == 4096) stream_tiles_kernel<4><<<grid, block, 0, s>>>(kb, vb, tiles, jobs, split, sink);
  else if (tile_bytes == 8192) stream_tiles_kernel<8><<<grid, block, 0, s>>>(kb, vb, tiles, jobs, split, sink);
  else stream_tiles_kernel<16><<<grid, block, 0, s>>>(kb, vb, tiles, jobs, split, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
