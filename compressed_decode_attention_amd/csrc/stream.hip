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
// reads tile tiles[j / 2] of k (j even) or of v (j odd).  A tile is
// tile_kb loads of 16 bytes per lane.
__global__ __launch_bounds__(64 * kMaxWaves) void stream_tiles_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ tiles, int n_jobs, int tile_kb, int split,
    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * (blockDim.x >> 6) + wave;
  if (j >= n_jobs) return;
  const int i = split ? j >> 1 : j;
  const int64_t t = tiles ? tiles[i] : i;
  const int64_t off = t * (int64_t)tile_kb * 1024 + lane * 16;
  const uint8_t* first = (split && (j & 1)) ? v + off : k + off;
  u32x4 acc = u32x4{0, 0, 0, 0};
  for (int c = 0; c < tile_kb; ++c)
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(first + c * 1024));
  if (!split)
    for (int c = 0; c < tile_kb; ++c)
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off + c * 1024));
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if (lane == 0) sink[j] = x;
}

}  // namespace

extern "C" {

// Reads n_tiles tiles of tile_bytes (a multiple of 1024) from k and from v:
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
  if (n_tiles < 0 || n_tiles > (1 << 29) || tile_bytes <= 0 || tile_bytes % 1024 != 0 ||
      waves < 1 || waves > kMaxWaves || (split != 0 && split != 1) || !k || !v || !sink)
    return 1;
  if (n_tiles == 0) return 0;
  const int jobs = split ? 2 * n_tiles : n_tiles;
  const int grid = (jobs + waves - 1) / waves;
  stream_tiles_kernel<<<grid, 64 * waves, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), tiles, jobs,
      tile_bytes / 1024, split, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
