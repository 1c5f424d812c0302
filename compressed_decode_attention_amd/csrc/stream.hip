// Measurement kernel of the benchmark (libcda_stream.so, not part of the
// C ABI of the attention library): a plain streaming read of 64-row tiles in
// the decode attention's own access pattern -- one 64-lane wave per tile,
// 16-byte nontemporal loads, first the K tile, then the V tile, eight waves
// per workgroup -- with no arithmetic beyond folding the words read into one
// value per wave (so that the loads are not dropped).  Timed over a large
// buffer it gives the read ceiling of this pattern on the device; over the
// tiles of one layer's compact store, the load-only floor of one attention
// launch; read by a counter run, it calibrates FETCH_SIZE.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWaves = 8;

// Wave w of workgroup g reads tile tiles[8g + w] (or 8g + w without a list)
// of both buffers: tile_bytes / 1024 loads of 16 bytes per lane from each.
__global__ __launch_bounds__(64 * kWaves) void stream_tiles_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ tiles, int n_tiles, int tile_kb, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * kWaves + wave;
  if (j >= n_tiles) return;
  const int64_t t = tiles ? tiles[j] : j;
  const uint8_t* kt = k + t * (int64_t)tile_kb * 1024 + lane * 16;
  const uint8_t* vt = v + t * (int64_t)tile_kb * 1024 + lane * 16;
  u32x4 acc = u32x4{0, 0, 0, 0};
  for (int c = 0; c < tile_kb; ++c)
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + c * 1024));
  for (int c = 0; c < tile_kb; ++c)
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vt + c * 1024));
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if (lane == 0) sink[j] = x;
}

}  // namespace

extern "C" {

// Reads n_tiles tiles of tile_bytes (a multiple of 1024) from k and from v:
// tile tiles[j] (or tile j if tiles is NULL) at byte tiles[j] * tile_bytes of
// each buffer, all of which the caller guarantees to be inside them.
// sink: n_tiles words written.  Returns 0, 1 for invalid arguments, 4 for a
// launch error.
int32_t cda_stream_tiles(const void* k, const void* v, const int32_t* tiles, int32_t n_tiles,
                         int32_t tile_bytes, uint32_t* sink, void* stream) {
  if (n_tiles < 0 || tile_bytes <= 0 || tile_bytes % 1024 != 0 || !k || !v || !sink) return 1;
  if (n_tiles == 0) return 0;
  const int grid = (n_tiles + kWaves - 1) / kWaves;
  stream_tiles_kernel<<<grid, 64 * kWaves, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), tiles, n_tiles,
      tile_bytes / 1024, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
