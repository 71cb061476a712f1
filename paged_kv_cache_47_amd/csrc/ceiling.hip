// HBM read ceilings (pa_ceiling.h): a stream read and a decode-shaped tile
// gather.  Neither computes anything of the attention; they give the rates a
// roofline of the table-walking decode kernels is read against.
#include "pa_ceiling.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCeilThreads = 256;
constexpr uint32_t kSinkMagic = 0x9e3779b9u;   // contents that are never expected: keeps the loads

// Grid-stride read of n 16-byte words, U loads in flight per lane.
template <int U>
__global__ __launch_bounds__(kCeilThreads) void stream_read_kernel(const u32x4_t* __restrict__ p, size_t n,
                                                                   uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kCeilThreads;
  size_t i = (size_t)blockIdx.x * kCeilThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4_t w = __builtin_nontemporal_load(p + i);
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == kSinkMagic) *sink = acc;
}

// One wave reads a run of the id list: for each id the K tile and the V tile
// (4 KiB each: 64 lanes x 4 x 16 B), P further pairs in flight.
template <int P>
__global__ __launch_bounds__(kCeilThreads) void gather_kernel(const u32x4_t* __restrict__ k,
                                                              const u32x4_t* __restrict__ v, int64_t num_tiles,
                                                              const int32_t* __restrict__ ids, int64_t num_ids,
                                                              int per_wave, uint32_t* sink) {
  constexpr int kWords = 4096 / 16;   // 16-byte words per tile
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * (kCeilThreads / 64) + (threadIdx.x >> 6)) * per_wave;
  if (i0 >= num_ids) return;   // uniform per wave
  const int n = (int)min((int64_t)per_wave, num_ids - i0);
  u32x4_t buf[P + 1][8];
  uint32_t acc = 0;
  auto load = [&](int t, u32x4_t* d) {
    if (t >= n) return;   // uniform per wave
    int64_t tile = ids[i0 + t];
    if (tile < 0 || tile >= num_tiles) tile = 0;
    const size_t base = (size_t)tile * kWords + lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = __builtin_nontemporal_load(k + base + c * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) d[4 + c] = __builtin_nontemporal_load(v + base + c * 64);
  };
#pragma unroll
  for (int p = 0; p < P; ++p) load(p, buf[p]);
  for (int t = 0; t < n; t += P + 1) {
#pragma unroll
    for (int s = 0; s <= P; ++s) {
      load(t + s + P, buf[(s + P) % (P + 1)]);
      if (t + s < n) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc ^= buf[s][c].x ^ buf[s][c].y ^ buf[s][c].z ^ buf[s][c].w;
      }
    }
  }
  if (acc == kSinkMagic) *sink = acc;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_ceiling_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                                            hipStream_t stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes == 0 || bytes % 16 || (uintptr_t)buf % 16 || workgroups < 0 || workgroups > 65536) return PA_ERR_SHAPE;
  const int grid = workgroups ? workgroups : 2048;
  stream_read_kernel<8><<<grid, kCeilThreads, 0, stream>>>((const u32x4_t*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_ceiling_gather(const void* k_tiles, const void* v_tiles, int64_t num_tiles,
                                       const int32_t* tile_ids, int64_t num_ids, int32_t ids_per_wave, int32_t depth,
                                       uint32_t* sink, hipStream_t stream) {
  if (!k_tiles || !v_tiles || !tile_ids || !sink) return PA_ERR_NULL;
  if (num_tiles < 1 || num_tiles > ((int64_t)1 << 28) || num_ids < 1 || ids_per_wave < 1 ||
      (depth != 1 && depth != 2) || (uintptr_t)k_tiles % 16 || (uintptr_t)v_tiles % 16)
    return PA_ERR_SHAPE;
  const int64_t waves = (num_ids + ids_per_wave - 1) / ids_per_wave;
  const int64_t grid = (waves + kCeilThreads / 64 - 1) / (kCeilThreads / 64);
  if (grid > INT32_MAX) return PA_ERR_SHAPE;
  const u32x4_t* k = (const u32x4_t*)k_tiles;
  const u32x4_t* v = (const u32x4_t*)v_tiles;
  if (depth == 1)
    gather_kernel<1><<<(int)grid, kCeilThreads, 0, stream>>>(k, v, num_tiles, tile_ids, num_ids, ids_per_wave, sink);
  else
    gather_kernel<2><<<(int)grid, kCeilThreads, 0, stream>>>(k, v, num_tiles, tile_ids, num_ids, ids_per_wave, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
