// KV writes through a slot mapping, and whole-block copies for copy-on-write.
//
// [pytorch] "How to implement paged attention: the minimal data flow": token at
// position p of a sequence goes to block table[p / bs] at offset p % bs; the
// caller hands the resulting slot numbers (block * bs + offset) to the device.
// [engine] "INT8 KV cache design": int8 blocks are requantised on every token
// write with one max-abs fp16 scale per block per head.
#include "pa_internal.h"

namespace pa {

// Pools hold every layer of a block: tile (block, layer, head) starts at
// ((block * num_layers + layer) * hkv + head) * block_size * head_dim.  The
// launchers offset the pool (and scale) pointers to the addressed layer's
// first tile, so kernels index tiles as block * blk_tiles + head with
// blk_tiles = num_layers * hkv.
__host__ __device__ inline int64_t layer_tile0(const pa_cache_desc& d) {
  return (int64_t)d.layer * d.num_kv_heads;
}
__host__ __device__ inline int32_t blk_tiles_of(const pa_cache_desc& d) {
  return (d.num_layers > 0 ? d.num_layers : 1) * d.num_kv_heads;
}

// ---------------------------------------------------------------- fp16 ----
// One thread moves 16 bytes (8 halves) of one token's K and V for one head.
// Consecutive threads cover consecutive 16-byte chunks of a token row, so both
// the read of k/v and the write into the block are contiguous per token-head.
__global__ __launch_bounds__(256) void write_f16_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                        const int32_t* __restrict__ slots, int32_t T,
                                                        int32_t hkv, int32_t blk_tiles, int32_t chunks_per_row,
                                                        int64_t num_slots, uint4* __restrict__ kc,
                                                        uint4* __restrict__ vc) {
  const int64_t per_token = (int64_t)hkv * chunks_per_row;
  const int64_t n = (int64_t)T * per_token;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int64_t r = i - t * per_token;
    const int32_t h = (int32_t)(r / chunks_per_row);
    const int32_t c = (int32_t)(r - (int64_t)h * chunks_per_row);
    const int32_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const int64_t blk = s / kBlockSize, off = s % kBlockSize;
    const int64_t dst = ((blk * blk_tiles + h) * kBlockSize + off) * chunks_per_row + c;
    kc[dst] = k[i];
    vc[dst] = v[i];
  }
}

hipError_t launch_write_f16(const pa_cache_desc& d, const void* k, const void* v, const int32_t* slots,
                            int32_t T, void* kc, void* vc, hipStream_t s) {
  const int cpr = d.head_dim / 8;
  const int64_t n = (int64_t)T * d.num_kv_heads * cpr;
  const int64_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  const int64_t off = layer_tile0(d) * kBlockSize * cpr;   // in 16-byte chunks
  write_f16_kernel<<<grid, 256, 0, s>>>((const uint4*)k, (const uint4*)v, slots, T, d.num_kv_heads, blk_tiles_of(d),
                                        cpr, (int64_t)d.num_blocks * kBlockSize, (uint4*)kc + off,
                                        (uint4*)vc + off);
  return hipGetLastError();
}

// ---------------------------------------------------------------- int8 ----
// A run starts at a token whose predecessor does not write the previous slot
// of the same block; it continues while the next token writes the next slot.
// A wave replays a run on one (block, KV head, K or V): the block's codes live
// in registers as exact small floats (EPL dims per lane), and each token of
// the run is replayed in order:
//   x_j = code_j * scale (j < o), x_o = new, scale = fp16(max|x| / 127),
//   code_j = clamp(rint(x_j / scale), -127, 127)   (zero if scale == 0).
// fp32 division is IEEE (the build does not use fast-math) so the codes match
// a CPU evaluation of the same formula bit for bit.
//
// Two exact shortcuts keep the per-token cost low:
// * max|x_j| over the earlier rows is |scale| * max|code_j| (products of an
//   fp16 scale and a 7-bit code are exact in fp32), so the wave tracks the
//   largest code instead of re-reading every row;
// * when the new scale equals the old one (positive and finite) and every
//   earlier code is within +-127, requantising leaves every earlier code as
//   it is: code_j * scale is exact and dividing it by the same scale gives
//   code_j back exactly.  Only the new row is then quantised.
template <int D>
__device__ void replay_run_i8(const half_t* __restrict__ src, const int32_t s, const int t, const int n,
                              const int h, const int hkv, const int blk_tiles, int8_t* __restrict__ cache,
                              half_t* __restrict__ scales) {
  constexpr int EPL = D / 64;  // dims per lane: 2 (d128) or 1 (d64)
  const int lane = threadIdx.x;
  const int64_t blk = s / kBlockSize;
  const int o0 = s % kBlockSize;
  int8_t* tile = cache + (blk * blk_tiles + h) * (int64_t)kBlockSize * D;
  const int64_t sidx = blk * blk_tiles + h;

  float c[kBlockSize][EPL];
  float sc = (float)scales[sidx];
  float cm = 0.f;   // largest |code| of the rows before the current one (whole wave)
#pragma unroll
  for (int j = 0; j < kBlockSize; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      c[j][e] = (j < o0) ? (float)tile[j * D + lane * EPL + e] : 0.f;
      cm = fmaxf(cm, fabsf(c[j][e]));
    }
  cm = wave_max(cm);

  for (int r = 0; r < n; ++r) {
    const int o = o0 + r;
    const half_t* row = src + ((int64_t)(t + r) * hkv + h) * D + lane * EPL;
    float xo[EPL];
    float xm = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xo[e] = (float)row[e];
      xm = fmaxf(xm, fabsf(xo[e]));
    }
    xm = wave_max(xm);
    const float amax = fmaxf(cm * fabsf(sc), xm);
    const float sn = (float)(half_t)(amax / 127.0f);
    // wave-uniform: every value above is
    const bool keep = sn == sc && sn > 0.f && sn <= 65504.f && cm <= 127.f;
    float lm = cm;
    if (!keep) {
      lm = 0.f;
#pragma unroll
      for (int j = 0; j < kBlockSize; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          if (j < o) {
            const float qv = (sn == 0.f) ? 0.f : __builtin_rintf((c[j][e] * sc) / sn);
            c[j][e] = fminf(127.f, fmaxf(-127.f, qv));
            lm = fmaxf(lm, fabsf(c[j][e]));
          }
        }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float qv = (sn == 0.f) ? 0.f : __builtin_rintf(xo[e] / sn);
      const float q = fminf(127.f, fmaxf(-127.f, qv));
      lm = fmaxf(lm, fabsf(q));
#pragma unroll
      for (int j = 0; j < kBlockSize; ++j)
        if (j == o) c[j][e] = q;
    }
    cm = wave_max(lm);
    sc = sn;
  }
  const int olast = o0 + n - 1;
#pragma unroll
  for (int j = 0; j < kBlockSize; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (j <= olast) tile[j * D + lane * EPL + e] = (int8_t)(int)c[j][e];
  if (lane == 0) scales[sidx] = (half_t)sc;
}

// One wave per (kI8Window consecutive tokens, KV head, K or V): it replays, in
// token order, every run that starts in its window (a run may continue past
// the window; the tokens it covers there are not run starts and are skipped
// by the next window's wave).
constexpr int kI8Window = 8;

template <int D>
__global__ __launch_bounds__(64) void write_i8_kernel(const half_t* __restrict__ k, const half_t* __restrict__ v,
                                                      const int32_t* __restrict__ slots, int32_t T, int32_t hkv,
                                                      int32_t blk_tiles, int64_t num_slots, int8_t* __restrict__ kc,
                                                      int8_t* __restrict__ vc, half_t* __restrict__ ks,
                                                      half_t* __restrict__ vs) {
  const int h = blockIdx.y, which = blockIdx.z;
  const half_t* src = which ? v : k;
  int8_t* cache = which ? vc : kc;
  half_t* scales = which ? vs : ks;
  const int t_end = min(T, (int)(blockIdx.x + 1) * kI8Window);
  for (int t = blockIdx.x * kI8Window; t < t_end; ++t) {
    const int32_t s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    if (t > 0 && (s % kBlockSize) != 0 && slots[t - 1] == s - 1) continue;  // inside a run started earlier
    int n = 1;
    while (t + n < T && ((s + n) % kBlockSize) != 0 && slots[t + n] == s + n) ++n;
    replay_run_i8<D>(src, s, t, n, h, hkv, blk_tiles, cache, scales);
  }
}

hipError_t launch_write_i8(const pa_cache_desc& d, const void* k, const void* v, const int32_t* slots,
                           int32_t T, void* kc, void* vc, void* ks, void* vs, hipStream_t s) {
  dim3 grid((T + kI8Window - 1) / kI8Window, d.num_kv_heads, 2);
  const int64_t ns = (int64_t)d.num_blocks * kBlockSize;
  const int64_t t0 = layer_tile0(d), off = t0 * kBlockSize * d.head_dim;
  const int bt = blk_tiles_of(d);
  if (d.head_dim == 128)
    write_i8_kernel<128><<<grid, 64, 0, s>>>((const half_t*)k, (const half_t*)v, slots, T, d.num_kv_heads, bt, ns,
                                             (int8_t*)kc + off, (int8_t*)vc + off, (half_t*)ks + t0,
                                             (half_t*)vs + t0);
  else
    write_i8_kernel<64><<<grid, 64, 0, s>>>((const half_t*)k, (const half_t*)v, slots, T, d.num_kv_heads, bt, ns,
                                            (int8_t*)kc + off, (int8_t*)vc + off, (half_t*)ks + t0,
                                            (half_t*)vs + t0);
  return hipGetLastError();
}

// ---------------------------------------------------------- block copies ----
// blockIdx.x = pair; threads stride over the 16-byte chunks of the K and V
// tiles of every layer and head of the source block, then copy the int8
// scales (one per layer and head).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                          half_t* __restrict__ ks, half_t* __restrict__ vs,
                                                          const int32_t* __restrict__ pairs, int32_t num_blocks,
                                                          int32_t chunks_per_block, int32_t blk_tiles) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  const int64_t so = (int64_t)src * chunks_per_block, d = (int64_t)dst * chunks_per_block;
  for (int i = threadIdx.x; i < chunks_per_block; i += blockDim.x) {
    kc[d + i] = kc[so + i];
    vc[d + i] = vc[so + i];
  }
  if (ks != nullptr) {
    for (int i = threadIdx.x; i < blk_tiles; i += blockDim.x) {
      ks[(int64_t)dst * blk_tiles + i] = ks[(int64_t)src * blk_tiles + i];
      vs[(int64_t)dst * blk_tiles + i] = vs[(int64_t)src * blk_tiles + i];
    }
  }
}

hipError_t launch_copy(const pa_cache_desc& d, void* kc, void* vc, void* ks, void* vs, const int32_t* pairs,
                       int32_t n, hipStream_t s) {
  const int eb = d.kv_dtype == PA_KV_I8 ? 1 : 2;
  const int chunks = blk_tiles_of(d) * kBlockSize * d.head_dim * eb / 16;
  const bool i8 = d.kv_dtype == PA_KV_I8;
  copy_blocks_kernel<<<n, 256, 0, s>>>((uint4*)kc, (uint4*)vc, i8 ? (half_t*)ks : nullptr, i8 ? (half_t*)vs : nullptr,
                                       pairs, d.num_blocks, chunks, blk_tiles_of(d));
  return hipGetLastError();
}

}  // namespace pa
