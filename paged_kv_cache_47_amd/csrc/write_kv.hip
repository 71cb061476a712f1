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
// A wave replays a run on one (block, KV head, K or V), EPL dims per lane,
// with the result of replaying each token of the run in order:
//   x_j = code_j * scale (j < o), x_o = new, scale = fp16(max|x| / 127),
//   code_j = clamp(rint(x_j / scale), -127, 127)   (zero if scale == 0).
// fp32 division is IEEE (the build does not use fast-math) so the codes match
// a CPU evaluation of the same formula bit for bit.
//
// The replay is split so that nothing in the token order waits on memory, on
// another lane, or on a pass over the block:
// * every load of the run is issued first: the block's codes (all rows: the
//   tile is whole, and no other wave writes the block in the same call), its
//   old scale and the run's new rows;
// * max|x| of every new row is reduced across the wave in one batch;
// * the scales follow from wave-uniform arithmetic alone.  Quantising at a
//   scale s >= 0 is odd and monotone in x (IEEE division by s, rint and the
//   clamp all are), so the largest |code| of a set of values is the code of
//   their largest |x|; and the largest |x_j| of the earlier rows is
//   cm * |scale| for their largest |code| cm (a 7-bit code times an fp16
//   scale is exact in fp32).  The largest code after a token is therefore
//   max(q(cm * |scale|), q(max|x_o|)), and the token's new scale needs no
//   codes at all;
// * the codes come last, row by row: a row's code is quantised at its own
//   token's scale and requantised at every later token that changed the
//   scale, in token order, which is the value the token-by-token replay
//   leaves in it.
// When the new scale equals the old one (positive and finite) and every
// earlier code is within +-127, requantising leaves every earlier code as it
// is (code_j * scale is exact and dividing it by the same scale gives code_j
// back), so such a token changes no earlier code.

// code of x at scale sn (every code is zero when sn == 0)
__device__ __forceinline__ float quant_i8(float x, float sn) {
  const float q = (sn == 0.f) ? 0.f : __builtin_rintf(x / sn);
  return fminf(127.f, fmaxf(-127.f, q));
}

// max over the wave of COUNT values at once; every lane gets the results.
// The row-wide butterfly steps of different values are independent, so they
// fill each other's DPP wait states; the four rows then meet through readlane.
template <int COUNT>
__device__ __forceinline__ void wave_max_all(float* x) {
#pragma unroll
  for (int k = 0; k < COUNT; ++k) x[k] = fmaxf(x[k], dpp<0xB1>(x[k]));    // quad_perm [1,0,3,2]
#pragma unroll
  for (int k = 0; k < COUNT; ++k) x[k] = fmaxf(x[k], dpp<0x4E>(x[k]));    // quad_perm [2,3,0,1]
#pragma unroll
  for (int k = 0; k < COUNT; ++k) x[k] = fmaxf(x[k], dpp<0x141>(x[k]));   // row_half_mirror
#pragma unroll
  for (int k = 0; k < COUNT; ++k) x[k] = fmaxf(x[k], dpp<0x140>(x[k]));   // row_mirror
#pragma unroll
  for (int k = 0; k < COUNT; ++k) {
    const int b = __builtin_bit_cast(int, x[k]);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    x[k] = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
  }
}

template <int EPL> struct LaneWords;
template <> struct LaneWords<1> { typedef uint8_t codes; typedef uint16_t halves; };
template <> struct LaneWords<2> { typedef uint16_t codes; typedef uint32_t halves; };

// The run of n tokens t.. writing slots s.. of one block, for KV head h.
template <int D>
__device__ __forceinline__ void replay_run_i8(const half_t* __restrict__ src, const int32_t s, const int t,
                                              const int n, const int h, const int hkv, const int blk_tiles,
                                              int8_t* __restrict__ cache, half_t* __restrict__ scales) {
  constexpr int EPL = D / 64;  // dims per lane: 2 (d128) or 1 (d64)
  typedef typename LaneWords<EPL>::codes cw_t;   // a lane's codes of one row
  typedef typename LaneWords<EPL>::halves xw_t;  // a lane's halves of one new row
  const int lane = threadIdx.x & 63;
  const int o0 = s % kBlockSize;
  const int64_t sidx = (int64_t)(s / kBlockSize) * blk_tiles + h;
  int8_t* tile = cache + sidx * (kBlockSize * D) + lane * EPL;
  const half_t* row0 = src + ((int64_t)t * hkv + h) * D + lane * EPL;
  const int64_t rstride = (int64_t)hkv * D;

  // every load first (rows past the run re-read its last row)
  cw_t cw[kBlockSize];
  xw_t xw[kBlockSize];
#pragma unroll
  for (int j = 0; j < kBlockSize; ++j) cw[j] = *(const cw_t*)(tile + j * D);
#pragma unroll
  for (int r = 0; r < kBlockSize; ++r) xw[r] = *(const xw_t*)(row0 + min(r, n - 1) * rstride);
  float sc = (float)scales[sidx];

  // a new row's value (exact fp16 -> fp32), a code as a float
  auto xval = [&](int r, int e) {
    return (float)__builtin_bit_cast(half_t, (uint16_t)(xw[r] >> (16 * e)));
  };
  auto code = [&](cw_t w, int e) { return (float)(int8_t)(w >> (8 * e)); };
  auto pack = [&](const float* q) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) w |= (uint32_t)(uint8_t)(int8_t)(int)q[e] << (8 * e);
    return (cw_t)w;
  };
  auto lane_val = [](float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };

  // max|x| of each new row and the largest earlier |code|, in one batch
  float xm[kBlockSize + 1];
  float cm = 0.f;
#pragma unroll
  for (int j = 0; j < kBlockSize; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) cm = fmaxf(cm, (j < o0) ? fabsf(code(cw[j], e)) : 0.f);
#pragma unroll
  for (int r = 0; r < kBlockSize; ++r) {
    xm[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) xm[r] = fmaxf(xm[r], fabsf(xval(r, e)));
  }
  xm[kBlockSize] = cm;
  wave_max_all<kBlockSize + 1>(xm);
  cm = xm[kBlockSize];
  float xmv = 0.f;   // lane r: max|x| of new row r
#pragma unroll
  for (int r = 0; r < kBlockSize; ++r) xmv = lane == r ? xm[r] : xmv;

  // The scale recurrence, token by token, on wave-uniform values only.  Lane r
  // of spv / snv keeps the scale before / after token r; bit r of steps marks
  // a token that changed the scale (every earlier code is then requantised).
  float spv = 0.f, snv = 0.f;
  uint32_t steps = 0;
  for (int r = 0; r < n; ++r) {
    const float x = lane_val(xmv, r);
    const float amax = fmaxf(cm * fabsf(sc), x);
    const float sn = (float)(half_t)(amax / 127.0f);
    const bool keep = sn == sc && sn > 0.f && sn <= 65504.f && cm <= 127.f;
    if (!keep) {
      cm = o0 + r > 0 ? fabsf(quant_i8(cm * fabsf(sc), sn)) : 0.f;
      steps |= 1u << r;
    }
    if (cm < 127.f) cm = fmaxf(cm, fabsf(quant_i8(x, sn)));   // no code exceeds 127
    spv = lane == r ? sc : spv;
    snv = lane == r ? sn : snv;
    sc = sn;
  }

  // The run's rows: each quantised at its own token's scale, then requantised
  // at every later scale change, in token order.
  float cn[kBlockSize][EPL];
#pragma unroll
  for (int p = 0; p < kBlockSize; ++p)
    if (p < n) {
      const float sn = lane_val(snv, p);
#pragma unroll
      for (int e = 0; e < EPL; ++e) cn[p][e] = quant_i8(xval(p, e), sn);
    }
  for (uint32_t m = steps & ~1u; m != 0; m &= m - 1) {
    const int k = __builtin_ctz(m);
    const float sp = lane_val(spv, k), sn = lane_val(snv, k);
#pragma unroll
    for (int p = 0; p < kBlockSize - 1; ++p)
      if (p < k) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) cn[p][e] = quant_i8(cn[p][e] * sp, sn);
      }
  }
#pragma unroll
  for (int p = 0; p < kBlockSize; ++p)
    if (p < n) *(cw_t*)(tile + (o0 + p) * D) = pack(cn[p]);

  // The block's earlier rows: requantised at every scale change of the run.
  if (o0 > 0 && steps != 0) {
    for (uint32_t m = steps; m != 0; m &= m - 1) {
      const int k = __builtin_ctz(m);
      const float sp = lane_val(spv, k), sn = lane_val(snv, k);
#pragma unroll
      for (int j = 0; j < kBlockSize - 1; ++j)
        if (j < o0) {
          float q[EPL];
#pragma unroll
          for (int e = 0; e < EPL; ++e) q[e] = quant_i8(code(cw[j], e) * sp, sn);
          cw[j] = pack(q);
        }
    }
#pragma unroll
    for (int j = 0; j < kBlockSize - 1; ++j)
      if (j < o0) *(cw_t*)(tile + j * D) = cw[j];
  }
  if (lane == 0) scales[sidx] = (half_t)sc;
}

// Work item i = (window i / (2 * hkv), KV head and K or V i % (2 * hkv)), one
// wave each: it replays, in token order, every run that starts in its
// kI8Window tokens (a run may continue past the window; the tokens it covers
// there are not run starts and are skipped by the next window's wave).  Runs
// start every 16 tokens inside a chunk, so only some windows hold work; with
// the head index varying fastest, consecutive workgroups (which the hardware
// deals out to the XCDs in turn) carry equal work whichever windows those are.
// Lane i holds the slot of token t0 - 1 + i, so run starts and lengths come
// from one load and a ballot.
#ifndef PA_I8_WINDOW
#define PA_I8_WINDOW 4
#endif
constexpr int kI8Window = PA_I8_WINDOW;
constexpr int kI8MaxGrid = 1 << 20;
static_assert(kI8Window >= 1 && kI8Window + kBlockSize <= 64, "a window's slots and the run tails past it fit one wave");

template <int D>
__global__ __launch_bounds__(64) void write_i8_kernel(const half_t* __restrict__ k, const half_t* __restrict__ v,
                                                      const int32_t* __restrict__ slots, int32_t T, int32_t hkv,
                                                      int32_t blk_tiles, int64_t num_slots, int8_t* __restrict__ kc,
                                                      int8_t* __restrict__ vc, half_t* __restrict__ ks,
                                                      half_t* __restrict__ vs) {
  const int lane = threadIdx.x;
  const int64_t items = (((int64_t)T + kI8Window - 1) / kI8Window) * (2 * hkv);
  for (int64_t id = blockIdx.x; id < items; id += gridDim.x) {
    const int hw = (int)(id % (2 * hkv));
    const int t0 = (int)(id / (2 * hkv)) * kI8Window;
    const int h = hw >> 1, which = hw & 1;
    const half_t* src = which ? v : k;
    int8_t* cache = which ? vc : kc;
    half_t* scales = which ? vs : ks;
    const int ti = t0 - 1 + lane;
    const int32_t sl = (lane < kI8Window + kBlockSize && ti >= 0 && ti < T) ? slots[ti] : -1;
    for (int q = 0; q < kI8Window && t0 + q < T; ++q) {
      const int32_t s = __builtin_amdgcn_readlane(sl, q + 1);
      if (s < 0 || s >= num_slots) continue;
      if ((s % kBlockSize) != 0 && __builtin_amdgcn_readlane(sl, q) == s - 1) continue;  // inside an earlier run
      // token t0 + q + i (i >= 1) continues the run when it writes slot s + i of the same block
      const int i = lane - (q + 1);
      const bool more = i >= 1 && i < kBlockSize && sl == s + i && ((s + i) % kBlockSize) != 0;
      const uint64_t m = __ballot(more) >> (q + 2);   // bit i - 1 for token t0 + q + i
      const int n = 1 + __builtin_ctzll(~m);
      replay_run_i8<D>(src, s, t0 + q, n, h, hkv, blk_tiles, cache, scales);
    }
  }
}

hipError_t launch_write_i8(const pa_cache_desc& d, const void* k, const void* v, const int32_t* slots,
                           int32_t T, void* kc, void* vc, void* ks, void* vs, hipStream_t s) {
  const int64_t items = (((int64_t)T + kI8Window - 1) / kI8Window) * (2 * d.num_kv_heads);
  const int grid = (int)std::min<int64_t>(items, kI8MaxGrid);
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
