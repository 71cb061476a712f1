// Paged attention for query groups of 16 or 32 rows on the matrix cores
// (decode and other single-row-per-sequence work with G = 16 or 32), for gfx950.
//
// What is computed is the vector path's ([pytorch] "Compute reference
// attention without hiding the layout": KV head = query head / group, which
// may leave 16 or more query heads per KV head): for one query row of a
// sequence, its G query heads attend over the keys they may see ([engine]
// "03 Correctness, and the bugs a real model found"), walking the block
// table in the kernel ([pytorch] "Map the PyTorch design to vLLM
// PagedAttention").  With G = 16 or 32 rows per KV head the work is a dense
// contraction (16 or 32 rows x 16 keys x head_dim per block), so it runs on
// the matrix cores; it is still bound by the K/V bytes.
//
// Work units are the vector path's (one query row, one KV head, one split-K
// partition; see units.h); partials go through the same merge kernel.  Four
// waves take the unit's 16-key blocks in turn.  Per block:
//   S^T = K Q^T  on v_mfma_f32_16x16x32: K rows are loaded straight into the
//                A-operand layout (lane: key l % 16, eight dims), Q sits in
//                registers as the B operand (lane: query row l % 16);
//   the online softmax on the accumulator (lane: query row l % 16, keys
//                4 * (l / 16) + e), whose layout is also the B operand of
//   O^T += V^T P^T  on v_mfma_f32_16x16x16: V is written to a per-wave LDS
//                tile in its natural layout and read back transposed
//                (ds_read_b64_tr_b16), four keys per lane.
// int8 blocks ([engine] "INT8 KV cache design"): K and V codes become exact
// fp16; the K scale multiplies the scores, the V scale the weights.
#include "units.h"

namespace pa {

constexpr int kMfmaDecodeWaves = 4;
#ifndef PA_MFD_NTV
#define PA_MFD_NTV 1   // V tile loads (whole 128-byte lines per instruction) with the nontemporal hint
#endif
#ifndef PA_MFD_NTK
#define PA_MFD_NTK 0   // K tile loads (half lines per instruction, the other half read by the next) likewise
#endif
#ifndef PA_MFD_KLDS
#define PA_MFD_KLDS 1  // K loaded like V (whole lines, nontemporal) and read as operands from LDS
#endif
template <typename T>
__device__ __forceinline__ T ldk(const char* p) {
  if constexpr (PA_MFD_NTK) return __builtin_nontemporal_load((const T*)p);
  else return *(const T*)p;
}
#ifndef PA_MFD_DEPTH
#define PA_MFD_DEPTH 2   // tiles in flight per wave while one is processed (groups of 16: 1 or 2)
#endif

__device__ __forceinline__ float bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(half_t, b); }

__device__ __forceinline__ float4_t mfma16x16x16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16x16x16(bf164_t a, bf164_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a), __builtin_bit_cast(short4_t, b),
                                                    c, 0, 0, 0);
}

template <int D, int G, int KV>
__global__ __launch_bounds__(64 * kMfmaDecodeWaves) void decode_mfma_kernel(AttnArgs a) {
  constexpr bool I8 = KV == kKvI8;
  using act_t = typename Act<KV>::t;
  using act4_t = typename Act<KV>::t4;
  using act8_t = typename Act<KV>::t8;
  constexpr int NW = kMfmaDecodeWaves;
  constexpr int RB = G / 16;   // 16-row blocks of the query group
  constexpr int KS = D / 32;   // k-steps of S over the head dim
  constexpr int NT = D / 16;   // 16-wide column tiles of O
  constexpr int EB = I8 ? 1 : 2;
  constexpr int LDV = D + 16;  // LDS row stride of a V tile (halves)
  constexpr int VL = kBlockSize * D * EB / (64 * 16);   // 16-byte V loads per lane per block
  constexpr int64_t TILE = (int64_t)kBlockSize * D * EB;
  // Lazy-rescale thresholds (log2 units): weights stay below 2^thr.  int8
  // weights are multiplied by the block's V scale (up to 516) in fp16, so
  // 2^6.5 * 516 < 65504 keeps them finite.
  constexpr float kThr = I8 ? 6.5f : 8.0f;
  static_assert(G == 16 || G == 32, "groups of 16 or 32");
  constexpr bool DEPTH2 = G == 16 && PA_MFD_DEPTH == 2;
  // K rows are loaded whole (like V, every instruction covering whole 128-byte
  // lines, nontemporal) and staged through a per-wave LDS tile (int8: as exact
  // fp16 codes) from which the A operands are read; loading them straight into
  // the operand layout reads half (int8: quarter) lines per instruction.
  constexpr bool KLDS = PA_MFD_KLDS;
  constexpr int LDK = D + 8;   // LDS row stride of a K tile (halves): conflict-free operand reads

  // one V (and K) tile per wave: a wave's LDS accesses stay in program order
  __shared__ __attribute__((aligned(16))) half_t vtile[NW][kBlockSize * LDV];
  __shared__ __attribute__((aligned(16))) half_t ktile[KLDS ? NW : 1][KLDS ? kBlockSize * LDK : 8];
  __shared__ float sm[NW][G];
  // merge buffer of the waves' accumulators; rows padded by 4 floats so the 16
  // rows a column tile writes at once fall on different LDS banks
  constexpr int LDA = D + 4;
  __shared__ float sacc[G * LDA];
  __shared__ float ssum[G];

  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  Unit un;
  if (!resolve_unit<NW * 64>(a, h, un)) return;
  const int64_t row0 = (int64_t)(un.q_start + un.t) * a.hq + (int64_t)h * G;   // first of the G query rows
  const int32_t* tbl = a.block_tables + (int64_t)un.seq * a.max_blocks;

  // Q as the B operand of S^T: lane (grp, l16) holds query row rb * 16 + l16, dims ks * 32 + 8 * grp + [0, 8).
  // From 16 rows at head dim 128 up the operands are read from LDS at each use instead of being
  // held in 16-32 registers, which keeps one more wave per SIMD (three at G = 16, two at G = 32).
  constexpr bool QLDS = G * D >= 2048;
  constexpr int LDQ = D + 8;
  __shared__ __attribute__((aligned(16))) act_t sq[QLDS ? G * LDQ : 8];
  act8_t qop[QLDS ? 1 : RB][KS];
  if constexpr (QLDS) {
    for (int c = threadIdx.x; c < G * D / 8; c += NW * 64)
      *(act8_t*)&sq[(c / (D / 8)) * LDQ + (c % (D / 8)) * 8] = *((const act8_t*)((const act_t*)a.q + row0 * D) + c);
    __syncthreads();
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qop[rb][ks] = *(const act8_t*)((const act_t*)a.q + (row0 + rb * 16 + l16) * D + ks * 32 + 8 * grp);
  }
  auto q_operand = [&](int rb, int ks) -> act8_t {
    if constexpr (QLDS) return *(const act8_t*)&sq[(rb * 16 + l16) * LDQ + ks * 32 + 8 * grp];
    else return qop[rb][ks];
  };

  float4_t o[RB][NT];
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    lsum[rb] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[rb][nt] = (float4_t)0.f;
  }

  // A block's registers: K in the A-operand layout (16-bit pools: one 16-byte
  // load per k-step; int8: eight codes per k-step), V in its natural layout
  // (chunk c = i * 64 + lane: key c / (D * EB / 16), 16 bytes at (c % (D * EB / 16)) * 16).
  struct Tile {
    u32x4_t k[KLDS ? VL : (I8 ? KS / 2 : KS)];
    u32x4_t v[VL];
    float ksc, vsc;
  };
  const __amdgpu_buffer_rsrc_t ks_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.ks, 0, I8 ? (int)(a.scale_count * 2 < INT32_MAX ? a.scale_count * 2 : INT32_MAX) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t vs_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.vs, 0, I8 ? (int)(a.scale_count * 2 < INT32_MAX ? a.scale_count * 2 : INT32_MAX) : 0, 0x00020000);
  const int bend = (un.kend + kBlockSize - 1) / kBlockSize;
  auto load_tile = [&](int blk, Tile& tl) {
    const int ph = clamp_block(tbl[blk], a.num_blocks);
    const int64_t tile = (int64_t)ph * a.blk_tiles + h;
    const char* kt = (const char*)a.kc + tile * TILE;
    const char* vt = (const char*)a.vc + tile * TILE;
    if constexpr (KLDS) {
#pragma unroll
      for (int i = 0; i < VL; ++i) tl.k[i] = __builtin_nontemporal_load((const u32x4_t*)(kt + (i * 64 + lane) * 16));
    }
    if constexpr (I8) {
      // codes of key l16, dims 32 * ks + 8 * grp + [0, 8): 8 bytes per k-step, two k-steps per register quad
#pragma unroll
      for (int j = 0; j < (KLDS ? 0 : KS / 2); ++j) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t lo = ldk<u32x2_t>(kt + l16 * D + (2 * j) * 32 + 8 * grp);
        const u32x2_t hi = ldk<u32x2_t>(kt + l16 * D + (2 * j + 1) * 32 + 8 * grp);
        tl.k[j] = (u32x4_t){lo.x, lo.y, hi.x, hi.y};
      }
      // a zero K scale becomes the least normal float: masked scores stay -inf, not -inf * 0
      tl.ksc = fmaxf(a.scale_log2 * bits_to_float(__builtin_amdgcn_raw_buffer_load_b16(ks_rs, (int)(tile * 2), 0, 0)),
                     1.17549435e-38f);
      tl.vsc = bits_to_float(__builtin_amdgcn_raw_buffer_load_b16(vs_rs, (int)(tile * 2), 0, 0));
    } else {
#pragma unroll
      for (int ks = 0; ks < (KLDS ? 0 : KS); ++ks) tl.k[ks] = ldk<u32x4_t>(kt + (l16 * D + ks * 32 + 8 * grp) * 2);
      tl.ksc = a.scale_log2;
      tl.vsc = 1.f;
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const u32x4_t* vp = (const u32x4_t*)(vt + (i * 64 + lane) * 16);
      tl.v[i] = PA_MFD_NTV ? __builtin_nontemporal_load(vp) : *vp;
    }
  };

  auto process = [&](const Tile& tl, int blk) {
    // V into this wave's LDS tile (fp16 codes for int8), read back transposed below
    half_t* vd = vtile[wave];
    if constexpr (KLDS && I8) {
      // K codes into this wave's K tile as exact fp16, read back below as A operands
      constexpr int CPR = D / 16;   // 16-code chunks per key row
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int c = i * 64 + lane, key = c / CPR, col = (c % CPR) * 16;
        const uint32_t w[4] = {tl.k[i][0], tl.k[i][1], tl.k[i][2], tl.k[i][3]};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const half2_t a0 = sdwa_pair<0, 1>(w[2 * q], w[2 * q]), a1 = sdwa_pair<2, 3>(w[2 * q], w[2 * q]);
          const half2_t a2 = sdwa_pair<0, 1>(w[2 * q + 1], w[2 * q + 1]);
          const half2_t a3 = sdwa_pair<2, 3>(w[2 * q + 1], w[2 * q + 1]);
          *(half8_t*)(ktile[wave] + key * LDK + col + 8 * q) = (half8_t){a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        }
      }
    } else if constexpr (KLDS) {
      // K rows into this wave's K tile, read back below as A operands
      constexpr int CPR = D / 8;
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int c = i * 64 + lane;
        *(u32x4_t*)(ktile[wave] + (c / CPR) * LDK + (c % CPR) * 8) = tl.k[i];
      }
    }
    if constexpr (I8) {
      constexpr int CPR = D / 16;   // 16-code chunks per key row
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int c = i * 64 + lane, key = c / CPR, col = (c % CPR) * 16;
        const uint32_t w[4] = {tl.v[i][0], tl.v[i][1], tl.v[i][2], tl.v[i][3]};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const half2_t a0 = sdwa_pair<0, 1>(w[2 * q], w[2 * q]), a1 = sdwa_pair<2, 3>(w[2 * q], w[2 * q]);
          const half2_t a2 = sdwa_pair<0, 1>(w[2 * q + 1], w[2 * q + 1]);
          const half2_t a3 = sdwa_pair<2, 3>(w[2 * q + 1], w[2 * q + 1]);
          *(half8_t*)(vd + key * LDV + col + 8 * q) = (half8_t){a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        }
      }
    } else {
      constexpr int CPR = D / 8;    // 8-element chunks per key row
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int c = i * 64 + lane;
        *(u32x4_t*)(vd + (c / CPR) * LDV + (c % CPR) * 8) = tl.v[i];
      }
    }
    __builtin_amdgcn_wave_barrier();   // the wave's own LDS writes precede its transposed reads

    // S^T = K Q^T: lane (grp, l16) gets keys 4 * grp + e of the block for query row rb * 16 + l16
    float4_t s[RB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      act8_t kop;
      if constexpr (KLDS) {
        kop = *(const act8_t*)(ktile[wave] + l16 * LDK + ks * 32 + 8 * grp);
      } else if constexpr (I8) {
        const uint32_t w0 = tl.k[ks / 2][2 * (ks & 1)], w1 = tl.k[ks / 2][2 * (ks & 1) + 1];
        const half2_t c0 = sdwa_pair<0, 1>(w0, w0), c1 = sdwa_pair<2, 3>(w0, w0);
        const half2_t c2 = sdwa_pair<0, 1>(w1, w1), c3 = sdwa_pair<2, 3>(w1, w1);
        kop = (half8_t){c0.x, c0.y, c1.x, c1.y, c2.x, c2.y, c3.x, c3.y};
      } else {
        kop = __builtin_bit_cast(act8_t, tl.k[ks]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb] = mfma16x16x32(kop, q_operand(rb, ks), ks == 0 ? (float4_t)0.f : s[rb]);
    }
    // keys outside [klo, kend): only the block holding the range's start or end has any
    if (blk * kBlockSize < un.klo || blk * kBlockSize + kBlockSize > un.kend) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = blk * kBlockSize + 4 * grp + e;
        if (key < un.klo || key >= un.kend)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[rb][e] = -__builtin_inff();
      }
    }
    // online softmax, base 2, with lazy rescaling (the row max moves only past kThr)
    float mb[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      mb[rb] = fmaxf(fmaxf(s[rb][0], s[rb][1]), fmaxf(s[rb][2], s[rb][3])) * tl.ksc;
      grow |= mb[rb] > m[rb] + kThr;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float x = fmaxf(mb[rb], __shfl_xor(mb[rb], 16, 64));
        x = fmaxf(x, __shfl_xor(x, 32, 64));
        const bool g = x > m[rb] + kThr;   // the same for the row's four lanes
        const float al = g ? fast_exp2(m[rb] - x) : 1.f;
        m[rb] = g ? x : m[rb];
        lsum[rb] *= al;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[rb][nt] *= al;
      }
    }
    act4_t p[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = fast_exp2(fmaf(s[rb][e], tl.ksc, -m[rb]));
        if constexpr (I8) {
          lsum[rb] += w;
          p[rb][e] = (act_t)(w * tl.vsc);
        } else {
          p[rb][e] = (act_t)w;
          lsum[rb] += (float)p[rb][e];   // the rounded weights the product uses
        }
      }
    }
    // O^T += V^T P^T, one 16-dim column tile at a time
    typedef __attribute__((address_space(3))) short4_t lds_short4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const half_t* p1 = vd + (4 * grp + (l16 >> 2)) * LDV + nt * 16 + 4 * (l16 & 3);
      const act4_t vq = __builtin_bit_cast(act4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p1));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][nt] = mfma16x16x16(vq, p[rb], o[rb][nt]);
    }
    __builtin_amdgcn_wave_barrier();   // the reads of this tile precede the next write to it
  };

  // the wave's blocks in turn, the next block's tile in flight while one is
  // processed; with 16 rows two tiles in flight (a three-tile ring)
  int b = un.kbeg / kBlockSize + wave;
  if constexpr (DEPTH2) {
    Tile ta, tb, tc;
    if (b < bend) load_tile(b, ta);
    if (b + NW < bend) load_tile(b + NW, tb);
    while (b < bend) {
      if (b + 2 * NW < bend) load_tile(b + 2 * NW, tc);
      process(ta, b);
      b += NW;
      if (b >= bend) break;
      if (b + 2 * NW < bend) load_tile(b + 2 * NW, ta);
      process(tb, b);
      b += NW;
      if (b >= bend) break;
      if (b + 2 * NW < bend) load_tile(b + 2 * NW, tb);
      process(tc, b);
      b += NW;
    }
  } else {
    Tile ta, tb;
    if (b < bend) load_tile(b, ta);
    while (b < bend) {
      if (b + NW < bend) load_tile(b + NW, tb);
      process(ta, b);
      b += NW;
      if (b >= bend) break;
      if (b + NW < bend) load_tile(b + NW, ta);
      process(tb, b);
      b += NW;
    }
  }

  // row sums over the row's four lanes, then the waves merged in turn through LDS
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += __shfl_xor(lsum[rb], 16, 64);
    lsum[rb] += __shfl_xor(lsum[rb], 32, 64);
    if (grp == 0) sm[wave][rb * 16 + l16] = m[rb];
  }
  __syncthreads();
  float f[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float M = sm[0][rb * 16 + l16];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][rb * 16 + l16]);
    f[rb] = fast_exp2(m[rb] - M);
  }
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + l16;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* dst = &sacc[row * LDA + nt * 16 + 4 * grp + e];
            *dst = (w == 0 ? 0.f : *dst) + o[rb][nt][e] * f[rb];
          }
        if (grp == 0) ssum[row] = (w == 0 ? 0.f : ssum[row]) + lsum[rb] * f[rb];
      }
    }
    __syncthreads();
  }
  const bool split = un.parts > 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D, d = idx % D;
    float M = sm[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][g]);
    const float L = ssum[g], O = sacc[g * LDA + d];
    if (!split) {
      ((act_t*)a.out)[(row0 + g) * D + d] = (act_t)(O / L);
    } else {
      const int64_t pr = (int64_t)un.u * a.hq + (int64_t)h * G + g;
      a.po[pr * D + d] = O / L;
      if (d == 0) a.plse[pr] = M + __builtin_log2f(L);
    }
  }
}

template <int D, int KV>
static hipError_t decode_mfma_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  const dim3 grid(n, a.hkv);
  switch (g) {
    case 16: decode_mfma_kernel<D, 16, KV><<<grid, 64 * kMfmaDecodeWaves, 0, s>>>(a); break;
    case 32: decode_mfma_kernel<D, 32, KV><<<grid, 64 * kMfmaDecodeWaves, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t decode_mfma_d(const AttnArgs& a, int g, int kv, int n, hipStream_t s) {
  switch (kv) {
    case kKvF16: return decode_mfma_g<D, kKvF16>(a, g, n, s);
    case kKvI8: return decode_mfma_g<D, kKvI8>(a, g, n, s);
    case kKvBF16: return decode_mfma_g<D, kKvBF16>(a, g, n, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const AttnArgs& a, int head_dim, int group, int kv, int n, hipStream_t s) {
  return head_dim == 128 ? decode_mfma_d<128>(a, group, kv, n, s) : decode_mfma_d<64>(a, group, kv, n, s);
}

}  // namespace pa
