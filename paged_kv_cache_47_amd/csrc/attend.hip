// Paged attention kernels for gfx950.
//
// What is computed ([pytorch] "Compute reference attention without hiding
// the layout"): for each query row, scores q.k * scale over the keys it may
// see, softmax, weighted sum of V; KV head = query head / group.  The block
// table is walked inside the kernels, so no contiguous K/V copy is made
// ([pytorch] "Map the PyTorch design to vLLM PagedAttention").  Query row t of
// a sequence with q_len rows and kv_len keys sits at position
// kv_len - q_len + t and sees keys 0 .. that position ([engine] "03
// Correctness, and the bugs a real model found").  int8 blocks are
// dequantised in registers before each of the two products ([engine] "INT8
// KV cache design").
//
// Two paths:
//  * vector path (decode and other short query groups): one workgroup per
//    (query row, KV head, split-K partition); the G query heads of the KV head
//    are processed together so every K/V element loaded from HBM serves all G
//    rows.  K/V tiles arrive as 16-byte loads (one (block, head) tile is a
//    contiguous 2-4 KB run); fp32 online softmax with a running max.  Rows
//    split over several partitions are merged in log-sum-exp form by
//    `reduce_kernel` (a kernel boundary, not a device-scope fence: each XCD
//    has its own L2, so a device-wide release/acquire inside the kernel would
//    write back and invalidate whole caches).
//  * MFMA path (prefill / chunked prefill, q_len * G >= 16 rows): 128 query
//    rows per workgroup (4 waves x 32), 64 keys per step, S^T = K Q^T and
//    O^T = V^T P^T on v_mfma_f32_16x16x32_f16.  Computing the transposes makes
//    each lane own one query row in both accumulators, and the P accumulator
//    already sits in the B-operand layout of the second product.  V is staged
//    in LDS and read with the gfx950 transposing LDS read.
#include "pa_internal.h"

namespace pa {

// bytes b0 b1 of a dword of int8 codes -> exact fp16 pair, via 0x64XX = 1024 + XX
__device__ __forceinline__ void i8x4_to_h2(uint32_t w, half2_t& lo, half2_t& hi) {
  const uint32_t u = w ^ 0x80808080u;  // biased: XX = code + 128
  const uint32_t l = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t h = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  lo = __builtin_bit_cast(half2_t, l) - bias;
  hi = __builtin_bit_cast(half2_t, h) - bias;
}

// V of two token rows (same dims) -> (row0, row1) fp16 pairs per dim, the
// operand layout of v_dot2 over tokens.  fp16: one byte permute per pair.
// int8: interleave the two rows' codes, then the 0x64XX fp16 trick.
// N dwords of one lane's share of a token row (8 or 16 bytes per load).
template <int N>
struct Dw {
  uint32_t v[N];
};

template <bool I8, int N>
__device__ __forceinline__ void v_token_pairs(const Dw<N>& r0, const Dw<N>& r1, half2_t* vp) {
  if constexpr (I8) {
    const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint32_t x = r0.v[c] ^ 0x80808080u, y = r1.v[c] ^ 0x80808080u;
      const uint32_t t01 = __builtin_amdgcn_perm(y, x, 0x05010400u);  // x.b0 y.b0 x.b1 y.b1
      const uint32_t t23 = __builtin_amdgcn_perm(y, x, 0x07030602u);  // x.b2 y.b2 x.b3 y.b3
      vp[4 * c + 0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t01, 0x04010400u)) - bias;
      vp[4 * c + 1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t01, 0x04030402u)) - bias;
      vp[4 * c + 2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t23, 0x04010400u)) - bias;
      vp[4 * c + 3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, t23, 0x04030402u)) - bias;
    }
  } else {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      vp[2 * c + 0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(r1.v[c], r0.v[c], 0x05040100u));
      vp[2 * c + 1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(r1.v[c], r0.v[c], 0x07060302u));
    }
  }
}

constexpr float kRescale = 8.0f;

// fp16 scale at a wave-uniform index, read as the aligned dword that holds it
// (a scalar load; 16-bit loads would go through the vector memory path).
__device__ __forceinline__ float scale_at(const half_t* base, int64_t idx) {
  const uint32_t w = ((const uint32_t*)base)[idx >> 1];
  const uint16_t bits = (idx & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(half_t, bits);
}

// ============================================================ vector path ===
#ifndef PA_DECODE_NW
#define PA_DECODE_NW 4   // waves per workgroup
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1   // 1: K/V tile loads carry the nontemporal hint (each tile is read once)
#endif

template <int N>
__device__ __forceinline__ Dw<N> load_dw(const uint32_t* p) {
  typedef uint32_t vec_t __attribute__((ext_vector_type(N)));
#if PA_DECODE_NT
  const vec_t x = __builtin_nontemporal_load((const vec_t*)p);
#else
  const vec_t x = *(const vec_t*)p;
#endif
  Dw<N> r;
#pragma unroll
  for (int c = 0; c < N; ++c) r.v[c] = x[c];
  return r;
}

template <int D, int G, bool I8, int NW, int VB>
__global__ __launch_bounds__(NW * 64) void decode_kernel(AttnArgs a) {
  constexpr int EB = I8 ? 1 : 2;       // bytes per element
  constexpr int ND = VB / 4;           // dwords per lane per load (VB = 8 or 16 bytes)
  constexpr int E = VB / EB;           // elements per lane per load
  constexpr int LPT = D / E;           // lanes per token row
  constexpr int TPL = 64 / LPT;        // token rows per wave-wide load
  constexpr int NL = kBlockSize / TPL; // loads per (block, head) tile
  constexpr int E2 = E / 2;            // fp16 pairs per lane per row
  constexpr int64_t TILE = (int64_t)kBlockSize * D * EB;
#ifndef PA_DECODE_PINGPONG_I8
#define PA_DECODE_PINGPONG_I8 0
#endif
  // two alternating tile buffers for fp16; int8 keeps one loop body (fewer live registers)
  constexpr bool PINGPONG = I8 ? (PA_DECODE_PINGPONG_I8 != 0) : true;

  __shared__ float sm[NW][G], sl[NW][G];
  __shared__ float so[NW][G][D];

  const int u = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps block indices scalar
  const int2 un = a.vunit[u];
  if (un.x < 0) return;
  const VTok vt = a.vtok[un.x];
  if (vt.seq < 0) return;
  const SeqInfo si = a.seqs[vt.seq];
  const int nvis = si.kv_len - si.q_len + vt.t + 1;
  const int kbeg = un.y * a.part;
  const int kend = min(nvis, kbeg + a.part);
  const int grp = lane / LPT, sub = lane % LPT;
  const int64_t row0 = (int64_t)(si.q_start + vt.t) * a.hq + (int64_t)h * G;
  const int32_t* tbl = a.block_tables + (int64_t)vt.seq * a.max_blocks;

  half2_t qh[G][E2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4* qp = (const uint4*)(a.q + (row0 + g) * D + sub * E);
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const uint4 w = qp[c];
      qh[g][4 * c + 0] = __builtin_bit_cast(half2_t, w.x);
      qh[g][4 * c + 1] = __builtin_bit_cast(half2_t, w.y);
      qh[g][4 * c + 2] = __builtin_bit_cast(half2_t, w.z);
      qh[g][4 * c + 3] = __builtin_bit_cast(half2_t, w.w);
    }
  }

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const int bend = (kend + kBlockSize - 1) / kBlockSize;
  int b = kbeg / kBlockSize + wave;
  auto load_tile = [&](int blk, Dw<ND>* kd, Dw<ND>* vd, int& ph) {
    ph = clamp_block(tbl[blk], a.num_blocks);
    const int64_t off = ((int64_t)ph * a.hkv + h) * TILE;
    const uint32_t* kt = (const uint32_t*)((const char*)a.kc + off);
    const uint32_t* vt2 = (const uint32_t*)((const char*)a.vc + off);
#pragma unroll
    for (int i = 0; i < NL; ++i) kd[i] = load_dw<ND>(kt + (i * 64 + lane) * ND);
#pragma unroll
    for (int i = 0; i < NL; ++i) vd[i] = load_dw<ND>(vt2 + (i * 64 + lane) * ND);
  };
  // One block of this wave: scores, softmax bookkeeping, P.V.  `kr`/`vr` hold
  // the block's K and V tile rows of this lane.
  auto process = [&](Dw<ND>* kr, Dw<ND>* vr, const int phys, const int blk) {
    float ksc = a.scale_log2, vsc = 1.f;
    if constexpr (I8) {
      ksc *= scale_at(a.ks, (int64_t)phys * a.hkv + h);
      vsc = scale_at(a.vs, (int64_t)phys * a.hkv + h);
    }
    const int tok0 = blk * kBlockSize + grp;
    const bool tail = blk * kBlockSize + kBlockSize > kend;  // wave-uniform: last block of the range
    if (tail) {  // drop V of keys past the range (their slots may hold anything)
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (tok0 + i * TPL >= kend) vr[i] = Dw<ND>{};
    }

    // raw dot products q.k of this lane group's NL tokens for the G rows;
    // the score (base 2) is d * ksc, ksc > 0
    float s[NL][G];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      half2_t kh[E2];
      if constexpr (I8) {
#pragma unroll
        for (int c = 0; c < ND; ++c) i8x4_to_h2(kr[i].v[c], kh[2 * c], kh[2 * c + 1]);
      } else {
#pragma unroll
        for (int c = 0; c < ND; ++c) kh[c] = __builtin_bit_cast(half2_t, kr[i].v[c]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < E2; ++c) d = __builtin_amdgcn_fdot2(qh[g][c], kh[c], d, false);
        s[i][g] = d;
      }
    }
    group_sum_all<LPT, NL * G>(&s[0][0]);
    if (tail) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (tok0 + i * TPL >= kend) s[i][g] = -__builtin_inff();
    }

    // The running max moves only when a score exceeds it by more than
    // kRescale (log2 units), so weights stay <= 2^kRescale and the
    // accumulators are rescaled rarely.
    bool grow = false;
    float mb[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = s[0][g];
#pragma unroll
      for (int i = 1; i < NL; ++i) x = fmaxf(x, s[i][g]);
      mb[g] = x * ksc;
      grow |= mb[g] > m[g] + kRescale;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (mb[g] > m[g] + kRescale) {
          const float al = fast_exp2(m[g] - mb[g]);
          m[g] = mb[g];
          l[g] *= al;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] *= al;
        }
      }
    }

    if constexpr (NL >= 2) {
      // P.V on v_dot2_f32_f16 over token pairs: vp[e] = (V[tok 2j][e], V[tok 2j+1][e])
#pragma unroll
      for (int j = 0; j < NL / 2; ++j) {
        half2_t vp[E];
        v_token_pairs<I8, ND>(vr[2 * j], vr[2 * j + 1], vp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p0 = fast_exp2(fmaf(s[2 * j][g], ksc, -m[g]));
          const float p1 = fast_exp2(fmaf(s[2 * j + 1][g], ksc, -m[g]));
          half2_t pp;
          if constexpr (I8) {
            l[g] += p0 + p1;
            pp = (half2_t){(half_t)(p0 * vsc), (half_t)(p1 * vsc)};
          } else {
            pp = (half2_t){(half_t)p0, (half_t)p1};
            // sum the rounded weights the product uses, so the output stays a convex combination
            l[g] = __builtin_amdgcn_fdot2(pp, (half2_t){(half_t)1.f, (half_t)1.f}, l[g], false);
          }
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = __builtin_amdgcn_fdot2(pp, vp[e], acc[g][e], false);
        }
      }
    } else {
      // one token row per lane per block (int8, head_dim 64)
      float vf[E];
#pragma unroll
      for (int c = 0; c < ND; ++c) {
        half2_t lo, hi;
        i8x4_to_h2(vr[0].v[c], lo, hi);
        vf[4 * c + 0] = (float)lo.x * vsc;
        vf[4 * c + 1] = (float)lo.y * vsc;
        vf[4 * c + 2] = (float)hi.x * vsc;
        vf[4 * c + 3] = (float)hi.y * vsc;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p0 = fast_exp2(fmaf(s[0][g], ksc, -m[g]));
        l[g] += p0;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p0, vf[e], acc[g][e]);
      }
    }
  };

  // The wave's next block is in flight while the current one is processed.
  if constexpr (PINGPONG) {
    // two tile buffers used in turn (no register copies between iterations)
    Dw<ND> ka[NL], va[NL], kb[NL], vb[NL];
    int pha = 0, phb = 0;
    if (b < bend) load_tile(b, ka, va, pha);
    while (b < bend) {
      if (b + NW < bend) load_tile(b + NW, kb, vb, phb);
      process(ka, va, pha, b);
      b += NW;
      if (b >= bend) break;
      if (b + NW < bend) load_tile(b + NW, ka, va, pha);
      process(kb, vb, phb, b);
      b += NW;
    }
  } else {
    // one loop body; the prefetched tile moves into the current one
    Dw<ND> kc[NL], vc[NL];
    int phc = 0;
    if (b < bend) load_tile(b, kc, vc, phc);
    while (b < bend) {
      Dw<ND> kn[NL], vn[NL];
      int phn = 0;
      if (b + NW < bend) load_tile(b + NW, kn, vn, phn);
      process(kc, vc, phc, b);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        kc[i] = kn[i];
        vc[i] = vn[i];
      }
      phc = phn;
      b += NW;
    }
  }

  // merge the TPL token-row streams of this wave (lane groups), then the waves
#pragma unroll
  for (int msk = LPT; msk < 64; msk <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], msk, 64);
      const float lo = __shfl_xor(l[g], msk, 64);
      const float mn = fmaxf(m[g], mo);
      const float fa = fast_exp2(m[g] - mn), fb = fast_exp2(mo - mn);
      l[g] = l[g] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = acc[g][e] * fa + __shfl_xor(acc[g][e], msk, 64) * fb;
      m[g] = mn;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) so[wave][g][sub * E + e] = acc[g][e];
      if (sub == 0) {
        sm[wave][g] = m[g];
        sl[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  const bool split = vt.parts > 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D, d = idx % D;
    float M = sm[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][g]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm[w][g] - M);
      Ls += sl[w][g] * f;
      O += so[w][g][d] * f;
    }
    if (!split) {
      a.out[(row0 + g) * D + d] = (half_t)(O / Ls);
    } else {
      const int64_t pr = (int64_t)u * a.hq + (int64_t)h * G + g;
      a.po[pr * D + d] = O / Ls;
      if (d == 0) a.plse[pr] = M + __builtin_log2f(Ls);
    }
  }
}

// Merge the split-K partials of one (query row, KV head): its G query heads,
// base-2 log-sum-exp: out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
template <int D, int G>
__global__ __launch_bounds__(256) void reduce_kernel(AttnArgs a) {
  const VTok vt = a.vtok[blockIdx.x];
  if (vt.seq < 0 || vt.parts <= 1) return;
  const int h = blockIdx.y;
  const SeqInfo si = a.seqs[vt.seq];
  const int64_t row0 = (int64_t)(si.q_start + vt.t) * a.hq + (int64_t)h * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D, d = idx % D;
    const int64_t col = (int64_t)h * G + g;
    float M = -__builtin_inff();
    for (int p = 0; p < vt.parts; ++p) M = fmaxf(M, a.plse[(int64_t)(vt.u0 + p) * a.hq + col]);
    float S = 0.f, O = 0.f;
    for (int p = 0; p < vt.parts; ++p) {
      const int64_t pr = (int64_t)(vt.u0 + p) * a.hq + col;
      const float wgt = fast_exp2(a.plse[pr] - M);
      S += wgt;
      O = fmaf(wgt, a.po[pr * D + d], O);
    }
    a.out[(row0 + g) * D + d] = (half_t)(O / S);
  }
}

// ============================================================== MFMA path ===
// One workgroup = 4 waves = 128 query rows of one (sequence, KV head); each
// wave owns 32 rows as two 16-row MFMA blocks, so every K or V operand read
// from LDS feeds two MFMAs.  Keys advance 64 at a time (four 16-key blocks):
// the next 64-key K and V tiles are loaded from HBM into registers while the
// current tiles in LDS are used, then written to the other LDS buffer; one
// barrier per step.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaBN = 64;
#ifndef PA_PF_PADK
#define PA_PF_PADK 16  // K tile row padding (halves)
#endif
#ifndef PA_PF_PADV
#define PA_PF_PADV 16  // V tile row padding (halves)
#endif
#ifndef PA_PF_WSWAP
#define PA_PF_WSWAP 0  // int8 tiles: stagger the order of each thread's two LDS stores
#endif
// Lazy-rescale threshold of the MFMA path (log2 units): weights stay below
// 2^6, so an int8 weight times its V scale (at most 65504 / 127) stays finite in fp16.
constexpr float kRescalePf = 6.0f;

template <int D, int G, bool I8>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnArgs a) {
  constexpr int KS = D / 32;        // k-steps of 32 over the head dim
  constexpr int NT = D / 16;        // 16-wide output column tiles
  constexpr int BN = kMfmaBN;       // keys per step
  constexpr int KB = BN / 16;       // 16-key blocks per step
  constexpr int RB = 2;             // 16-row MFMA blocks per wave
  constexpr int LDK = D + PA_PF_PADK;  // LDS row strides (halves) of the K and V tiles
  constexpr int LDV = D + PA_PF_PADV;
  constexpr int EB = I8 ? 1 : 2;
  constexpr int CPR = D * EB / 16;  // 16-byte chunks per key row in the pool
  constexpr int PT = BN * CPR / 256;  // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) half_t ldk[2][BN * LDK];  // [buffer]
  __shared__ __attribute__((aligned(16))) half_t ldv[2][BN * LDV];

  const int id = blockIdx.x;
  const int h = id % a.hkv;         // consecutive workgroups = consecutive KV heads (one XCD each when hkv = 8)
  const int2 mu = a.munit[id / a.hkv];
  if (mu.x < 0) return;
  const SeqInfo si = a.seqs[mu.x];
  const int L = si.kv_len, Q = si.q_len, rows = Q * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps block indices scalar
  const int l16 = lane & 15, grp = lane >> 4;
  const int r0 = mu.y * kMfmaRows;
  const int last_row = min(rows, r0 + kMfmaRows) - 1;
  const int kmax = min(L, L - Q + last_row / G + 1);
  const int32_t* tbl = a.block_tables + (int64_t)mu.x * a.max_blocks;
  const int qmin = L - Q + (r0 + wave * 32) / G;  // query position of this wave's first row

  int qpos[RB];
  int64_t orow[RB];
  bool rvalid[RB];
  half8_t qop[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = r0 + wave * 32 + rb * 16 + l16;
    rvalid[rb] = row < rows;
    const int tq = rvalid[rb] ? row / G : 0;
    qpos[rb] = rvalid[rb] ? L - Q + tq : -1;
    orow[rb] = ((int64_t)(si.q_start + tq) * a.hq + (int64_t)h * G + row % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[rb][ks] = rvalid[rb] ? *(const half8_t*)(a.q + orow[rb] + ks * 32 + 8 * grp) : (half8_t)(half_t)0.f;
  }

  float4_t o[RB][NT];
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    lsum[rb] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[rb][nt] = (float4_t)0.f;
  }

  uint4 stk[PT], stv[PT];
  float nks[KB], nvs[KB];  // int8: K and V scales of the 16-key blocks of the tiles in flight
  // Physical blocks, read one step before the tiles they address: per 16-key
  // block of the step (int8: for its scales), and per staging chunk of this
  // wave (its 64 lanes cover 64 / CPR <= 16 aligned keys, one 16-key block).
  // Blocks past the sequence repeat its last block (always inside the table
  // row); no key of theirs is loaded, and their scores are masked.  The reads
  // go through the vector memory path (vz is a zero the compiler cannot prove
  // uniform): scalar loads share a counter with LDS reads, so every LDS read
  // of the step would wait for them.
  const int last_blk = (L - 1) / kBlockSize;   // L >= q_len >= 1 for a row tile
  const int vz = lane & (a.hkv >> 30);          // 0 (hkv is small and positive)
  struct Blocks {
    int kb[KB];
    int chunk[PT];
  };
  auto table = [&](int kt, Blocks& t) {
    if constexpr (I8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) t.kb[kb] = tbl[min(kt / kBlockSize + kb, last_blk) + vz];
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int key0 = (64 * wave + 256 * i) / CPR;
      t.chunk[i] = tbl[min((kt + key0) / kBlockSize, last_blk) + vz];
    }
  };
  auto gload = [&](int kt, const Blocks& t) {
    if constexpr (I8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int64_t sidx = (int64_t)clamp_block(t.kb[kb], a.num_blocks) * a.hkv + h;
        nks[kb] = (float)a.ks[sidx];
        nvs[kb] = (float)a.vs[sidx];
      }
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int key = c / CPR, ch = c % CPR;
      const int kg = kt + key;
      if (kg < L) {
        const int ph = clamp_block(t.chunk[i], a.num_blocks);
        const int64_t off = ((((int64_t)ph * a.hkv + h) * kBlockSize + (kg % kBlockSize)) * D) * EB + ch * 16;
        stk[i] = *(const uint4*)((const char*)a.kc + off);
        stv[i] = *(const uint4*)((const char*)a.vc + off);
      } else {
        stk[i] = make_uint4(0, 0, 0, 0);
        stv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int key = c / CPR, ch = c % CPR;
      if constexpr (I8) {
        half_t* kd = &ldk[buf][key * LDK + ch * 16];
        half_t* vd = &ldv[buf][key * LDV + ch * 16];
        const uint32_t kw[4] = {stk[i].x, stk[i].y, stk[i].z, stk[i].w};
        const uint32_t vw[4] = {stv[i].x, stv[i].y, stv[i].z, stv[i].w};
        half8_t k0, k1, v0, v1;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          half2_t a0, a1, a2, a3, b0, b1, b2, b3;
          i8x4_to_h2(kw[2 * c2], a0, a1);
          i8x4_to_h2(kw[2 * c2 + 1], a2, a3);
          i8x4_to_h2(vw[2 * c2], b0, b1);
          i8x4_to_h2(vw[2 * c2 + 1], b2, b3);
          const half8_t kk = (half8_t){a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
          const half8_t vv = (half8_t){b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
          if (c2 == 0) { k0 = kk; v0 = vv; } else { k1 = kk; v1 = vv; }
        }
        if (PA_PF_WSWAP && (ch & 4)) {  // upper half of the row first: the two stores of 8 lanes hit distinct banks
          *(half8_t*)(kd + 8) = k1;
          *(half8_t*)(vd + 8) = v1;
          *(half8_t*)kd = k0;
          *(half8_t*)vd = v0;
        } else {
          *(half8_t*)kd = k0;
          *(half8_t*)vd = v0;
          *(half8_t*)(kd + 8) = k1;
          *(half8_t*)(vd + 8) = v1;
        }
      } else {
        *(uint4*)&ldk[buf][key * LDK + ch * 8] = stk[i];
        *(uint4*)&ldv[buf][key * LDV + ch * 8] = stv[i];
      }
    }
  };

  Blocks tn, tn2;
  table(0, tn);
  gload(0, tn);
  lstore(0);
  table(BN, tn);
  __syncthreads();
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  int buf = 0;
  // One 64-key step: S = K Q^T for the four 16-key blocks (this lane: query
  // row l16 of each row block, keys 16*kb + 4*grp + e), the online-softmax
  // max, then the fp16 weights and O^T += V^T P^T per 32-key half, so that the
  // second half's vector work sits beside the first half's matrix products,
  // and the next tiles' staging beside the second half's.
  //
  // Only steps that reach past this wave's first query position need the
  // causal mask (a wave-uniform test); it sets the hidden raw scores to -inf.
  // The max is taken on raw scores and scaled once per 16-key block (scales
  // are positive), and the scale rides in the exponent's FMA.  The running max
  // moves only when a score exceeds it by more than kRescalePf (log2 units),
  // so the accumulators are rescaled rarely.
  for (int kt = 0; kt < kmax; kt += BN, buf ^= 1) {
    const bool more = kt + BN < kmax;
    // score scale per 16-key block (base 2; int8 folds in the block's K scale).  A zero K scale
    // (an all-zero block) becomes the least normal float: its scores stay 0, and -inf stays -inf.
    float cks[KB], vscl[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      cks[kb] = I8 ? fmaxf(a.scale_log2 * nks[kb], 1.17549435e-38f) : a.scale_log2;
      vscl[kb] = I8 ? nvs[kb] : 1.f;
    }
    // the staging at the end of the step is unconditional, so it can share a block with the
    // matrix work; after the last step it rewrites the idle buffer with tiles nothing reads
    if (more) {
      gload(kt + BN, tn);
      table(kt + 2 * BN, tn2);
    }

    float4_t s[RB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kb] = (float4_t)0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const half8_t kop = *(const half8_t*)&ldk[buf][(kb * 16 + l16) * LDK + ks * 32 + 8 * grp];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[rb][ks], s[rb][kb], 0, 0, 0);
      }
    }
    if (kt + BN - 1 > qmin) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kt + kb * 16 + 4 * grp + e > qpos[rb]) s[rb][kb][e] = -__builtin_inff();
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mb = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float r = fmaxf(fmaxf(s[rb][kb][0], s[rb][kb][1]), fmaxf(s[rb][kb][2], s[rb][kb][3]));
        mb = fmaxf(mb, r * cks[kb]);
      }
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const bool grow = mb > m[rb] + kRescalePf;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float al = grow ? fast_exp2(m[rb] - mb) : 1.f;
        m[rb] = grow ? mb : m[rb];
        lsum[rb] *= al;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[rb][nt] *= al;
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      half8_t p[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kb = 2 * hh + j / 4;
          const float w = fast_exp2(fmaf(s[rb][kb][j % 4], cks[kb], -m[rb]));
          half_t ph;
          if constexpr (I8) {
            ps += w;
            ph = (half_t)(w * vscl[kb]);
          } else {
            ph = (half_t)w;  // the weight the product uses is also the one summed
            ps += (float)ph;
          }
          // slot j of the k-step: keys 4*grp + [0..3] of the half's first and second 16-key block
          p[rb][j] = ph;
        }
        lsum[rb] += ps;   // this lane's share of the row sum; the row's four lanes are added at the end
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const half_t* p1 = &ldv[buf][(hh * 32 + 4 * grp + (l16 >> 2)) * LDV + nt * 16 + 4 * (l16 & 3)];
        const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p1);
        const short4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1 + 16 * LDV));
        const half4_t h1 = __builtin_bit_cast(half4_t, v1), h2 = __builtin_bit_cast(half4_t, v2);
        const half8_t vop = (half8_t){h1.x, h1.y, h1.z, h1.w, h2.x, h2.y, h2.z, h2.w};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, p[rb], o[rb][nt], 0, 0, 0);
      }
    }
    lstore(buf ^ 1);
    if (more) tn = tn2;
    __syncthreads();
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += __shfl_xor(lsum[rb], 16, 64);
    lsum[rb] += __shfl_xor(lsum[rb], 32, 64);
    if (!rvalid[rb]) continue;
    const float inv = 1.f / lsum[rb];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      half4_t r;
      r.x = (half_t)(o[rb][nt][0] * inv);
      r.y = (half_t)(o[rb][nt][1] * inv);
      r.z = (half_t)(o[rb][nt][2] * inv);
      r.w = (half_t)(o[rb][nt][3] * inv);
      *(half4_t*)(a.out + orow[rb] + nt * 16 + 4 * grp) = r;
    }
  }
}

// =============================================================== dispatch ===
#ifndef PA_DECODE_VB_I8
#define PA_DECODE_VB_I8 16  // bytes per lane per load for int8 pools (8: twice the lanes per row)
#endif

template <int D, bool I8>
static hipError_t decode_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  // 16-byte loads per lane; 8-byte int8 loads halve the per-lane registers
  // (4 waves/SIMD) but add reduction and softmax work, and measure slower
  constexpr int kVB = I8 ? PA_DECODE_VB_I8 : 16;
  dim3 grid(n, a.hkv);
  switch (g) {
    case 1: decode_kernel<D, 1, I8, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    case 2: decode_kernel<D, 2, I8, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    case 4: decode_kernel<D, 4, I8, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    case 8: decode_kernel<D, 8, I8, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, int head_dim, int group, bool i8, int n, hipStream_t s) {
  if (head_dim == 128) return i8 ? decode_g<128, true>(a, group, n, s) : decode_g<128, false>(a, group, n, s);
  return i8 ? decode_g<64, true>(a, group, n, s) : decode_g<64, false>(a, group, n, s);
}

template <int D>
static hipError_t reduce_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  dim3 grid(n, a.hkv);
  switch (g) {
    case 1: reduce_kernel<D, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: reduce_kernel<D, 2><<<grid, 256, 0, s>>>(a); break;
    case 4: reduce_kernel<D, 4><<<grid, 256, 0, s>>>(a); break;
    case 8: reduce_kernel<D, 8><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const AttnArgs& a, int head_dim, int group, int n_vtok, hipStream_t s) {
  return head_dim == 128 ? reduce_g<128>(a, group, n_vtok, s) : reduce_g<64>(a, group, n_vtok, s);
}

template <int D, bool I8>
static hipError_t prefill_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  const dim3 grid(n * a.hkv);   // workgroup id = row tile * hkv + KV head
  switch (g) {
    case 1: prefill_kernel<D, 1, I8><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 2: prefill_kernel<D, 2, I8><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 4: prefill_kernel<D, 4, I8><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 8: prefill_kernel<D, 8, I8><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnArgs& a, int head_dim, int group, bool i8, int n, hipStream_t s) {
  if (head_dim == 128) return i8 ? prefill_g<128, true>(a, group, n, s) : prefill_g<128, false>(a, group, n, s);
  return i8 ? prefill_g<64, true>(a, group, n, s) : prefill_g<64, false>(a, group, n, s);
}

}  // namespace pa
