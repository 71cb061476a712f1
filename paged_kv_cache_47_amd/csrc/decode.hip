// Paged attention, vector path (decode and other short query groups), for gfx950.
//
// What is computed ([pytorch] "Compute reference attention without hiding
// the layout"): for each query row, scores q.k * scale over the keys it may
// see, softmax, weighted sum of V; KV head = query head / group.  The block
// table is walked inside the kernel, so no contiguous K/V copy is made
// ([pytorch] "Map the PyTorch design to vLLM PagedAttention").  Query row t of
// a sequence with q_len rows and kv_len keys sits at position
// kv_len - q_len + t and sees keys 0 .. that position ([engine] "03
// Correctness, and the bugs a real model found"), or only the last `window`
// of them ([pytorch] "PagedAttention vs sliding-window attention,
// RadixAttention, and SSMs"); the walk then starts at the 16-key block that
// holds the window's first key, and earlier blocks are never read.  int8 blocks are
// dequantised in registers before each of the two products ([engine] "INT8
// KV cache design").
//
// One workgroup per (query row, KV head, split-K partition); the G query
// heads of the KV head are processed together so every K/V element loaded
// from HBM serves all G rows.  K/V tiles arrive as 16-byte loads (one
// (block, head) tile is a contiguous 2-4 KB run); fp32 online softmax with a
// running max.  Rows split over several partitions are merged in
// log-sum-exp form by `reduce_kernel` (a kernel boundary, not a device-scope
// fence: each XCD has its own L2, so a device-wide release/acquire inside
// the kernel would write back and invalidate whole caches).
#include "units.h"

namespace pa {

// V of two token rows (same dims) -> (row0, row1) fp16 pairs per dim, the
// operand layout of v_dot2 over tokens.  fp16: one byte permute per pair.
// int8: interleave the two rows' codes, then the 0x64XX fp16 trick.
// N dwords of one lane's share of a token row (8 or 16 bytes per load).
template <int N>
struct Dw {
  uint32_t v[N];
};

__device__ __forceinline__ float dot2_first(half2_t a, half2_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float dot2_first(bf162_t a, bf162_t b) { return dot2(a, b, 0.f); }

template <bool I8, int N, typename T2>
__device__ __forceinline__ void v_token_pairs(const Dw<N>& r0, const Dw<N>& r1, T2* vp) {
  if constexpr (I8 && PA_I8_SDWA) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      vp[4 * c + 0] = sdwa_pair<0, 0>(r0.v[c], r1.v[c]);
      vp[4 * c + 1] = sdwa_pair<1, 1>(r0.v[c], r1.v[c]);
      vp[4 * c + 2] = sdwa_pair<2, 2>(r0.v[c], r1.v[c]);
      vp[4 * c + 3] = sdwa_pair<3, 3>(r0.v[c], r1.v[c]);
    }
  } else if constexpr (I8) {
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
      vp[2 * c + 0] = __builtin_bit_cast(T2, __builtin_amdgcn_perm(r1.v[c], r0.v[c], 0x05040100u));
      vp[2 * c + 1] = __builtin_bit_cast(T2, __builtin_amdgcn_perm(r1.v[c], r0.v[c], 0x07060302u));
    }
  }
}

// Lazy-rescale thresholds (log2 units): weights stay below 2^threshold.  For
// int8 pools a weight is multiplied by its block's V scale in fp16 before the
// product; scales reach 65504 / 127 (fp16 516), so 2^6.5 * 516 < 65504 keeps
// that product finite.
constexpr float kRescaleF16 = 8.0f;
constexpr float kRescaleI8 = 6.5f;

// fp16 scales are read with 16-bit buffer loads: any alignment, and the
// descriptor's range check keeps every read inside the array.  The loads of a
// tile's two scales are issued before its K and V loads (vector loads return
// in order), so waiting for the scales never waits for the tile behind them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scale_rsrc(const half_t* base, int64_t count) {
  const int64_t bytes = count > 0 ? 2 * count : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(bytes < INT32_MAX ? bytes : INT32_MAX), 0x00020000);
}
__device__ __forceinline__ uint16_t scale_bits(__amdgpu_buffer_rsrc_t rs, int64_t idx) {
  return __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(idx * 2), 0, 0);
}
__device__ __forceinline__ float half_bits_to_float(uint16_t b) { return (float)__builtin_bit_cast(half_t, b); }

// ============================================================ vector path ===
#ifndef PA_DECODE_NW
#define PA_DECODE_NW 4   // waves per workgroup
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1   // 1: K/V tile loads carry the nontemporal hint (each tile is read once)
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 2   // tiles in flight per wave while one is processed (fp16/bf16, some groups: 1 or 2)
#endif
#ifndef PA_DECODE_KQ
#define PA_DECODE_KQ 1      // int8 d128, G = 8: K read four lanes per token row (see the kernel)
#endif
#ifndef PA_DECODE_G8_OCC
#define PA_DECODE_G8_OCC 1  // d128, G = 8, 16-bit pools: registers bounded for two waves per SIMD
#endif
#ifndef PA_DECODE_RS
#define PA_DECODE_RS 1      // d128, G = 4: scores summed by reduce-scatter (see the kernel)
#endif

template <int N, bool NT = PA_DECODE_NT>
__device__ __forceinline__ Dw<N> load_dw(const uint32_t* p) {
  typedef uint32_t vec_t __attribute__((ext_vector_type(N)));
  vec_t x;
  if constexpr (NT) x = __builtin_nontemporal_load((const vec_t*)p);
  else x = *(const vec_t*)p;
  Dw<N> r;
#pragma unroll
  for (int c = 0; c < N; ++c) r.v[c] = x[c];
  return r;
}

// Waves per SIMD the compiler must leave room for.  16-bit pools at head dim
// 128 with eight rows otherwise take all 256 vector registers plus one
// accumulator register as spill room, which leaves one wave per SIMD.
template <int D, int G, int KV>
constexpr int decode_min_waves() {
  return (PA_DECODE_G8_OCC && D == 128 && G == 8 && KV != kKvI8) ? 2 : 1;
}

template <int D, int G, int KV, int NW, int VB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(decode_min_waves<D, G, KV>())))
void decode_kernel(AttnArgs a) {
  constexpr bool I8 = KV == kKvI8;
  using act_t = typename Act<KV>::t;   // 16-bit type of queries, weights and outputs
  using act2_t = typename Act<KV>::t2;
  constexpr int EB = I8 ? 1 : 2;       // bytes per element
  constexpr int ND = VB / 4;           // dwords per lane per load (VB = 8 or 16 bytes)
  constexpr int E = VB / EB;           // elements per lane per load
  constexpr int LPT = D / E;           // lanes per token row
  constexpr int TPL = 64 / LPT;        // token rows per wave-wide load
  constexpr int NL = kBlockSize / TPL; // loads per (block, head) tile
  constexpr int E2 = E / 2;            // fp16 pairs per lane per row
  constexpr int64_t TILE = (int64_t)kBlockSize * D * EB;
  // Two alternating tile buffers (no register copies between iterations).
  // int8 with G >= 4 gets them by keeping Q in LDS (below); with smaller
  // groups one loop body keeps more waves resident.
  constexpr bool PINGPONG = I8 ? G >= 4 : true;
  // 16-bit pools whose group fits beside a third buffer (G * D of 256 or 512:
  // d128 with G 2 or 4, d64 with G 4 or 8) keep two tiles in flight per wave
  // while a third is processed: fewer waves fit (two per SIMD at d128 G = 4
  // instead of three) but more bytes are in flight per compute unit.
  constexpr bool DEPTH2 = !I8 && PA_DECODE_DEPTH == 2 && G * D >= 256 && G * D <= 512;

  __shared__ float sm[NW][G], sl[NW][G];
  __shared__ float so[NW][G][D];
  // int8, G >= 4: the G query rows sit in LDS and each row's slice is read
  // just before its dot products, so 8 rather than G * 8 registers of Q are
  // live at a time, which makes room for the second tile buffer
  constexpr bool QLDS = I8 && G >= 4;
  __shared__ __attribute__((aligned(16))) act_t qs[QLDS ? G * D : 8];
  // int8 at head dim 128 with eight rows (8-byte V loads, 16 lanes per V row):
  // K is read four lanes per token row (32 bytes each: dims 16c + [0,16) and
  // 64 + 16c + [0,16) for lane c of the quad), so a score is summed in two
  // butterfly steps inside the quad instead of four across 16 lanes, and each
  // quad forms only its own token's weights.  A V lane group (16 lanes, tokens
  // grp + 4i) holds four quads, quad q owning token grp + 4q; the other tokens'
  // weights reach it with one DPP move each (row half-mirror: quad q ^ 1; row
  // rotate by 8: q ^ 2; row mirror: q ^ 3), and the lane loads its V rows in
  // that order (row i is token grp + 4 (q ^ i)), so pairs of loaded rows meet
  // pairs of weights.  Measured on 64 query heads over 8 int8 KV heads: 5%
  // faster than the 16-lane sums; with four rows (8 lanes per row) the same
  // layout was 7-13% slower than three butterfly steps, so it is not used there.
  constexpr bool KQ = I8 && QLDS && D == 128 && NL == 4 && PA_DECODE_KQ;
  // Head dim 128 with four rows (16-byte loads: an int8 token row spans 8
  // lanes, two token rows per lane; a 16-bit one spans 16 lanes, four token
  // rows per lane): the lanes of a token row hold the four query rows in a
  // lane-dependent order, slot j holding row fr ^ j, with fr chosen so that
  // the partner of each DPP step holds in the same register the rows this
  // lane keeps.  The sums then reduce-scatter without selects: two halving
  // steps (int8: row half-mirror, lane ^ 7, then quad xor 1; 16-bit: row
  // mirror, lane ^ 15, then row half-mirror) and all-reduce steps over the
  // rest of the row (quad xor 2; quad xor 1 and 2), and each lane ends with its
  // own row's scores: 8 DPP adds instead of 24 (int8), 20 instead of 64
  // (16-bit), and the softmax of one row (a quarter of the exponentials).  The
  // other rows' weight pairs come back with three DPP moves per pair (from1:
  // row fr ^ 1, from2: row fr ^ 2, both: fr ^ 3), so accumulator slot j is row
  // fr ^ j too; the rows return to their order once, after the last block.
  constexpr bool RS = D == 128 && G == 4 && PA_DECODE_RS &&
                      ((I8 && QLDS && LPT == 8 && NL == 2) || (!I8 && LPT == 16 && NL == 4));

  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps block indices scalar
  // this workgroup's unit: its sequence, query row, partition and the row's partition count
  Unit un;
  if (!resolve_unit<NW * 64>(a, h, un)) return;
  const int u = un.u, seq = un.seq, t = un.t, parts = un.parts, q_start = un.q_start;
  const int klo = un.klo, kbeg = un.kbeg, kend = un.kend;
  const int grp = lane / LPT, sub = lane % LPT;
  const int kquad = sub >> 2;   // KQ: the lane's quad inside its V lane group
  // RS: the row in slot 0 (int8: bits b0 ^ b2, b2 of the lane in its row; 16-bit: b2 ^ b3, b3)
  const int fr = LPT == 8 ? (((sub ^ (sub >> 2)) & 1) | (sub & 4) >> 1) : ((((sub >> 2) ^ (sub >> 3)) & 1) | (sub >> 2 & 2));
  // RS: the same register of the lane holding row fr ^ 1, and of the one holding fr ^ 2
  auto from1 = [&](float x) {
    if constexpr (LPT == 8) return dpp<0xB1>(x);
    else return dpp<0x141>(x);
  };
  auto from2 = [&](float x) {
    if constexpr (LPT == 8) return dpp<0x141>(x);
    else return dpp<0x140>(x);
  };
  const int64_t row0 = (int64_t)(q_start + t) * a.hq + (int64_t)h * G;
  const int32_t* tbl = a.block_tables + (int64_t)seq * a.max_blocks;

  // Fused KV write: the unit that walks the row's last key (the new token's
  // position) loads the token's K and V rows of this KV head and uses them
  // from registers in place of the pool's copy of that slot when it
  // processes the last block, so nothing in this kernel reads the slot; it
  // stores them into the slot after its walk (a store issued at the start
  // would hold up the wave's first tile loads until its data arrived).  Only the lanes that hold that
  // token in the last block's loads (in the wave that loads the block) take
  // part: each loads and stores its 16-byte chunk of the two rows.  No other
  // unit reads the slot: it lies past the row's other units and belongs to
  // this sequence alone.
  bool fused_last = false;   // wave-uniform: this wave processes the block holding the new token
  int new_i = 0, new_g = 0;  // the load (of NL) and the lane group holding the new token in that block
  int32_t new_slot = -1;     // where the rows are stored (after the walk: the store waits for its data)
  Dw<ND> new_kr{}, new_vr{};
  if constexpr (!I8) {
    const int last_blk = (kend + kBlockSize - 1) / kBlockSize - 1;
    if (a.new_k != nullptr && kend == un.kv_len && wave == (last_blk - kbeg / kBlockSize) % NW) {
      fused_last = true;
      const int o = (kend - 1) % kBlockSize;
      new_i = o / TPL;
      new_g = o % TPL;
      if (grp == new_g) {
        const int64_t tok = (int64_t)q_start + t;
        const int64_t row = (tok * a.hkv + h) * D;
        new_kr = load_dw<ND, false>((const uint32_t*)((const act_t*)a.new_k + row) + sub * ND);
        new_vr = load_dw<ND, false>((const uint32_t*)((const act_t*)a.new_v + row) + sub * ND);
        new_slot = a.new_slots[tok];
      }
    }
  }

  act2_t qh[QLDS ? 1 : G][E2];
  if constexpr (QLDS) {
    // the workgroup's G rows are contiguous: G * D / 8 chunks of 16 bytes
    const uint4* qp = (const uint4*)((const act_t*)a.q + row0 * D);
    for (int c = threadIdx.x; c < G * D / 8; c += NW * 64) ((uint4*)qs)[c] = qp[c];
    __syncthreads();
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4* qp = (const uint4*)((const act_t*)a.q + (row0 + (RS ? (fr ^ g) : g)) * D + sub * E);
#pragma unroll
      for (int c = 0; c < E / 8; ++c) {
        const uint4 w = qp[c];
        qh[g][4 * c + 0] = __builtin_bit_cast(act2_t, w.x);
        qh[g][4 * c + 1] = __builtin_bit_cast(act2_t, w.y);
        qh[g][4 * c + 2] = __builtin_bit_cast(act2_t, w.z);
        qh[g][4 * c + 3] = __builtin_bit_cast(act2_t, w.w);
      }
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
  const __amdgpu_buffer_rsrc_t ks_rs = scale_rsrc(a.ks, I8 ? a.scale_count : 0);
  const __amdgpu_buffer_rsrc_t vs_rs = scale_rsrc(a.vs, I8 ? a.scale_count : 0);
  // Physical block of a logical one (0 past the range, which is never loaded).
  // The entry is read one iteration before its tile's loads are issued, so
  // the scalar round trip overlaps the current block's work.
  // (The raw entry is kept; the range check happens when it is used.)
  auto table_at = [&](int blk) { return blk < bend ? tbl[blk] : 0; };
  // Issue the loads of one tile (for int8, first its two scales `kq`/`vq`,
  // fetched with the tile rather than when it is processed so that their
  // latency overlaps the current block's work too).
  auto load_tile = [&](int entry, Dw<ND>* kd, Dw<ND>* vd, uint16_t& kq, uint16_t& vq) {
    const int ph = clamp_block(entry, a.num_blocks);
    if constexpr (I8) {
      const int64_t sidx = (int64_t)ph * a.blk_tiles + h;
      kq = scale_bits(ks_rs, sidx);
      vq = scale_bits(vs_rs, sidx);
    }
    const int64_t off = ((int64_t)ph * a.blk_tiles + h) * TILE;
    const uint32_t* kt = (const uint32_t*)((const char*)a.kc + off);
    const uint32_t* vt2 = (const uint32_t*)((const char*)a.vc + off);
    if constexpr (KQ) {
      // token grp + TPL * kquad, two 16-byte pieces half a row apart, spread over the NL * ND dwords
      const uint32_t* kp = kt + (grp + TPL * kquad) * (D / 4) + (lane & 3) * 4;
      // each load covers half of every row of the tile, so the rows stay cached for the other
      const Dw<4> x0 = load_dw<4, false>(kp), x1 = load_dw<4, false>(kp + D / 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kd[w / ND].v[w % ND] = x0.v[w];
        kd[(w + 4) / ND].v[(w + 4) % ND] = x1.v[w];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) kd[i] = load_dw<ND>(kt + (i * 64 + lane) * ND);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) vd[i] = load_dw<ND>(vt2 + ((KQ ? (kquad ^ i) : i) * 64 + lane) * ND);
  };
  // One block of this wave: scores, softmax bookkeeping, P.V.  `kr`/`vr` hold
  // the block's K and V tile rows of this lane, `kq`/`vq` its int8 scales.
  auto process = [&](Dw<ND>* kr, Dw<ND>* vr, const uint16_t kq, const uint16_t vq, const int blk) {
    float ksc = a.scale_log2, vsc = 1.f;
    if constexpr (I8) {
      // a zero K scale (a block whose K rows are all zero) becomes the least
      // normal float: its scores stay 0 and masked ones stay -inf, not -inf * 0
      ksc = fmaxf(ksc * half_bits_to_float(kq), 1.17549435e-38f);
      vsc = half_bits_to_float(vq);
    }
    const int tok0 = blk * kBlockSize + grp;
    // wave-uniform: the last block of the range, or the block the window starts in
    const bool edge = blk * kBlockSize + kBlockSize > kend || blk * kBlockSize < klo;
    if constexpr (!I8) {
      // fused write: the new token's rows come from registers, not from the slot being stored
      if (fused_last && blk * kBlockSize + kBlockSize >= kend) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if (i == new_i && grp == new_g) {
            kr[i] = new_kr;
            vr[i] = new_vr;
          }
      }
    }
    // keys outside [klo, kend) (the slots past the range may hold anything)
    auto hidden = [&](int tok) { return (unsigned)(tok - klo) >= (unsigned)(kend - klo); };
    if (edge) {  // drop their V
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if (hidden(tok0 + (KQ ? (kquad ^ i) : i) * TPL)) vr[i] = Dw<ND>{};
    }

    if constexpr (KQ) {
      act2_t kh[16];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t x = kr[w / ND].v[w % ND];
        kh[2 * w] = sdwa_pair<0, 1>(x, x);
        kh[2 * w + 1] = sdwa_pair<2, 3>(x, x);
      }
      const int c = lane & 3;
      float s[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        act2_t qg[16];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const uint4 w = *(const uint4*)(qs + g * D + r * (D / 2) + 16 * c + 8 * h2);
            qg[8 * r + 4 * h2 + 0] = __builtin_bit_cast(act2_t, w.x);
            qg[8 * r + 4 * h2 + 1] = __builtin_bit_cast(act2_t, w.y);
            qg[8 * r + 4 * h2 + 2] = __builtin_bit_cast(act2_t, w.z);
            qg[8 * r + 4 * h2 + 3] = __builtin_bit_cast(act2_t, w.w);
          }
        float d = dot2_first(qg[0], kh[0]);
#pragma unroll
        for (int k = 1; k < 16; ++k) d = dot2(qg[k], kh[k], d);
        s[g] = d;
      }
      group_sum_all<4, G>(s);
      if (edge && hidden(tok0 + kquad * TPL)) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = -__builtin_inff();
      }
      // lazy rescale as below; the running max covers the lane group's NL tokens
      bool grow = false;
#pragma unroll
      for (int g = 0; g < G; ++g) grow |= s[g] * ksc > m[g] + kRescaleI8;
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float x = s[g] * ksc;
          x = fmaxf(x, dpp<0x141>(x));
          x = fmaxf(x, dpp<0x128>(x));
          if (x > m[g] + kRescaleI8) {
            const float al = fast_exp2(m[g] - x);
            m[g] = x;
            l[g] *= al;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] *= al;
          }
        }
      }
      // weights of the quad's own token (its own row sum), then the group's other tokens
      float wt[NL][G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(fmaf(s[g], ksc, -m[g]));
        l[g] += p;
        wt[0][g] = p * vsc;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        wt[1][g] = dpp<0x141>(wt[0][g]);
        wt[2][g] = dpp<0x128>(wt[0][g]);
        wt[3][g] = dpp<0x140>(wt[0][g]);
      }
#pragma unroll
      for (int j = 0; j < NL / 2; ++j) {
        act2_t vp[E];
        v_token_pairs<I8, ND>(vr[2 * j], vr[2 * j + 1], vp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const act2_t pp = (act2_t){(act_t)wt[2 * j][g], (act_t)wt[2 * j + 1][g]};
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = dot2(pp, vp[e], acc[g][e]);
        }
      }
      return;
    }

    if constexpr (RS) {
      float s[NL][G];   // token i, row slot j (row fr ^ j)
      if constexpr (I8) {
        act2_t kh[NL][E2];
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int c = 0; c < ND; ++c) {
            kh[i][2 * c] = sdwa_pair<0, 1>(kr[i].v[c], kr[i].v[c]);
            kh[i][2 * c + 1] = sdwa_pair<2, 3>(kr[i].v[c], kr[i].v[c]);
          }
#pragma unroll
        for (int j = 0; j < G; ++j) {
          act2_t qg[E2];
#pragma unroll
          for (int c = 0; c < E2 / 4; ++c) {
            const uint4 w = ((const uint4*)(qs + (fr ^ j) * D + sub * E))[c];
            qg[4 * c + 0] = __builtin_bit_cast(act2_t, w.x);
            qg[4 * c + 1] = __builtin_bit_cast(act2_t, w.y);
            qg[4 * c + 2] = __builtin_bit_cast(act2_t, w.z);
            qg[4 * c + 3] = __builtin_bit_cast(act2_t, w.w);
          }
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            float d = dot2_first(qg[0], kh[i][0]);
#pragma unroll
            for (int c = 1; c < E2; ++c) d = dot2(qg[c], kh[i][c], d);
            s[i][j] = d;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          act2_t kh[E2];
#pragma unroll
          for (int c = 0; c < ND; ++c) kh[c] = __builtin_bit_cast(act2_t, kr[i].v[c]);
#pragma unroll
          for (int j = 0; j < G; ++j) {   // qh[j] holds row fr ^ j
            float d = dot2_first(qh[j][0], kh[0]);
#pragma unroll
            for (int c = 1; c < E2; ++c) d = dot2(qh[j][c], kh[c], d);
            s[i][j] = d;
          }
        }
      }
      // halving steps, then the rest of the row
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) s[i][j] += from2(s[i][j ^ 2]);
#pragma unroll
      for (int i = 0; i < NL; ++i) s[i][0] += from1(s[i][1]);
      if constexpr (LPT == 16) {
#pragma unroll
        for (int i = 0; i < NL; ++i) s[i][0] += dpp<0xB1>(s[i][0]);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) s[i][0] += dpp<0x4E>(s[i][0]);
      if (edge) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if (hidden(tok0 + i * TPL)) s[i][0] = -__builtin_inff();
      }
      // lazy rescale as below, each lane testing its own row; the maxima of
      // the other slots' rows come from their owners
      constexpr float kRescale = I8 ? kRescaleI8 : kRescaleF16;
      float mb = s[0][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mb = fmaxf(mb, s[i][0]);
      mb *= ksc;
      if (__builtin_amdgcn_ballot_w64(mb > m[0] + kRescale)) {
        float mbs[G];
        mbs[0] = mb;
        mbs[1] = from1(mb);
        mbs[2] = from2(mb);
        mbs[3] = from2(mbs[1]);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          if (mbs[j] > m[j] + kRescale) {
            const float al = fast_exp2(m[j] - mbs[j]);
            m[j] = mbs[j];
            l[j] *= al;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] *= al;
          }
        }
      }
#pragma unroll
      for (int jp = 0; jp < NL / 2; ++jp) {
        const float p0 = fast_exp2(fmaf(s[2 * jp][0], ksc, -m[0]));
        const float p1 = fast_exp2(fmaf(s[2 * jp + 1][0], ksc, -m[0]));
        act2_t pw;
        if constexpr (I8) {
          l[0] += p0 + p1;   // only the own row's sum is kept (slot 0)
          pw = (act2_t){(act_t)(p0 * vsc), (act_t)(p1 * vsc)};
        } else {
          pw = (act2_t){(act_t)p0, (act_t)p1};
          // sum the rounded weights the product uses, so the output stays a convex combination
          l[0] = dot2(pw, (act2_t){(act_t)1.f, (act_t)1.f}, l[0]);
        }
        float pp[G];   // the weight pair of each slot's row, as raw bits
        pp[0] = __builtin_bit_cast(float, pw);
        pp[1] = from1(pp[0]);
        pp[2] = from2(pp[0]);
        pp[3] = from2(pp[1]);
        act2_t vp[E];
        v_token_pairs<I8, ND>(vr[2 * jp], vr[2 * jp + 1], vp);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const act2_t pj = __builtin_bit_cast(act2_t, pp[j]);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[j][e] = dot2(pj, vp[e], acc[j][e]);
        }
      }
      return;
    }

    // raw dot products q.k of this lane group's NL tokens for the G rows;
    // the score (base 2) is d * ksc, ksc > 0
    float s[NL][G];
    if constexpr (QLDS) {
      // both token rows' K as fp16 first, then one query row at a time from LDS
      act2_t kh[NL][E2];
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int c = 0; c < ND; ++c) {
          if constexpr (PA_I8_SDWA) {
            kh[i][2 * c] = sdwa_pair<0, 1>(kr[i].v[c], kr[i].v[c]);
            kh[i][2 * c + 1] = sdwa_pair<2, 3>(kr[i].v[c], kr[i].v[c]);
          } else {
            i8x4_to_h2(kr[i].v[c], kh[i][2 * c], kh[i][2 * c + 1]);
          }
        }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        act2_t qg[E2];
#pragma unroll
        for (int c = 0; c < E2 / 4; ++c) {
          const uint4 w = ((const uint4*)(qs + g * D + sub * E))[c];
          qg[4 * c + 0] = __builtin_bit_cast(act2_t, w.x);
          qg[4 * c + 1] = __builtin_bit_cast(act2_t, w.y);
          qg[4 * c + 2] = __builtin_bit_cast(act2_t, w.z);
          qg[4 * c + 3] = __builtin_bit_cast(act2_t, w.w);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float d = dot2_first(qg[0], kh[i][0]);
#pragma unroll
          for (int c = 1; c < E2; ++c) d = dot2(qg[c], kh[i][c], d);
          s[i][g] = d;
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      act2_t kh[E2];
      if constexpr (I8) {
#pragma unroll
        for (int c = 0; c < ND; ++c) {
          if constexpr (PA_I8_SDWA) {
            kh[2 * c] = sdwa_pair<0, 1>(kr[i].v[c], kr[i].v[c]);
            kh[2 * c + 1] = sdwa_pair<2, 3>(kr[i].v[c], kr[i].v[c]);
          } else {
            i8x4_to_h2(kr[i].v[c], kh[2 * c], kh[2 * c + 1]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < ND; ++c) kh[c] = __builtin_bit_cast(act2_t, kr[i].v[c]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // the first pair product starts the sum (the three-operand form takes a
        // zero addend, so no register has to be cleared first)
        float d = dot2_first(qh[g][0], kh[0]);
#pragma unroll
        for (int c = 1; c < E2; ++c) d = dot2(qh[g][c], kh[c], d);
        s[i][g] = d;
      }
    }
    }
    group_sum_all<LPT, NL * G>(&s[0][0]);
    if (edge) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (hidden(tok0 + i * TPL)) s[i][g] = -__builtin_inff();
    }

    // The running max moves only when a score exceeds it by more than
    // kRescale (log2 units), so weights stay <= 2^kRescale and the
    // accumulators are rescaled rarely.
    constexpr float kRescale = I8 ? kRescaleI8 : kRescaleF16;
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
        act2_t vp[E];
        v_token_pairs<I8, ND>(vr[2 * j], vr[2 * j + 1], vp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p0 = fast_exp2(fmaf(s[2 * j][g], ksc, -m[g]));
          const float p1 = fast_exp2(fmaf(s[2 * j + 1][g], ksc, -m[g]));
          act2_t pp;
          if constexpr (I8) {
            l[g] += p0 + p1;
            pp = (act2_t){(act_t)(p0 * vsc), (act_t)(p1 * vsc)};
          } else {
            pp = (act2_t){(act_t)p0, (act_t)p1};
            // sum the rounded weights the product uses, so the output stays a convex combination
            l[g] = dot2(pp, (act2_t){(act_t)1.f, (act_t)1.f}, l[g]);
          }
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = dot2(pp, vp[e], acc[g][e]);
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
  if constexpr (DEPTH2) {
    // three tile buffers used in turn: two tiles in flight while one is processed
    Dw<ND> ka[NL], va[NL], kb[NL], vb[NL], kc[NL], vc[NL];
    uint16_t kqa = 0, vqa = 0, kqb = 0, vqb = 0, kqc = 0, vqc = 0;
    if (b < bend) load_tile(table_at(b), ka, va, kqa, vqa);
    if (b + NW < bend) load_tile(table_at(b + NW), kb, vb, kqb, vqb);
    int pn = table_at(b + 2 * NW);
    while (b < bend) {
      if (b + 2 * NW < bend) load_tile(pn, kc, vc, kqc, vqc);
      pn = table_at(b + 3 * NW);
      process(ka, va, kqa, vqa, b);
      b += NW;
      if (b >= bend) break;
      if (b + 2 * NW < bend) load_tile(pn, ka, va, kqa, vqa);
      pn = table_at(b + 3 * NW);
      process(kb, vb, kqb, vqb, b);
      b += NW;
      if (b >= bend) break;
      if (b + 2 * NW < bend) load_tile(pn, kb, vb, kqb, vqb);
      pn = table_at(b + 3 * NW);
      process(kc, vc, kqc, vqc, b);
      b += NW;
    }
  } else if constexpr (PINGPONG) {
    // two tile buffers used in turn (no register copies between iterations)
    Dw<ND> ka[NL], va[NL], kb[NL], vb[NL];
    uint16_t kqa = 0, vqa = 0, kqb = 0, vqb = 0;
    int pn = table_at(b + NW);
    if (b < bend) load_tile(table_at(b), ka, va, kqa, vqa);
    while (b < bend) {
      if (b + NW < bend) load_tile(pn, kb, vb, kqb, vqb);
      pn = table_at(b + 2 * NW);
      process(ka, va, kqa, vqa, b);
      b += NW;
      if (b >= bend) break;
      if (b + NW < bend) load_tile(pn, ka, va, kqa, vqa);
      pn = table_at(b + 2 * NW);
      process(kb, vb, kqb, vqb, b);
      b += NW;
    }
  } else {
    // one loop body; the prefetched tile moves into the current one
    Dw<ND> kc[NL], vc[NL];
    uint16_t kqc = 0, vqc = 0;
    int pn = table_at(b + NW);
    if (b < bend) load_tile(table_at(b), kc, vc, kqc, vqc);
    while (b < bend) {
      Dw<ND> kn[NL], vn[NL];
      uint16_t kqn = 0, vqn = 0;
      if (b + NW < bend) load_tile(pn, kn, vn, kqn, vqn);
      pn = table_at(b + 2 * NW);
      process(kc, vc, kqc, vqc, b);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        kc[i] = kn[i];
        vc[i] = vn[i];
      }
      kqc = kqn;
      vqc = vqn;
      b += NW;
    }
  }

  // the fused write's store, once the walk no longer waits on this wave's loads
  if constexpr (!I8) {
    if (fused_last && grp == new_g && new_slot >= 0 && (int64_t)new_slot < (int64_t)a.num_blocks * kBlockSize) {
      const int64_t off =
          ((int64_t)(new_slot / kBlockSize) * a.blk_tiles + h) * TILE + (int64_t)(new_slot % kBlockSize) * D * EB;
      // the pools are the caller's writable memory; the attention reads them through const pointers
      uint32_t* dk = (uint32_t*)((char*)const_cast<void*>(a.kc) + off) + sub * ND;
      uint32_t* dv = (uint32_t*)((char*)const_cast<void*>(a.vc) + off) + sub * ND;
#pragma unroll
      for (int c = 0; c < ND; ++c) {
        dk[c] = new_kr.v[c];
        dv[c] = new_vr.v[c];
      }
    }
  }

  if constexpr (RS) {
    // the row sums from their owners (slot j holds row fr ^ j), then every
    // lane's rows back in order
    float ls[G];
    ls[0] = l[0];
    ls[1] = from1(l[0]);
    ls[2] = from2(l[0]);
    ls[3] = from2(ls[1]);
    auto pick = [&](int k, float x0, float x1, float x2, float x3) {
      return k == 0 ? x0 : k == 1 ? x1 : k == 2 ? x2 : x3;
    };
    float mr[G], lr[G], ar[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int k = g ^ fr;
      mr[g] = pick(k, m[0], m[1], m[2], m[3]);
      lr[g] = pick(k, ls[0], ls[1], ls[2], ls[3]);
#pragma unroll
      for (int e = 0; e < E; ++e) ar[g][e] = pick(k, acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = mr[g];
      l[g] = lr[g];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = ar[g][e];
    }
  }
  if constexpr (KQ) {
    // each quad summed its own token's weights: the lane group's row sums
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] += dpp<0x141>(l[g]);
      l[g] += dpp<0x128>(l[g]);
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
  const bool split = parts > 1;
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
      ((act_t*)a.out)[(row0 + g) * D + d] = (act_t)(O / Ls);
    } else {
      const int64_t pr = (int64_t)u * a.hq + (int64_t)h * G + g;
      a.po[pr * D + d] = O / Ls;
      if (d == 0) a.plse[pr] = M + __builtin_log2f(Ls);
    }
  }
}

// Merge the split-K partials of one (query row, KV head): its G query heads,
// base-2 log-sum-exp: out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
// The kernel is a short chain of dependent loads (where the row's units are,
// then their log-sum-exps and partials), so the partials of the first
// kPrefetch units are loaded before the weights are formed.
template <int D, int G, typename OUT>
__global__ __launch_bounds__(256) void reduce_kernel(AttnArgs a) {
  const int h = blockIdx.y;
  int u0, parts;
  int64_t row0;
  if (a.selfplan) {
    // grid x = sequence; its first unit recorded where the row's units are
    // (written every call by that unit: one query row per sequence, each with units)
    const int2 ru = a.row_u0[blockIdx.x];
    u0 = ru.x;
    parts = ru.y;
    if (parts <= 1) return;
    if (u0 < 0 || (int64_t)u0 + parts > a.n_units) return;   // only if device and host lengths disagree
    row0 = (int64_t)blockIdx.x * a.hq + (int64_t)h * G;
  } else {
    const VTok vt = a.vtok[blockIdx.x];
    if (vt.seq < 0 || vt.parts <= 1) return;
    const SeqInfo si = a.seqs[vt.seq];
    u0 = vt.u0;
    parts = vt.parts;
    row0 = (int64_t)(si.q_start + vt.t) * a.hq + (int64_t)h * G;
  }
  // Up to kMaxParts partials: the weights 2^(lse_p - M) / sum_p 2^(lse_p - M)
  // of each query head are formed once in LDS, and every output element is a
  // plain weighted sum of its partials (the element loop below otherwise
  // re-reads the log-sum-exps of every partial for each of the G * D elements).
  constexpr int kMaxParts = 64;
  constexpr int kPer = (G * D + 255) / 256;   // output elements per thread
  constexpr int kPrefetch = 4;
  __shared__ float wsh[G][kMaxParts];
  if (parts <= kMaxParts) {
    float pre[kPer][kPrefetch];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = threadIdx.x + 256 * k;
      const int g = idx / D, d = idx % D;
#pragma unroll
      for (int p = 0; p < kPrefetch; ++p)
        pre[k][p] = (idx < G * D && p < parts)
                        ? a.po[((int64_t)(u0 + p) * a.hq + (int64_t)h * G + g) * D + d] : 0.f;
    }
    for (int i = threadIdx.x; i < G * parts; i += 256)
      wsh[i / parts][i % parts] = a.plse[(int64_t)(u0 + i % parts) * a.hq + (int64_t)h * G + i / parts];
    __syncthreads();
    if (threadIdx.x < G) {
      float* w = wsh[threadIdx.x];
      float M = -__builtin_inff();
      for (int p = 0; p < parts; ++p) M = fmaxf(M, w[p]);
      float S = 0.f;
      for (int p = 0; p < parts; ++p) {
        w[p] = fast_exp2(w[p] - M);
        S += w[p];
      }
      const float inv = 1.f / S;
      for (int p = 0; p < parts; ++p) w[p] *= inv;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = threadIdx.x + 256 * k;
      if (idx >= G * D) break;
      const int g = idx / D, d = idx % D;
      const float* po = a.po + ((int64_t)u0 * a.hq + (int64_t)h * G + g) * D + d;
      float O = 0.f;
#pragma unroll
      for (int p = 0; p < kPrefetch; ++p)
        if (p < parts) O = fmaf(wsh[g][p], pre[k][p], O);
      for (int p = kPrefetch; p < parts; ++p) O = fmaf(wsh[g][p], po[(int64_t)p * a.hq * D], O);
      ((OUT*)a.out)[(row0 + g) * D + d] = (OUT)O;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int g = idx / D, d = idx % D;
    const int64_t col = (int64_t)h * G + g;
    float M = -__builtin_inff();
    for (int p = 0; p < parts; ++p) M = fmaxf(M, a.plse[(int64_t)(u0 + p) * a.hq + col]);
    float S = 0.f, O = 0.f;
    for (int p = 0; p < parts; ++p) {
      const int64_t pr = (int64_t)(u0 + p) * a.hq + col;
      const float wgt = fast_exp2(a.plse[pr] - M);
      S += wgt;
      O = fmaf(wgt, a.po[pr * D + d], O);
    }
    ((OUT*)a.out)[(row0 + g) * D + d] = (OUT)(O / S);
  }
}

// =============================================================== dispatch ===
#ifndef PA_DECODE_VB_I8
#define PA_DECODE_VB_I8 16  // bytes per lane per load for int8 pools (8: twice the lanes per row)
#endif

template <int D, int KV>
static hipError_t decode_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  // 16-byte loads per lane; 8-byte int8 loads halve the per-lane registers
  // (4 waves/SIMD) but add reduction and softmax work, and measure slower
  constexpr int kVB = KV == kKvI8 ? PA_DECODE_VB_I8 : 16;
  dim3 grid(n, a.hkv);
  switch (g) {
    case 1: decode_kernel<D, 1, KV, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    case 2: decode_kernel<D, 2, KV, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    case 4: decode_kernel<D, 4, KV, PA_DECODE_NW, kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    // int8 with eight rows: 8-byte loads, so the accumulators (G x elements per lane) fit two waves per SIMD
    case 8: decode_kernel<D, 8, KV, PA_DECODE_NW, KV == kKvI8 ? 8 : kVB><<<grid, PA_DECODE_NW * 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t decode_d(const AttnArgs& a, int g, int kv, int n, hipStream_t s) {
  switch (kv) {
    case kKvF16: return decode_g<D, kKvF16>(a, g, n, s);
    case kKvI8: return decode_g<D, kKvI8>(a, g, n, s);
    case kKvBF16: return decode_g<D, kKvBF16>(a, g, n, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const AttnArgs& a, int head_dim, int group, int kv, int n, hipStream_t s) {
  // groups of 16 or more rows: the same units on the matrix cores (decode_mfma.hip)
  if (group >= 16) return launch_decode_mfma(a, head_dim, group, kv, n, s);
  return head_dim == 128 ? decode_d<128>(a, group, kv, n, s) : decode_d<64>(a, group, kv, n, s);
}

template <int D, typename OUT>
static hipError_t reduce_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  dim3 grid(n, a.hkv);
  switch (g) {
    case 1: reduce_kernel<D, 1, OUT><<<grid, 256, 0, s>>>(a); break;
    case 2: reduce_kernel<D, 2, OUT><<<grid, 256, 0, s>>>(a); break;
    case 4: reduce_kernel<D, 4, OUT><<<grid, 256, 0, s>>>(a); break;
    case 8: reduce_kernel<D, 8, OUT><<<grid, 256, 0, s>>>(a); break;
    case 16: reduce_kernel<D, 16, OUT><<<grid, 256, 0, s>>>(a); break;
    case 32: reduce_kernel<D, 32, OUT><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const AttnArgs& a, int head_dim, int group, int kv, int n_vtok, hipStream_t s) {
  if (kv == kKvBF16)
    return head_dim == 128 ? reduce_g<128, bf16_t>(a, group, n_vtok, s) : reduce_g<64, bf16_t>(a, group, n_vtok, s);
  return head_dim == 128 ? reduce_g<128, half_t>(a, group, n_vtok, s) : reduce_g<64, half_t>(a, group, n_vtok, s);
}

}  // namespace pa
