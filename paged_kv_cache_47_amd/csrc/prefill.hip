// Paged attention, MFMA path (prefill and chunked prefill), for gfx950.
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
// RadixAttention, and SSMs").  int8 blocks are dequantised before the two
// products ([engine] "INT8 KV cache design").
//
// Sequences with q_len * G >= 16 rows take this path: kMfmaRows query rows
// per workgroup (kMfmaWaves waves x 32), 64 keys per step, S^T = K Q^T and O^T = V^T P^T
// on v_mfma_f32_16x16x32_f16 (_bf16 for bf16 pools).  Computing the transposes makes each lane own
// one query row in both accumulators, and the P accumulator already sits in
// the B-operand layout of the second product.  V is staged in LDS and read
// with the gfx950 transposing LDS read.
#include "mfma_tile.h"

namespace pa {

// ============================================================== MFMA path ===
// One workgroup = kMfmaWaves waves = kMfmaRows query rows of one (sequence,
// KV head); each wave owns 32 rows as two 16-row MFMA blocks, so every K or V
// operand read from LDS feeds two MFMAs.  Keys advance 64 at a time (four
// 16-key blocks): the next 64-key K and V tiles are loaded from HBM into
// registers while the current tiles in LDS are used, then written to the
// other LDS buffer; one barrier per step.  The more waves share a tile, the
// less staging (loads, int8 conversion, LDS stores) each wave does per step.
#ifndef PA_PF_PRIO
#define PA_PF_PRIO 0   // 1: raise the wave's issue priority over the S = K Q^T products
#endif
#ifndef PA_PF_PADK
#define PA_PF_PADK 16  // K tile row padding (halves)
#endif
#ifndef PA_PF_PADV
#define PA_PF_PADV 16  // V tile row padding (halves)
#endif
// Lazy-rescale threshold of the MFMA path (log2 units): weights stay below 2^8.
constexpr float kRescalePf = 8.0f;

template <int D, int G, int KV>
__global__ __launch_bounds__(64 * kMfmaWaves, 8 / kMfmaWaves) void prefill_kernel(AttnArgs a) {
  constexpr bool I8 = KV == kKvI8;
  using act_t = typename Act<KV>::t;     // 16-bit operand type of both products (int8 pools: fp16)
  using act4_t = typename Act<KV>::t4;
  using act8_t = typename Act<KV>::t8;
  constexpr int KS = D / 32;        // k-steps of 32 over the head dim
  constexpr int NT = D / 16;        // 16-wide output column tiles
  constexpr int BN = kMfmaBN;       // keys per step
  constexpr int KB = BN / 16;       // 16-key blocks per step
  constexpr int RB = 2;             // 16-row MFMA blocks per wave
  constexpr int LDK = D + PA_PF_PADK;  // LDS row strides (halves) of the K and V tiles
  constexpr int LDV = D + PA_PF_PADV;
  constexpr int EB = I8 ? 1 : 2;
  constexpr int CPR = D * EB / 16;  // 16-byte chunks per key row in the pool
  constexpr int NTH = 64 * kMfmaWaves;
  constexpr int NCH = BN * CPR;                    // 16-byte chunks per tile
  constexpr int PT = NCH >= NTH ? NCH / NTH : 1;   // chunks per thread per tile
  static_assert(NCH % NTH == 0 || NTH % NCH == 0, "chunks must tile the workgroup");
  __shared__ __attribute__((aligned(16))) half_t ldk[2][BN * LDK];  // [buffer]
  __shared__ __attribute__((aligned(16))) half_t ldv[2][BN * LDV];

  const int id = blockIdx.x;
  const int h = id % a.hkv;         // consecutive workgroups = consecutive KV heads (one XCD each when hkv = 8)
  const int4 mu = a.munit[id / a.hkv];   // {sequence, row tile, part | parts << 16, partial slot}
  if (mu.x < 0) return;
  const SeqInfo si = a.seqs[mu.x];
  const int L = si.kv_len, Q = si.q_len, rows = Q * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps block indices scalar
  const int l16 = lane & 15, grp = lane >> 4;
  const int r0 = mu.y * kMfmaRows;
  const TileSpan span = tile_span(L, Q, G, mu.y, a.window);
  const int kmax = span.kmax;
  const int32_t* tbl = a.block_tables + (int64_t)mu.x * a.max_blocks;
  const int qmin = L - Q + (r0 + wave * 32) / G;  // query position of this wave's first row
  // With a window the tile starts at the 64-key step holding its first row's
  // first visible key (klo); keys before klo are read from klo instead, so
  // blocks the window has left behind are never addressed.  A step needs the
  // window mask while it starts before the wave's last row's window does.
  const int klo = window_lo(L - Q + r0 / G, a.window);
  const int kt0 = span.k0;   // klo, step-aligned
  // a part of a split tile walks its share of the tile's steps: keys [kbeg, kend)
  const int part = mu.z & 0xFFFF, parts = mu.z >> 16;
  const int psteps = part_steps(span.steps, parts);
  const int kbeg = kt0 + part * psteps * BN;
  const int kend = min(kmax, kbeg + psteps * BN);
  const int wlo_last = window_lo(L - Q + (min(rows, r0 + wave * 32 + 32) - 1) / G, a.window);

  int qpos[RB], qlo[RB];
  int64_t orow[RB];
  bool rvalid[RB];
  act8_t qop[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = r0 + wave * 32 + rb * 16 + l16;
    rvalid[rb] = row < rows;
    const int tq = rvalid[rb] ? row / G : 0;
    qpos[rb] = rvalid[rb] ? L - Q + tq : -1;
    qlo[rb] = window_lo(qpos[rb], a.window);
    orow[rb] = ((int64_t)(si.q_start + tq) * a.hq + (int64_t)h * G + row % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[rb][ks] = rvalid[rb] ? *(const act8_t*)((const act_t*)a.q + orow[rb] + ks * 32 + 8 * grp)
                               : (act8_t)(act_t)0.f;
  }

  float4_t o[RB][NT];
  float m[RB];
  float4_t lsum[RB];   // row sums of the fp16 weights, accumulated on the matrix cores (all 4 entries equal)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    lsum[rb] = (float4_t)0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[rb][nt] = (float4_t)0.f;
  }

  // native vectors: an array of HIP's uint4 class type was kept in private memory (80 B per lane
  // of scratch traffic each step on 16-bit pools); these stay in registers
  u32x4_t stk[PT], stv[PT];
  float nks[KB];  // int8: K scales of the four 16-key blocks of the tiles in flight
  float nvc[PT];  // int8: V scale of the 16-key block of each of this thread's staging chunks
  // Physical blocks, read one step before the tiles they address: per 16-key
  // block of the step (int8: for its scales), and per staging chunk of this
  // wave (its 64 lanes cover 64 / CPR <= 16 aligned keys, one 16-key block).
  // The reads go through the vector memory path at a uniform address (vz is a
  // zero the compiler cannot prove uniform): scalar loads share a counter with
  // LDS reads, so every LDS read of the step would wait for them.  The values
  // are made scalar again when used.
  const int last_blk = (L - 1) / kBlockSize;   // L >= q_len >= 1 for a row tile
  const int first_blk = klo / kBlockSize;
  const int vz = lane & (a.hkv >> 30);          // 0 (hkv is small and positive)
  struct Blocks {
    int kb[KB];
    int chunk[PT];
  };
  auto table = [&](int kt, Blocks& t) {
    if constexpr (I8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) t.kb[kb] = (tbl + min(max(kt / kBlockSize + kb, first_blk), last_blk))[vz];
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int key0 = ((64 * wave + NTH * i) % NCH) / CPR;
      t.chunk[i] = (tbl + min(max(kt + key0, klo) / kBlockSize, last_blk))[vz];
    }
  };
  // Keys past the sequence are read from its last key instead, and keys
  // before klo from klo (real, finite rows): their scores are masked to -inf
  // and their weights are 0, so no stale slot is read and no zero fill is
  // needed.  Per lane only a 32-bit
  // offset inside the (block, head) tile varies; the tile base is scalar.
  constexpr int64_t kTileBytes = (int64_t)kBlockSize * D * EB;
  auto gload = [&](int kt, const Blocks& t) {
    if constexpr (I8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int64_t sidx =
            (int64_t)clamp_block(__builtin_amdgcn_readfirstlane(t.kb[kb]), a.num_blocks) * a.blk_tiles + h;
        nks[kb] = (float)(a.ks + sidx)[vz];
      }
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = (threadIdx.x + NTH * i) % NCH;   // threads past the chunks repeat the first ones
      const int key = c / CPR, ch = c % CPR;
      const int kg = min(max(kt + key, klo), L - 1);
      const int64_t tile =
          (int64_t)clamp_block(__builtin_amdgcn_readfirstlane(t.chunk[i]), a.num_blocks) * a.blk_tiles + h;
      if constexpr (I8) nvc[i] = (float)(a.vs + tile)[vz];
      const uint32_t off = (uint32_t)((kg % kBlockSize) * D * EB + ch * 16);
      stk[i] = *(const u32x4_t*)((const char*)a.kc + tile * kTileBytes + off);
      stv[i] = *(const u32x4_t*)((const char*)a.vc + tile * kTileBytes + off);
    }
  };
  // int8 tiles become fp16: K as exact codes (its scale multiplies the
  // scores), V as code * (scale / 2) of its 16-key block, rounded to fp16, so
  // the weights that multiply V are the plain softmax weights.  The half keeps
  // 127 * scale finite (scale <= 65504 / 127 rounds up to 516); the output
  // takes the factor 2 back.
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = (threadIdx.x + NTH * i) % NCH;   // threads past the chunks repeat the first ones
      const int key = c / CPR, ch = c % CPR;
      if constexpr (I8) {
        const half_t vh = (half_t)(0.5f * nvc[i]);
        const half2_t vs2 = {vh, vh};
        half_t* kd = &ldk[buf][key * LDK + ch * 16];
        half_t* vd = &ldv[buf][key * LDV + ch * 16];
        const uint32_t kw[4] = {stk[i][0], stk[i][1], stk[i][2], stk[i][3]};
        const uint32_t vw[4] = {stv[i][0], stv[i][1], stv[i][2], stv[i][3]};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const half2_t a0 = sdwa_pair<0, 1>(kw[2 * c2], kw[2 * c2]), a1 = sdwa_pair<2, 3>(kw[2 * c2], kw[2 * c2]);
          const half2_t a2 = sdwa_pair<0, 1>(kw[2 * c2 + 1], kw[2 * c2 + 1]);
          const half2_t a3 = sdwa_pair<2, 3>(kw[2 * c2 + 1], kw[2 * c2 + 1]);
          half2_t b0 = sdwa_pair<0, 1>(vw[2 * c2], vw[2 * c2]), b1 = sdwa_pair<2, 3>(vw[2 * c2], vw[2 * c2]);
          half2_t b2 = sdwa_pair<0, 1>(vw[2 * c2 + 1], vw[2 * c2 + 1]);
          half2_t b3 = sdwa_pair<2, 3>(vw[2 * c2 + 1], vw[2 * c2 + 1]);
          b0 *= vs2;
          b1 *= vs2;
          b2 *= vs2;
          b3 *= vs2;
          *(half8_t*)(kd + 8 * c2) = (half8_t){a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
          *(half8_t*)(vd + 8 * c2) = (half8_t){b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
        }
      } else {
        *(u32x4_t*)&ldk[buf][key * LDK + ch * 8] = stk[i];
        *(u32x4_t*)&ldv[buf][key * LDV + ch * 8] = stv[i];
      }
    }
  };

  Blocks tn, tn2;
  table(kbeg, tn);
  gload(kbeg, tn);
  lstore(0);
  table(kbeg + BN, tn);
  __syncthreads();
  typedef __attribute__((address_space(3))) short4_t lds_short4;
  int buf = 0;
  const act8_t kOnes8 = (act8_t)(act_t)1.0f;

  // One 64-key step: S = K Q^T for the four 16-key blocks (this lane: query
  // row l16 of each row block, keys 16*kb + 4*grp + e), the online-softmax
  // max, then the fp16 weights and O^T += V^T P^T per 32-key half, so that the
  // second half's vector work sits beside the first half's matrix products,
  // and the next tiles' staging beside the second half's.
  //
  // Only steps that reach past this wave's first query position, or start
  // before its last row's window does, need the mask (a wave-uniform test);
  // it sets the hidden raw scores to -inf.
  // The max is taken on raw scores and scaled once per 16-key block (scales
  // are positive), and the scale rides in the exponent's FMA.  The running max
  // moves only when a score exceeds it by more than kRescalePf (log2 units),
  // so the accumulators are rescaled rarely.
  for (int kt = kbeg; kt < kend; kt += BN, buf ^= 1) {
    const bool more = kt + BN < kend;
    // score scale per 16-key block (base 2; int8 folds in the block's K scale).  A zero K scale
    // (an all-zero block) becomes the least normal float: its scores stay 0, and -inf stays -inf.
    float cks[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) cks[kb] = I8 ? fmaxf(a.scale_log2 * nks[kb], 1.17549435e-38f) : a.scale_log2;
    // the staging at the end of the step is unconditional, so it can share a block with the
    // matrix work; after the last step it rewrites the idle buffer with tiles nothing reads
    if (more) {
      gload(kt + BN, tn);
      table(kt + 2 * BN, tn2);
    }

    // S^T = K Q^T, k-step outer so the eight accumulators interleave, with the
    // next k-step's four K operands read from LDS while this one's products run
    float4_t s[RB][KB];
    act8_t kq[2][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      kq[0][kb] = __builtin_bit_cast(act8_t, *(const half8_t*)&ldk[buf][(kb * 16 + l16) * LDK + 8 * grp]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kq[(ks + 1) & 1][kb] = __builtin_bit_cast(
              act8_t, *(const half8_t*)&ldk[buf][(kb * 16 + l16) * LDK + (ks + 1) * 32 + 8 * grp]);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][kb] = mfma16x16x32(kq[ks & 1][kb], qop[rb][ks], ks == 0 ? (float4_t)0.f : s[rb][kb]);
    }
    if (kt + BN - 1 > qmin || kt < wlo_last) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kt + kb * 16 + 4 * grp + e;
            if (key > qpos[rb] || key < qlo[rb]) s[rb][kb][e] = -__builtin_inff();
          }
    }
    // Each lane tests its own 16 scores against its row's running max; only
    // when some score of the wave exceeds it by more than kRescalePf are the
    // row maxima formed across the row's four lanes and the rows rescaled.
    float mloc[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mb = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float r = fmaxf(fmaxf(s[rb][kb][0], s[rb][kb][1]), fmaxf(s[rb][kb][2], s[rb][kb][3]));
        mb = fmaxf(mb, r * cks[kb]);
      }
      mloc[rb] = mb;
      grow |= mb > m[rb] + kRescalePf;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mb = fmaxf(mloc[rb], __shfl_xor(mloc[rb], 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const bool g = mb > m[rb] + kRescalePf;   // the same for the row's four lanes
        const float al = g ? fast_exp2(m[rb] - mb) : 1.f;
        m[rb] = g ? mb : m[rb];
        lsum[rb] *= al;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[rb][nt] *= al;
      }
    }
#pragma unroll
    for (int hh = 0; hh < KB / 2; ++hh) {
      // this half's V operands (transposing LDS reads) are requested before its weights are formed
      act8_t vq[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const half_t* p1 = &ldv[buf][(hh * 32 + 4 * grp + (l16 >> 2)) * LDV + nt * 16 + 4 * (l16 & 3)];
        const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p1);
        const short4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1 + 16 * LDV));
        const half4_t h1 = __builtin_bit_cast(half4_t, v1), h2 = __builtin_bit_cast(half4_t, v2);
        vq[nt] = __builtin_bit_cast(act8_t, (half8_t){h1.x, h1.y, h1.z, h1.w, h2.x, h2.y, h2.z, h2.w});
      }
      act8_t p[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // slot j of the k-step: keys 4*grp + [0..3] of the half's first and second 16-key block
          const int kb = 2 * hh + j / 4;
          p[rb][j] = (act_t)fast_exp2(fmaf(s[rb][kb][j % 4], cks[kb], -m[rb]));
        }
        // row sums of exactly the weights the product uses: ones^T P^T on the matrix cores
        lsum[rb] = mfma16x16x32(kOnes8, p[rb], lsum[rb]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][nt] = mfma16x16x32(vq[nt], p[rb], o[rb][nt]);
    }
    lstore(buf ^ 1);
    if (more) tn = tn2;
    __syncthreads();
  }

  if (mu.w >= 0) {
    // a part of a split tile: its rows' normalised outputs and base-2
    // log-sum-exps go to its partial slot (a row that saw no key of this
    // part: output 0, log-sum-exp -inf), for the merge kernel
    const int64_t prow = ((int64_t)mu.w * a.hkv + h) * kMfmaRows + wave * 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!rvalid[rb]) continue;
      const float l = lsum[rb][0];
      const float inv = l > 0.f ? (I8 ? 2.f : 1.f) / l : 0.f;
      const int64_t pr = prow + rb * 16 + l16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) *(float4_t*)(a.mpo + pr * D + nt * 16 + 4 * grp) = o[rb][nt] * inv;
      if (grp == 0) a.mlse[pr] = l > 0.f ? m[rb] + __builtin_log2f(l) : -__builtin_inff();
    }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rvalid[rb]) continue;
    const float inv = (I8 ? 2.f : 1.f) / lsum[rb][0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      act4_t r;
      r.x = (act_t)(o[rb][nt][0] * inv);
      r.y = (act_t)(o[rb][nt][1] * inv);
      r.z = (act_t)(o[rb][nt][2] * inv);
      r.w = (act_t)(o[rb][nt][3] * inv);
      *(act4_t*)((act_t*)a.out + orow[rb] + nt * 16 + 4 * grp) = r;
    }
  }
}

// Merge of split row tiles: for each of the tile's rows, the parts' outputs
// weighted by 2^(lse_p - max lse) over the sum of those weights (the
// log-sum-exp merge of split-K partitions).  One wave per row: lane p holds
// part p's log-sum-exp (64 parts at a time), each lane D / 64 dims of the
// output; a workgroup of four waves takes four rows of one (split tile, KV
// head), so the grid has 64 workgroups per split tile and head and the
// rows' loads are spread over the machine instead of queued in one wave.
constexpr int kMergeRowsPerGroup = 4;

template <int D, int G, int KV>
__global__ __launch_bounds__(64 * kMergeRowsPerGroup) void prefill_merge_kernel(AttnArgs a) {
  using act_t = typename Act<KV>::t;
  constexpr int E = D / 64;
  constexpr int GROUPS = kMfmaRows / kMergeRowsPerGroup;   // workgroups per (split tile, head)
  const int gid = blockIdx.x % GROUPS;
  const int h = (blockIdx.x / GROUPS) % a.hkv;
  const int4 ms = a.msplit[blockIdx.x / GROUPS / a.hkv];   // {sequence, row tile, parts, first slot}
  if (ms.x < 0) return;
  const SeqInfo si = a.seqs[ms.x];
  const int lane = threadIdx.x & 63;
  const int tr = gid * kMergeRowsPerGroup + (threadIdx.x >> 6);   // row within the tile
  const int row = ms.y * kMfmaRows + tr;
  if (row >= si.q_len * G) return;
  const int64_t base = (int64_t)ms.w * a.hkv + h;   // partial record of part p: (base + p * hkv) * kMfmaRows + tr
  auto rec = [&](int p) { return (base + (int64_t)p * a.hkv) * kMfmaRows + tr; };
  float mx = -__builtin_inff();
  for (int c = 0; c < ms.z; c += 64)
    mx = fmaxf(mx, c + lane < ms.z ? a.mlse[rec(c + lane)] : -__builtin_inff());
  mx = wave_max(mx);
  float acc[E] = {}, wsum = 0.f;
  for (int c = 0; c < ms.z; c += 64) {
    const float lse = c + lane < ms.z ? a.mlse[rec(c + lane)] : -__builtin_inff();
    const float wl = lse == -__builtin_inff() ? 0.f : fast_exp2(lse - mx);   // lane's part weight
    const int n = min(64, ms.z - c);
    for (int j = 0; j < n; ++j) {
      const float wt = __shfl(wl, j, 64);
      wsum += wt;
      const float* src = a.mpo + rec(c + j) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(wt, src[e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  act_t* dst = (act_t*)a.out + ((int64_t)(si.q_start + row / G) * a.hq + (int64_t)h * G + row % G) * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (act_t)(acc[e] * inv);
}

template <int D, int KV>
static hipError_t prefill_merge_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  // workgroup x: split tile x / (hkv * GROUPS), head (x / GROUPS) % hkv, rows of group x % GROUPS
  const dim3 grid(n * a.hkv * (kMfmaRows / kMergeRowsPerGroup));
  constexpr int NT = 64 * kMergeRowsPerGroup;
  switch (g) {
    case 1: prefill_merge_kernel<D, 1, KV><<<grid, NT, 0, s>>>(a); break;
    case 2: prefill_merge_kernel<D, 2, KV><<<grid, NT, 0, s>>>(a); break;
    case 4: prefill_merge_kernel<D, 4, KV><<<grid, NT, 0, s>>>(a); break;
    case 8: prefill_merge_kernel<D, 8, KV><<<grid, NT, 0, s>>>(a); break;
    case 16: prefill_merge_kernel<D, 16, KV><<<grid, NT, 0, s>>>(a); break;
    case 32: prefill_merge_kernel<D, 32, KV><<<grid, NT, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t prefill_merge_d(const AttnArgs& a, int g, int kv, int n, hipStream_t s) {
  // the merged outputs take the type of q: bf16 for bf16 pools, fp16 otherwise
  return kv == kKvBF16 ? prefill_merge_g<D, kKvBF16>(a, g, n, s) : prefill_merge_g<D, kKvF16>(a, g, n, s);
}

hipError_t launch_prefill_merge(const AttnArgs& a, int head_dim, int group, int kv, int n, hipStream_t s) {
  return head_dim == 128 ? prefill_merge_d<128>(a, group, kv, n, s) : prefill_merge_d<64>(a, group, kv, n, s);
}

template <int D, int KV>
static hipError_t prefill_g(const AttnArgs& a, int g, int n, hipStream_t s) {
  const dim3 grid(n * a.hkv);   // workgroup id = row tile * hkv + KV head
  switch (g) {
    case 1: prefill_kernel<D, 1, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 2: prefill_kernel<D, 2, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 4: prefill_kernel<D, 4, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 8: prefill_kernel<D, 8, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 16: prefill_kernel<D, 16, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    case 32: prefill_kernel<D, 32, KV><<<grid, 64 * kMfmaWaves, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t prefill_d(const AttnArgs& a, int g, int kv, int n, hipStream_t s) {
  switch (kv) {
    case kKvF16: return prefill_g<D, kKvF16>(a, g, n, s);
    case kKvI8: return prefill_g<D, kKvI8>(a, g, n, s);
    case kKvBF16: return prefill_g<D, kKvBF16>(a, g, n, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const AttnArgs& a, int head_dim, int group, int kv, int n, hipStream_t s) {
  return head_dim == 128 ? prefill_d<128>(a, group, kv, n, s) : prefill_d<64>(a, group, kv, n, s);
}

}  // namespace pa
