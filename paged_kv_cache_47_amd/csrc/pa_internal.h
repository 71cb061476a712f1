// Internal declarations shared by the libpa.so translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16_t;
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf164_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Pool element kinds the kernels are built for (the pa_kv_dtype values).
constexpr int kKvF16 = PA_KV_F16, kKvI8 = PA_KV_I8, kKvBF16 = PA_KV_BF16;

// The 16-bit activation type of a pool kind (queries, new rows, outputs, the
// softmax weights fed to the products): bf16 for bf16 pools, fp16 otherwise.
template <int KV>
struct Act {
  using t = half_t;
  using t2 = half2_t;
  using t4 = half4_t;
  using t8 = half8_t;
};
template <>
struct Act<kKvBF16> {
  using t = bf16_t;
  using t2 = bf162_t;
  using t4 = bf164_t;
  using t8 = bf168_t;
};

constexpr int kBlockSize = 16;     // tokens per block (the only size built)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

// Per-sequence values after host/device agreement checks (written by the plan kernel).
struct SeqInfo {
  int32_t kv_len;   // keys after this step's writes, clamped to the table width
  int32_t q_len;    // query rows, clamped to kv_len and to the packed batch
  int32_t q_start;  // first packed row of the sequence
  int32_t pad;
};

// One query row of the vector path: sequence, row within sequence, first unit, units.
struct VTok {
  int32_t seq, t, u0, parts;
};

struct AttnArgs {
  const void* q;       // fp16, or bf16 for bf16 pools
  const void* kc;
  const void* vc;
  const half_t* ks;
  const half_t* vs;
  const int32_t* block_tables;
  const SeqInfo* seqs;
  const VTok* vtok;
  const int2* vunit;   // {vtok index, partition}
  const int32_t* vorder;  // dispatch order of the vector units: workgroup x takes unit vorder[x]
  const int4* munit;   // {sequence, row tile, part | parts << 16, partial slot (-1: unsplit)}
  const int4* msplit;  // split row tiles: {sequence, row tile, parts, first partial slot}
  float* mpo;          // [slot][hkv][kMfmaRows][D] normalised partial outputs of split row tiles
  float* mlse;         // [slot][hkv][kMfmaRows] base-2 log-sum-exp of each (-inf: no visible key)
  float* po;           // [n_vunit][Hq][D] normalised partial outputs
  float* plse;         // [n_vunit][Hq] base-2 log-sum-exp of each partial
  void* out;           // the type of q
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t hq, hkv;
  int32_t blk_tiles;   // (layer, KV head) tiles per physical block: num_layers * hkv;
                       // kc/vc/ks/vs point at the addressed layer's first tile of block 0
  int32_t part;        // largest partition in keys (a multiple of 16); a split row's units are equal
  int32_t window;      // sliding window in keys; 0 = none
  float scale_log2;    // scale * log2(e)
  int64_t scale_count; // int8: scales from ks (or vs) to the end of its array (bounds of the scale reads)
  // direct != 0: a batch of one query row per sequence, unsplit, that needs no
  // plan: decode workgroup x serves sequence x, reading its length here
  // (clamped as the plan kernel clamps it: to max_kv, and the rows to the keys)
  const int32_t* seq_lens;
  const int32_t* q_lens;
  int32_t max_kv;
  int32_t direct;
  // selfplan != 0: a self-planned decode batch (see kSelfPlanMaxSeqs): decode
  // workgroup x takes the x-th unit of the bucketed order it derives from
  // seq_lens / q_lens; the first unit of each row records its index and the
  // row's unit count in row_u0[row] for the merge kernel
  int32_t selfplan;
  int32_t num_seqs;
  int32_t n_units;     // units of the launch (the decode grid's x extent)
  int2* row_u0;        // [num_seqs] {first unit, units}
  // Fused KV write (pa_write_attend; NULL otherwise): a batch of one query row
  // per sequence over a 16-bit pool, token i the new token of sequence i.  The
  // unit that walks a row's last key first writes the token's K and V rows of
  // its KV head into slot new_slots[i] of the pools (kc / vc, the same memory
  // the attention reads).
  const void* new_k;   // [num_seqs][hkv][D], the type of q
  const void* new_v;
  const int32_t* new_slots;
};

// First key a query at position `pos` sees (0 without a window).
__host__ __device__ __forceinline__ int window_lo(int pos, int window) {
  return window > 0 ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
}

// Split-K partitions of a row of `nkeys` keys (part <= 0: never split).
__host__ __device__ __forceinline__ int parts_for(int nkeys, int part) {
  return part <= 0 ? 1 : (nkeys + part - 1) / part;
}

// Keys the vector path walks for the query at position `pos`: from the
// 16-aligned start of its window (0 without one) to the query itself.
__host__ __device__ __forceinline__ int vector_keys(int pos, int window) {
  return pos + 1 - (window_lo(pos, window) & ~(kBlockSize - 1));
}

// Self-planned decode batches (one query row per sequence, at most
// kSelfPlanMaxSeqs sequences, no MFMA rows): no plan kernel runs; each decode
// workgroup finds its own unit.  Units are ordered by cost bucket (the size
// of the row's equal units in 64-key steps, capped), largest first, then by
// sequence, then by partition, so a row's units are consecutive.
constexpr int kSelfPlanMaxSeqs = 1024;
constexpr int kSelfPlanBuckets = 64;
#ifndef PA_SELFPLAN
#define PA_SELFPLAN 1   // 0: such batches go through the plan kernel too
#endif

struct PlanArgs {
  const int32_t* seq_lens;
  const int32_t* q_lens;
  SeqInfo* seqs;
  VTok* vtok;
  int2* vunit;
  int32_t* vorder;     // vector units, longest first (a permutation of 0 .. cap_vunit-1)
  int32_t* vcost;      // cost bucket of each vector unit (scratch for the ordering)
  int4* munit;         // row-tile units (a tile, or one part of a split tile), longest first
  int4* munit_tmp;     // the same units in sequence order, before the ordering
  int4* msplit;        // split row tiles, for the merge
  int32_t split_steps; // a row tile spanning more 64-key steps is split into equal parts (<= 0: never)
  int32_t num_seqs;
  int32_t group;
  int32_t part;        // <= 0: one partition per row
  int32_t window;      // sliding window in keys; 0 = none
  int32_t min_rows;
  int32_t max_kv;      // max_blocks_per_seq * block_size
  int32_t total_q;
  int32_t cap_vtok, cap_vunit, cap_munit, cap_msplit, cap_mslot;
};

// Launchers (one translation unit each); all return hipGetLastError() after launch.
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_decode(const AttnArgs& a, int head_dim, int group, int kv, int n_vunit, hipStream_t s);
hipError_t launch_decode_mfma(const AttnArgs& a, int head_dim, int group, int kv, int n_vunit, hipStream_t s);
hipError_t launch_reduce(const AttnArgs& a, int head_dim, int group, int kv, int n_vtok, hipStream_t s);
hipError_t launch_prefill(const AttnArgs& a, int head_dim, int group, int kv, int n_munit, hipStream_t s);
hipError_t launch_prefill_merge(const AttnArgs& a, int head_dim, int group, int kv, int n_msplit, hipStream_t s);
hipError_t launch_write_f16(const pa_cache_desc& d, const void* k, const void* v, const int32_t* slots,
                            int32_t T, void* kc, void* vc, hipStream_t s);
hipError_t launch_write_i8(const pa_cache_desc& d, const void* k, const void* v, const int32_t* slots,
                           int32_t T, void* kc, void* vc, void* ks, void* vs, hipStream_t s);
hipError_t launch_copy(const pa_cache_desc& d, void* kc, void* vc, void* ks, void* vs,
                       const int32_t* pairs, int32_t n, hipStream_t s);

// Metadata checks (check.hip): each clears `st` and records a violation there.
hipError_t launch_check_write(const pa_cache_desc& d, const int32_t* slots, int32_t T, int32_t* st, hipStream_t s);
hipError_t launch_check_attend(const pa_cache_desc& d, const int32_t* tables, int32_t max_blocks,
                               const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                               const int32_t* hL, const int32_t* hQ, int32_t window, int32_t* st, hipStream_t s);
hipError_t launch_check_copy(const pa_cache_desc& d, const int32_t* pairs, int32_t n, int32_t* st, hipStream_t s);
#ifndef PA_DEBUG
#define PA_DEBUG 0
#endif
#if PA_DEBUG
// Debug builds: run the check on the library's own status words, wait, and
// return PA_ERR_METADATA on a violation.
pa_status debug_check_write(const pa_cache_desc& d, const int32_t* slots, int32_t T, hipStream_t s);
pa_status debug_check_attend(const pa_cache_desc& d, const int32_t* tables, int32_t max_blocks,
                             const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs, const int32_t* hL,
                             const int32_t* hQ, int32_t window, hipStream_t s);
pa_status debug_check_copy(const pa_cache_desc& d, const int32_t* pairs, int32_t n, hipStream_t s);
#endif

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// Pair dot products with an fp32 accumulator, and the 16x16x32 matrix
// product, for either 16-bit type.
__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
__device__ __forceinline__ float dot2(bf162_t a, bf162_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16x16x32(bf168_t a, bf168_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the group ends with the sum.
// After the quad steps all lanes of a quad agree, so the row half-mirror (lane i <-> 7-i) acts
// as an exchange with the other quad and the row mirror (lane i <-> 15-i) as one with the other
// half-row.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
  return x;
}

// group_sum over COUNT independent values, step-major: the COUNT adds of
// one butterfly step are independent, so they fill the wait states a DPP read
// of a just-written register needs.
template <int N, int COUNT>
__device__ __forceinline__ void group_sum_all(float* x) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) x[k] += dpp<0xB1>(x[k]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) x[k] += dpp<0x4E>(x[k]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) x[k] += dpp<0x141>(x[k]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) x[k] += dpp<0x140>(x[k]);
  }
}

__device__ __forceinline__ float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ int clamp_block(int b, int nb) { return (unsigned)b < (unsigned)nb ? b : 0; }

#ifndef PA_I8_SDWA
#define PA_I8_SDWA 1
#endif
// int8 codes -> exact fp16 with sub-dword operand selection: one conversion
// per code, written straight into the low or high half of the result
// (signed byte -> int16 -> fp16 is exact for |code| <= 127).
template <int B0, int B1>
__device__ __forceinline__ half2_t sdwa_pair(uint32_t lo_src, uint32_t hi_src) {
  uint32_t r;
  asm(
      "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_%c3\n\t"
      "v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_%c4"
      : "=&v"(r)
      : "v"(lo_src), "v"(hi_src), "n"(B0), "n"(B1));
  return __builtin_bit_cast(half2_t, r);
}

// bytes b0 b1 of a dword of int8 codes -> exact fp16 pair, via 0x64XX = 1024 + XX
__device__ __forceinline__ void i8x4_to_h2(uint32_t w, half2_t& lo, half2_t& hi) {
  const uint32_t u = w ^ 0x80808080u;  // biased: XX = code + 128
  const uint32_t l = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t h = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  lo = __builtin_bit_cast(half2_t, l) - bias;
  hi = __builtin_bit_cast(half2_t, h) - bias;
}

}  // namespace pa
