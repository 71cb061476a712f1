// Work units of the vector-path attention kernels (the fp16/bf16/int8
// decode kernel and the matrix-core decode kernel for groups of 16 or more):
// one unit = one query row of one sequence, one KV head, one split-K
// partition of the row's keys.  A unit comes from the plan kernel's lists,
// from the sequence index (plan-free batches), or is located by the
// workgroup itself (self-planned batches).
#pragma once

#include "pa_internal.h"

namespace pa {

// ===================================================== self-planned units ===
// Row i of a self-planned batch as every workgroup derives it from the device
// lengths (clamped as the plan kernel clamps them): the keys its query walks,
// its equal units and their cost bucket.  No query row: no units.
struct SPRow {
  int keys, parts, bucket;
};

__device__ __forceinline__ SPRow sp_row(const AttnArgs& a, int i) {
  SPRow r = {0, 0, 0};
  const int L = min(max(a.seq_lens[i], 0), a.max_kv);
  if (min(a.q_lens[i], L) < 1) return r;
  r.keys = vector_keys(L - 1, a.window);
  r.parts = parts_for(r.keys, a.part);
  const int sz = r.parts > 1 ? (((r.keys + r.parts - 1) / r.parts + 15) & ~15) : r.keys;
  r.bucket = min(sz >> 6, kSelfPlanBuckets - 1);
  return r;
}

// The x-th unit of the order every workgroup derives alike (cost bucket
// descending, then sequence, then partition): a count of units per bucket,
// a scan over the buckets to find x's bucket and its rank there, then a scan
// over the sequences of that bucket to find the row.  Returns false when x
// is past the last unit (the device lengths then disagree with the host's).
struct SPUnit {
  int seq, part, parts;
};

template <int NT>
__device__ bool sp_locate(const AttnArgs& a, int x, SPUnit& out) {
  static_assert(kSelfPlanBuckets == 64, "one lane per bucket");
  constexpr int PER = kSelfPlanMaxSeqs / NT;   // sequences per thread, in order
  __shared__ int cnt[kSelfPlanBuckets];
  __shared__ int wsum[NT / 64];
  __shared__ int sel[5];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < kSelfPlanBuckets) cnt[tid] = 0;
  if (tid == 0) sel[0] = -1;
  __syncthreads();
  SPRow rows[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    rows[k] = i < a.num_seqs ? sp_row(a, i) : SPRow{0, 0, 0};
    if (rows[k].parts > 0) atomicAdd(&cnt[rows[k].bucket], rows[k].parts);
  }
  __syncthreads();
  if (wv == 0) {
    const int b = kSelfPlanBuckets - 1 - lane;   // lane 0 holds the largest bucket
    const int c = cnt[b];
    int inc = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off, 64);
      if (lane >= off) inc += t;
    }
    if (x >= inc - c && x < inc) {
      sel[0] = b;
      sel[1] = x - (inc - c);
    }
  }
  __syncthreads();
  const int B = sel[0], r = sel[1];
  if (B < 0) return false;
  int mine = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) mine += rows[k].bucket == B ? rows[k].parts : 0;
  int inc = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off, 64);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int base = inc - mine;
  for (int w = 0; w < wv; ++w) base += wsum[w];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int c = rows[k].bucket == B ? rows[k].parts : 0;
    if (r >= base && r < base + c) {
      sel[2] = tid * PER + k;
      sel[3] = r - base;
      sel[4] = rows[k].parts;
    }
    base += c;
  }
  __syncthreads();
  out.seq = sel[2];
  out.part = sel[3];
  out.parts = sel[4];
  return true;
}


// The unit workgroup blockIdx.x serves (for KV head h), and its key range.
struct Unit {
  int u;         // unit index (partials are stored by it)
  int seq, t;    // sequence and query row within it
  int part_idx, parts;
  int kv_len, q_len, q_start;
  int klo;       // first visible key of the row
  int kbeg, kend;  // this unit's keys: [kbeg, kend), kbeg 16-aligned
};

// Returns false when the workgroup has nothing to do (no such unit, a row
// with no query, or device lengths that disagree with the host's plan).
template <int NT>
__device__ __forceinline__ bool resolve_unit(const AttnArgs& a, int h, Unit& w) {
  if (a.direct) {
    w.u = w.seq = blockIdx.x;
    w.t = w.part_idx = 0;
    w.parts = 1;
    w.kv_len = min(max(a.seq_lens[w.seq], 0), a.max_kv);
    w.q_len = min(max(a.q_lens[w.seq], 0), w.kv_len);
    if (w.q_len == 0) return false;
    w.q_start = w.seq;
  } else if (a.selfplan) {
    SPUnit su;
    if (!sp_locate<NT>(a, blockIdx.x, su)) return false;
    w.u = blockIdx.x;
    w.seq = su.seq;
    w.t = 0;
    w.part_idx = su.part;
    w.parts = su.parts;
    w.kv_len = min(max(a.seq_lens[w.seq], 0), a.max_kv);
    w.q_len = 1;
    w.q_start = w.seq;   // one query row per sequence: packed row = sequence
    if (w.part_idx == 0 && h == 0 && threadIdx.x == 0) a.row_u0[w.seq] = make_int2(w.u, w.parts);
  } else {
    w.u = a.vorder[blockIdx.x];   // units go out longest first
    const int2 un = a.vunit[w.u];
    if (un.x < 0) return false;
    const VTok vt = a.vtok[un.x];
    if (vt.seq < 0) return false;
    const SeqInfo si = a.seqs[vt.seq];
    w.seq = vt.seq;
    w.t = vt.t;
    w.part_idx = un.y;
    w.parts = vt.parts;
    w.kv_len = si.kv_len;
    w.q_len = si.q_len;
    w.q_start = si.q_start;
  }
  // device lengths that split a row the host's lengths did not: no partial buffer to write to
  if (w.parts > 1 && a.po == nullptr) return false;
  const int nvis = w.kv_len - w.q_len + w.t + 1;
  w.klo = window_lo(nvis - 1, a.window);        // first visible key
  const int k0 = w.klo & ~(kBlockSize - 1);
  // a split row's units are equal (rounded up to 16 keys), not full partitions and a remainder
  const int sz = w.parts > 1 ? (((nvis - k0 + w.parts - 1) / w.parts + 15) & ~15) : a.part;
  w.kbeg = k0 + w.part_idx * sz;
  w.kend = min(nvis, w.kbeg + sz);
  return true;
}

}  // namespace pa
