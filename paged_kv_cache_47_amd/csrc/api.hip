// C ABI of libpa.so: argument validation, workspace layout, dispatch.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>

#include "mfma_tile.h"

namespace pa {

// ------------------------------------------------------------------ plan ----
// One workgroup turns the device lengths into the work lists the attention
// kernels consume: per-sequence (kv_len, q_len, q_start) after clamping, the
// vector-path rows and their split-K units, and the MFMA row tiles.  The
// host computes the same counts from its copies of the lengths to size the
// launches (caps); every list is filled up to its cap, unused entries marked
// with seq = -1, so kernels never read an unwritten entry even if the host and
// device lengths disagree.
constexpr int kPlanThreads = 1024;
constexpr int64_t kDirectMaxGroups = 1024;   // decode workgroups of a batch that may skip the plan (about one round)
constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive scan of four counters over the workgroup (one sequence per
// thread): wave-level shuffles, then one wave scans the 16 wave totals and
// every thread reads its wave's prefix back (one LDS read, instead of a loop
// over the waves that kept 16 partial sums live and spilled registers).
__device__ __forceinline__ int4 add4(int4 a, int4 b) { return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ int4 shfl_up4(int4 v, int off) {
  return make_int4(__shfl_up(v.x, off, 64), __shfl_up(v.y, off, 64), __shfl_up(v.z, off, 64), __shfl_up(v.w, off, 64));
}

__device__ int4 block_exclusive_scan4(int4 v, int4* lds, int4& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int4 inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int4 t = shfl_up4(inc, off);
    if (lane >= off) inc = add4(inc, t);
  }
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int4 w = lane < kPlanWaves ? lds[lane] : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int off = 1; off < kPlanWaves; off <<= 1) {
      const int4 t = shfl_up4(w, off);
      if (lane >= off) w = add4(w, t);
    }
    if (lane < kPlanWaves) lds[lane] = w;   // inclusive prefixes of the wave totals
  }
  __syncthreads();
  const int4 before = wave > 0 ? lds[wave - 1] : make_int4(0, 0, 0, 0);
  total = lds[kPlanWaves - 1];
  __syncthreads();   // the next scan reuses lds
  return make_int4(before.x + inc.x - v.x, before.y + inc.y - v.y, before.z + inc.z - v.z, before.w + inc.w - v.w);
}

// Row-tile units of the MFMA path go out longest first.  A unit's cost is
// the number of 64-key steps it walks (a whole tile: up to its last row's
// position, from its first row's window start; a part of a split tile: its
// share), and units that attend over long contexts would otherwise start
// late and finish after the rest of the grid; with 64-key cost buckets in
// descending order (a counting sort over the workgroup) the dispatcher fills
// the machine greedily, longest job first.  The order within a bucket is
// whatever the atomics give: every unit writes its own rows (or its own
// partial slot), so the results do not depend on it.
constexpr int kCostBuckets = kPlanThreads;

__device__ int tile_cost_bucket(const PlanArgs& a, int4 mu) {
  if (mu.x < 0) return 0;   // the parts of a split tile dropped for lack of room: nothing to run
  const SeqInfo si = a.seqs[mu.x];
  const int steps = tile_span(si.kv_len, si.q_len, a.group, mu.y, a.window).steps;
  const int part = mu.z & 0xFFFF, parts = mu.z >> 16;
  const int ps = part_steps(steps, parts);
  return min(min(ps, steps - part * ps), kCostBuckets - 1);
}

// Vector-path units go out longest first too (a unit's cost: its keys, in
// 64-key buckets), so a long row's partitions do not start last and set the
// kernel's tail; the decode kernel's workgroup x takes unit vorder[x].  The
// units keep their own indices (partials are stored by unit), so the merge
// does not depend on the order.
__device__ void order_vector_units(const PlanArgs& a, int n) {
  __shared__ int slot[kCostBuckets];
  __shared__ int4 scan_lds[kPlanWaves];
  slot[threadIdx.x] = 0;
  __syncthreads();   // also makes this workgroup's writes of vcost visible to all its threads
  for (int u = threadIdx.x; u < n; u += kPlanThreads) atomicAdd(&slot[kCostBuckets - 1 - a.vcost[u]], 1);
  __syncthreads();
  int4 tot;
  const int first = block_exclusive_scan4(make_int4(slot[threadIdx.x], 0, 0, 0), scan_lds, tot).x;
  slot[threadIdx.x] = first;
  __syncthreads();
  for (int u = threadIdx.x; u < n; u += kPlanThreads) a.vorder[atomicAdd(&slot[kCostBuckets - 1 - a.vcost[u]], 1)] = u;
}

__device__ void order_row_tiles(const PlanArgs& a, int n) {
  __shared__ int slot[kCostBuckets];
  __shared__ int4 scan_lds[kPlanWaves];
  slot[threadIdx.x] = 0;
  __syncthreads();   // also makes this workgroup's writes of seqs and munit_tmp visible to all its threads
  for (int u = threadIdx.x; u < n; u += kPlanThreads)
    atomicAdd(&slot[kCostBuckets - 1 - tile_cost_bucket(a, a.munit_tmp[u])], 1);
  __syncthreads();
  int4 tot;
  const int first = block_exclusive_scan4(make_int4(slot[threadIdx.x], 0, 0, 0), scan_lds, tot).x;
  slot[threadIdx.x] = first;
  __syncthreads();
  for (int u = threadIdx.x; u < n; u += kPlanThreads) {
    const int4 mu = a.munit_tmp[u];
    a.munit[atomicAdd(&slot[kCostBuckets - 1 - tile_cost_bucket(a, mu)], 1)] = mu;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int4 lds[kPlanWaves];
  int base_q = 0, base_vt = 0, base_vu = 0, base_mu = 0, base_ms = 0, base_sl = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += kPlanThreads) {
    const int i = c0 + threadIdx.x;
    int L = 0, Q = 0;
    if (i < a.num_seqs) {
      L = min(max(a.seq_lens[i], 0), a.max_kv);
      Q = min(max(a.q_lens[i], 0), L);
    }
    // the packed row offsets come from the unclamped-by-batch row counts
    int4 tot;
    const int qs = base_q + block_exclusive_scan4(make_int4(Q, 0, 0, 0), lds, tot).x;
    const int qsum = tot.x;
    int nvt = 0, nvu = 0, nmu = 0, ntile = 0, nms = 0, nsl = 0;
    if (i < a.num_seqs) {
      Q = max(0, min(Q, a.total_q - qs));   // rows beyond the batch the host sized are dropped
      if (Q > 0 && Q * a.group >= a.min_rows) {
        ntile = (Q * a.group + kMfmaRows - 1) / kMfmaRows;
        for (int r = 0; r < ntile; ++r) {
          const int parts = tile_parts(tile_span(L, Q, a.group, r, a.window).steps, a.split_steps);
          nmu += parts;
          if (parts > 1) {
            nms += 1;
            nsl += parts;
          }
        }
      } else {
        nvt = Q;
        for (int t = 0; t < Q; ++t) nvu += parts_for(vector_keys(L - Q + t, a.window), a.part);
      }
    }
    const int4 ex = block_exclusive_scan4(make_int4(nvt, nvu, nmu, nms), lds, tot);
    const int vt0 = base_vt + ex.x, vu0 = base_vu + ex.y, mu0 = base_mu + ex.z, ms0 = base_ms + ex.w;
    int4 tot2;
    const int sl0 = base_sl + block_exclusive_scan4(make_int4(nsl, 0, 0, 0), lds, tot2).x;
    if (i < a.num_seqs) {
      SeqInfo si;
      si.kv_len = L;
      si.q_len = Q;
      si.q_start = qs;
      si.pad = 0;
      a.seqs[i] = si;
      // the row tiles' units; a split tile's parts take consecutive partial
      // slots, and the tile is listed for the merge (dropped with its units
      // when the device lengths need more than the host sized)
      int mu = mu0, ms = ms0, sl = sl0;
      for (int r = 0; r < ntile; ++r) {
        const int parts = tile_parts(tile_span(L, Q, a.group, r, a.window).steps, a.split_steps);
        if (parts == 1) {
          if (mu < a.cap_munit) a.munit_tmp[mu] = make_int4(i, r, 1 << 16, -1);
        } else {
          const bool fits = ms < a.cap_msplit && sl + parts <= a.cap_mslot && mu + parts <= a.cap_munit;
          if (ms < a.cap_msplit) a.msplit[ms] = make_int4(fits ? i : -1, r, parts, sl);
          for (int p = 0; p < parts; ++p)
            if (mu + p < a.cap_munit) a.munit_tmp[mu + p] = make_int4(fits ? i : -1, r, p | parts << 16, sl + p);
          ms += 1;
          sl += parts;
        }
        mu += parts;
      }
      int u = vu0;
      for (int t = 0; t < nvt; ++t) {
        const int parts = parts_for(vector_keys(L - Q + t, a.window), a.part);
        const int k = vt0 + t;
        const bool fits = k < a.cap_vtok && u + parts <= a.cap_vunit;
        if (k < a.cap_vtok) {
          VTok vt;
          vt.seq = fits ? i : -1;
          vt.t = t;
          vt.u0 = u;
          vt.parts = parts;
          a.vtok[k] = vt;
        }
        const int keys = vector_keys(L - Q + t, a.window);
        for (int p = 0; p < parts; ++p) {
          if (u + p < a.cap_vunit) {
            a.vunit[u + p] = make_int2(fits ? k : -1, p);
            const int sz = parts > 1 ? (((keys + parts - 1) / parts + 15) & ~15) : keys;
            const int ck = min(sz, keys - p * sz);
            a.vcost[u + p] = fits ? min(ck / 64, kCostBuckets - 1) : 0;
          }
        }
        u += parts;
      }
    }
    base_q += qsum;
    base_vt += tot.x;
    base_vu += tot.y;
    base_mu += tot.z;
    base_ms += tot.w;
    base_sl += tot2.x;
  }
  for (int k = base_vt + threadIdx.x; k < a.cap_vtok; k += kPlanThreads) {
    VTok vt;
    vt.seq = -1;
    vt.t = vt.u0 = vt.parts = 0;
    a.vtok[k] = vt;
  }
  for (int u = base_vu + threadIdx.x; u < a.cap_vunit; u += kPlanThreads) {
    a.vunit[u] = make_int2(-1, 0);
    a.vcost[u] = 0;
  }
  for (int u = base_mu + threadIdx.x; u < a.cap_munit; u += kPlanThreads) a.munit[u] = make_int4(-1, 0, 1 << 16, -1);
  for (int k = base_ms + threadIdx.x; k < a.cap_msplit; k += kPlanThreads) a.msplit[k] = make_int4(-1, 0, 1, 0);
  order_row_tiles(a, min(base_mu, a.cap_munit));
  __syncthreads();   // the two orderings share nothing but reuse the scan's LDS pattern
  order_vector_units(a, a.cap_vunit);
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  plan_kernel<<<1, kPlanThreads, 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------ host plan ----
struct HostPlan {
  int32_t part = 0, min_rows = 16, total_q = 0, window = 0;
  int64_t n_vtok = 0, n_vunit = 0, n_munit = 0, n_mtile = 0, n_msplit = 0, n_mslot = 0;
  int32_t max_parts = 0;
  int32_t split_steps = 0;   // row tiles spanning more 64-key steps are split (0: never)
  bool direct = false;     // one decode workgroup per sequence, no plan kernel (see make_plan)
  bool selfplan = false;   // decode workgroups find their own units, no plan kernel (see make_plan)
  size_t off_seqs = 0, off_vtok = 0, off_vunit = 0, off_vorder = 0, off_vcost = 0, off_munit = 0, off_munit_tmp = 0,
         off_lse = 0, off_po = 0, off_row_u0 = 0, off_msplit = 0, off_mlse = 0, off_mpo = 0;
  size_t bytes = 0;
};

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The kernels move q, k, v, out, pool tiles and workspace records in 16-byte
// vectors and read int32 metadata and fp16 scales one element at a time.
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
static bool scales_aligned(const pa_cache_desc* d, const void* ks, const void* vs) {
  return d->kv_dtype != PA_KV_I8 || (aligned(ks, 2) && aligned(vs, 2));
}

static pa_status check_desc(const pa_cache_desc* d) {
  if (d == nullptr) return PA_ERR_NULL;
  if (d->kv_dtype != PA_KV_F16 && d->kv_dtype != PA_KV_I8 && d->kv_dtype != PA_KV_BF16) return PA_ERR_DTYPE;
  if (d->num_blocks <= 0 || d->num_kv_heads <= 0 || d->block_size <= 0 || d->head_dim <= 0) return PA_ERR_SHAPE;
  if (d->num_layers < 0 || d->layer < 0 || d->layer >= std::max(d->num_layers, 1)) return PA_ERR_SHAPE;
  if (d->block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if ((int64_t)d->num_blocks * d->block_size >= ((int64_t)1 << 31)) return PA_ERR_SHAPE;
  return PA_OK;
}

static pa_status check_heads(const pa_cache_desc* d, int32_t hq) {
  if (hq <= 0 || hq % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int g = hq / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16 && g != 32) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Largest split-K partition when the caller leaves it to the library (a row
// is then split into equal parts of at most this many keys): aim
// for about 16 workgroups per compute unit over the whole vector path, but
// give every partition at least 1 MiB of K and V (2048 keys of fp16 at head
// dim 128): each unit pays for filling and draining its waves' load
// pipelines, its merge and its partials, which shorter units amortise worse
// (256 decode rows of 1-4096 keys: 1536-key units 0.365 ms, 2048-3072 keys
// 0.360 ms; 1k-key rows and 32-sequence decode steps also lose to smaller
// units); twice that with groups of 16 or 32, whose units merge and write 4-8
// times the rows (the same rows unsplit: 0.444 -> 0.429 ms at G = 16, 0.486 ->
// 0.465 ms at G = 32); at most 4096 keys.
static int32_t auto_part(int64_t total_keys, int32_t hkv, int32_t head_dim, int32_t elem_bytes, int32_t group) {
  const int64_t target_units = 256 * 16;
  const int64_t min_keys = (int64_t)(group >= 16 ? 2 << 20 : 1 << 20) / (2 * head_dim * elem_bytes);
  int64_t p = std::max(total_keys * hkv / target_units, min_keys);
  p = (p + 255) / 256 * 256;
  return (int32_t)std::min<int64_t>(4096, p);
}

// Longest row-tile walk (in 64-key steps) when the caller leaves it to the
// library.  One row-tile workgroup fills a compute unit, so a batch with
// fewer row-tile workgroups than two rounds of the 256 compute units leaves
// part of the machine idle while its long tiles run: such a batch is split
// at about one workgroup's share of its row-tile work per compute unit, but
// at least 16 steps (1024 keys), which amortise a part's start and its share
// of the merge.  Measured with 512-query chunks over 8192 cached keys (fp16,
// 32/8 heads, d128): one chunk 0.272 -> 0.115 ms, two 0.288 -> 0.228 ms,
// four 0.359 -> 0.336 ms; one chunk over 32768 keys 0.948 -> 0.342 ms; finer
// splits (8 or 16 steps) were slower.  Larger grids are not split: the packed
// batch of eight chunks and 192 decode rows (512 row-tile workgroups) ran
// 0.289 -> 0.300 ms with its longest tiles split.
constexpr int64_t kComputeUnits = 256;
constexpr int32_t kMinSplitSteps = 16;
static int32_t auto_split_steps(int64_t tiles, int64_t tile_steps_total, int32_t hkv) {
  if (tiles * hkv >= 2 * kComputeUnits) return 0;
  const int64_t share = (tile_steps_total * hkv + kComputeUnits - 1) / kComputeUnits;
  return (int32_t)std::min<int64_t>(INT32_MAX / 2, std::max<int64_t>(share, kMinSplitSteps));
}

static pa_status make_plan(const pa_cache_desc* d, int32_t hq, int32_t num_seqs, const int32_t* hL,
                           const int32_t* hQ, int32_t max_blocks, const pa_attend_opts* opts, HostPlan& P) {
  pa_status st = check_desc(d);
  if (st != PA_OK) return st;
  if ((st = check_heads(d, hq)) != PA_OK) return st;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (hL == nullptr || hQ == nullptr)) return PA_ERR_NULL;
  const int g = hq / d->num_kv_heads;
  int32_t req_part = opts ? opts->partition_tokens : 0;
  // Row-tile (prefill) kernel from 16 rows of a sequence up; with groups of 16
  // or 32 a single query row already has that many, and its G rows go to the
  // matrix-core decode kernel instead (split-K units, one row per unit), so
  // there the row tiles start at two query rows.
  P.min_rows = (opts && opts->mfma_min_rows > 0) ? opts->mfma_min_rows : (g >= 16 ? 2 * g : 16);
  P.window = opts ? opts->window : 0;
  if (req_part > 0 && req_part % kBlockSize != 0) return PA_ERR_SHAPE;
  if (P.window < 0) return PA_ERR_SHAPE;
  const int64_t max_kv = (int64_t)max_blocks * kBlockSize;
  int64_t total_q = 0, vec_keys = 0;
  for (int i = 0; i < num_seqs; ++i) {
    if (hL[i] < 0 || hQ[i] < 0 || hQ[i] > hL[i] || hL[i] > max_kv) return PA_ERR_SHAPE;
    total_q += hQ[i];
    if (!(hQ[i] > 0 && (int64_t)hQ[i] * g >= P.min_rows))
      for (int t = 0; t < hQ[i]; ++t) vec_keys += vector_keys(hL[i] - hQ[i] + t, P.window);
  }
  if (total_q >= INT32_MAX / 2) return PA_ERR_SHAPE;
  P.total_q = (int32_t)total_q;
  P.part = req_part > 0 ? req_part
                       : (req_part < 0 ? 0 : auto_part(vec_keys, d->num_kv_heads, d->head_dim,
                                                       d->kv_dtype == PA_KV_I8 ? 1 : 2, g));
  // row tiles: their total walk picks the split (unless the caller fixed it), then units and parts are counted
  const int32_t req_split = opts ? opts->mfma_split_steps : 0;
  int64_t tile_steps = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int L = hL[i], Q = hQ[i];
    if (!(Q > 0 && (int64_t)Q * g >= P.min_rows)) continue;
    const int64_t nt = ((int64_t)Q * g + kMfmaRows - 1) / kMfmaRows;
    P.n_mtile += nt;
    for (int64_t r = 0; r < nt; ++r) tile_steps += tile_span(L, Q, g, (int)r, P.window).steps;
  }
  P.split_steps = req_split > 0 ? req_split
                  : (req_split < 0 || P.n_mtile == 0 ? 0 : auto_split_steps(P.n_mtile, tile_steps, d->num_kv_heads));
  for (int i = 0; i < num_seqs; ++i) {
    const int L = hL[i], Q = hQ[i];
    if (Q > 0 && (int64_t)Q * g >= P.min_rows) {
      const int64_t nt = ((int64_t)Q * g + kMfmaRows - 1) / kMfmaRows;
      for (int64_t r = 0; r < nt; ++r) {
        const int parts = tile_parts(tile_span(L, Q, g, (int)r, P.window).steps, P.split_steps);
        P.n_munit += parts;
        if (parts > 1) {
          P.n_msplit += 1;
          P.n_mslot += parts;
        }
      }
    } else {
      P.n_vtok += Q;
      for (int t = 0; t < Q; ++t) {
        const int parts = parts_for(vector_keys(L - Q + t, P.window), P.part);
        P.n_vunit += parts;
        P.max_parts = std::max(P.max_parts, parts);
      }
    }
  }
  if (P.n_vunit >= INT32_MAX / 2 || P.n_munit >= INT32_MAX / 2) return PA_ERR_SHAPE;
  // partial outputs of split row tiles: one float per (slot, KV head, tile row, dim)
  if (P.n_mslot * d->num_kv_heads * kMfmaRows >= INT32_MAX / 2) return PA_ERR_SHAPE;
  // A batch of one query row per sequence that no row splits and that fits in
  // about one round of workgroups needs no plan: the decode kernel reads each
  // sequence's length itself (longest-first ordering matters only when the
  // workgroups queue), which saves the plan kernel's launch and latency.
  bool one_row_each = P.n_munit == 0 && num_seqs > 0;
  for (int32_t i = 0; one_row_each && i < num_seqs; ++i) one_row_each = hQ[i] == 1;
  P.direct = one_row_each && P.max_parts <= 1 && (int64_t)num_seqs * d->num_kv_heads <= kDirectMaxGroups;
  // Other pure-decode batches of up to kSelfPlanMaxSeqs sequences need no plan
  // either: every decode workgroup derives the same bucketed unit order from
  // the device lengths and takes its own unit (a few LDS scans at its start,
  // beside other workgroups' loads, instead of a serial kernel in front).
  P.selfplan = PA_SELFPLAN && one_row_each && !P.direct && num_seqs <= kSelfPlanMaxSeqs;
  size_t off = 0;
  P.off_seqs = off;
  off = align_up(off + sizeof(SeqInfo) * (size_t)std::max(num_seqs, 1), 256);
  P.off_vtok = off;
  off = align_up(off + sizeof(VTok) * (size_t)std::max<int64_t>(P.n_vtok, 1), 256);
  P.off_vunit = off;
  off = align_up(off + sizeof(int2) * (size_t)std::max<int64_t>(P.n_vunit, 1), 256);
  P.off_vorder = off;
  off = align_up(off + sizeof(int32_t) * (size_t)std::max<int64_t>(P.n_vunit, 1), 256);
  P.off_vcost = off;
  off = align_up(off + sizeof(int32_t) * (size_t)std::max<int64_t>(P.n_vunit, 1), 256);
  P.off_munit = off;
  off = align_up(off + sizeof(int4) * (size_t)std::max<int64_t>(P.n_munit, 1), 256);
  P.off_munit_tmp = off;
  off = align_up(off + sizeof(int4) * (size_t)std::max<int64_t>(P.n_munit, 1), 256);
  P.off_msplit = off;
  off = align_up(off + sizeof(int4) * (size_t)std::max<int64_t>(P.n_msplit, 1), 256);
  const size_t mrows = (size_t)P.n_mslot * d->num_kv_heads * kMfmaRows;
  P.off_mlse = off;
  off = align_up(off + sizeof(float) * mrows, 256);
  P.off_mpo = off;
  off = align_up(off + sizeof(float) * mrows * d->head_dim, 256);
  const bool split = P.max_parts > 1;
  P.off_lse = off;
  if (split) off = align_up(off + sizeof(float) * (size_t)P.n_vunit * hq, 256);
  P.off_po = off;
  if (split) off = align_up(off + sizeof(float) * (size_t)P.n_vunit * hq * d->head_dim, 256);
  P.off_row_u0 = off;
  if (P.selfplan) off = align_up(off + sizeof(int2) * (size_t)num_seqs, 256);
  P.bytes = off;
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes are inconsistent, or an array is misaligned";
    case PA_ERR_DTYPE: return "unknown kv dtype";
    case PA_ERR_UNSUPPORTED: return "unsupported block size, head dim or group size";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_METADATA: return "device metadata breaks a precondition (debug build check)";
  }
  return "unknown status";
}

pa_status pa_write_kv(const pa_cache_desc* desc, const void* k, const void* v, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                      hipStream_t stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  if (desc->kv_dtype == PA_KV_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 4) || !scales_aligned(desc, k_scale, v_scale))
    return PA_ERR_SHAPE;
#if PA_DEBUG
  if ((st = debug_check_write(*desc, slot_mapping, num_tokens, stream)) != PA_OK) return st;
#endif
  hipError_t e;
  if (desc->kv_dtype == PA_KV_I8) {
    e = launch_write_i8(*desc, k, v, slot_mapping, num_tokens, k_cache, v_cache, k_scale, v_scale, stream);
  } else {
    e = launch_write_f16(*desc, k, v, slot_mapping, num_tokens, k_cache, v_cache, stream);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                         const int32_t* src_dst, int32_t num_pairs, hipStream_t stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst) return PA_ERR_NULL;
  if (desc->kv_dtype == PA_KV_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(src_dst, 4) ||
      !scales_aligned(desc, k_scale, v_scale))
    return PA_ERR_SHAPE;
#if PA_DEBUG
  if ((st = debug_check_copy(*desc, src_dst, num_pairs, stream)) != PA_OK) return st;
#endif
  hipError_t e = launch_copy(*desc, k_cache, v_cache, k_scale, v_scale, src_dst, num_pairs, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_check_write(const pa_cache_desc* desc, const int32_t* slot_mapping, int32_t num_tokens,
                         int32_t* status, hipStream_t stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (!status || (num_tokens > 0 && !slot_mapping)) return PA_ERR_NULL;
  if (!aligned(status, 4) || !aligned(slot_mapping, 4)) return PA_ERR_SHAPE;
  return launch_check_write(*desc, slot_mapping, num_tokens, status, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_check_attend(const pa_cache_desc* desc, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                          const int32_t* h_seq_lens, const int32_t* h_q_lens, const pa_attend_opts* opts,
                          int32_t* status, hipStream_t stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  if (opts && opts->window < 0) return PA_ERR_SHAPE;
  if (!status || (num_seqs > 0 && (!block_tables || !seq_lens || !q_lens || !h_seq_lens || !h_q_lens)))
    return PA_ERR_NULL;
  if (!aligned(status, 4) || !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(q_lens, 4))
    return PA_ERR_SHAPE;
  return launch_check_attend(*desc, block_tables, max_blocks_per_seq, seq_lens, q_lens, num_seqs, h_seq_lens,
                             h_q_lens, opts ? opts->window : 0, status, stream) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_check_copy(const pa_cache_desc* desc, const int32_t* src_dst, int32_t num_pairs, int32_t* status,
                        hipStream_t stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (!status || (num_pairs > 0 && !src_dst)) return PA_ERR_NULL;
  if (!aligned(status, 4) || !aligned(src_dst, 4)) return PA_ERR_SHAPE;
  return launch_check_copy(*desc, src_dst, num_pairs, status, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_attend_workspace_bytes(const pa_cache_desc* desc, int32_t num_q_heads, int32_t num_seqs,
                                 const int32_t* h_seq_lens, const int32_t* h_q_lens, const pa_attend_opts* opts) {
  HostPlan P;
  // the table width only bounds lengths; size the workspace for any width that fits them
  if (make_plan(desc, num_q_heads, num_seqs, h_seq_lens, h_q_lens, INT32_MAX / kBlockSize, opts, P) != PA_OK)
    return 0;
  return P.bytes;
}

pa_status pa_attend_plan_info(const pa_cache_desc* desc, int32_t num_q_heads, int32_t num_seqs,
                              const int32_t* h_seq_lens, const int32_t* h_q_lens, const pa_attend_opts* opts,
                              pa_attend_info* info) {
  if (info == nullptr) return PA_ERR_NULL;
  HostPlan P;
  const pa_status st = make_plan(desc, num_q_heads, num_seqs, h_seq_lens, h_q_lens, INT32_MAX / kBlockSize, opts, P);
  if (st != PA_OK) return st;
  info->partition_tokens = P.part;
  info->vector_rows = (int32_t)P.n_vtok;
  info->vector_units = (int32_t)P.n_vunit;
  info->max_parts = P.max_parts;
  info->mfma_tiles = (int32_t)P.n_mtile;
  info->mfma_units = (int32_t)P.n_munit;
  info->mfma_split_steps = P.split_steps;
  info->plan_free = P.direct ? 1 : (P.selfplan ? 2 : 0);
  info->workspace_bytes = P.bytes;
  return PA_OK;
}

}  // extern "C"

namespace pa {

// The new rows of a fused write (pa_write_attend): token i is the new token of
// sequence i.  NULL k: no fused write.
struct FusedWrite {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* slots = nullptr;
};

// pa_attend, with the KV write of a fused call folded into the decode units
// when the batch takes them alone (otherwise the write kernel runs first).
static pa_status attend_impl(const pa_cache_desc* desc, const void* q, int32_t num_q_heads, const void* k_cache,
                             const void* v_cache, const void* k_scale, const void* v_scale,
                             const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             const int32_t* q_lens, int32_t num_seqs, const int32_t* h_seq_lens,
                             const int32_t* h_q_lens, float scale, void* out, void* workspace, size_t workspace_bytes,
                             const pa_attend_opts* opts, hipStream_t stream, FusedWrite fw) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq < 0) return PA_ERR_SHAPE;
  HostPlan P;
  if ((st = make_plan(desc, num_q_heads, num_seqs, h_seq_lens, h_q_lens, max_blocks_per_seq, opts, P)) != PA_OK)
    return st;
  if (P.total_q == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !q_lens || !out || !workspace) return PA_ERR_NULL;
  if (desc->kv_dtype == PA_KV_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(workspace, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(q_lens, 4) ||
      !scales_aligned(desc, k_scale, v_scale))
    return PA_ERR_SHAPE;
  // the decode kernel's scale reads are range-checked against a 31-bit byte count
  if (desc->kv_dtype == PA_KV_I8 &&
      (int64_t)desc->num_blocks * std::max(desc->num_layers, 1) * desc->num_kv_heads * 2 > INT32_MAX)
    return PA_ERR_UNSUPPORTED;
  if (max_blocks_per_seq == 0) return PA_ERR_SHAPE;
  if (!(scale > 0.f) || scale > 3.0e38f) return PA_ERR_SHAPE;   // positive and finite
  if (opts && opts->side_stream && (!opts->side_fork || !opts->side_join)) return PA_ERR_NULL;
  if (workspace_bytes < P.bytes) return PA_ERR_WORKSPACE;
#if PA_DEBUG
  if ((st = debug_check_attend(*desc, block_tables, max_blocks_per_seq, seq_lens, q_lens, num_seqs, h_seq_lens,
                               h_q_lens, P.window, stream)) != PA_OK)
    return st;
#endif

  char* ws = (char*)workspace;
  const int g = num_q_heads / desc->num_kv_heads;
  const bool i8 = desc->kv_dtype == PA_KV_I8;

  PlanArgs pl;
  pl.seq_lens = seq_lens;
  pl.q_lens = q_lens;
  pl.seqs = (SeqInfo*)(ws + P.off_seqs);
  pl.vtok = (VTok*)(ws + P.off_vtok);
  pl.vunit = (int2*)(ws + P.off_vunit);
  pl.vorder = (int32_t*)(ws + P.off_vorder);
  pl.vcost = (int32_t*)(ws + P.off_vcost);
  pl.munit = (int4*)(ws + P.off_munit);
  pl.munit_tmp = (int4*)(ws + P.off_munit_tmp);
  pl.msplit = (int4*)(ws + P.off_msplit);
  pl.split_steps = P.split_steps;
  pl.num_seqs = num_seqs;
  pl.group = g;
  pl.part = P.part;
  pl.window = P.window;
  pl.min_rows = P.min_rows;
  pl.max_kv = (int32_t)std::min<int64_t>((int64_t)max_blocks_per_seq * kBlockSize, INT32_MAX);
  pl.total_q = P.total_q;
  pl.cap_vtok = (int32_t)P.n_vtok;
  pl.cap_vunit = (int32_t)P.n_vunit;
  pl.cap_munit = (int32_t)P.n_munit;
  pl.cap_msplit = (int32_t)P.n_msplit;
  pl.cap_mslot = (int32_t)P.n_mslot;
  const bool direct = P.direct;
  if (!direct && !P.selfplan && !(opts && opts->reuse_plan) && launch_plan(pl, stream) != hipSuccess)
    return PA_ERR_HIP;

  // the addressed layer's first tile of block 0; tiles of one block are num_layers * hkv apart
  const int64_t tile0 = (int64_t)desc->layer * desc->num_kv_heads;
  const int64_t tile_bytes = (int64_t)kBlockSize * desc->head_dim * (i8 ? 1 : 2);
  AttnArgs a;
  a.q = q;
  a.kc = (const char*)k_cache + tile0 * tile_bytes;
  a.vc = (const char*)v_cache + tile0 * tile_bytes;
  a.ks = i8 ? (const half_t*)k_scale + tile0 : nullptr;
  a.vs = i8 ? (const half_t*)v_scale + tile0 : nullptr;
  a.block_tables = block_tables;
  a.seqs = pl.seqs;
  a.vtok = pl.vtok;
  a.vunit = pl.vunit;
  a.vorder = pl.vorder;
  a.munit = pl.munit;
  a.msplit = pl.msplit;
  a.mlse = (float*)(ws + P.off_mlse);
  a.mpo = (float*)(ws + P.off_mpo);
  a.plse = P.max_parts > 1 ? (float*)(ws + P.off_lse) : nullptr;
  a.po = P.max_parts > 1 ? (float*)(ws + P.off_po) : nullptr;
  a.out = out;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = desc->num_blocks;
  a.hq = num_q_heads;
  a.hkv = desc->num_kv_heads;
  a.blk_tiles = std::max(desc->num_layers, 1) * desc->num_kv_heads;
  a.part = P.part > 0 ? P.part : INT32_MAX / 2;
  a.window = P.window;
  a.scale_log2 = scale * kLog2e;
  a.scale_count = (int64_t)desc->num_blocks * a.blk_tiles - tile0;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.max_kv = pl.max_kv;
  a.direct = direct ? 1 : 0;
  a.selfplan = P.selfplan ? 1 : 0;
  a.num_seqs = num_seqs;
  a.n_units = (int32_t)P.n_vunit;
  a.row_u0 = P.selfplan ? (int2*)(ws + P.off_row_u0) : nullptr;
  a.new_k = a.new_v = nullptr;
  a.new_slots = nullptr;
  if (fw.k != nullptr) {
    if (P.n_munit == 0 && g < 16) {
      a.new_k = fw.k;
      a.new_v = fw.v;
      a.new_slots = fw.slots;
    } else if (launch_write_f16(*desc, fw.k, fw.v, fw.slots, num_seqs, const_cast<void*>(k_cache),
                                const_cast<void*>(v_cache), stream) != hipSuccess) {
      return PA_ERR_HIP;   // rows on the matrix cores: the write kernel first, as pa_write_kv
    }
  }

  auto mark = [&](hipEvent_t ev, hipStream_t s) { return ev == nullptr || hipEventRecord(ev, s) == hipSuccess; };
  // With a side stream the row tiles run there, beside the decode units on `stream`.
  const bool side = opts && opts->side_stream && P.n_vunit > 0 && P.n_munit > 0;
  const hipStream_t rs = side ? opts->side_stream : stream;
  auto row_tiles = [&]() {
    if (!mark(opts ? opts->mfma_begin : nullptr, rs)) return false;
    if (launch_prefill(a, desc->head_dim, g, desc->kv_dtype, (int)P.n_munit, rs) != hipSuccess) return false;
    // the parts of split row tiles, merged into their rows
    if (P.n_msplit > 0 &&
        launch_prefill_merge(a, desc->head_dim, g, desc->kv_dtype, (int)P.n_msplit, rs) != hipSuccess)
      return false;
    return mark(opts ? opts->mfma_end : nullptr, rs);
  };
  if (side && (hipEventRecord(opts->side_fork, stream) != hipSuccess ||
               hipStreamWaitEvent(opts->side_stream, opts->side_fork, 0) != hipSuccess || !row_tiles()))
    return PA_ERR_HIP;
  if (P.n_vunit > 0) {
    if (!mark(opts ? opts->vector_begin : nullptr, stream)) return PA_ERR_HIP;
    if (launch_decode(a, desc->head_dim, g, desc->kv_dtype, (int)P.n_vunit, stream) != hipSuccess) return PA_ERR_HIP;
    if (!mark(opts ? opts->vector_end : nullptr, stream)) return PA_ERR_HIP;
    // one merge workgroup per vector row (self-planned: per sequence, the same count)
    if (P.max_parts > 1 && launch_reduce(a, desc->head_dim, g, desc->kv_dtype, (int)P.n_vtok, stream) != hipSuccess)
      return PA_ERR_HIP;
  }
  if (side) {
    if (hipEventRecord(opts->side_join, opts->side_stream) != hipSuccess ||
        hipStreamWaitEvent(stream, opts->side_join, 0) != hipSuccess)
      return PA_ERR_HIP;
  } else if (P.n_munit > 0 && !row_tiles()) {
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace pa

extern "C" {

pa_status pa_attend(const pa_cache_desc* desc, const void* q, int32_t num_q_heads, const void* k_cache,
                    const void* v_cache, const void* k_scale, const void* v_scale, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                    const int32_t* h_seq_lens, const int32_t* h_q_lens, float scale, void* out, void* workspace,
                    size_t workspace_bytes, const pa_attend_opts* opts, hipStream_t stream) {
  return attend_impl(desc, q, num_q_heads, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                     seq_lens, q_lens, num_seqs, h_seq_lens, h_q_lens, scale, out, workspace, workspace_bytes, opts,
                     stream, FusedWrite{});
}

pa_status pa_write_attend(const pa_cache_desc* desc, const void* k, const void* v, const int32_t* slot_mapping,
                          int32_t num_tokens, const void* q, int32_t num_q_heads, void* k_cache, void* v_cache,
                          void* k_scale, void* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                          const int32_t* h_seq_lens, const int32_t* h_q_lens, float scale, void* out,
                          void* workspace, size_t workspace_bytes, const pa_attend_opts* opts, hipStream_t stream) {
  // The fused form: a 16-bit pool, one new token and one query row per
  // sequence, the token of sequence i at index i, the write's own arguments
  // valid.  Debug builds always take the two calls, so that each one's
  // metadata check runs.
  bool fused = !PA_DEBUG && check_desc(desc) == PA_OK && desc->kv_dtype != PA_KV_I8 && num_seqs > 0 &&
               num_tokens == num_seqs && h_q_lens != nullptr && k && v && slot_mapping && k_cache && v_cache &&
               aligned(k, 16) && aligned(v, 16) && aligned(slot_mapping, 4) && aligned(k_cache, 16) &&
               aligned(v_cache, 16);
  for (int32_t i = 0; fused && i < num_seqs; ++i) fused = h_q_lens[i] == 1;
  if (!fused) {
    const pa_status st = pa_write_kv(desc, k, v, slot_mapping, num_tokens, k_cache, v_cache, k_scale, v_scale, stream);
    if (st != PA_OK) return st;
    return pa_attend(desc, q, num_q_heads, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                     seq_lens, q_lens, num_seqs, h_seq_lens, h_q_lens, scale, out, workspace, workspace_bytes, opts,
                     stream);
  }
  FusedWrite fw;
  fw.k = k;
  fw.v = v;
  fw.slots = slot_mapping;
  return attend_impl(desc, q, num_q_heads, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                     seq_lens, q_lens, num_seqs, h_seq_lens, h_q_lens, scale, out, workspace, workspace_bytes, opts,
                     stream, fw);
}

}  // extern "C"

// ------------------------------------------------------ fixed scratch ----
// pa_attend_noalloc's workspace: one array per GPU, allocated with the code
// object when the library is first used on that device and held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it names a stand-in, not device memory): the device address is looked
// up once per device and kept.
namespace pa {

static __device__ __align__(256) char scratch[PA_ATTEND_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
static pa_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

}  // namespace pa

extern "C" pa_status pa_attend_noalloc(const pa_cache_desc* desc, const void* q, int32_t num_q_heads,
                                       const void* k_cache, const void* v_cache, const void* k_scale,
                                       const void* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                                       const int32_t* h_seq_lens, const int32_t* h_q_lens, float scale, void* out,
                                       const pa_attend_opts* opts, hipStream_t stream) {
  // the size check needs only the host arguments: an oversized batch is refused before the GPU is touched
  HostPlan P;
  const int32_t width = max_blocks_per_seq >= 0 ? max_blocks_per_seq : 0;
  pa_status st = make_plan(desc, num_q_heads, num_seqs, h_seq_lens, h_q_lens, width, opts, P);
  if (st != PA_OK) return st;
  // the automatic split of long row tiles adds partial outputs; without room for them the tiles stay whole
  pa_attend_opts whole;
  if (P.bytes > (size_t)PA_ATTEND_SCRATCH_BYTES && P.n_msplit > 0 && (opts == nullptr || opts->mfma_split_steps == 0)) {
    if (opts) whole = *opts;
    else std::memset(&whole, 0, sizeof(whole));
    whole.mfma_split_steps = -1;
    HostPlan unsplit;
    if ((st = make_plan(desc, num_q_heads, num_seqs, h_seq_lens, h_q_lens, width, &whole, unsplit)) != PA_OK) return st;
    P = unsplit;
    opts = &whole;
  }
  if (P.bytes > (size_t)PA_ATTEND_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  if (P.total_q == 0) return PA_OK;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != PA_OK) return st;
  return pa_attend(desc, q, num_q_heads, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks_per_seq,
                   seq_lens, q_lens, num_seqs, h_seq_lens, h_q_lens, scale, out, ws, PA_ATTEND_SCRATCH_BYTES, opts,
                   stream);
}
