// Device-side checks of the metadata the kernels take on trust: slot numbers,
// block table entries, lengths and copy pairs (the preconditions pa.h lists).
// pa_check_write / pa_check_attend / pa_check_copy run them on the caller's
// stream into a caller-provided status buffer; a library built with
// PA_DEBUG=1 runs them itself before every write, attention and copy and
// refuses the call with PA_ERR_METADATA when one fails.
#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace pa {

// status[0] = violation code (0: none), [1] index, [2] value, [3] bound;
// [4..7] length sums of the attention check (compared with the host's).
__device__ void record(int32_t* st, int code, int index, int value, int bound) {
  if (atomicCAS(&st[0], 0, code) == 0) {
    st[1] = index;
    st[2] = value;
    st[3] = bound;
  }
}

// A fill kernel, not a memset, so the checks can sit in a captured graph.
__global__ void check_reset_kernel(int32_t* st) {
  if (threadIdx.x < PA_CHECK_STATUS_WORDS) st[threadIdx.x] = 0;
}

// Slots: in range (negative = skipped), pairwise distinct, and for int8 pools
// the tokens of one block consecutive with consecutive offsets (the replay
// order the int8 write relies on).  Thread t compares its slot with every
// later one.
__global__ __launch_bounds__(256) void check_write_kernel(const int32_t* __restrict__ slots, int32_t T,
                                                          int64_t num_slots, int32_t runs, int32_t* st) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int s = slots[t];
  if (s < 0) return;
  if (s >= num_slots) {
    record(st, PA_CHECK_SLOT_RANGE, t, s, (int)(num_slots < INT32_MAX ? num_slots : INT32_MAX));
    return;
  }
  for (int u = t + 1; u < T; ++u) {
    const int su = slots[u];
    if (su < 0 || su >= num_slots) continue;
    if (su == s) {
      record(st, PA_CHECK_SLOT_DUPLICATE, u, su, t);
      return;
    }
    if (runs && su / kBlockSize == s / kBlockSize && su - s != u - t) {
      record(st, PA_CHECK_SLOT_RUN, u, su, t);
      return;
    }
  }
}

// One workgroup per sequence: 0 <= q_len <= seq_len <= table width, the
// length sums (plain and position-weighted, mod 2^32) for the comparison with
// the host copies, and every table entry a query of the step can read (from
// the block holding the earliest key in a sliding window to the last key) a
// block id in [0, num_blocks).
struct CheckAttendArgs {
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* q_lens;
  int32_t max_blocks, num_blocks, window;
  int64_t max_kv;
};

__global__ __launch_bounds__(256) void check_attend_kernel(CheckAttendArgs a, int32_t* st) {
  const int i = blockIdx.x;
  const int L = a.seq_lens[i], Q = a.q_lens[i];
  if (threadIdx.x == 0) {
    atomicAdd((uint32_t*)&st[4], (uint32_t)L);
    atomicAdd((uint32_t*)&st[5], (uint32_t)L * (uint32_t)(i + 1));
    atomicAdd((uint32_t*)&st[6], (uint32_t)Q);
    atomicAdd((uint32_t*)&st[7], (uint32_t)Q * (uint32_t)(i + 1));
    if (Q < 0 || Q > L || L > a.max_kv) record(st, PA_CHECK_LENGTHS, i, L, Q);
  }
  if (Q < 0 || Q > L || L > a.max_kv || Q == 0) return;
  const int lo = a.window > 0 ? max(0, L - Q - a.window + 1) : 0;
  const int32_t* tbl = a.block_tables + (int64_t)i * a.max_blocks;
  for (int b = lo / kBlockSize + threadIdx.x; b < (L + kBlockSize - 1) / kBlockSize; b += blockDim.x) {
    const int id = tbl[b];
    if (id < 0 || id >= a.num_blocks) record(st, PA_CHECK_BLOCK_ID, i, id, b);
  }
}

// The sums of the device lengths against the host copies' (after the check).
__global__ void check_lengths_kernel(int32_t* st, uint32_t sum_l, uint32_t wsum_l, uint32_t sum_q, uint32_t wsum_q) {
  if (threadIdx.x != 0) return;
  if ((uint32_t)st[4] != sum_l || (uint32_t)st[5] != wsum_l) record(st, PA_CHECK_HOST_LENGTHS, -1, 0, 0);
  if ((uint32_t)st[6] != sum_q || (uint32_t)st[7] != wsum_q) record(st, PA_CHECK_HOST_LENGTHS, -1, 1, 0);
}

// Copy pairs: ids in range; no destination is another pair's source or destination.
__global__ __launch_bounds__(256) void check_copy_kernel(const int2* __restrict__ pairs, int32_t n, int32_t nb,
                                                         int32_t* st) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n) return;
  const int2 pr = pairs[p];
  if (pr.x < 0 || pr.x >= nb || pr.y < 0 || pr.y >= nb) {
    record(st, PA_CHECK_COPY_PAIR, p, pr.x < 0 || pr.x >= nb ? pr.x : pr.y, nb);
    return;
  }
  for (int q = 0; q < n; ++q) {
    if (q == p) continue;
    const int2 o = pairs[q];
    if (o.x == pr.y || o.y == pr.y) {
      record(st, PA_CHECK_COPY_PAIR, p, pr.y, q);
      return;
    }
  }
}

static int grid_for(int64_t n) { return (int)((n + 255) / 256); }

hipError_t launch_check_write(const pa_cache_desc& d, const int32_t* slots, int32_t T, int32_t* st, hipStream_t s) {
  check_reset_kernel<<<1, 64, 0, s>>>(st);
  if (T > 0)
    check_write_kernel<<<grid_for(T), 256, 0, s>>>(slots, T, (int64_t)d.num_blocks * kBlockSize,
                                                    d.kv_dtype == PA_KV_I8 ? 1 : 0, st);
  return hipGetLastError();
}

hipError_t launch_check_attend(const pa_cache_desc& d, const int32_t* tables, int32_t max_blocks,
                               const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                               const int32_t* hL, const int32_t* hQ, int32_t window, int32_t* st, hipStream_t s) {
  uint32_t sl = 0, wsl = 0, sq = 0, wsq = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    sl += (uint32_t)hL[i];
    wsl += (uint32_t)hL[i] * (uint32_t)(i + 1);
    sq += (uint32_t)hQ[i];
    wsq += (uint32_t)hQ[i] * (uint32_t)(i + 1);
  }
  CheckAttendArgs a;
  a.block_tables = tables;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.max_blocks = max_blocks;
  a.num_blocks = d.num_blocks;
  a.window = window;
  a.max_kv = (int64_t)max_blocks * kBlockSize;
  check_reset_kernel<<<1, 64, 0, s>>>(st);
  if (num_seqs > 0) check_attend_kernel<<<num_seqs, 256, 0, s>>>(a, st);
  check_lengths_kernel<<<1, 64, 0, s>>>(st, sl, wsl, sq, wsq);
  return hipGetLastError();
}

hipError_t launch_check_copy(const pa_cache_desc& d, const int32_t* pairs, int32_t n, int32_t* st, hipStream_t s) {
  check_reset_kernel<<<1, 64, 0, s>>>(st);
  if (n > 0) check_copy_kernel<<<grid_for(n), 256, 0, s>>>((const int2*)pairs, n, d.num_blocks, st);
  return hipGetLastError();
}

#if PA_DEBUG
// The debug build's own status words: one array per GPU, its device address
// looked up once per device (host code never passes the array's name to a
// kernel).
static __device__ __align__(256) int32_t debug_status[PA_CHECK_STATUS_WORDS];
static std::atomic<int32_t*> g_debug_status[64];
static std::mutex g_debug_mu;

static pa_status debug_status_ptr(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= 64) return PA_ERR_UNSUPPORTED;
  int32_t* p = g_debug_status[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_debug_mu);
    p = g_debug_status[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* v = nullptr;
      if (hipGetSymbolAddress(&v, HIP_SYMBOL(debug_status)) != hipSuccess || v == nullptr) return PA_ERR_HIP;
      p = (int32_t*)v;
      g_debug_status[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

// Waits for the checks just enqueued and turns a violation into a status.
static pa_status debug_outcome(int32_t* st, hipStream_t s) {
  int32_t h[4] = {0, 0, 0, 0};
  if (hipMemcpyAsync(h, st, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess) return PA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  return h[0] == 0 ? PA_OK : PA_ERR_METADATA;
}

pa_status debug_check_write(const pa_cache_desc& d, const int32_t* slots, int32_t T, hipStream_t s) {
  int32_t* st = nullptr;
  pa_status r = debug_status_ptr(&st);
  if (r != PA_OK) return r;
  if (launch_check_write(d, slots, T, st, s) != hipSuccess) return PA_ERR_HIP;
  return debug_outcome(st, s);
}

pa_status debug_check_attend(const pa_cache_desc& d, const int32_t* tables, int32_t max_blocks,
                             const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs, const int32_t* hL,
                             const int32_t* hQ, int32_t window, hipStream_t s) {
  int32_t* st = nullptr;
  pa_status r = debug_status_ptr(&st);
  if (r != PA_OK) return r;
  if (launch_check_attend(d, tables, max_blocks, seq_lens, q_lens, num_seqs, hL, hQ, window, st, s) != hipSuccess)
    return PA_ERR_HIP;
  return debug_outcome(st, s);
}

pa_status debug_check_copy(const pa_cache_desc& d, const int32_t* pairs, int32_t n, hipStream_t s) {
  int32_t* st = nullptr;
  pa_status r = debug_status_ptr(&st);
  if (r != PA_OK) return r;
  if (launch_check_copy(d, pairs, n, st, s) != hipSuccess) return PA_ERR_HIP;
  return debug_outcome(st, s);
}
#endif

}  // namespace pa
