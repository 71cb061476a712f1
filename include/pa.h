/*
 * pa.h - C ABI of libpa.so: paged KV writes and paged attention on one
 * AMD Instinct MI355X (gfx950).
 *
 * The pages this library follows (cited by title and section):
 *   [pytorch]   "How to Implement Paged Attention in PyTorch and vLLM"
 *   [engine]    "Building a paged inference engine from scratch, and measuring
 *               it honestly"
 *   [manager]   "Build a paged KV cache manager from scratch"
 *   [nanoserve] "Day 14: the block allocator, paging for attention starts as
 *               pure bookkeeping"
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every buffer argument is a DEVICE pointer unless its name starts with
 *   h_ (host memory).  The caller owns every buffer, including the attention
 *   workspace; the library allocates no device memory and keeps no global
 *   mutable state (except the fixed per-GPU scratch of pa_attend_noalloc).
 * - Work is enqueued on `stream` and returns without synchronising.  The
 *   status only covers what the host can check: argument validation and kernel
 *   launch errors.  Arguments are checked before anything is enqueued.
 * - KV pool layout (a reading: the pages store K and V either in one per-block
 *   slab, [manager] "Step 1: The Block", or as two tensors, [pytorch]
 *   "Allocate, append, and free KV-cache blocks"): two pools, K and V, each
 *       [num_blocks][num_layers][num_kv_heads][block_size][head_dim]
 *   of fp16 (PA_KV_F16), bf16 (PA_KV_BF16) or int8 codes (PA_KV_I8), so one
 *   (block, layer, KV
 *   head) tile is one contiguous run of block_size * head_dim elements.  A
 *   physical block holds its tokens for every layer ([pytorch] "Allocate,
 *   append, and free KV-cache blocks" keeps the layer axis inside the block),
 *   so one block table and one slot mapping serve all layers; num_layers = 1
 *   is the single-layer pool [num_blocks][num_kv_heads][block_size][head_dim].
 *   int8 pools carry per-block-per-layer-per-head fp16 scales k_scale,
 *   v_scale [num_blocks][num_layers][num_kv_heads] ([engine] "INT8 KV cache
 *   design": symmetric, no zero point, one scale per block per head).
 * - Supported shapes: block_size 16, head_dim 64 or 128, num_q_heads a
 *   multiple of num_kv_heads with a group size of 1, 2, 4, 8, 16 or 32,
 *   num_blocks * block_size < 2^31, and for int8 pools scale arrays of
 *   less than 2^31 bytes (pa_attend).  Anything else returns
 *   PA_ERR_UNSUPPORTED (or PA_ERR_SHAPE for inconsistent sizes).
 * - Device arrays: q, k, v, out, the pools and the workspace 16-byte
 *   aligned (the kernels move them in 16-byte vectors), int32 arrays 4-byte
 *   and fp16 scale arrays 2-byte aligned; PA_ERR_SHAPE otherwise.
 * - Device-side integer data (slots, block ids, lengths) are preconditions.
 *   Kernels never read or write outside the pools for out-of-range values:
 *   an out-of-range slot is skipped and an out-of-range block id reads block
 *   0, so bad metadata gives wrong numbers, never a memory fault.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL                       */
  PA_ERR_SHAPE = 2,        /* sizes inconsistent with each other, or a
                              misaligned device array                        */
  PA_ERR_DTYPE = 3,        /* unknown kv_dtype                                 */
  PA_ERR_UNSUPPORTED = 4,  /* valid but not built: block size, head dim, group */
  PA_ERR_WORKSPACE = 5,    /* workspace smaller than pa_attend_workspace_bytes */
  PA_ERR_HIP = 6,          /* a HIP launch failed                              */
  PA_ERR_METADATA = 7      /* debug builds: device metadata breaks a precondition
                              (see pa_check_write / pa_check_attend)           */
} pa_status;

/* Element type of the pools.  The activations a call takes and returns (new
 * K/V rows, queries, outputs) are bf16 for PA_KV_BF16 and fp16 otherwise
 * ([pytorch] "Compute reference attention without hiding the layout" tests
 * fp16 and bf16 caches, each against its own tolerance). */
typedef enum { PA_KV_F16 = 0, PA_KV_I8 = 1, PA_KV_BF16 = 2 } pa_kv_dtype;

/* Shape of one KV pool pair (see the layout above) and the layer a call
 * addresses. */
typedef struct {
  int32_t num_blocks;    /* physical blocks in each pool                  */
  int32_t block_size;    /* tokens per block (16)                         */
  int32_t num_kv_heads;
  int32_t head_dim;      /* 64 or 128                                     */
  int32_t kv_dtype;      /* pa_kv_dtype                                   */
  int32_t num_layers;    /* layers per block; 0 is taken as 1             */
  int32_t layer;         /* the layer pa_write_kv / pa_attend address,
                            0 <= layer < num_layers (pa_copy_blocks copies
                            every layer of a block and ignores it)        */
} pa_cache_desc;

/*
 * pa_write_kv - write this step's new K/V rows into the pools through a slot
 * mapping ([pytorch] "How to implement paged attention: the minimal data
 * flow", steps 2-3; "Map the PyTorch design to vLLM PagedAttention": slot
 * mappings are integer tensors handed over each step).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], row-major: fp16
 *                 (bf16 for PA_KV_BF16 pools).
 *   slot_mapping  int32 [num_tokens]; slot = block_id * block_size + offset.
 *                 A negative slot skips that token (padding).  Slots of one
 *                 call must be distinct.
 *   k_cache, v_cache  the pools (fp16, bf16 or int8 codes, per desc->kv_dtype).
 *   k_scale, v_scale  fp16 [num_blocks][num_layers][num_kv_heads] for
 *                 PA_KV_I8, else ignored (may be NULL).
 * Rows go to layer desc->layer of the pools; the other layers are untouched.
 *
 * fp16 and bf16: token t's K/V of every head are copied bit-for-bit to offset
 * slot % block_size of block slot / block_size.
 *
 * int8 ([engine] "INT8 KV cache design": on every token write the block's
 * entries are dequantised, the new token appended, a new max-abs scale taken
 * and everything requantised).  For each token in increasing t, separately
 * for K and V and for each KV head, with o = slot % block_size and entries
 * 0..o-1 of the block taken as valid:
 *     x_j = float(code_j) * float(scale)  (j < o),  x_o = float(new)
 *     scale' = fp16_rne(max_j |x_j| / 127.0f)        (IEEE fp32 division)
 *     code_j = clamp(rint_half_even(x_j / float(scale')), -127, 127)
 *              (all zero if scale' == 0), for j = 0..o.
 * Entries past o are not touched.  Tokens that write the same block in one
 * call must be consecutive in t with consecutive offsets (a sequence's new
 * tokens packed in position order), which is how the replay order is found.
 */
pa_status pa_write_kv(const pa_cache_desc* desc, const void* k, const void* v,
                      const int32_t* slot_mapping, int32_t num_tokens,
                      void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                      hipStream_t stream);

/*
 * Dispatch options of pa_attend (NULL = defaults; zero-initialise unused fields).
 *   partition_tokens  largest split-K partition of the vector path, in
 *                     keys: a row of n keys is split into ceil(n / p) equal
 *                     partitions (rounded up to 16 keys; the last one takes
 *                     what remains).  0 = p chosen from the batch, > 0 = p
 *                     (a multiple of 16), < 0 = never split.
 *   mfma_min_rows     a sequence whose q_len * group rows reach this count
 *                     runs on the row-tile (prefill) kernel, otherwise its
 *                     query rows are split-K units of the decode kernel:
 *                     0 = default (16; 2 * group for groups of 16 or 32),
 *                     1 = every sequence on row tiles, INT32_MAX = every
 *                     query row as decode units.  Groups of 16 or 32 run
 *                     their decode units on the matrix cores too (one query
 *                     row is already 16 or 32 rows of a dense product); the
 *                     smaller groups on the vector ALUs.
 *   vector_begin/end  optional caller-created HIP events, recorded on
 *   mfma_begin/end    `stream` immediately before and after the vector-path
 *                     (resp. MFMA-path) attention kernel when that kernel is
 *                     launched; NULL = not recorded.  For per-kernel timing.
 *   window            sliding window ([pytorch] "PagedAttention vs
 *                     sliding-window attention, RadixAttention, and SSMs":
 *                     each query attends only to the most recent `window`
 *                     tokens): 0 = none; w > 0 = the query at position P
 *                     sees keys max(0, P - w + 1) .. P.  Table entries of
 *                     blocks that hold no key at or after the earliest one a
 *                     step's queries see (seq_len - q_len - w + 1) are never
 *                     read, so the caller may have released those blocks.
 *                     Negative: PA_ERR_SHAPE.
 *   reuse_plan        0 = plan the batch (one small kernel that turns the
 *                     device lengths into work lists in the workspace);
 *                     1 = use the plan an earlier pa_attend call left in
 *                     this workspace.  The caller promises that the call is
 *                     ordered after that one on the device and that the
 *                     lengths (host and device), the table width, num_q_heads,
 *                     num_kv_heads and the other options are the same: the
 *                     case of the layers of one model step, which share the
 *                     block tables and lengths ([engine] "07 Open items":
 *                     build the step's block table and batch metadata once
 *                     per step, not once per layer).
 *   side_stream       optional second stream (same device, default priority)
 *   side_fork         with two caller-created events (hipEventDisableTiming
 *   side_join         is enough): when a batch has both decode units and row
 *                     tiles ([engine] "02 The engine": one packed batch of
 *                     prefill chunks and decode rows), the row-tile kernel
 *                     runs on side_stream beside the decode kernels on
 *                     `stream` (side_stream waits for side_fork, recorded on
 *                     `stream` after the plan; `stream` waits for side_join,
 *                     recorded on side_stream after the row tiles), so the
 *                     HBM-bound and the matrix-bound kernels can share the
 *                     GPU.  All three NULL: everything on `stream`.  Either
 *                     way the call's work is complete when `stream` reaches
 *                     the point after the call.
 *   mfma_split_steps  longest key range, in 64-key steps, that one
 *                     workgroup of the row-tile kernel walks: a row tile
 *                     (256 query rows of a sequence) whose keys span more
 *                     steps is split into ceil(steps / s) parts of equal
 *                     step counts, each run by its own workgroup, and the
 *                     parts' (max, sum, output) are merged in log-sum-exp
 *                     form into the tile's rows (the split-K of the decode
 *                     path, applied to long chunked-prefill contexts).
 *                     0 = chosen from the batch: a batch with fewer than
 *                     512 row-tile workgroups (two per compute unit) is
 *                     split at about one workgroup's share of its row-tile
 *                     work per compute unit (at least 16 steps), a larger
 *                     one is not; > 0 = s, < 0 = never split.
 */
typedef struct {
  int32_t partition_tokens;
  int32_t mfma_min_rows;
  hipEvent_t vector_begin;
  hipEvent_t vector_end;
  hipEvent_t mfma_begin;
  hipEvent_t mfma_end;
  int32_t window;
  int32_t reuse_plan;
  hipStream_t side_stream;
  hipEvent_t side_fork;
  hipEvent_t side_join;
  int32_t mfma_split_steps;
} pa_attend_opts;

/*
 * pa_attend_workspace_bytes - device workspace pa_attend needs for this batch
 * (same arguments as pa_attend's host side).  Returns 0 when the arguments
 * are invalid (pa_attend then reports why).  The size depends only on the
 * host lengths, the head counts and the options.
 */
size_t pa_attend_workspace_bytes(const pa_cache_desc* desc, int32_t num_q_heads,
                                 int32_t num_seqs, const int32_t* h_seq_lens,
                                 const int32_t* h_q_lens, const pa_attend_opts* opts);

/*
 * pa_attend_plan_info - how pa_attend would run this batch, decided from the
 * host lengths alone (no device work; same arguments as
 * pa_attend_workspace_bytes).  For callers that size buffers once for an
 * upper bound on the lengths: with partition_tokens fixed to the value
 * returned here, the workspace a batch needs never grows when its lengths
 * shrink.
 *   partition_tokens  the largest split-K partition in keys (0: rows are never
 *                     split); rows longer than it are split
 *   vector_rows       query rows on the vector path
 *   vector_units      (row, partition) units of the vector path, per KV head
 *   max_parts         the most partitions of one row (> 1: the merge kernel runs)
 *   mfma_tiles        row tiles of the MFMA path, per KV head
 *   plan_free         0 when a plan kernel turns the device lengths into work
 *                     lists first; 1 for a batch of one query row per
 *                     sequence, no row split and at most 1024 (sequence, KV
 *                     head) pairs: decode workgroup x serves sequence x and
 *                     reads its length itself; 2 for any other batch of one
 *                     query row per sequence with at most 1024 sequences:
 *                     every decode workgroup derives the same unit order
 *                     (largest units first) from the device lengths and
 *                     takes its own unit
 *   workspace_bytes   what pa_attend_workspace_bytes returns
 *   mfma_units        row-tile workgroups per KV head (a split tile counts
 *                     once per part)
 *   mfma_split_steps  the split of long row tiles (0: none is split); with
 *                     mfma_split_steps fixed to this value as well, the
 *                     workspace never grows when the lengths shrink
 * Returns the status pa_attend would return for these host arguments.
 */
typedef struct {
  int32_t partition_tokens;
  int32_t vector_rows;
  int32_t vector_units;
  int32_t max_parts;
  int32_t mfma_tiles;
  int32_t plan_free;
  size_t workspace_bytes;
  int32_t mfma_units;
  int32_t mfma_split_steps;
} pa_attend_info;

pa_status pa_attend_plan_info(const pa_cache_desc* desc, int32_t num_q_heads, int32_t num_seqs,
                              const int32_t* h_seq_lens, const int32_t* h_q_lens,
                              const pa_attend_opts* opts, pa_attend_info* info);

/*
 * pa_attend - scaled dot-product attention of a packed batch over paged K/V,
 * walking each sequence's block table ([pytorch] "Compute reference attention
 * without hiding the layout" for what is computed; "Map the PyTorch design to
 * vLLM PagedAttention": fused kernels read the block table directly, so no
 * contiguous copy is made; [engine] "02 The engine": kernel parameters
 * block_table, q_len_per_seq, kv_len_per_seq, block_size, and one packed
 * batch of prefill and decode rows).
 *
 *   q             [total_q][num_q_heads][head_dim], sequence-major (fp16;
 *                 bf16 for PA_KV_BF16 pools):
 *                 sequence i's q_lens[i] rows follow sequence i-1's.
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entry b of row i is
 *                 the physical block of logical block b of sequence i.
 *   seq_lens      int32 [num_seqs]: keys of sequence i after this step's
 *                 writes (its new tokens included: write, then attend).
 *   q_lens        int32 [num_seqs]: query rows of sequence i (0 allowed).
 *   h_seq_lens, h_q_lens  host copies of the same values; the launch shape is
 *                 chosen from them, so they must equal the device arrays.
 *   scale         multiplier of q.k (normally head_dim ** -0.5); must be
 *                 positive and finite (PA_ERR_SHAPE otherwise).
 *   out           [total_q][num_q_heads][head_dim], the type of q.
 *   workspace     device scratch of at least pa_attend_workspace_bytes.
 *
 * Query row t (0-based) of sequence i sits at position
 * seq_lens[i] - q_lens[i] + t and attends to keys 0 .. that position (the
 * last opts->window of them with a sliding window)
 * ([engine] "03 Correctness, and the bugs a real model found": the mask uses
 * the query's real position).  Query head h reads KV head h / group
 * ([pytorch] reference attention: each KV head repeated group times along a
 * new axis).  Softmax runs in fp32 with a running max; long key ranges are
 * split into partitions whose (max, sum, output) are merged in log-sum-exp
 * form.  Requires q_lens[i] <= seq_lens[i] and
 * ceil(seq_lens[i] / block_size) <= max_blocks_per_seq.
 */
pa_status pa_attend(const pa_cache_desc* desc, const void* q, int32_t num_q_heads,
                    const void* k_cache, const void* v_cache,
                    const void* k_scale, const void* v_scale,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                    const int32_t* h_seq_lens, const int32_t* h_q_lens,
                    float scale, void* out, void* workspace, size_t workspace_bytes,
                    const pa_attend_opts* opts, hipStream_t stream);

/*
 * pa_write_attend - pa_write_kv followed by pa_attend on the same stream, as
 * one call (the arguments of both; the write's k, v, slot_mapping, num_tokens
 * first).  Results are those of the two calls.  For a decode step ([pytorch]
 * "How to implement paged attention: the minimal data flow": write the new
 * token's K/V, then attend over the sequence including it) the write runs
 * inside the attention kernel: when the pool is fp16 or bf16, every sequence
 * has exactly one query row (h_q_lens all 1), num_tokens == num_seqs and the
 * rows take the decode units (no row tiles, group below 16), the workgroup
 * that walks a row's last key takes that key's K and V rows of its KV head
 * from k and v (not from the pool) and stores them into the slot after its
 * walk, which saves the write kernel's launch.  That form
 * requires token i to be the new token of sequence i: slot_mapping[i] is the
 * slot of position seq_lens[i] - 1 of sequence i (the slot its table
 * names); otherwise results are undefined (no access outside the pools).
 * Any other batch (int8 pools, several query rows, row tiles) runs the two
 * calls.  Debug builds always run the two calls, each with its metadata
 * check.  Errors: those of pa_write_kv and pa_attend; a refused fused call
 * enqueues nothing.
 */
pa_status pa_write_attend(const pa_cache_desc* desc, const void* k, const void* v,
                          const int32_t* slot_mapping, int32_t num_tokens,
                          const void* q, int32_t num_q_heads, void* k_cache, void* v_cache,
                          void* k_scale, void* v_scale, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, const int32_t* q_lens,
                          int32_t num_seqs, const int32_t* h_seq_lens, const int32_t* h_q_lens,
                          float scale, void* out, void* workspace, size_t workspace_bytes,
                          const pa_attend_opts* opts, hipStream_t stream);

/*
 * pa_attend_noalloc - pa_attend without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, results and errors are
 * those of pa_attend; the workspace is a fixed device array of
 * PA_ATTEND_SCRATCH_BYTES that the library holds per GPU (created with the
 * library's code object on that device and kept until the process ends; its
 * address is looked up on the first call on each device, with that device
 * current).  The call itself allocates nothing.
 *   - A batch whose pa_attend_workspace_bytes exceeds PA_ATTEND_SCRATCH_BYTES
 *     returns PA_ERR_WORKSPACE, checked on the host before the GPU is used;
 *     except that when the excess comes from the automatic split of long
 *     row tiles (opts NULL or mfma_split_steps 0), the call runs with row
 *     tiles unsplit if that fits (the same results up to the merge's
 *     rounding).
 *   - Every call on one GPU shares that GPU's array.  Calls that may overlap
 *     on the device (other streams, other threads) race on it and give wrong
 *     results; order them on one stream.  opts->reuse_plan = 1 takes the plan
 *     that the previous pa_attend_noalloc call on the device left there.
 *   - The device current at the call must be the one `stream` belongs to.
 * This is the one exception to "the library keeps no global mutable state".
 */
#define PA_ATTEND_SCRATCH_BYTES ((size_t)64 << 20)

pa_status pa_attend_noalloc(const pa_cache_desc* desc, const void* q, int32_t num_q_heads,
                            const void* k_cache, const void* v_cache,
                            const void* k_scale, const void* v_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                            const int32_t* h_seq_lens, const int32_t* h_q_lens,
                            float scale, void* out, const pa_attend_opts* opts,
                            hipStream_t stream);

/*
 * pa_copy_blocks - copy whole blocks (every layer, every KV head, every slot,
 * and the scales of int8 pools) from src to dst, for copy-on-write of a shared block
 * before its first divergent write ([pytorch] "Map the PyTorch design to vLLM
 * PagedAttention": shared blocks are copied only on the first divergent write;
 * [manager] "Architecture Overview": the diverging block is duplicated).
 *
 *   src_dst  int32 [num_pairs][2] = (src, dst) pairs.  No dst may also be a
 *            src or another pair's dst in the same call.
 */
pa_status pa_copy_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                         void* k_scale, void* v_scale, const int32_t* src_dst,
                         int32_t num_pairs, hipStream_t stream);

/*
 * Metadata checks.  The kernels take slots, block ids and lengths on trust
 * (out-of-range values give wrong numbers, never an access outside the
 * pools).  These calls check them on the device, on `stream`, and record a
 * violation in `status`, a caller-owned device buffer of
 * PA_CHECK_STATUS_WORDS int32:
 *   status[0]  0 when every check passed, else a pa_check_code
 *   status[1]  the offending index (token, sequence or pair; -1 when the
 *              violation is a disagreement of sums)
 *   status[2]  the offending value,  status[3]  the bound or the other index
 * When several checks fail, one of the violations is recorded.  The buffer
 * is cleared by the call itself (a fill kernel, no memset), so the calls can
 * sit in a captured graph; read it after the stream has reached it.
 *
 * A library built with PA_DEBUG=1 (libpa_debug.so: `python -m
 * paged_kv_cache_47_amd.build --debug`) runs the matching check before every
 * pa_write_kv, pa_attend and pa_copy_blocks, waits for it, and returns
 * PA_ERR_METADATA without enqueueing the call's work when it fails; those
 * calls then synchronise the stream.
 */
#define PA_CHECK_STATUS_WORDS 8
typedef enum {
  PA_CHECK_OK = 0,
  PA_CHECK_SLOT_RANGE = 1,      /* slot >= num_blocks * block_size           */
  PA_CHECK_SLOT_DUPLICATE = 2,  /* two tokens of one call share a slot       */
  PA_CHECK_SLOT_RUN = 3,        /* int8: a block's tokens are not consecutive
                                   in t with consecutive offsets             */
  PA_CHECK_LENGTHS = 4,         /* not 0 <= q_len <= seq_len <= table width  */
  PA_CHECK_HOST_LENGTHS = 5,    /* device lengths differ from the host copies */
  PA_CHECK_BLOCK_ID = 6,        /* a table entry a query reads is outside
                                   [0, num_blocks)                           */
  PA_CHECK_COPY_PAIR = 7        /* a copy id out of range, or a destination
                                   that is another pair's source or destination */
} pa_check_code;

/* The preconditions of pa_write_kv: every non-negative slot below
 * num_blocks * block_size, all distinct, and for int8 pools each block's
 * tokens consecutive in t with consecutive offsets ([engine] "INT8 KV cache
 * design": the replay appends tokens in order). */
pa_status pa_check_write(const pa_cache_desc* desc, const int32_t* slot_mapping, int32_t num_tokens,
                         int32_t* status, hipStream_t stream);

/* The preconditions of pa_attend with the same arguments: per sequence
 * 0 <= q_len <= seq_len <= max_blocks_per_seq * block_size, the device
 * lengths equal to the host copies (compared through their plain and
 * position-weighted sums), and every table entry a query of the step reads
 * (from the block holding the earliest key any of its queries sees, with
 * opts->window, to its last key) in [0, num_blocks) ([pytorch] "Trace a
 * block-table lookup during one decode step"). */
pa_status pa_check_attend(const pa_cache_desc* desc, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* q_lens, int32_t num_seqs,
                          const int32_t* h_seq_lens, const int32_t* h_q_lens, const pa_attend_opts* opts,
                          int32_t* status, hipStream_t stream);

/* The preconditions of pa_copy_blocks: ids in [0, num_blocks), and no
 * destination that is another pair's source or destination. */
pa_status pa_check_copy(const pa_cache_desc* desc, const int32_t* src_dst, int32_t num_pairs,
                        int32_t* status, hipStream_t stream);

/* Static description of a status code. */
const char* pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
