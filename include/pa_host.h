/*
 * pa_host.h - host-side block bookkeeping of libpa.so: the block allocator,
 * per-sequence block tables, reference counts, fork / copy-on-write, the
 * sliding-window release, and the per-step metadata arrays that pa_write_kv,
 * pa_copy_blocks and pa_attend consume (pa.h).  Pure integer work on the CPU;
 * no call here touches a GPU.
 *
 * The pages this follows (cited by title and section):
 *   [nanoserve] "Day 14: the block allocator, paging for attention starts as
 *               pure bookkeeping", "What I learned": a block id is either on
 *               a LIFO free stack or allocated; freeing an id that is not
 *               allocated is an error; a multi-block reserve takes all of its
 *               blocks or none.
 *   [pytorch]   "How to Implement Paged Attention in PyTorch and vLLM",
 *               "Allocate, append, and free KV-cache blocks": first pops give
 *               0, 1, 2, ...; a sequence takes a new block when
 *               pos % block_size == 0; position pos lives in block
 *               table[pos / block_size] at offset pos % block_size, so its
 *               slot is table[pos / block_size] * block_size + pos % block_size.
 *               "Map the PyTorch design to vLLM PagedAttention": a shared block
 *               is copied on its first divergent write (copy-on-write).
 *               "PagedAttention vs sliding-window attention, RadixAttention,
 *               and SSMs": with a window of w tokens, blocks that hold only
 *               positions no query can see any more may be freed.
 *   [manager]   "Build a paged KV cache manager from scratch", steps 2-3:
 *               retain / release reference counts; fork shares every block.
 *   [engine]    "Building a paged inference engine from scratch, and
 *               measuring it honestly", "02 The engine": can-allocate checks
 *               for admission.
 *
 * Conventions
 * -----------
 * - Every pointer is HOST memory owned by the caller.  Arrays are int32.
 * - A manager is not thread-safe: calls on one manager must not overlap.
 *   Different managers are independent.
 * - Every call returns a pa_host_status; on any error nothing changed (calls
 *   are atomic), except pa_mgr_free_all, which stops at the first bad id.
 * - A block whose reference count drops to zero goes back on the free stack
 *   at once, unless it is published in the prefix cache (below).
 */
#ifndef PA_HOST_H
#define PA_HOST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_HOST_OK = 0,
  PA_HOST_ERR_ARG = -1,          /* invalid argument (size, id, duplicate, NULL)         */
  PA_HOST_ERR_EXHAUSTED = -2,    /* the pool cannot supply the blocks ([nanoserve])      */
  PA_HOST_ERR_NOT_ALLOCATED = -3,/* retain / release / free of a block that is not held  */
  PA_HOST_ERR_SHARED = -4,       /* free of a block with more than one reference         */
  PA_HOST_ERR_CAPACITY = -5,     /* an output array is too small (see each call)         */
  PA_HOST_ERR_RELEASED = -6      /* positions in blocks the sliding window released      */
} pa_host_status;

typedef struct pa_mgr pa_mgr;

/* Human-readable text of a status (static storage). */
const char* pa_host_status_str(int32_t status);

/*
 * pa_mgr_create - a pool of num_blocks block ids of block_size tokens.
 *   first_pops  NULL (pops give 0, 1, 2, ...) or a permutation of
 *               0 .. num_blocks-1: successive pops return its entries in order.
 *   window      0 = full causal attention; w > 0 = sliding window of w tokens:
 *               pa_mgr_step releases blocks that leave every window.
 * Returns NULL for invalid arguments (num_blocks or block_size <= 0, a
 * first_pops that is not a permutation, window < 0) or when out of memory.
 */
pa_mgr* pa_mgr_create(int32_t num_blocks, int32_t block_size, const int32_t* first_pops, int32_t window);
void pa_mgr_destroy(pa_mgr* m);

/* ---- allocator ---------------------------------------------------------- */
int32_t pa_mgr_num_blocks(const pa_mgr* m);
int32_t pa_mgr_block_size(const pa_mgr* m);
int32_t pa_mgr_num_free(const pa_mgr* m);
/* Pop n blocks (all or none) into out[n]; each starts with one reference. */
int32_t pa_mgr_allocate(pa_mgr* m, int32_t n, int32_t* out);
/* Reference count of block b (0 when free; -1 when b is out of range). */
int32_t pa_mgr_refcount(const pa_mgr* m, int32_t b);
int32_t pa_mgr_retain(pa_mgr* m, int32_t b);
/* Drop one reference; *freed (may be NULL) = 1 when b went back on the stack. */
int32_t pa_mgr_release(pa_mgr* m, int32_t b, int32_t* freed);
/* Return a block held by exactly one owner (PA_HOST_ERR_SHARED otherwise). */
int32_t pa_mgr_free(pa_mgr* m, int32_t b);
/* pa_mgr_free of ids[0..n-1] in order; stops at the first error. */
int32_t pa_mgr_free_all(pa_mgr* m, const int32_t* ids, int32_t n);
/* The free stack, bottom first (out[cap]); returns the count or
 * PA_HOST_ERR_CAPACITY when cap is smaller. */
int32_t pa_mgr_free_ids(const pa_mgr* m, int32_t* out, int32_t cap);
/* Reference counts of all blocks (out[cap], cap >= num_blocks); returns
 * num_blocks or PA_HOST_ERR_CAPACITY. */
int32_t pa_mgr_refcounts(const pa_mgr* m, int32_t* out, int32_t cap);

/* ---- sequences ---------------------------------------------------------- */
/*
 * pa_mgr_add_sequence - a new sequence holding num_tokens cached tokens; its
 * id goes to *sid (ids count up from 0).  With shared_from >= 0, its first
 * shared_tokens tokens (a whole number of blocks, at most that sequence's
 * length and at most num_tokens) reuse that sequence's blocks (one more
 * reference each) and only the rest is allocated.
 */
int32_t pa_mgr_add_sequence(pa_mgr* m, int32_t num_tokens, int32_t shared_from, int32_t shared_tokens,
                            int32_t* sid);
/* A new sequence sharing every block of sid (one more reference each). */
int32_t pa_mgr_fork(pa_mgr* m, int32_t sid, int32_t* child);
/* Release every block of sid; a second finish is harmless. */
int32_t pa_mgr_finish(pa_mgr* m, int32_t sid);
int32_t pa_mgr_num_seqs(const pa_mgr* m);
/* Length of sid in tokens (-1 for an unknown id). */
int32_t pa_mgr_seq_len(const pa_mgr* m, int32_t sid);
/* The block table of sid (released entries are -1) into out[cap]; returns
 * the number of entries or an error (PA_HOST_ERR_CAPACITY when cap is smaller). */
int32_t pa_mgr_seq_blocks(const pa_mgr* m, int32_t sid, int32_t* out, int32_t cap);
/* Slots of the existing positions start .. start+n-1 of sid into out[n]. */
int32_t pa_mgr_slots(const pa_mgr* m, int32_t sid, int32_t start, int32_t n, int32_t* out);

/* ---- prefix cache --------------------------------------------------------- */
/*
 * [manager] "Architecture Overview" and "Step 4: The Prefix Tree (Radix
 * Trie)": a tree
 * whose edges are the token ids of one full block maps prompt prefixes to the
 * blocks that hold them, so a request whose prompt starts with a known prefix
 * reuses those blocks; "Step 2: The Block Pool": blocks whose reference count
 * has dropped to zero are reclaimed least recently used first.  Here a published block whose count
 * drops to zero is cached (neither free nor allocated, still in the tree);
 * allocation takes the free stack first and, when it is empty, evicts the
 * least recently released cached block together with its subtree (cached
 * nodes go back on the stack, children before parents; nodes still in use
 * only leave the tree).  Blocks never published are freed at once as before.
 * Free-capacity checks (allocation, steps) count cached blocks as available.
 */

/*
 * pa_mgr_add_sequence_prefix - a new sequence for a prompt of n tokens that
 * starts with the longest chain of published full blocks matching its
 * tokens (at most (n - 1) / block_size blocks: one prompt token is always
 * left to compute).  The sequence holds those blocks (one more reference
 * each; cached ones are revived) and has *cached_tokens = their tokens as its
 * length; the rest of the prompt is reserved by later steps.
 */
int32_t pa_mgr_add_sequence_prefix(pa_mgr* m, const int32_t* tokens, int32_t n, int32_t* sid,
                                   int32_t* cached_tokens);

/*
 * pa_mgr_publish - enter sid's full blocks that hold tokens[0 .. n-1] (after
 * their K/V have been written, or ordered before any later read) into the
 * tree, root first.  A path that already leads to another block, a block that
 * is already a node elsewhere, or a released block ends the walk.
 */
int32_t pa_mgr_publish(pa_mgr* m, int32_t sid, const int32_t* tokens, int32_t n);

/* Cached blocks (refcount 0, still in the tree). */
int32_t pa_mgr_num_cached(const pa_mgr* m);

/* ---- steps -------------------------------------------------------------- */
/*
 * pa_mgr_append - reserve the next n positions of sid: a new block when a
 * position starts one; a block with more than one reference is first copied
 * into a fresh block (its (src, dst) pair goes to copies, the old block loses
 * a reference).  slots[n] receives the positions' slots; copies[2 * cap_copies]
 * the pairs and *n_copies their count (cap_copies >= n / block_size + 2 always
 * suffices).  No window release.
 */
int32_t pa_mgr_append(pa_mgr* m, int32_t sid, int32_t n, int32_t* slots, int32_t* copies, int32_t cap_copies,
                      int32_t* n_copies);

/* Release the blocks of sid that hold no position at or after
 * seq_len - q_len - window + 1 (entries become -1); nothing without a window. */
int32_t pa_mgr_release_out_of_window(pa_mgr* m, int32_t sid, int32_t q_len);

/* Block-table width a step of these sequences needs (the largest table after
 * it, at least 1); the state is not changed.  Returns the width or an error. */
int32_t pa_mgr_step_width(const pa_mgr* m, const int32_t* sids, const int32_t* q_lens, int32_t num_seqs);

/*
 * pa_mgr_step - one step: for each listed sequence in order (ids distinct),
 * pa_mgr_append of q_lens[i] positions, then (with a window) its release.
 * Outputs, the metadata of pa_copy_blocks / pa_write_kv / pa_attend:
 *   slot_mapping  [sum q_lens]
 *   copies        [2 * cap_copies] (src, dst) pairs, *n_copies of them, to run
 *                 before the step's writes
 *   block_tables  [num_seqs][width] (NULL: not written); entries past a table
 *                 are 0, released entries -1; width must be at least
 *                 pa_mgr_step_width (PA_HOST_ERR_CAPACITY otherwise)
 *   seq_lens      [num_seqs] lengths after the step (NULL: not written)
 * Either every sequence's positions are reserved or nothing changes
 * (PA_HOST_ERR_EXHAUSTED when the pool cannot supply the step, counting
 * the blocks its own window releases free before they are needed).
 */
int32_t pa_mgr_step(pa_mgr* m, const int32_t* sids, const int32_t* q_lens, int32_t num_seqs, int32_t width,
                    int32_t* slot_mapping, int32_t* copies, int32_t cap_copies, int32_t* n_copies,
                    int32_t* block_tables, int32_t* seq_lens);

/* [num_seqs][width] tables of the listed sequences (0 past a table). */
int32_t pa_mgr_block_tables(const pa_mgr* m, const int32_t* sids, int32_t num_seqs, int32_t width,
                            int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_HOST_H */
