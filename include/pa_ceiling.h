/*
 * pa_ceiling.h - HBM read ceilings of one MI355X, measured by two plain
 * read kernels exported from libpa.so beside the paged-attention calls.
 *
 * The decode kernels of pa.h are bound by HBM reads: every (block, KV head)
 * tile a sequence's table names is read once per step, at a position the
 * table chooses ([pytorch] "Trace a block-table lookup during one decode
 * step": consecutive logical blocks land on unrelated physical blocks).
 * What the memory system delivers for such reads is lower than its
 * published peak.  These calls give the two reference rates a roofline of
 * those kernels can be read against:
 *   - a stream read: one buffer read front to back in 16-byte loads;
 *   - a tile gather: K and V tiles of 4 KiB each (16 tokens x 128 fp16,
 *     one (block, KV head) tile of a d128 pool) read in the order a list of
 *     tile ids gives, each wave reading a run of the list with the next
 *     pairs already in flight, as the decode kernel walks a table.
 * Both only read (one 4-byte store to `sink` that the contents decide, so
 * the loads are kept) and compute nothing of the method.  Time them with
 * events on `stream`.
 *
 * Conventions as in pa.h: device pointers, work enqueued on `stream`,
 * arguments checked on the host before anything is enqueued, pa_status
 * codes.
 */
#ifndef PA_CEILING_H
#define PA_CEILING_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads buf[0, bytes) once with 16-byte nontemporal loads, `workgroups`
 * workgroups of 256 threads in a grid-stride loop (0: 2048).
 *   buf    16-byte aligned, bytes a multiple of 16 (PA_ERR_SHAPE otherwise)
 *   sink   one uint32, written only when the xor of the data read equals a
 *          fixed constant
 * Errors: PA_ERR_NULL (buf or sink NULL), PA_ERR_SHAPE (bytes 0, not a
 * multiple of 16, misaligned buf, workgroups negative or above 65536),
 * PA_ERR_HIP. */
pa_status pa_ceiling_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                                 hipStream_t stream);

/* Reads, for each entry i of tile_ids[0, num_ids), the 4 KiB tile
 * tile_ids[i] of k_tiles and of v_tiles (both [num_tiles][4096 bytes]).
 * Wave w reads entries [w * ids_per_wave, (w + 1) * ids_per_wave), keeping
 * `depth` further pairs in flight (1 or 2) beyond the one it works on.
 *   tile_ids  device int32; an id outside [0, num_tiles) reads tile 0 (no
 *             access outside the pools for any value)
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_tiles < 1, num_tiles * 4096 above
 * 2^40 bytes, num_ids < 1, ids_per_wave < 1, depth not 1 or 2, k_tiles or
 * v_tiles not 16-byte aligned), PA_ERR_HIP. */
pa_status pa_ceiling_gather(const void* k_tiles, const void* v_tiles, int64_t num_tiles, const int32_t* tile_ids,
                            int64_t num_ids, int32_t ids_per_wave, int32_t depth, uint32_t* sink,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_CEILING_H */
