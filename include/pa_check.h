/*
 * pa_check.h -- checks of the device-side arguments of pa.h's compute calls,
 * part of libpa.so.
 *
 * pa_decode, pa_prefill, pa_reshape_and_cache and pa_copy_blocks validate
 * what the host can see (pointers, shapes, alignment) but take the contents
 * of their device arrays on trust: block-table ids, sequence lengths, query
 * starts, slots and (src, dst) pairs.  The kernels stay in bounds whatever
 * those hold (ids are clamped, out-of-range slots and pairs skipped), so a
 * bad entry gives wrong results or a lost write, never a fault.  The calls
 * here find such entries.  They follow the pages' convention that an
 * impossible request is an error the caller is told about ("KV Cache memory
 * core", section 2.3: the pool refuses an allocation it cannot serve and the
 * caller checks capacity first).
 *
 * Each call runs small kernels on the caller's stream, then waits for that
 * stream and returns PA_OK, or PA_ERR_INVALID_ARG with the first problem
 * (ordered by kind, then by index) and the number of problems found in
 * pa_last_error().  Host-side argument errors return as in pa.h and launch
 * nothing.  They are for debugging and tests, not for a serving loop: each
 * call synchronises.
 *
 * scratch: caller-owned device memory of at least pa_check_scratch_bytes(pool)
 * bytes, 8-byte aligned; its contents are overwritten.  Calls that run
 * concurrently need separate scratch buffers.
 */
#ifndef PA_CHECK_H
#define PA_CHECK_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Scratch bytes the checks below need for this pool: a 256-byte report plus
 * one bit per slot of the pool.  0 for an invalid descriptor. */
size_t pa_check_scratch_bytes(const pa_kv_pool* pool);

/* pa_decode's device arguments ("vLLM intro part 2", section 3: the block
 * table maps a sequence's logical blocks to physical ids):
 *   0 <= seq_lens[s] <= max_seq_len;
 *   cdiv(seq_lens[s], block_size) <= max_blocks_per_seq;
 *   block_tables[s][j] in [0, num_blocks) for every block the query reads
 *   (with a sliding window, entries wholly before the window may hold
 *   anything, e.g. -1 for a released block). */
int pa_check_decode_inputs(const pa_kv_pool* pool, int32_t num_seqs,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, void* scratch,
                           size_t scratch_bytes, hipStream_t stream);

/* pa_prefill's device arguments:
 *   0 <= q_start[0] <= q_start[1] <= ... <= q_start[num_seqs] <= total_q;
 *   q_len = q_start[s + 1] - q_start[s] <= max_q_len and <= seq_lens[s];
 *   seq_lens[s] >= 0 and cdiv(seq_lens[s], block_size) <= max_blocks_per_seq;
 *   block_tables[s][j] in [0, num_blocks) for every block a query of sequence
 *   s reads (from the window start of its first new token). */
int pa_check_prefill_inputs(const pa_kv_pool* pool, int32_t total_q, const int32_t* q_start,
                            int32_t num_seqs, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t max_q_len, void* scratch, size_t scratch_bytes,
                            hipStream_t stream);

/* pa_reshape_and_cache's slot_mapping ("vLLM intro part 2", section 3.2):
 * every non-negative slot below num_blocks * block_size and no slot listed
 * twice.  Negative slots (padding) are allowed. */
int pa_check_slot_mapping(const pa_kv_pool* pool, const int64_t* slot_mapping,
                          int64_t num_tokens, void* scratch, size_t scratch_bytes,
                          hipStream_t stream);

/* pa_copy_blocks's block_mapping ("GPU memory & KV cache", copy-on-write):
 * both ids of every pair in [0, num_blocks), no block the destination of two
 * pairs, and no destination also a source. */
int pa_check_block_mapping(const pa_kv_pool* pool, const int64_t* block_mapping,
                           int64_t num_pairs, void* scratch, size_t scratch_bytes,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_CHECK_H */
