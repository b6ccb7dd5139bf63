/*
 * pa_blocks.h -- host block pool with prefix caching, part of libpa.so.
 *
 * The pool hands out physical block ids for the device pools of pa.h and keeps
 * the bookkeeping the pages describe: reference counts, one LRU free queue
 * that also holds the cached blocks, chained block hashes and the hash index
 * used for prefix hits ("KV Cache memory core", sections 2.3 and 4.1;
 * "vLLM intro part 2", sections 5 and 6; "GPU memory & KV cache",
 * copy-on-write steps).
 *
 *   * Blocks with count 0 form one doubly linked free queue.  Allocation takes
 *     from the head; a block that still carries a hash loses it then (the
 *     eviction).  A block whose count returns to 0 goes to the tail if it
 *     carries a hash, to the head otherwise.
 *   * A full block's hash is SHA-256(parent hash | its token ids as
 *     little-endian int32 | extra-key bytes), the first block's parent being
 *     32 zero bytes.  Lookups walk the chain and stop at the first miss.
 *     SHA-256 runs on the x86 SHA extensions when the CPU has them (setting
 *     PA_SHA256_PORTABLE=1 in the environment selects the portable code).
 *   * A request's lookup never covers its last token: at most
 *     (num_tokens - 1) / block_size blocks hit.
 *
 * All functions are host functions and touch no device memory.  A pool is
 * not thread-safe: use one pool per scheduling thread, or serialise calls.
 * Functions returning int give PA_OK (0) or a negative pa_status; the message
 * is in pa_bp_last_error() on the calling thread.  A failed call changes
 * nothing.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_pool pa_block_pool;
typedef struct {
  uint8_t bytes[32];
} pa_block_hash;

/* A pool of num_blocks blocks of block_size tokens, all free, queue order
 * 0, 1, ..., num_blocks - 1.  NULL on bad arguments. */
pa_block_pool* pa_bp_create(int32_t num_blocks, int32_t block_size);
void pa_bp_destroy(pa_block_pool* pool);
const char* pa_bp_last_error(void);

/* Free blocks (count 0), cached or not. */
int32_t pa_bp_num_free(const pa_block_pool* pool);
/* Count of one block (or a negative status for a bad id). */
int32_t pa_bp_ref_count(const pa_block_pool* pool, int32_t block);
/* 1 and the hash if the block carries one, 0 if not, negative on a bad id. */
int pa_bp_block_hash(const pa_block_pool* pool, int32_t block, pa_block_hash* out);
/* Free queue from head to tail: writes up to cap ids, returns the length. */
int32_t pa_bp_free_queue(const pa_block_pool* pool, int32_t* out, int32_t cap);

/* Take n blocks from the head of the free queue (evicting hashes they carry);
 * each gets count 1.  PA_ERR_NO_BLOCKS if fewer than n are free. */
int pa_bp_get_new_blocks(pa_block_pool* pool, int32_t n, int32_t* out);
/* Drop one count per listed id, in the order given (callers pass a request's
 * blocks last to first).  Every id must be held at least as often as listed. */
int pa_bp_free_blocks(pa_block_pool* pool, const int32_t* ids, int32_t n);
/* Prefix hit: one more count per listed id; free blocks leave the queue. */
int pa_bp_touch(pa_block_pool* pool, const int32_t* ids, int32_t n);
/* Register a held, full block under its hash (no-op if it already has one). */
int pa_bp_cache_block(pa_block_pool* pool, int32_t block, const pa_block_hash* hash);
/* Blocks cached under the leading run of hashes (no side effects): returns
 * the run length and writes the ids; among equal hashes the first cached. */
int32_t pa_bp_lookup(const pa_block_pool* pool, const pa_block_hash* hashes, int32_t n,
                     int32_t* out);
/* out = SHA-256(parent or 32 zero bytes | tokens as int32 LE | extra). */
void pa_hash_block_tokens(const pa_block_hash* parent, const int32_t* tokens, int32_t n,
                          const void* extra, int32_t extra_len, pa_block_hash* out);
/* The chained hashes of the full blocks of a token sequence ("vLLM intro
 * part 2", section 6.1): out[i] hashes block i with out[i - 1] (32 zero bytes
 * for block 0) as parent.  Writes min(full blocks, cap) hashes and returns the
 * number of full blocks, or a negative status on bad arguments. */
int32_t pa_hash_blocks(const int32_t* tokens, int32_t num_tokens, int32_t block_size,
                       const void* extra, int32_t extra_len, pa_block_hash* out, int32_t cap);

/* Request-level calls.  allocate: hash the full blocks of the prompt, take
 * the cached prefix (touch), allocate the rest; *num_cached_tokens = hits *
 * block_size.  cache: after the K/V are written, register the request's full
 * blocks.  append: grow to num_tokens_after tokens.  free: release last to
 * first.  request_blocks: the block table row (returns its length). */
int pa_bp_allocate_request(pa_block_pool* pool, int64_t request, const int32_t* tokens,
                           int32_t num_tokens, const void* extra, int32_t extra_len,
                           int32_t* num_cached_tokens);
int pa_bp_cache_request(pa_block_pool* pool, int64_t request, const int32_t* tokens,
                        int32_t num_tokens, const void* extra, int32_t extra_len);
int pa_bp_append_slots(pa_block_pool* pool, int64_t request, int32_t num_tokens_after);
int pa_bp_free_request(pa_block_pool* pool, int64_t request);
/* One scheduler step of growth: request requests[i] grows to
 * num_tokens_after[i] tokens, for i < n (each request listed at most once).
 * All or nothing: PA_ERR_NO_BLOCKS when the step needs more blocks than are
 * free, PA_ERR_INVALID_ARG for an unknown or repeated request; either way the
 * pool is unchanged.  Blocks are taken in list order. */
int pa_bp_append_slots_batch(pa_block_pool* pool, const int64_t* requests,
                             const int32_t* num_tokens_after, int32_t n);
int32_t pa_bp_request_blocks(const pa_block_pool* pool, int64_t request, int32_t* out,
                             int32_t cap);

/* Sliding-window layers: once a request holds num_tokens tokens, its next
 * query (position num_tokens) sees positions num_tokens - window + 1 onward;
 * release every block lying wholly before that position ("Paging saves no KV
 * bytes", section 5: out-of-window blocks are released directly).  Released
 * entries of the block table read back as -1 and are skipped when the request
 * is freed.  Returns the number of blocks released. */
int32_t pa_bp_remove_skipped_blocks(pa_block_pool* pool, int64_t request, int32_t num_tokens,
                                    int32_t window);

/* Fork: child shares every block of parent (each count + 1). */
int pa_bp_fork_request(pa_block_pool* pool, int64_t parent, int64_t child);
/* Before writing the token at this position: if its block is shared (count
 * > 1), move the request to a new block (count 1, old block's count - 1) and
 * write the (src, dst) pair for pa_copy_blocks into copy_pair; returns 1.
 * Returns 0 when the block is the request's own. */
int pa_bp_prepare_write(pa_block_pool* pool, int64_t request, int32_t position,
                        int64_t* copy_pair);

#ifdef __cplusplus
}
#endif
#endif /* PA_BLOCKS_H */
