/*
 * pa.h -- paged-attention decode for AMD MI355X (gfx950): the C ABI of libpa.so.
 *
 * The operation, as the pages state it:
 *   - One layer's KV cache is a K pool and a V pool, each
 *     [num_blocks, block_size, num_kv_heads, head_dim]; block_size tokens share
 *     a block ("KV Cache memory core", section 2.2 layout sketch; "vLLM intro
 *     part 2", section 3.1: one pool per layer, separate K and V blocks).
 *   - A sequence's logical block j lives in physical block block_table[j]; the
 *     tables of a batch are stacked into a 2-D [num_seqs, max_num_blocks]
 *     array and handed to the kernel together with slot_mapping, the absolute
 *     pool slot (block * block_size + offset) of every new token ("vLLM intro
 *     part 2", section 3.2).
 *   - Decode reads the blocks of block_table[seq] in order and scores the query
 *     against each block's keys, softmax over all scores, then weights the
 *     values ("KV Cache memory core", section 3, read path); scores are
 *     scale * dot(q, k) and the softmax subtracts the running max ("vLLM intro
 *     part 2", section 4.2); partial results of different blocks are merged
 *     with the online-softmax rule ("PagedAttention & vLLM", PagedAttention
 *     kernel steps).
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads): consecutive
 *     query heads share one KV head ("KV Cache memory core", section 4.2).
 *   - Copy-on-write duplicates a whole block before a shared block is written
 *     ("GPU memory & KV cache", copy-on-write steps and incident code).
 *   - fp8 KV is quantised on write and dequantised inside the attention kernel
 *     on read ("KV Cache memory core", section 4.4); the format is OCP e4m3fn
 *     ("Paging saves no KV bytes", section 4) or OCP e5m2 ("vLLM intro part 2",
 *     section 7), with one fp32 scale per pool.
 *
 * Conventions for every entry point:
 *   - All pointers named as device pointers point to device memory the caller
 *     owns.  The library allocates nothing, keeps no per-call state and never
 *     synchronises: work is enqueued on the caller's stream and the call returns.
 *   - Host-checkable arguments are validated before anything is launched; a
 *     failed check returns a negative pa_status and launches nothing.  The
 *     message is available from pa_last_error() on the same thread.
 *   - Device contents are not validated.  Indices that would leave a buffer are
 *     made harmless instead (see each function), so a bad table cannot fault
 *     the GPU, but the affected outputs are then unspecified.
 *   - With PA_LOG set (to anything but "0") in the environment when the
 *     library is first used, pa_reshape_and_cache, pa_copy_blocks, pa_decode,
 *     pa_decode_grouped and pa_prefill print one line each to stderr ("[pa] "
 *     then the entry point, its shapes, the schedule chosen and the launch
 *     size), including calls with nothing to do.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t* hipStream_t; /* same type as HIP's own declaration */
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad size or shape                    */
  PA_ERR_UNSUPPORTED = -2, /* head_dim, block_size, dtype or GQA ratio not built  */
  PA_ERR_ALIGNMENT = -3,   /* a pointer or stride is not 16-byte aligned          */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required          */
  PA_ERR_HIP = -5,         /* the HIP runtime rejected a launch                   */
  PA_ERR_NO_BLOCKS = -6    /* host block pool (pa_blocks.h): not enough free blocks */
} pa_status;

typedef enum {
  PA_KV_F16 = 0,        /* IEEE binary16 elements                                */
  PA_KV_FP8_E4M3FN = 1, /* OCP e4m3fn bytes; value = e4m3(byte) * pool scale      */
  PA_KV_FP8_E5M2 = 2    /* OCP e5m2 bytes; value = e5m2(byte) * pool scale (the
                           pages' second fp8 KV format: wider range, one fewer
                           mantissa bit; "vLLM intro part 2", section 7)        */
} pa_kv_dtype;

/* One layer's KV pool.
 * Element (block b, slot o, KV head h, dim d) of the K pool is at byte
 *   k_base + b * block_stride + ((o * num_kv_heads + h) * head_dim + d) * elem_bytes
 * and likewise in the V pool.  block_stride_bytes = 0 means dense blocks,
 * block_size * num_kv_heads * head_dim * elem_bytes; a larger stride (a
 * multiple of 16) lets K and V blocks interleave in one allocation.
 * Supported: head_dim 64, 128 or 256 (256, the head size of one of the pages'
 * model examples, "Paging saves no KV bytes", section 5); block_size 8, 16,
 * 32, 64 or 128 (the range the pages give the block size, 16 being the
 * default: "vLLM intro part 2", section 3.3); k_base, v_base 16-byte
 * aligned.  k_scale / v_scale are the per-pool fp8 scales (ignored for f16);
 * k_head_scales / v_head_scales optionally give one scale per KV head.
 * flags: PA_POOL_SHARED_BLOCKS when some blocks are read by several sequences
 * of one pa_decode batch (shared prefixes, forked sequences: "PagedAttention
 * & vLLM", memory sharing); decode then keeps K/V reads cacheable so that the
 * other readers of a block find it in cache.  Without it, K/V tiles are read
 * with the streaming (non-temporal) cache policy, the faster choice when every
 * block has one reader.  The flag changes speed only, never results.
 * sliding_window > 0 makes the layer a sliding-window layer: a query at
 * position p attends to positions p - sliding_window + 1 .. p only (0: every
 * earlier position); blocks wholly before a sequence's window are never read,
 * so the host may release them ("Paging saves no KV bytes", section 5). */
#define PA_POOL_SHARED_BLOCKS 1u
typedef struct {
  void* k_base;                /* device */
  void* v_base;                /* device */
  int64_t num_blocks;
  int64_t block_stride_bytes;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;               /* pa_kv_dtype */
  float k_scale;
  float v_scale;
  uint32_t flags;              /* PA_POOL_* bits */
  int32_t sliding_window;      /* 0: full attention */
  /* Optional finer fp8 scale grain: device arrays of num_kv_heads float32
   * scales, one per KV head, for K and for V ("KV Cache memory core",
   * section 4.4 names scale granularity finer than per tensor).  Both NULL
   * (per-tensor k_scale / v_scale) or both set, fp8 pools only, 4-byte
   * aligned; when set, k_scale and v_scale are ignored. */
  const float* k_head_scales;
  const float* v_head_scales;
  /* Optional per-block fp8 scale grain: device arrays of num_blocks *
   * num_kv_heads float32 scales, [block][KV head], for K and for V, kept
   * beside the pools ("KV Cache memory core", section 4.4: scale granularity
   * finer than per tensor; quantised KV stays managed per block with its
   * scale metadata).  The library reads AND writes them:
   * pa_reshape_and_cache sets a block's scales as it writes the block (see
   * there), pa_copy_blocks copies them with the block, and every decode and
   * prefill call dequantises a row with its block's scale.  Both NULL or both
   * set, fp8 pools only, not together with k_head_scales / v_head_scales,
   * num_kv_heads <= 512, 4-byte aligned; when set, k_scale and v_scale are
   * ignored.  A block's scales are defined once its slot 0 has been
   * written. */
  float* k_block_scales;
  float* v_block_scales;
} pa_kv_pool;

/* Write num_tokens new tokens into their slots (the write side of slot_mapping,
 * "vLLM intro part 2", section 3.2).
 *   k_new, v_new  device, [num_tokens, num_kv_heads, head_dim] binary16, contiguous,
 *                 16-byte aligned.
 *   slot_mapping  device, [num_tokens] int64; token i goes to block
 *                 slot / block_size, offset slot % block_size.  A negative slot,
 *                 or one at or beyond num_blocks * block_size, skips the token.
 *                 Slots must be distinct within one call.
 * f16 pools receive the bits unchanged.  fp8 pools receive
 * enc(float(x) / scale), rounded to nearest even and saturated to the
 * format's largest finite value (448 for e4m3fn, 57344 for e5m2; infinities
 * saturate too), NaN stays NaN.  num_tokens == 0 is a no-op.
 * With per-block scales the tokens are taken in runs -- consecutive entries
 * of slot_mapping that lie in one block -- and every block a call writes
 * must be written by one run (a decode step appends one token per block; a
 * prefill writes each block's new positions consecutively); blocks written
 * by two runs of one call are a race.  For each run, KV head, and K and V
 * separately, in fp32, with a = the largest finite |x| of the run and m = the
 * format's largest finite value:
 *   c = max(a / m, smallest normal fp32);
 *   new = c when the run writes the block's slot 0 (a block starts over),
 *   else max(old, c);
 *   if the run does not write slot 0 and new > old, every slot of the block
 *   the run does not write is re-encoded, byte -> enc((value(byte) * old) / new);
 *   the run's values are stored as enc(x / new) and new becomes the scale.
 * Values are never saturated by a scale that is too small. */
int pa_reshape_and_cache(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int64_t num_tokens, hipStream_t stream);

/* Copy whole blocks, K and V, for copy-on-write ("GPU memory & KV cache",
 * copy_blocks(blk, new) in the incident fix).
 *   block_mapping device, [num_pairs, 2] int64 of (src, dst).  Destinations must
 *                 be distinct and must not also be sources in the same call.
 *                 Pairs with an id outside [0, num_blocks) are skipped. */
int pa_copy_blocks(const pa_kv_pool* pool, const int64_t* block_mapping, int64_t num_pairs,
                   hipStream_t stream);

/* The schedule pa_decode will use for these arguments:
 *   0   single pass: one workgroup per (sequence, KV head);
 *   1   flat schedule: the (sequence, 16-token) units of the whole batch are
 *       cut into equal ranges, each walked by one wavefront per KV head, so
 *       long and short contexts cost the same; contexts cut by range
 *       boundaries are merged by a log-sum-exp kernel;
 *   >=16 split pass with that many tokens per partition, followed by a
 *       log-sum-exp reduce kernel.
 * partition_size follows pa_decode.  Returns a negative pa_status on bad
 * arguments. */
int32_t pa_decode_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_seq_len, int32_t partition_size);

/* Bytes of workspace pa_decode needs for these arguments (0 for the single
 * pass).  Returns 0 as well when the arguments are invalid; pa_decode then
 * reports the error. */
size_t pa_decode_workspace_size(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_seq_len, int32_t partition_size);

/* Decode attention for one new query token per sequence.
 *   out           device, [num_seqs, num_q_heads, head_dim] binary16 (written).
 *   q             device, [num_seqs, num_q_heads, head_dim] binary16.
 *   block_tables  device, [num_seqs, max_blocks_per_seq] int32 physical ids; only
 *                 the first cdiv(seq_lens[s], block_size) entries of a row are
 *                 read.  Ids are clamped into [0, num_blocks).
 *   seq_lens      device, [num_seqs] int32 context lengths, including the token
 *                 this step wrote; each must be <= max_seq_len and
 *                 <= max_blocks_per_seq * block_size (larger values are clamped).
 *                 A length of 0 gives an all-zero output row.
 *   max_seq_len   host upper bound of seq_lens; sizes the grid and workspace.
 *   scale         softmax scale applied to q.k (e.g. 1/sqrt(head_dim)).
 *   partition_size  -1 single pass, 0 library choice (the flat schedule for up
 *                 to 8000 sequences), 1 flat schedule, >= 16 split pass with
 *                 that many tokens per partition (a multiple of 16) followed by
 *                 a log-sum-exp reduce of the partitions.
 *   workspace     device scratch of at least pa_decode_workspace_size(...) bytes,
 *                 16-byte aligned; may be NULL when that size is 0.  Calls
 *                 that run concurrently need separate workspaces.
 * num_q_heads must be a multiple of num_kv_heads with a ratio of at most 16.
 * Outputs are bitwise reproducible for the same inputs and do not depend on
 * which physical ids hold the blocks. */
int pa_decode(const pa_kv_pool* pool, void* out, const void* q, int32_t num_seqs,
              int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* seq_lens, int32_t max_seq_len, float scale, int32_t partition_size,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode with shared prefixes read once per group of sequences ("PagedAttention
 * & vLLM", memory sharing: several sequences list the same physical blocks,
 * e.g. parallel samples forked from one prompt, or requests hitting the same
 * cached prefix).  Same arguments, results and output as pa_decode, plus a
 * grouping of the batch:
 *   group i is the sequences members[member_start[i] .. member_start[i+1])
 *   (device int32 arrays, [num_seqs] and [num_groups + 1]); every sequence
 *   must be listed exactly once (a sequence left out gets no output row).  A
 *   group holds at most 16 / (num_q_heads / num_kv_heads) sequences (further
 *   members are ignored).  member_shared[p] (device int32 [num_seqs]) is the
 *   number of leading positions the member at position p of members shares
 *   with the member listed just before it in the same group: both tables
 *   list the same physical blocks for those positions (whole 16-token tiles,
 *   at most both lengths; other values are rounded down and clamped; the
 *   entry of a group's first member is ignored).
 *   The query heads of all members of a group form the columns of one
 *   matrix-core operand; a tile that several consecutive members share is
 *   read once and feeds all of their columns, so every distinct (position
 *   range, physical block) of a group is read once.
 *   schedule: 0 library choice, 1 flat ranges over the groups' tiles (needs
 *   2 num_groups + 4 num_seqs + 2 <= 16384 and a workspace of
 *   pa_decode_grouped_workspace_size bytes; chosen for fewer than 1024
 *   (group, KV head) items), 2 one workgroup per (group, KV head) (no
 *   workspace).
 * pa_decode_group_plan builds such a grouping on the host from host copies
 * of the tables.  Ids in members and member_start are clamped into their
 * arrays; nothing faults on bad contents, but outputs are then unspecified.
 * Pools with a sliding window are refused (PA_ERR_UNSUPPORTED).  Outputs are
 * bitwise reproducible for the same inputs, grouping and schedule, and for a
 * given grouping they do not depend on which physical ids hold the blocks
 * (the planner's member order does: it sorts by table rows). */
int pa_decode_grouped(const pa_kv_pool* pool, void* out, const void* q, int32_t num_seqs,
                      int32_t num_q_heads, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                      float scale, int32_t num_groups, const int32_t* members,
                      const int32_t* member_start, const int32_t* member_shared,
                      int32_t schedule, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* The grouped schedule pa_decode_grouped will use (1 or 2, see above), or a
 * negative pa_status for bad arguments. */
int32_t pa_decode_grouped_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_seq_len, int32_t num_groups, int32_t schedule);

/* Workspace bytes pa_decode_grouped needs (0 for schedule 2, and for bad
 * arguments, which pa_decode_grouped then reports). */
size_t pa_decode_grouped_workspace_size(const pa_kv_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_seq_len,
                                        int32_t num_groups, int32_t schedule);

/* Host planner for pa_decode_grouped.  block_tables [num_seqs,
 * max_blocks_per_seq] and seq_lens [num_seqs] are HOST int32 arrays; members
 * [num_seqs], member_start [num_seqs + 1] and member_shared [num_seqs] are
 * host outputs.  Sequences whose first table entry names the same physical
 * block form a family; a family is sorted by its table rows, so that rows
 * with long common prefixes are neighbours, and cut into groups: runs of at
 * most 16 / (num_q_heads / num_kv_heads) consecutive members each of which
 * shares at least one whole 16-token tile with the one before it.
 * member_shared is that shared length (the common run of leading table
 * entries, within both lengths, in whole tiles; 0 for a group's first
 * member).  Groups are listed longest first.  Returns the number of groups,
 * or a negative pa_status. */
int32_t pa_decode_group_plan(const int32_t* block_tables, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t* members, int32_t* member_start, int32_t* member_shared);

/* pa_decode for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results as pa_decode, but the flat and
 * split schedules use the library's own scratch instead of a workspace
 * argument.  The scratch is one static device array of
 * PA_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until
 * the process ends; its address is looked up on the first call on each
 * device.  Nothing is allocated and nothing is synchronised.
 * Returns PA_ERR_WORKSPACE, launching nothing, when the planned schedule
 * needs more workspace than that (pa_decode_workspace_size tells beforehand;
 * the default flat schedule needs at most about 35 MB).  Every call on a
 * GPU uses that GPU's one array: calls that may overlap on one GPU (on
 * different streams, or from different threads) race on it and must be
 * serialised by the caller, e.g. by issuing them on one stream.  The array
 * keeps whatever the last call left; the kernels read only what the same
 * call wrote, so nothing needs clearing. */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
int pa_decode_noalloc(const pa_kv_pool* pool, void* out, const void* q, int32_t num_seqs,
                      int32_t num_q_heads, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                      float scale, int32_t partition_size, hipStream_t stream);

/* Prefill and chunked-prefill attention over the paged cache.  A prompt's new
 * tokens are written first (pa_reshape_and_cache, on the same stream) and then
 * each attends to itself and every earlier position of its sequence ("vLLM
 * intro part 2", section 3: bulk write on prefill, reads through the block
 * table); with a prefix-cache hit only the uncached tail is new (same page,
 * section 6 example).
 *   out           device, [total_q, num_q_heads, head_dim] binary16 (written).
 *   q             device, [total_q, num_q_heads, head_dim] binary16: the new
 *                 tokens of every sequence, sequence after sequence.
 *   q_start       device, [num_seqs + 1] int32: sequence s owns q rows
 *                 [q_start[s], q_start[s + 1]).  q_len = q_start[s + 1] -
 *                 q_start[s] is clamped to [0, max_q_len] and to seq_lens[s];
 *                 rows outside [0, total_q) are neither read nor written.
 *   block_tables  device, [num_seqs, max_blocks_per_seq] int32, as in pa_decode.
 *   seq_lens      device, [num_seqs] int32 context lengths including the new
 *                 tokens: q row i of sequence s sits at position
 *                 seq_lens[s] - q_len + i and attends to positions 0 .. that
 *                 (causal).  Clamped to max_blocks_per_seq * block_size.
 *   max_q_len     host upper bound of q_len; sizes the grid.
 *   scale         softmax scale applied to q.k; finite and > 0.
 * num_q_heads must be a multiple of num_kv_heads with a ratio of at most 16.
 * No workspace is needed.  total_q, num_seqs or max_q_len of 0 is a no-op.
 * Outputs are bitwise reproducible and do not depend on which physical ids
 * hold the blocks.  At head_dim 128 a workgroup takes 128 or 192 query rows
 * (32 or 48 new tokens at 4 query heads per KV head): 192 when the grid has
 * at least four workgroups per CU and max_q_len pads no worse, else 128; the
 * two differ only in rounding order.  PA_PREFILL_GROUPS=2 (128 rows) or 3
 * (192 rows) in the environment, read at every call, fixes the choice.
 * Non-finite pool data: the K and V rows of a 32-position tile are shared by
 * the query rows of a wave (16 to 48 rows), so an infinite V element at an
 * in-context position that a query does not see (a later position of the
 * same tile) can reach that query as 0 * inf = NaN; positions outside the
 * context or the window never do.  fp8 pools written by pa_reshape_and_cache
 * hold no infinities (the encoders saturate), but binary16 pools receive the
 * bits unchanged, so an infinite element written there does this.  Pools
 * with per-block scales are read at head_dim 128 and 256; at head_dim 64
 * they are refused with PA_ERR_UNSUPPORTED. */
int pa_prefill(const pa_kv_pool* pool, void* out, const void* q, int32_t total_q,
               const int32_t* q_start, int32_t num_seqs, int32_t num_q_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
               int32_t max_q_len, float scale, hipStream_t stream);

/* Query rows ((token, query head) pairs) per workgroup that pa_prefill will
 * use for these arguments: a workgroup takes n new tokens of one sequence and
 * all g = num_q_heads / num_kv_heads query heads of one KV head, n g rows,
 * with n = floor(R / g) for R = 128 at head_dim 64 and 256 and R = 128 or
 * 192 at head_dim 128 (the library's choice described at pa_prefill, or the
 * one PA_PREFILL_GROUPS fixes).  Returns n g, or a negative pa_status on
 * arguments pa_prefill would refuse for the same reason. */
int32_t pa_prefill_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                        int32_t max_q_len);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
