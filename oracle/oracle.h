/*
 * oracle.h -- plain CPU reference for paged-attention decode, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load liboracle.so.  It is written from the definitions on the pages, not
 * from the GPU code, and shares no header, helper or table with it.
 *
 * What it computes (the pages' definition, written out):
 *   - A layer's K pool and V pool are each [num_blocks, block_size,
 *     num_kv_heads, head_dim] ("KV Cache memory core", section 2.2 sketch).
 *   - A sequence's logical block j lives in physical block block_table[j]
 *     ("vLLM intro part 2", section 3.2); token t sits at offset t % block_size
 *     of logical block t / block_size.
 *   - Decode: for each block of the table, score the query against the block's
 *     keys, then softmax over all scores and weight the values ("KV Cache memory
 *     core", section 3, read path; the scores are scale * dot(q, k) and the
 *     softmax subtracts the max, "vLLM intro part 2", section 4.2).  The oracle
 *     gathers K/V to contiguous fp64 rows and evaluates that formula directly.
 *   - Query head h reads KV head h / (Hq / Hkv): consecutive query heads share a
 *     KV head ("KV Cache memory core", section 4.2 GQA diagram).
 *   - Writing a token stores its K/V at its absolute slot, block*bs + offset
 *     ("vLLM intro part 2", section 3.2 slot_mapping); fp8 pools store
 *     e4m3fn(x / scale) or e5m2(x / scale) (quantise on write, "KV Cache memory
 *     core", section 4.4; the two fp8 formats of "vLLM intro part 2", section 7).
 *     The scale is one per tensor, one per KV head, or one per (block, KV
 *     head) kept beside the block (the finer granularities the quantisation
 *     passage of "KV Cache memory core", section 4.4, names).
 *   - copy_blocks copies a whole block for copy-on-write ("GPU memory & KV
 *     cache", COW incident code; "vLLM intro part 2", section 5).
 *   - A sliding-window layer lets a query see only the last sliding_window
 *     positions; blocks wholly outside the window are released ("Paging saves
 *     no KV bytes", section 5, sliding-window block release).
 *   - Prefill writes a prompt's K/V in bulk and then attends over the paged
 *     context ("vLLM intro part 2", section 3, KV lifecycle: prefill writes
 *     blocks in bulk, decode appends one slot); with a prefix-cache hit only the
 *     uncached tail is computed (same page, section 6 worked example).  Each new
 *     token attends to itself and every earlier position: the oracle runs the
 *     decode formula once per query position over that position's prefix.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  void*   k;              /* host K pool                                      */
  void*   v;              /* host V pool                                      */
  int64_t num_blocks;
  int64_t block_stride;   /* bytes from one block to the next; 0 = dense      */
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t elem_bytes;     /* 2: IEEE binary16 elements, 1: fp8 bytes          */
  int32_t fp8_format;     /* for 1-byte elements: ORC_FP8_E4M3FN or _E5M2     */
  double  k_scale;        /* fp8 dequantisation scales (1.0 for binary16)     */
  double  v_scale;
  /* Optional finer grain: one scale per KV head ([num_kv_heads] each); when
   * non-NULL they replace k_scale / v_scale for fp8 pools.                    */
  const double* k_head_scales;
  const double* v_head_scales;
  /* Sliding-window attention: > 0 limits a query at position p to positions
   * p - sliding_window + 1 .. p (0: every earlier position).                  */
  int32_t sliding_window;
  /* Optional per-block grain (fp8 pools): [num_blocks][num_kv_heads] float32
   * scales for K and for V, kept beside the pools; orc_scatter updates them
   * and orc_copy_blocks copies them (see orc_scatter).  When non-NULL they
   * replace the per-tensor and per-head scales.                               */
  float*  k_block_scales;
  float*  v_block_scales;
} orc_pool;

#define ORC_FP8_E4M3FN 0
#define ORC_FP8_E5M2 1

/* Value of an IEEE-754 binary16 bit pattern. */
double orc_f16_value(uint16_t bits);
/* Value of an OCP e4m3fn byte (bias 7, no infinities, S.1111.111 = NaN). */
double orc_e4m3fn_value(uint8_t byte);
/* fp32 -> e4m3fn, round to nearest even, saturating to +-448, NaN -> NaN. */
uint8_t orc_e4m3fn_encode(float x);
/* Value of an OCP e5m2 byte (bias 15, infinities and NaN in exponent 31). */
double orc_e5m2_value(uint8_t byte);
/* fp32 -> e5m2, round to nearest even, saturating to +-57344, NaN -> NaN. */
uint8_t orc_e5m2_encode(float x);
/* Batch forms of the codec functions (n elements). */
void orc_f16_values(const uint16_t* bits, int64_t n, double* out);
void orc_e4m3fn_values(const uint8_t* bytes, int64_t n, double* out);
void orc_e4m3fn_encode_n(const float* x, int64_t n, uint8_t* out);
void orc_e5m2_values(const uint8_t* bytes, int64_t n, double* out);
void orc_e5m2_encode_n(const float* x, int64_t n, uint8_t* out);

/* Write T tokens: k_new/v_new are [T, Hkv, D] binary16 bit patterns; a slot
 * below 0 (padding) or at or beyond num_blocks * block_size skips the token.  fp8 pools receive enc(float(x) / float(scale)) with the
 * pool's fp8 encoder.
 * Per-block scales (quantise on write, with the scale kept beside the block,
 * "KV Cache memory core", section 4.4): the tokens are taken in runs, a run
 * being the consecutive entries of slots that lie in one block.  For each KV
 * head, and for K and V separately, with a = the largest finite |x| of the
 * run and m = the format's largest finite value (448, 57344), in fp32:
 *   c   = max(a / m, smallest normal fp32)
 *   new = c if the run writes the block's slot 0, else max(old, c)
 * If the run does not write slot 0 and new > old, every slot of the block the
 * run does not write is re-encoded: byte -> enc((value(byte) * old) / new).
 * The run's values are stored as enc(x / new) and new becomes the block's
 * scale.  Runs are taken in order, one after another. */
void orc_scatter(const orc_pool* p, const uint16_t* k_new, const uint16_t* v_new,
                 const int64_t* slots, int64_t T, int nthreads);

/* Copy whole blocks: pairs is [n, 2] of (src, dst), applied in order; a pair
 * naming a block outside [0, num_blocks) is skipped.  Per-block scales are
 * copied with their block. */
void orc_copy_blocks(const orc_pool* p, const int64_t* pairs, int64_t n);

/* Gather KV head kh of a sequence into contiguous fp64 rows Kc/Vc [len, D]. */
void orc_gather_head(const orc_pool* p, const int32_t* bt_row, int32_t len, int32_t kh,
                     double* Kc, double* Vc);

/* softmax(scale * q.K^T) V over len contiguous rows; len == 0 gives zeros. */
void orc_attend(const double* q, const double* Kc, const double* Vc, int32_t len,
                int32_t D, double scale, double* out);

/* Decode S sequences: q is [S, Hq, D] binary16 bits, block_tables [S, max_blocks],
 * seq_lens [S].  units lists (s, kh) pairs to evaluate (NULL = all S*Hkv); out is
 * [S, Hq, D] fp64 and only the selected rows are written. */
void orc_decode(const orc_pool* p, const uint16_t* q, int32_t S, int32_t Hq,
                const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                float scale, const int32_t* units, int64_t n_units, double* out, int nthreads);

/* Same result by another route: split each context into partitions of
 * partition_size tokens, keep (max, sum of exp, normalised output) per partition
 * and merge them by log-sum-exp. */
void orc_decode_split(const orc_pool* p, const uint16_t* q, int32_t S, int32_t Hq,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                      float scale, int32_t partition_size, const int32_t* units,
                      int64_t n_units, double* out, int nthreads);

/* Prefill (a prompt, or the uncached chunk of one): q is [total_q, Hq, D]
 * binary16 bits; sequence s owns q rows [q_start[s], q_start[s+1]).  Its
 * q_len = q_start[s+1] - q_start[s] new tokens are the last q_len of its
 * seq_lens[s] context positions (their K/V already written), so q row i of s
 * sits at position c = seq_lens[s] - q_len + i and attends to positions 0..c
 * (causal).  rows lists (s, kh, i) triples to evaluate, each for the gqa query
 * heads of KV head kh (NULL = every row of every sequence); out is
 * [total_q, Hq, D] fp64 and only the selected rows are written. */
void orc_prefill(const orc_pool* p, const uint16_t* q, const int32_t* q_start, int32_t S,
                 int32_t Hq, const int32_t* block_tables, int32_t max_blocks,
                 const int32_t* seq_lens, float scale, const int32_t* rows, int64_t n_rows,
                 double* out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
