// pa_internal.h -- argument blocks and launchers shared by the HIP sources of
// libpa.so.  Not installed; the public interface is include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Resolved geometry of one pool, computed on the host from pa_kv_pool.
struct PoolGeom {
  char* k;
  char* v;
  int64_t num_blocks;
  int64_t block_stride;  // bytes between consecutive blocks
  int32_t row_stride;    // bytes between consecutive slots of a block (Hkv*D*e)
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t elem_bytes;    // 2: binary16, 1: fp8
  int32_t fp8_e5m2;      // 1-byte elements: 0 e4m3fn, 1 e5m2
  float k_scale;
  float v_scale;
  uint32_t flags;        // pa_kv_pool.flags
  const float* k_hs;     // per-KV-head fp8 scales (device) or null
  const float* v_hs;
  int32_t window;        // sliding window in positions, 0: none
  float* k_bs;           // per-(block, KV head) fp8 scales (device) or null
  float* v_bs;
};

struct DecodeArgs {
  const char* k;
  const char* v;
  int64_t block_stride;
  int32_t row_stride;
  int32_t num_kv_heads;
  int32_t num_blocks_m1;      // largest valid physical id
  int32_t num_q_heads;
  int32_t gqa;                // query heads per KV head
  const _Float16* q;
  _Float16* out;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t len_cap;            // min(max_seq_len, max_blocks * block_size)
  const int32_t* seq_lens;
  float score_scale;          // scale * log2(e) * k_scale: scores in log2 units
  float v_scale;
  const float* k_hs;          // per-KV-head scales (device) or null: score_scale
  const float* v_hs;          //   and v_scale then take the head's factor
  int32_t window;             // sliding window: the query sees the last `window`
                              //   positions of its context (0: all)
  const float* k_bs;          // per-(block, KV head) scales [num_blocks][Hkv] (kv
  const float* v_bs;          //   formats 3 and 4) or null
  int32_t part_tokens;        // split pass: tokens per partition
  int32_t num_parts;          // split pass: partitions per (sequence, KV head)
  float* ws_o;                // split pass: [S][Hq][num_parts][D] normalised partials
  float2* ws_ml;              // split pass: [S][Hq][num_parts] (max in log2 units, sum)
};

// Flat schedule: the list of all (sequence, 16-token tile) units is cut into
// num_ranges equal ranges; range r is walked by waves r*Hkv .. r*Hkv+Hkv-1.
struct FlatArgs {
  int32_t num_seqs;
  int32_t num_ranges;
  int32_t* prefix;            // [S + 1] tiles before each sequence (written by the kernel)
  float* slots;               // [num_ranges * Hkv][2][gqa][head_dim + 2] partial records
};

// Grouped schedules: group i is the sequences members[member_start[i] ..
// member_start[i + 1]); the member at position p shares its first
// member_shared[p] positions (whole 16-token tiles) with the member before it
// in its group (device arrays).
struct GroupArgs {
  int32_t num_groups;
  int32_t num_seqs;
  int32_t num_members;          // length of members and member_shared
  const int32_t* members;
  const int32_t* member_start;  // [num_groups + 1]
  const int32_t* member_shared; // [num_members]
};

enum { kModeSingle = 0, kModeSplit = 1, kModeFlat = 2, kModeGroup = 3, kModeFlatGroup = 4 };

hipError_t launch_reshape_and_cache(const PoolGeom& g, const _Float16* k_new,
                                    const _Float16* v_new, const int64_t* slots, int64_t T,
                                    hipStream_t stream);
hipError_t launch_copy_blocks(const PoolGeom& g, const int64_t* pairs, int64_t n,
                              hipStream_t stream);
// stream_kv: read K/V tiles with the streaming cache policy (pools without
// blocks shared between sequences of the batch).
// kv: 0 binary16, 1 e4m3fn, 2 e5m2, 3 e4m3fn and 4 e5m2 with per-block scales.
hipError_t launch_decode(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                         int32_t num_seqs, int32_t head_dim, int32_t block_size, int kv,
                         bool stream_kv, int mode, hipStream_t stream);
// The decode launchers of one (head_dim, kv) pair (pa_decode.hip).
template <int D, int KV>
hipError_t launch_decode_dk(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                            int32_t num_seqs, int32_t block_size, bool stream_kv, int mode,
                            hipStream_t stream);

// Prefill over the paged cache: sequence s owns q rows [q_start[s], q_start[s+1]);
// its new tokens are the last q_len of its seq_lens[s] positions.
struct PrefillArgs {
  const char* k;
  const char* v;
  int64_t block_stride;
  int32_t row_stride;
  int32_t num_blocks_m1;      // largest valid physical id
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t gqa;
  const _Float16* q;          // [total_q, Hq, D]
  _Float16* out;              // [total_q, Hq, D]
  const int32_t* q_start;     // [num_seqs + 1]
  const int32_t* seq_lens;    // [num_seqs]
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t groups;             // 16-row query groups per wave (prefill_plan)
  int32_t tile_tokens;        // new tokens per workgroup: rows per workgroup / gqa
  int32_t num_qt;             // workgroups per (sequence, KV head): cdiv(max_q_len, tile)
  float score_scale;          // scale * log2(e) * k_scale
  float v_scale;
  const float* k_hs;          // per-KV-head scales (device) or null
  const float* v_hs;
  int32_t window;             // sliding window (0: none): position p sees p - window + 1 .. p
  const float* k_bs;          // per-(block, KV head) scales [num_blocks][Hkv] (kv codes 3, 4)
  const float* v_bs;          //   or null
};

// Sets the calling thread's pa_last_error() message and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Validates a pool descriptor and resolves its geometry (PA_OK or a status).
int check_pool(const pa_kv_pool* p, PoolGeom* g);

// The prefill launch shape for this head_dim, pool code (0 binary16, 1-4 fp8
// formats with or without block scales), query heads per KV head, number of
// (sequence, KV head) pairs and largest new-token count: 16-row query groups
// per wave, and new tokens per workgroup (its query rows / gqa).  force: 2 or
// 3 fixes the groups at head_dim 128; 0 lets the plan choose.
struct PrefillPlan {
  int groups;
  int tile_tokens;
};
PrefillPlan prefill_plan(int head_dim, int kv_code, int gqa, int64_t pairs, int max_q_len,
                         int force);

// kv: 0 binary16, 1 e4m3fn, 2 e5m2.
hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, int32_t block_size, int kv,
                          hipStream_t stream);

}  // namespace pa
