// pa_api.hip -- the extern "C" entry points of libpa.so (declared in include/pa.h).
//
// Host side only: validate what the host can see, resolve the pool geometry,
// choose single pass or split pass, and enqueue the kernels on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

// Dispatch log: with PA_LOG set (and not "0") in the environment, read once,
// every call that launches work prints one line to stderr naming its
// schedule and launch shape.
bool log_on() {
  static const bool on = [] {
    const char* e = std::getenv("PA_LOG");
    return e && e[0] && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void log_line(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void log_line(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[pa] %s\n", buf);
}

// PA_PREFILL_GROUPS=2 or 3 in the environment, read at every pa_prefill call,
// fixes the 16-row query groups per wave of head_dim 128 prefill instead of
// the library's choice (both give the same results up to rounding order).
int prefill_groups_override() {
  const char* e = std::getenv("PA_PREFILL_GROUPS");
  if (!e) return 0;
  if (std::strcmp(e, "2") == 0) return 2;
  if (std::strcmp(e, "3") == 0) return 3;
  return 0;
}

const char* kv_name(int dtype) {
  return dtype == PA_KV_F16 ? "f16" : (dtype == PA_KV_FP8_E4M3FN ? "fp8_e4m3fn" : "fp8_e5m2");
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

namespace pa {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_pool(const pa_kv_pool* p, PoolGeom* g) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool descriptor is NULL");
  if (!p->k_base || !p->v_base) return fail(PA_ERR_INVALID_ARG, "pool k_base/v_base is NULL");
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", p->head_dim);
  if (p->block_size != 8 && p->block_size != 16 && p->block_size != 32 && p->block_size != 64 &&
      p->block_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (8, 16, 32, 64, 128)",
                p->block_size);
  if (p->dtype != PA_KV_F16 && p->dtype != PA_KV_FP8_E4M3FN && p->dtype != PA_KV_FP8_E5M2)
    return fail(PA_ERR_UNSUPPORTED, "kv dtype %d not supported", p->dtype);
  if (p->num_kv_heads < 1 || p->num_kv_heads > 4096)
    return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d out of range", p->num_kv_heads);
  if (p->num_blocks < 1 || p->num_blocks > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)p->num_blocks);
  if (!aligned16(p->k_base) || !aligned16(p->v_base))
    return fail(PA_ERR_ALIGNMENT, "pool bases must be 16-byte aligned");
  const int32_t e = p->dtype == PA_KV_F16 ? 2 : 1;
  const int64_t row = (int64_t)p->num_kv_heads * p->head_dim * e;
  const int64_t dense = row * p->block_size;
  const int64_t stride = p->block_stride_bytes ? p->block_stride_bytes : dense;
  if (stride < dense)
    return fail(PA_ERR_INVALID_ARG, "block_stride_bytes %lld smaller than a block (%lld)",
                (long long)stride, (long long)dense);
  if (stride % 16) return fail(PA_ERR_ALIGNMENT, "block_stride_bytes must be a multiple of 16");
  if (row > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "token row too large");
  if (p->dtype != PA_KV_F16 &&
      (!(p->k_scale > 0.f) || !(p->v_scale > 0.f) || !std::isfinite(p->k_scale) ||
       !std::isfinite(p->v_scale)))
    return fail(PA_ERR_INVALID_ARG, "fp8 pools need finite positive k_scale and v_scale");
  if (p->flags & ~PA_POOL_SHARED_BLOCKS)
    return fail(PA_ERR_INVALID_ARG, "unknown pool flags 0x%x", (unsigned)p->flags);
  if (p->sliding_window < 0)
    return fail(PA_ERR_INVALID_ARG, "sliding_window %d < 0", p->sliding_window);
  if ((p->k_head_scales == nullptr) != (p->v_head_scales == nullptr))
    return fail(PA_ERR_INVALID_ARG, "k_head_scales and v_head_scales must be both set or both NULL");
  if (p->k_head_scales) {
    if (p->dtype == PA_KV_F16)
      return fail(PA_ERR_INVALID_ARG, "per-head scales are for fp8 pools only");
    if (((uintptr_t)p->k_head_scales & 3u) || ((uintptr_t)p->v_head_scales & 3u))
      return fail(PA_ERR_ALIGNMENT, "per-head scale arrays must be 4-byte aligned");
  }
  if ((p->k_block_scales == nullptr) != (p->v_block_scales == nullptr))
    return fail(PA_ERR_INVALID_ARG,
                "k_block_scales and v_block_scales must be both set or both NULL");
  if (p->k_block_scales) {
    if (p->dtype == PA_KV_F16)
      return fail(PA_ERR_INVALID_ARG, "per-block scales are for fp8 pools only");
    if (p->k_head_scales)
      return fail(PA_ERR_INVALID_ARG, "per-block and per-head scales cannot be combined");
    if (p->num_kv_heads > 512)
      return fail(PA_ERR_UNSUPPORTED, "per-block scales support at most 512 KV heads");
    if (((uintptr_t)p->k_block_scales & 3u) || ((uintptr_t)p->v_block_scales & 3u))
      return fail(PA_ERR_ALIGNMENT, "per-block scale arrays must be 4-byte aligned");
  }
  g->k = (char*)p->k_base;
  g->v = (char*)p->v_base;
  g->num_blocks = p->num_blocks;
  g->block_stride = stride;
  g->row_stride = (int32_t)row;
  g->block_size = p->block_size;
  g->num_kv_heads = p->num_kv_heads;
  g->head_dim = p->head_dim;
  g->elem_bytes = e;
  g->fp8_e5m2 = p->dtype == PA_KV_FP8_E5M2;
  g->k_scale = p->dtype == PA_KV_F16 ? 1.f : p->k_scale;
  g->v_scale = p->dtype == PA_KV_F16 ? 1.f : p->v_scale;
  g->flags = p->flags;
  g->window = p->sliding_window;
  g->k_hs = p->k_head_scales;
  g->v_hs = p->v_head_scales;
  g->k_bs = p->k_block_scales;
  g->v_bs = p->v_block_scales;
  if (g->k_hs || g->k_bs) g->k_scale = g->v_scale = 1.f;
  return PA_OK;
}

hipError_t launch_decode(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                         int32_t num_seqs, int32_t head_dim, int32_t block_size, int kv,
                         bool stream_kv, int mode, hipStream_t stream) {
#define PA_DK(D, KV)                                                                        \
  if (head_dim == D && kv == KV)                                                            \
    return launch_decode_dk<D, KV>(a, f, gr, num_seqs, block_size, stream_kv, mode, stream);
  PA_DK(128, 0) PA_DK(128, 1) PA_DK(128, 2) PA_DK(128, 3) PA_DK(128, 4)
  PA_DK(64, 0) PA_DK(64, 1) PA_DK(64, 2) PA_DK(64, 3) PA_DK(64, 4)
  PA_DK(256, 0) PA_DK(256, 1) PA_DK(256, 2) PA_DK(256, 3) PA_DK(256, 4)
#undef PA_DK
  return hipErrorInvalidValue;
}

}  // namespace pa

using pa::check_pool;
using pa::fail;

namespace {

// Planning.  The flat schedule balances any mix of context lengths, so it is
// the default unless the batch is many short contexts; it keeps per-sequence
// prefix and lengths in LDS (2 S + 1 ints).
constexpr int32_t kFlatMaxSeqs = 8000;
// Waves of the flat schedule, measured per size of a 16-token K+V tile (each
// wave keeps about one tile in flight).  4 KiB tiles (fp8 at head_dim 128,
// head_dim 64): 2048 waves, two per SIMD (1536 were 5-8% slower, 1024 10-27%).
// 8 KiB tiles (fp16 at head_dim 128): 768, three per CU (1024 were 3-4%
// slower, 640 8-9%, 704 2-3%, 896 2%; 832 was 2% faster on one shape and
// slower on another).  head_dim 256: 1024, one per SIMD (896 2% slower, 768
// 10%, 1152-1280 30-40%).
int64_t flat_waves(const pa::PoolGeom& g) {
#ifdef PA_FLAT_MAX_WAVES
  (void)g;
  return PA_FLAT_MAX_WAVES;
#else
  const int64_t tile_bytes = 16 * (int64_t)g.head_dim * g.elem_bytes * 2;
  if (g.head_dim > 128) return 1024;
  return tile_bytes <= 4096 ? 2048 : 768;
#endif
}
// The grouped flat schedule's waves: enough that about 8 MiB of tiles are in
// flight, 1024..2048 (for 8 KiB tiles 1024 beat 768 and 832 by 2-3% on 256
// fork groups of 4).
int64_t group_flat_waves(const pa::PoolGeom& g) {
#ifdef PA_FLAT_MAX_WAVES
  (void)g;
  return PA_FLAT_MAX_WAVES;
#else
  const int64_t tile_bytes = 16 * (int64_t)g.head_dim * g.elem_bytes * 2;
  int64_t w = (8 << 20) / tile_bytes;
  return w < 1024 ? 1024 : (w > 2048 ? 2048 : w);
#endif
}
constexpr int64_t kFlatMinTiles = 8;         // keep at least this many tiles per range
constexpr int32_t kPlanFlat = 1;             // pa_decode_plan's code for the flat schedule

// Beyond the flat schedule's limit: the single pass when there are enough
// (sequence, KV head) units to occupy the GPU and contexts are short, else a
// split pass with a few thousand workgroups of at least 256 tokens each.
int32_t choose_partition(int64_t units, int32_t max_seq_len) {
  if (max_seq_len <= 256) return 0;
  if (units >= 2048 && max_seq_len <= 2048) return 0;
  int32_t P = 512;
  while (P > 256 && units * cdiv64(max_seq_len, P) < 2048) P /= 2;
  return P;
}

struct Plan {
  int mode;             // pa::kMode*
  int32_t part;         // split pass: tokens per partition
  int32_t num_parts;
  int64_t waves;        // flat: number of ranges (one wave per KV head each)
};

int plan(const pa_kv_pool* pool, int32_t S, int32_t Hq, int32_t max_seq_len, int32_t req,
         pa::PoolGeom* g, Plan* pl) {
  int st = check_pool(pool, g);
  if (st) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", S);
  if (Hq < 1 || Hq % g->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq,
                g->num_kv_heads);
  if (Hq / g->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d > 16", Hq / g->num_kv_heads);
  if (max_seq_len < 0) return fail(PA_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if (req < -1 || (req > kPlanFlat && req % 16))
    return fail(PA_ERR_INVALID_ARG,
                "partition_size %d invalid (-1, 0, 1 or a multiple of 16)", req);
  const int64_t units = (int64_t)S * g->num_kv_heads;
  const int64_t tiles_ub = units * cdiv64(max_seq_len, 16);
  if (tiles_ub > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "too many 16-token tiles");
  pl->mode = pa::kModeSingle;
  pl->part = 0;
  pl->num_parts = 0;
  pl->waves = 0;
  // Many short contexts: one workgroup per (sequence, KV head) already fills
  // the GPU several times over and no context is long enough to unbalance it,
  // and the single pass has no range bookkeeping.
  const bool many_short = units >= 4096 && max_seq_len <= 1024;
  if (req == kPlanFlat || (req == 0 && !many_short && S <= kFlatMaxSeqs)) {
    if (S > kFlatMaxSeqs)
      return fail(PA_ERR_UNSUPPORTED, "flat schedule supports at most %d sequences", kFlatMaxSeqs);
    // ranges: about flat_waves() waves in all, at least kFlatMinTiles units each
    const int64_t per_head_ub = (int64_t)S * cdiv64(max_seq_len, 16);
    int64_t ranges = flat_waves(*g) / g->num_kv_heads;
    if (ranges > per_head_ub / kFlatMinTiles) ranges = per_head_ub / kFlatMinTiles;
    if (ranges < 1) ranges = 1;
    pl->mode = pa::kModeFlat;
    pl->waves = ranges;           // number of ranges
    return PA_OK;
  }
  int32_t P = req == -1 ? 0 : (req > 0 ? req : choose_partition(units, max_seq_len));
  if (P > 0 && max_seq_len > 0) {
    pl->mode = pa::kModeSplit;
    pl->part = P;
    pl->num_parts = (int32_t)cdiv64(max_seq_len, P);
    if (units * pl->num_parts > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "grid of %lld workgroups too large",
                  (long long)(units * pl->num_parts));
  }
  return PA_OK;
}

int32_t plan_code(const Plan& pl) {
  return pl.mode == pa::kModeFlat ? kPlanFlat : (pl.mode == pa::kModeSplit ? pl.part : 0);
}

// Workspace layouts.  Split: (m, l) pairs [S][Hq][parts] then o [S][Hq][parts][D].
// Flat: prefix [S + 1] int32 then partial records [ranges * Hkv][2][gqa][D + 2].
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t workspace_bytes_for(const Plan& pl, int64_t S, int64_t Hq, int64_t Hkv, int64_t D) {
  if (pl.mode == pa::kModeSplit) {
    const int64_t rows = S * Hq * pl.num_parts;
    return align256((size_t)rows * 8) + (size_t)(rows * D * 4);
  }
  if (pl.mode == pa::kModeFlat)
    return align256((size_t)((S + 1) * 4)) +
           (size_t)(pl.waves * Hkv * 2 * (Hq / Hkv) * (D + 2) * 4);
  return 0;
}

// Grouped schedules: 1 flat ranges over the groups' units (per-group and
// per-member tables in LDS, a workspace for the cut groups' records), 2 one
// workgroup per (group, KV head) (no workspace, any batch size).  Measured on
// the prefix-sharing batch (2,048 items): 124 us per group against 140 us
// flat; on batches of few groups the flat ranges keep every CU busy.
constexpr int32_t kGroupFlat = 1, kGroupPerGroup = 2;
constexpr int64_t kGroupFlatMaxLdsInts = 16384;   // 64 KiB of group and member tables
constexpr int64_t kGroupPerGroupMinItems = 1024;   // items from which one workgroup each pays

struct GroupPlan {
  int32_t mode;
  int64_t ranges;
  size_t workspace;
};

int group_plan(const pa_kv_pool* pool, int32_t S, int32_t Hq, int32_t max_seq_len, int32_t G,
               int32_t schedule, pa::PoolGeom* g, GroupPlan* gp) {
  Plan pl;
  int st = plan(pool, S, Hq, max_seq_len, -1, g, &pl);
  if (st) return st;
  if (g->window > 0)
    return fail(PA_ERR_UNSUPPORTED, "the grouped schedules do not take sliding-window pools");
  if (G < 0 || G > S) return fail(PA_ERR_INVALID_ARG, "num_groups %d out of range [0, %d]", G, S);
  if (schedule < 0 || schedule > kGroupPerGroup)
    return fail(PA_ERR_INVALID_ARG, "grouped schedule %d invalid (0, 1 or 2)", schedule);
  const int64_t lds_ints = 2 * (int64_t)G + 2 + 4 * (int64_t)S;
  const bool flat_fits = lds_ints <= kGroupFlatMaxLdsInts;
  if (schedule == kGroupFlat && !flat_fits)
    return fail(PA_ERR_UNSUPPORTED, "the flat grouped schedule needs 2 groups + 4 sequences + 2 "
                "<= %lld", (long long)kGroupFlatMaxLdsInts);
  if ((int64_t)G * g->num_kv_heads > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "too many groups");
  // enough (group, KV head) items to fill the GPU several times over: one
  // workgroup each; fewer, larger groups: balanced flat ranges
  const bool many_items = (int64_t)G * g->num_kv_heads >= kGroupPerGroupMinItems;
  gp->mode = schedule ? schedule : (flat_fits && !many_items ? kGroupFlat : kGroupPerGroup);
  gp->ranges = 0;
  gp->workspace = 0;
  if (gp->mode == kGroupFlat) {
    const int64_t per_head_ub = (int64_t)S * cdiv64(max_seq_len, 16);
    int64_t ranges = group_flat_waves(*g) / g->num_kv_heads;
    if (ranges > per_head_ub / kFlatMinTiles) ranges = per_head_ub / kFlatMinTiles;
    if (ranges < 1) ranges = 1;
    gp->ranges = ranges;
    gp->workspace = align256((size_t)(G + 1) * 4) +
                    (size_t)(ranges * g->num_kv_heads * 2 * 16 * (g->head_dim + 2) * 4);
  }
  return PA_OK;
}

// Host checks shared by every decode entry point, then the kernel arguments.
int decode_args(const pa::PoolGeom& g, void* out, const void* q, int32_t num_seqs,
                int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* seq_lens, int32_t max_seq_len, float scale, pa::DecodeArgs* ap) {
  if (!out || !q || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG, "out, q, block_tables and seq_lens must be non-NULL");
  if (!aligned16(out) || !aligned16(q))
    return fail(PA_ERR_ALIGNMENT, "q and out must be 16-byte aligned");
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  pa::DecodeArgs& a = *ap;
  a = pa::DecodeArgs{};
  a.k = g.k;
  a.v = g.v;
  a.block_stride = g.block_stride;
  a.row_stride = g.row_stride;
  a.num_kv_heads = g.num_kv_heads;
  a.num_blocks_m1 = (int32_t)(g.num_blocks - 1);
  a.num_q_heads = num_q_heads;
  a.gqa = num_q_heads / g.num_kv_heads;
  a.q = (const _Float16*)q;
  a.out = (_Float16*)out;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  const int64_t table_cap = (int64_t)max_blocks_per_seq * g.block_size;
  a.len_cap = (int32_t)(table_cap < max_seq_len ? table_cap : max_seq_len);
  a.seq_lens = seq_lens;
  a.score_scale = (float)((double)scale * 1.4426950408889634 * (double)g.k_scale);
  a.v_scale = g.v_scale;
  a.k_hs = g.k_hs;
  a.v_hs = g.v_hs;
  a.window = g.window;
  a.k_bs = g.k_bs;
  a.v_bs = g.v_bs;
  (void)num_seqs;
  return PA_OK;
}

int kv_code(const pa::PoolGeom& g) {
  return g.elem_bytes == 2 ? 0 : (g.fp8_e5m2 ? 2 : 1) + (g.k_bs ? 2 : 0);
}


}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_reshape_and_cache(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int64_t num_tokens, hipStream_t stream) {
  pa::PoolGeom g;
  int st = check_pool(pool, &g);
  if (st) return st;
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_tokens %lld out of range", (long long)num_tokens);
  log_line("pa_reshape_and_cache: %lld tokens, %s pool of %lld blocks x %d slots, %d kv heads, "
           "head_dim %d", (long long)num_tokens, kv_name(pool->dtype), (long long)g.num_blocks,
           g.block_size, g.num_kv_heads, g.head_dim);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "k_new, v_new and slot_mapping must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_ALIGNMENT, "k_new and v_new must be 16-byte aligned");
  if (hipError_t e = pa::launch_reshape_and_cache(g, (const _Float16*)k_new,
                                                  (const _Float16*)v_new, slot_mapping,
                                                  num_tokens, stream))
    return fail(PA_ERR_HIP, "reshape_and_cache launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_copy_blocks(const pa_kv_pool* pool, const int64_t* block_mapping, int64_t num_pairs,
                   hipStream_t stream) {
  pa::PoolGeom g;
  int st = check_pool(pool, &g);
  if (st) return st;
  if (num_pairs < 0 || num_pairs > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_pairs %lld out of range", (long long)num_pairs);
  log_line("pa_copy_blocks: %lld pairs (K and V blocks of %lld bytes each)", (long long)num_pairs,
           (long long)(g.row_stride * (int64_t)g.block_size));
  if (num_pairs == 0) return PA_OK;
  if (!block_mapping) return fail(PA_ERR_INVALID_ARG, "block_mapping is NULL");
  if (hipError_t e = pa::launch_copy_blocks(g, block_mapping, num_pairs, stream))
    return fail(PA_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int32_t pa_decode_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_seq_len, int32_t partition_size) {
  pa::PoolGeom g;
  Plan pl;
  int st = plan(pool, num_seqs, num_q_heads, max_seq_len, partition_size, &g, &pl);
  return st ? st : plan_code(pl);
}

size_t pa_decode_workspace_size(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_seq_len, int32_t partition_size) {
  pa::PoolGeom g;
  Plan pl;
  if (plan(pool, num_seqs, num_q_heads, max_seq_len, partition_size, &g, &pl)) return 0;
  return workspace_bytes_for(pl, num_seqs, num_q_heads, g.num_kv_heads, g.head_dim);
}


int pa_decode(const pa_kv_pool* pool, void* out, const void* q, int32_t num_seqs,
              int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* seq_lens, int32_t max_seq_len, float scale, int32_t partition_size,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  pa::PoolGeom g;
  Plan pl;
  int st = plan(pool, num_seqs, num_q_heads, max_seq_len, partition_size, &g, &pl);
  if (st) return st;
  if (log_on()) {
    const int64_t units = (int64_t)num_seqs * g.num_kv_heads;
    if (pl.mode == pa::kModeFlat)
      log_line("pa_decode: %d seqs, %d/%d heads, head_dim %d, bs %d, %s, max_seq_len %d: flat, "
               "%lld ranges x %d kv heads = %lld waves, then the merge of cut sequences",
               num_seqs, num_q_heads, g.num_kv_heads, g.head_dim, g.block_size,
               kv_name(pool->dtype), max_seq_len, (long long)pl.waves, g.num_kv_heads,
               (long long)(pl.waves * g.num_kv_heads));
    else if (pl.mode == pa::kModeSplit)
      log_line("pa_decode: %d seqs, %d/%d heads, head_dim %d, bs %d, %s, max_seq_len %d: split, "
               "%d-token partitions, %lld workgroups, then the log-sum-exp reduce", num_seqs,
               num_q_heads, g.num_kv_heads, g.head_dim, g.block_size, kv_name(pool->dtype),
               max_seq_len, pl.part, (long long)(units * pl.num_parts));
    else
      log_line("pa_decode: %d seqs, %d/%d heads, head_dim %d, bs %d, %s, max_seq_len %d: single "
               "pass, %lld workgroups", num_seqs, num_q_heads, g.num_kv_heads, g.head_dim,
               g.block_size, kv_name(pool->dtype), max_seq_len, (long long)units);
  }
  if (num_seqs == 0) return PA_OK;
  pa::DecodeArgs a;
  st = decode_args(g, out, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, seq_lens,
                   max_seq_len, scale, &a);
  if (st) return st;
  const size_t need = workspace_bytes_for(pl, num_seqs, num_q_heads, g.num_kv_heads, g.head_dim);
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "this schedule needs %zu workspace bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }

  pa::FlatArgs f{};
  if (pl.mode == pa::kModeSplit) {
    a.part_tokens = pl.part;
    a.num_parts = pl.num_parts;
    const int64_t rows = (int64_t)num_seqs * num_q_heads * pl.num_parts;
    a.ws_ml = (float2*)workspace;
    a.ws_o = (float*)((char*)workspace + align256((size_t)rows * 8));
  } else if (pl.mode == pa::kModeFlat) {
    f.num_seqs = num_seqs;
    f.num_ranges = (int32_t)pl.waves;
    f.prefix = (int32_t*)workspace;
    f.slots = (float*)((char*)workspace + align256((size_t)(num_seqs + 1) * 4));
  }
  const bool stream_kv = !(g.flags & PA_POOL_SHARED_BLOCKS);
  if (hipError_t e = pa::launch_decode(a, &f, nullptr, num_seqs, g.head_dim, g.block_size,
                                       kv_code(g), stream_kv, pl.mode, stream))
    return fail(PA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int32_t pa_decode_group_plan(const int32_t* block_tables, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t* members, int32_t* member_start, int32_t* member_shared) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_kv_heads < 1 ||
      num_q_heads < num_kv_heads || num_q_heads % num_kv_heads ||
      num_q_heads / num_kv_heads > 16)
    return fail(PA_ERR_INVALID_ARG, "bad sizes for the group plan");
  if (num_seqs && (!block_tables || !seq_lens || !members || !member_start || !member_shared))
    return fail(PA_ERR_INVALID_ARG, "group plan arrays must be non-NULL");
  const int32_t cap = 16 / (num_q_heads / num_kv_heads);
  const int64_t mb = max_blocks_per_seq;
  auto len_of = [&](int32_t s) {
    const int64_t n = seq_lens[s], m = mb * block_size;
    return (int32_t)(n < 0 ? 0 : (n > m ? m : n));
  };
  auto nblk = [&](int32_t s) { return (len_of(s) + block_size - 1) / block_size; };
  auto row = [&](int32_t s) { return block_tables + (int64_t)s * mb; };
  // positions shared by s and t: their common run of leading table entries,
  // within both lengths, in whole 16-token tiles
  auto shared = [&](int32_t s, int32_t t) {
    const int32_t n = std::min(nblk(s), nblk(t));
    const int32_t* a = row(s);
    const int32_t* b = row(t);
    int32_t k = 0;
    while (k < n && a[k] == b[k]) ++k;
    return (int32_t)(std::min((int64_t)k * block_size,
                              (int64_t)std::min(len_of(s), len_of(t))) & ~15);
  };
  // families: sequences whose first block is the same physical block, in
  // order of their first member; each family sorted by its table rows, so
  // that rows with long common prefixes are neighbours
  std::vector<std::vector<int32_t>> fam;
  std::unordered_map<int32_t, size_t> by_first;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (len_of(s) < 16 || cap < 2) {
      fam.push_back({s});
      continue;
    }
    auto it = by_first.find(row(s)[0]);
    if (it == by_first.end()) {
      by_first.emplace(row(s)[0], fam.size());
      fam.push_back({s});
    } else {
      fam[it->second].push_back(s);
    }
  }
  struct G { int32_t first, n; int64_t work; };
  std::vector<G> groups;
  std::vector<int32_t> order, share;
  order.reserve((size_t)num_seqs);
  share.reserve((size_t)num_seqs);
  for (auto& f : fam) {
    std::stable_sort(f.begin(), f.end(), [&](int32_t s, int32_t t) {
      return std::lexicographical_compare(row(s), row(s) + nblk(s), row(t), row(t) + nblk(t));
    });
    // chains of neighbours that share something, cut every `cap` members
    for (size_t i = 0; i < f.size(); ++i) {
      const int32_t sh = i ? shared(f[i - 1], f[i]) : 0;
      if (sh == 0 || groups.empty() || groups.back().n == cap ||
          order[(size_t)groups.back().first + groups.back().n - 1] != f[i - 1]) {
        groups.push_back({(int32_t)order.size(), 0, 0});
        share.push_back(0);
      } else {
        share.push_back(sh);
      }
      G& gr = groups.back();
      gr.work += (len_of(f[i]) + 15) / 16 - share.back() / 16;
      ++gr.n;
      order.push_back(f[i]);
    }
  }
  // the longest groups start first, so that the short ones fill in at the end
  std::vector<size_t> idx(groups.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(),
                   [&](size_t x, size_t y) { return groups[x].work > groups[y].work; });
  int32_t pos = 0;
  for (size_t k = 0; k < idx.size(); ++k) {
    const G& gr = groups[idx[k]];
    member_start[k] = pos;
    for (int32_t m = 0; m < gr.n; ++m, ++pos) {
      members[pos] = order[(size_t)gr.first + m];
      member_shared[pos] = m ? share[(size_t)gr.first + m] : 0;
    }
  }
  member_start[groups.size()] = pos;
  return (int32_t)groups.size();
}

int32_t pa_decode_grouped_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_seq_len, int32_t num_groups, int32_t schedule) {
  pa::PoolGeom g;
  GroupPlan gp;
  int st = group_plan(pool, num_seqs, num_q_heads, max_seq_len, num_groups, schedule, &g, &gp);
  return st ? st : gp.mode;
}

size_t pa_decode_grouped_workspace_size(const pa_kv_pool* pool, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_seq_len,
                                        int32_t num_groups, int32_t schedule) {
  pa::PoolGeom g;
  GroupPlan gp;
  if (group_plan(pool, num_seqs, num_q_heads, max_seq_len, num_groups, schedule, &g, &gp))
    return 0;
  return gp.workspace;
}

int pa_decode_grouped(const pa_kv_pool* pool, void* out, const void* q, int32_t num_seqs,
                      int32_t num_q_heads, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                      float scale, int32_t num_groups, const int32_t* members,
                      const int32_t* member_start, const int32_t* member_shared,
                      int32_t schedule, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  pa::PoolGeom g;
  GroupPlan gpl;
  int st = group_plan(pool, num_seqs, num_q_heads, max_seq_len, num_groups, schedule, &g, &gpl);
  if (st) return st;
  if (gpl.mode == kGroupFlat)
    log_line("pa_decode_grouped: %d seqs in %d groups, %d/%d heads, head_dim %d, %s: flat over "
             "groups, %lld ranges x %d kv heads, then the merge of cut groups", num_seqs,
             num_groups, num_q_heads, g.num_kv_heads, g.head_dim, kv_name(pool->dtype),
             (long long)gpl.ranges, g.num_kv_heads);
  else
    log_line("pa_decode_grouped: %d seqs in %d groups, %d/%d heads, head_dim %d, %s: one "
             "workgroup per (group, kv head), %lld workgroups", num_seqs, num_groups,
             num_q_heads, g.num_kv_heads, g.head_dim, kv_name(pool->dtype),
             (long long)num_groups * g.num_kv_heads);
  if (num_seqs == 0 || num_groups == 0) return PA_OK;
  if (!members || !member_start || !member_shared)
    return fail(PA_ERR_INVALID_ARG, "members, member_start and member_shared must be non-NULL");
  pa::DecodeArgs a;
  st = decode_args(g, out, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, seq_lens,
                   max_seq_len, scale, &a);
  if (st) return st;
  if (gpl.workspace) {
    if (!workspace || workspace_bytes < gpl.workspace)
      return fail(PA_ERR_WORKSPACE, "this schedule needs %zu workspace bytes, got %zu",
                  gpl.workspace, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PA_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  pa::GroupArgs gr{num_groups, num_seqs, num_seqs, members, member_start, member_shared};
  pa::FlatArgs f{};
  if (gpl.mode == kGroupFlat) {
    f.num_seqs = num_seqs;
    f.num_ranges = (int32_t)gpl.ranges;
    f.prefix = (int32_t*)workspace;
    f.slots = (float*)((char*)workspace + align256((size_t)(num_groups + 1) * 4));
  }
  // every tile is read by one wave: streaming loads whatever the pool flag says
  if (hipError_t e = pa::launch_decode(a, &f, &gr, num_seqs, g.head_dim, g.block_size,
                                       kv_code(g), true,
                                       gpl.mode == kGroupFlat ? pa::kModeFlatGroup
                                                              : pa::kModeGroup, stream))
    return fail(PA_ERR_HIP, "grouped decode launch: %s", hipGetErrorString(e));
  return PA_OK;
}

// Checks shared by pa_prefill and pa_prefill_plan.
int prefill_shape(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                  int32_t max_q_len, pa::PoolGeom* g) {
  int st = check_pool(pool, g);
  if (st) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "max_q_len %d < 0", max_q_len);
  if (num_q_heads < 1 || num_q_heads % g->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, g->num_kv_heads);
  if (num_q_heads / g->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d > 16",
                num_q_heads / g->num_kv_heads);
  if (g->k_bs && g->head_dim < 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill reads per-block scales at head_dim 128 and 256");
  return PA_OK;
}

int32_t pa_prefill_plan(const pa_kv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                        int32_t max_q_len) {
  pa::PoolGeom g;
  if (int st = prefill_shape(pool, num_seqs, num_q_heads, max_q_len, &g)) return st;
  const int32_t gqa = num_q_heads / g.num_kv_heads;
  const pa::PrefillPlan plan = pa::prefill_plan(g.head_dim, kv_code(g), gqa,
                                                (int64_t)num_seqs * g.num_kv_heads, max_q_len,
                                                prefill_groups_override());
  return plan.tile_tokens * gqa;
}

int pa_prefill(const pa_kv_pool* pool, void* out, const void* q, int32_t total_q,
               const int32_t* q_start, int32_t num_seqs, int32_t num_q_heads,
               const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
               int32_t max_q_len, float scale, hipStream_t stream) {
  pa::PoolGeom g;
  if (int st = prefill_shape(pool, num_seqs, num_q_heads, max_q_len, &g)) return st;
  if (total_q < 0) return fail(PA_ERR_INVALID_ARG, "total_q %d < 0", total_q);
  const int32_t gqa = num_q_heads / g.num_kv_heads;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !q_start || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG,
                "out, q, q_start, block_tables and seq_lens must be non-NULL");
  if (!aligned16(out) || !aligned16(q))
    return fail(PA_ERR_ALIGNMENT, "q and out must be 16-byte aligned");
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "scale must be finite and positive");
  const pa::PrefillPlan plan = pa::prefill_plan(g.head_dim, kv_code(g), gqa,
                                                (int64_t)num_seqs * g.num_kv_heads, max_q_len,
                                                prefill_groups_override());
  const int32_t tile = plan.tile_tokens;
  const int64_t num_qt = cdiv64(max_q_len, tile);
  if ((int64_t)num_seqs * g.num_kv_heads * num_qt > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_seqs * num_kv_heads * cdiv(max_q_len, %d) too large",
                tile);
  log_line("pa_prefill: %d seqs, %d new tokens (at most %d per sequence), %d/%d heads, "
           "head_dim %d, %s: %d new tokens per workgroup (%d row groups per wave), %lld "
           "workgroups", num_seqs, total_q, max_q_len, num_q_heads, g.num_kv_heads, g.head_dim,
           kv_name(pool->dtype), tile, plan.groups, (long long)num_seqs * g.num_kv_heads * num_qt);

  pa::PrefillArgs a{};
  a.k = g.k;
  a.v = g.v;
  a.block_stride = g.block_stride;
  a.row_stride = g.row_stride;
  a.num_blocks_m1 = (int32_t)(g.num_blocks - 1);
  a.num_kv_heads = g.num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.gqa = gqa;
  a.q = (const _Float16*)q;
  a.out = (_Float16*)out;
  a.q_start = q_start;
  a.seq_lens = seq_lens;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.groups = plan.groups;
  a.tile_tokens = tile;
  a.num_qt = (int32_t)num_qt;
  a.score_scale = (float)((double)scale * 1.4426950408889634 * (double)g.k_scale);
  a.v_scale = g.v_scale;
  a.k_hs = g.k_hs;
  a.v_hs = g.v_hs;
  a.window = g.window;
  a.k_bs = g.k_bs;
  a.v_bs = g.v_bs;
  if (hipError_t e = pa::launch_prefill(a, g.head_dim, g.block_size, kv_code(g), stream))
    return fail(PA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
