// pa_check.hip -- checks of the device-side arguments of the compute calls
// (declared in include/pa_check.h).
//
// The compute kernels stay in bounds whatever their device arrays hold; these
// kernels find the entries that would make them clamp or skip, and the
// preconditions they cannot see (distinct slots, distinct copy destinations).
// Every problem adds one to a counter and offers a (kind, index) key to an
// atomic minimum, so the reported problem does not depend on thread timing.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"
#include "pa_check.h"
#include "pa_internal.h"

namespace {

using pa::fail;

// The report at the start of the scratch buffer; bitmaps follow at kBitmapAt.
struct Report {
  uint32_t count;
  uint32_t pad;
  unsigned long long first;   // (kind << 48) | index of the first problem
};
constexpr size_t kBitmapAt = 256;
constexpr int kThreads = 256;

enum Kind : int {
  kLenRange = 1,   // seq_lens[s] < 0 or > max_seq_len          index: s
  kTableRow = 2,   // the sequence needs more blocks than a row  index: s
  kTableId = 3,    // table entry outside [0, num_blocks)        index: s * max_blocks + j
  kQStart = 4,     // q_start out of order or outside [0, T]     index: entry
  kQLen = 5,       // q_len > max_q_len or > seq_lens[s]         index: s
  kSlotRange = 6,  // slot >= num_blocks * block_size            index: token
  kSlotDup = 7,    // slot listed more than once                 index: slot
  kPairRange = 8,  // pair with an id outside [0, num_blocks)    index: pair
  kDstDup = 9,     // block is the destination of two pairs      index: block
  kDstIsSrc = 10,  // block is a destination and a source        index: block
};

__device__ __forceinline__ void report(Report* r, int kind, int64_t index) {
  atomicAdd(&r->count, 1u);
  atomicMin(&r->first, ((unsigned long long)kind << 48) | (unsigned long long)index);
}

// Zero the report and the bitmaps; the minimum starts at all ones.
__global__ void clear_kernel(uint32_t* w, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    w[i] = (i == 2 || i == 3) ? 0xffffffffu : 0u;
}

struct SeqCheck {
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* q_start;     // null: decode (one query, the last position)
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t block_size;
  int32_t window;
  int32_t max_seq_len;        // decode only
  int32_t total_q;            // prefill only
  int32_t max_q_len;          // prefill only
  int32_t num_seqs;
  Report* rep;
};

// One workgroup per sequence; the threads walk the table row.
__global__ __launch_bounds__(kThreads) void seq_check_kernel(SeqCheck c) {
  const int s = blockIdx.x;
  const bool lead = threadIdx.x == 0;
  const int len = c.lens[s];
  int q_len = 1;
  if (c.q_start) {
    const int a = c.q_start[s], b = c.q_start[s + 1];
    if (lead && s == 0 && (a < 0 || a > c.total_q)) report(c.rep, kQStart, 0);
    if (lead && (b < a || b > c.total_q)) report(c.rep, kQStart, s + 1);
    q_len = b - a;
    if (lead && q_len >= 0 && (q_len > c.max_q_len || q_len > len)) report(c.rep, kQLen, s);
    if (q_len <= 0) return;                 // nothing of this sequence is read
  } else if (lead && (len < 0 || len > c.max_seq_len)) {
    report(c.rep, kLenRange, s);
  }
  if (len <= 0) {
    if (lead && len < 0 && c.q_start) report(c.rep, kLenRange, s);
    return;
  }
  const int64_t need = ((int64_t)len + c.block_size - 1) / c.block_size;
  if (lead && need > c.max_blocks) report(c.rep, kTableRow, s);
  // first position any query of the sequence sees (the kernels clamp q_len to len)
  const int first_q = len - (q_len < len ? q_len : len);
  int lo = 0;
  if (c.window > 0) {
    lo = first_q - c.window + 1;
    if (lo < 0) lo = 0;
  }
  const int64_t end = need < c.max_blocks ? need : c.max_blocks;
  const int32_t* row = c.tables + (int64_t)s * c.max_blocks;
  for (int64_t j = lo / c.block_size + threadIdx.x; j < end; j += blockDim.x) {
    const int32_t id = row[j];
    if (id < 0 || id >= c.num_blocks) report(c.rep, kTableId, (int64_t)s * c.max_blocks + j);
  }
}

__global__ __launch_bounds__(kThreads) void slot_check_kernel(const int64_t* slots, int64_t n,
                                                              int64_t num_slots, uint32_t* seen,
                                                              Report* rep) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t x = slots[i];
    if (x < 0) continue;                    // padding
    if (x >= num_slots) {
      report(rep, kSlotRange, i);
      continue;
    }
    const uint32_t bit = 1u << (x & 31);
    if (atomicOr(&seen[x >> 5], bit) & bit) report(rep, kSlotDup, x);
  }
}

// Pass 1: ids in range, sources marked, repeated destinations found.
__global__ __launch_bounds__(kThreads) void pair_mark_kernel(const int64_t* pairs, int64_t n,
                                                             int64_t num_blocks, uint32_t* src_map,
                                                             uint32_t* dst_map, Report* rep) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) {
      report(rep, kPairRange, i);
      continue;
    }
    atomicOr(&src_map[s >> 5], 1u << (s & 31));
    const uint32_t bit = 1u << (d & 31);
    if (atomicOr(&dst_map[d >> 5], bit) & bit) report(rep, kDstDup, d);
  }
}

// Pass 2 (after pass 1 on the same stream): destinations that are sources.
__global__ __launch_bounds__(kThreads) void pair_src_kernel(const int64_t* pairs, int64_t n,
                                                            int64_t num_blocks,
                                                            const uint32_t* src_map,
                                                            Report* rep) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) continue;
    if ((src_map[d >> 5] >> (d & 31)) & 1u) report(rep, kDstIsSrc, d);
  }
}

int64_t bitmap_words(int64_t bits) { return (bits + 31) / 32; }

size_t scratch_for(const pa::PoolGeom& g) {
  const int64_t slot_words = bitmap_words(g.num_blocks * g.block_size);
  const int64_t pair_words = 2 * bitmap_words(g.num_blocks);
  const int64_t words = slot_words > pair_words ? slot_words : pair_words;
  return (kBitmapAt + 4 * (size_t)words + 255) / 256 * 256;
}

uint32_t grid_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (uint32_t)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

int check_scratch(const pa::PoolGeom& g, void* scratch, size_t bytes) {
  if (!scratch) return fail(PA_ERR_INVALID_ARG, "scratch is NULL");
  if ((uintptr_t)scratch & 7u) return fail(PA_ERR_ALIGNMENT, "scratch must be 8-byte aligned");
  if (bytes < scratch_for(g))
    return fail(PA_ERR_WORKSPACE, "scratch of %zu bytes is smaller than the %zu needed", bytes,
                scratch_for(g));
  return PA_OK;
}

// Clears the report and `bitmap_bits` bits after it.
hipError_t clear(void* scratch, int64_t bitmap_bits, hipStream_t stream) {
  const int64_t words = (int64_t)(kBitmapAt / 4) + bitmap_words(bitmap_bits);
  hipLaunchKernelGGL(clear_kernel, dim3(grid_for(words)), dim3(kThreads), 0, stream,
                     (uint32_t*)scratch, words);
  return hipGetLastError();
}

template <typename T>
T fetch(const T* dev, int64_t i) {
  T v{};
  if (hipMemcpy(&v, dev + i, sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) return T{};
  return v;
}

// Waits for the stream and turns the report into a status and a message.
// describe(kind, index) words the first problem.
template <typename F>
int finish(void* scratch, hipStream_t stream, const char* what, F describe) {
  Report r{};
  if (hipError_t e = hipMemcpyAsync(&r, scratch, sizeof r, hipMemcpyDeviceToHost, stream))
    return fail(PA_ERR_HIP, "%s: reading the report: %s", what, hipGetErrorString(e));
  if (hipError_t e = hipStreamSynchronize(stream))
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (r.count == 0) return PA_OK;
  const int kind = (int)(r.first >> 48);
  const int64_t index = (int64_t)(r.first & ((1ull << 48) - 1));
  const std::string msg = describe(kind, index);
  return fail(PA_ERR_INVALID_ARG, "%s: %s (%u problem%s found)", what, msg.c_str(), r.count,
              r.count == 1 ? "" : "s");
}

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char* f, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

std::string describe_seq(int kind, int64_t index, const SeqCheck& c) {
  switch (kind) {
    case kLenRange:
      if (c.q_start)
        return fmt("seq_lens[%lld] = %d is negative", (long long)index, fetch(c.lens, index));
      return fmt("seq_lens[%lld] = %d is negative or above max_seq_len %d", (long long)index,
                 fetch(c.lens, index), c.max_seq_len);
    case kTableRow:
      return fmt("seq_lens[%lld] = %d needs more than max_blocks_per_seq = %d blocks of %d",
                 (long long)index, fetch(c.lens, index), c.max_blocks, c.block_size);
    case kTableId:
      return fmt("block_tables[%lld][%lld] = %d is outside [0, %lld)",
                 (long long)(index / c.max_blocks), (long long)(index % c.max_blocks),
                 fetch(c.tables, index), (long long)c.num_blocks);
    case kQStart:
      return fmt("q_start[%lld] = %d is out of order or outside [0, total_q = %d]",
                 (long long)index, fetch(c.q_start, index), c.total_q);
    case kQLen:
      return fmt("sequence %lld has q_len %d, above max_q_len %d or its seq_lens %d",
                 (long long)index, fetch(c.q_start, index + 1) - fetch(c.q_start, index),
                 c.max_q_len, fetch(c.lens, index));
    default:
      return fmt("problem of kind %d at %lld", kind, (long long)index);
  }
}

int run_seq_check(const SeqCheck& c0, void* scratch, hipStream_t stream, const char* what) {
  SeqCheck c = c0;
  c.rep = (Report*)scratch;
  if (hipError_t e = clear(scratch, 0, stream))
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  hipLaunchKernelGGL(seq_check_kernel, dim3((uint32_t)c.num_seqs), dim3(kThreads), 0, stream, c);
  if (hipError_t e = hipGetLastError())
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  return finish(scratch, stream, what,
                [&](int kind, int64_t index) { return describe_seq(kind, index, c); });
}

}  // namespace

extern "C" {

size_t pa_check_scratch_bytes(const pa_kv_pool* pool) {
  pa::PoolGeom g;
  if (pa::check_pool(pool, &g)) return 0;
  return scratch_for(g);
}

int pa_check_decode_inputs(const pa_kv_pool* pool, int32_t num_seqs,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, void* scratch,
                           size_t scratch_bytes, hipStream_t stream) {
  pa::PoolGeom g;
  if (int st = pa::check_pool(pool, &g)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (max_seq_len < 0) return fail(PA_ERR_INVALID_ARG, "max_seq_len %d < 0", max_seq_len);
  if (int st = check_scratch(g, scratch, scratch_bytes)) return st;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG, "block_tables and seq_lens must be non-NULL");
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  SeqCheck c{};
  c.tables = block_tables;
  c.lens = seq_lens;
  c.num_blocks = g.num_blocks;
  c.max_blocks = max_blocks_per_seq;
  c.block_size = g.block_size;
  c.window = g.window;
  c.max_seq_len = max_seq_len;
  c.num_seqs = num_seqs;
  return run_seq_check(c, scratch, stream, "pa_decode inputs");
}

int pa_check_prefill_inputs(const pa_kv_pool* pool, int32_t total_q, const int32_t* q_start,
                            int32_t num_seqs, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t max_q_len, void* scratch, size_t scratch_bytes,
                            hipStream_t stream) {
  pa::PoolGeom g;
  if (int st = pa::check_pool(pool, &g)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (total_q < 0) return fail(PA_ERR_INVALID_ARG, "total_q %d < 0", total_q);
  if (max_q_len < 0) return fail(PA_ERR_INVALID_ARG, "max_q_len %d < 0", max_q_len);
  if (int st = check_scratch(g, scratch, scratch_bytes)) return st;
  if (num_seqs == 0) return PA_OK;
  if (!q_start || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG, "q_start, block_tables and seq_lens must be non-NULL");
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  SeqCheck c{};
  c.tables = block_tables;
  c.lens = seq_lens;
  c.q_start = q_start;
  c.num_blocks = g.num_blocks;
  c.max_blocks = max_blocks_per_seq;
  c.block_size = g.block_size;
  c.window = g.window;
  c.total_q = total_q;
  c.max_q_len = max_q_len;
  c.num_seqs = num_seqs;
  return run_seq_check(c, scratch, stream, "pa_prefill inputs");
}

int pa_check_slot_mapping(const pa_kv_pool* pool, const int64_t* slot_mapping,
                          int64_t num_tokens, void* scratch, size_t scratch_bytes,
                          hipStream_t stream) {
  pa::PoolGeom g;
  if (int st = pa::check_pool(pool, &g)) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (int st = check_scratch(g, scratch, scratch_bytes)) return st;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping) return fail(PA_ERR_INVALID_ARG, "slot_mapping is NULL");
  const int64_t num_slots = g.num_blocks * g.block_size;
  const char* what = "pa_reshape_and_cache slot_mapping";
  if (hipError_t e = clear(scratch, num_slots, stream))
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  hipLaunchKernelGGL(slot_check_kernel, dim3(grid_for(num_tokens)), dim3(kThreads), 0, stream,
                     slot_mapping, num_tokens, num_slots,
                     (uint32_t*)((char*)scratch + kBitmapAt), (Report*)scratch);
  if (hipError_t e = hipGetLastError())
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  return finish(scratch, stream, what, [&](int kind, int64_t index) {
    if (kind == kSlotRange)
      return fmt("slot_mapping[%lld] = %lld is at or beyond the pool's %lld slots",
                 (long long)index, (long long)fetch(slot_mapping, index), (long long)num_slots);
    return fmt("slot %lld is listed more than once", (long long)index);
  });
}

int pa_check_block_mapping(const pa_kv_pool* pool, const int64_t* block_mapping,
                           int64_t num_pairs, void* scratch, size_t scratch_bytes,
                           hipStream_t stream) {
  pa::PoolGeom g;
  if (int st = pa::check_pool(pool, &g)) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %lld < 0", (long long)num_pairs);
  if (int st = check_scratch(g, scratch, scratch_bytes)) return st;
  if (num_pairs == 0) return PA_OK;
  if (!block_mapping) return fail(PA_ERR_INVALID_ARG, "block_mapping is NULL");
  const int64_t words = bitmap_words(g.num_blocks);
  uint32_t* src_map = (uint32_t*)((char*)scratch + kBitmapAt);
  uint32_t* dst_map = src_map + words;
  const char* what = "pa_copy_blocks block_mapping";
  if (hipError_t e = clear(scratch, 64 * words, stream))
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  hipLaunchKernelGGL(pair_mark_kernel, dim3(grid_for(num_pairs)), dim3(kThreads), 0, stream,
                     block_mapping, num_pairs, g.num_blocks, src_map, dst_map, (Report*)scratch);
  hipLaunchKernelGGL(pair_src_kernel, dim3(grid_for(num_pairs)), dim3(kThreads), 0, stream,
                     block_mapping, num_pairs, g.num_blocks, (const uint32_t*)src_map,
                     (Report*)scratch);
  if (hipError_t e = hipGetLastError())
    return fail(PA_ERR_HIP, "%s: launch: %s", what, hipGetErrorString(e));
  return finish(scratch, stream, what, [&](int kind, int64_t index) {
    if (kind == kPairRange)
      return fmt("block_mapping[%lld] = (%lld, %lld) has an id outside [0, %lld)",
                 (long long)index, (long long)fetch(block_mapping, 2 * index),
                 (long long)fetch(block_mapping, 2 * index + 1), (long long)g.num_blocks);
    if (kind == kDstDup) return fmt("block %lld is the destination of more than one pair",
                                    (long long)index);
    return fmt("block %lld is both a destination and a source", (long long)index);
  });
}

}  // extern "C"
