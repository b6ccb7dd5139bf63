// pa_noalloc.hip -- pa_decode_noalloc: pa_decode with the library's own
// per-device scratch in place of a caller workspace (declared in include/pa.h).
//
// The scratch is one file-scope device array per GPU.  Its host-side name is
// only a stand-in, never a device address: the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and only
// that pointer is ever handed to kernels.  Nothing here allocates.
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

static __device__ __align__(256) char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];      // device address of `scratch` on each device

// Device address of this device's scratch array (looked up on first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev))
    return pa::fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
      return pa::fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                      hipGetErrorString(e));
    if (!p) return pa::fail(PA_ERR_HIP, "no address for the scratch array on device %d", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(const pa_kv_pool* pool, void* out, const void* q,
                                 int32_t num_seqs, int32_t num_q_heads,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                 int32_t partition_size, hipStream_t stream) {
  // the plan's own argument errors are reported by pa_decode below
  if (pa_decode_plan(pool, num_seqs, num_q_heads, max_seq_len, partition_size) >= 0) {
    const size_t need =
        pa_decode_workspace_size(pool, num_seqs, num_q_heads, max_seq_len, partition_size);
    if (need > (size_t)PA_DECODE_NOALLOC_SCRATCH_BYTES)
      return pa::fail(PA_ERR_WORKSPACE,
                      "this schedule needs %zu bytes of workspace, more than the %u bytes of "
                      "the library's scratch: call pa_decode with a workspace",
                      need, (unsigned)PA_DECODE_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if (int st = scratch_for_current_device(&ws)) return st;
  return pa_decode(pool, out, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq,
                   seq_lens, max_seq_len, scale, partition_size, ws,
                   (size_t)PA_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}
