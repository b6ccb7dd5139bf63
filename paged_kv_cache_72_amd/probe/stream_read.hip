// stream_read.hip -- HBM read-bandwidth ceiling probe (measurement only; not
// part of libpa's interface).  Every lane streams 16-byte loads over a large
// buffer in a grid-stride loop with UNROLL independent loads in flight, folds
// them with XOR and writes one word per thread so the loads cannot be elided.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr int kUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}
}  // namespace

extern "C" {
// Read `bytes` (a multiple of 16) from `src` once.  `sink` must hold
// blocks * 256 uint32 words.  Returns a hipError_t value.
int pa_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                         hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     (const u32x4*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}
}
