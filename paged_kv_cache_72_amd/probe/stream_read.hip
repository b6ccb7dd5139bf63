// stream_read.hip -- HBM read-bandwidth ceiling probes (measurement only; not
// part of libpa's interface).  Both fold what they read with XOR and write one
// word per thread so the loads cannot be elided.
//   grid-stride:  every lane streams 16-byte loads over the whole buffer with
//                 kUnroll independent loads in flight.
//   wave-chunk:   wave w reads its own contiguous chunk of the buffer, U KiB
//                 per step (U loads of 64 lanes x 16 bytes), like a decode wave
//                 walking its range of KV tiles.
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

// steps16: 1 KiB steps per wave (a multiple of U); waves = gridDim.x * 4.
template <int U>
__global__ __launch_bounds__(256) void wave_chunk_kernel(const u32x4* __restrict__ src,
                                                         int64_t steps_per_wave,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const u32x4* p = src + w * steps_per_wave * 64 + lane;
  uint32_t acc = 0;
  for (int64_t s = 0; s < steps_per_wave; s += U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + (s + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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

// Read the first waves * steps_per_wave KiB of `src` (which must hold that
// many bytes), wave w taking the w-th contiguous chunk, `unroll` (4, 8 or 16)
// KiB per step; steps_per_wave must be a multiple of unroll and waves a
// multiple of 4.  `sink` must hold waves * 64 uint32 words.
int pa_probe_wave_chunk(const void* src, int64_t waves, int64_t steps_per_wave, int32_t unroll,
                        uint32_t* sink, hipStream_t stream) {
  if (waves <= 0 || waves % 4 || steps_per_wave <= 0 || steps_per_wave % unroll)
    return (int)hipErrorInvalidValue;
  const dim3 grid((uint32_t)(waves / 4)), block(256);
  const u32x4* s = (const u32x4*)src;
  if (unroll == 4)
    hipLaunchKernelGGL(wave_chunk_kernel<4>, grid, block, 0, stream, s, steps_per_wave, sink);
  else if (unroll == 8)
    hipLaunchKernelGGL(wave_chunk_kernel<8>, grid, block, 0, stream, s, steps_per_wave, sink);
  else if (unroll == 16)
    hipLaunchKernelGGL(wave_chunk_kernel<16>, grid, block, 0, stream, s, steps_per_wave, sink);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
}
