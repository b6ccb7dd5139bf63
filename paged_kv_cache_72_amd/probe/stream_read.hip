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

// ---------------------------------------------------------------- tile gather
// The decode kernels' read pattern without their arithmetic: wave w serves KV
// head w % Hkv of range w / Hkv, a contiguous slice of `blocks` (physical ids
// of 16-token blocks, [nlisted]); for every block it reads the head's 16 rows
// of 256 bytes (head_dim 128, binary16) from the K pool and from the V pool
// with four 16-byte loads per lane, UT blocks in flight.  Pools are
// [*, 16, Hkv, 128] binary16.  Lane layouts of load u (0..3):
//   MAP 0: token l & 15, bytes (l >> 4) * 64 + 16 u   (64 pieces of 16 B)
//   MAP 1: token l & 15, bytes u * 64 + (l >> 4) * 16 (16 pieces of 64 B)
//   MAP 2: token 4 u + (l >> 4), bytes (l & 15) * 16  (4 whole 256-B rows)
namespace {
template <int MAP>
__device__ __forceinline__ int64_t lane_offset(int lane, int u, int64_t row) {
  if constexpr (MAP == 0) return (lane & 15) * row + (lane >> 4) * 64 + 16 * u;
  else if constexpr (MAP == 1) return (lane & 15) * row + u * 64 + (lane >> 4) * 16;
  else return (4 * u + (lane >> 4)) * row + (lane & 15) * 16;
}

template <int UT, int MAP>
__global__ __launch_bounds__(256) void tile_gather_kernel(const char* __restrict__ kp,
                                                          const char* __restrict__ vp,
                                                          const int32_t* __restrict__ blocks,
                                                          int64_t nlisted, int32_t hkv,
                                                          int64_t ranges,
                                                          uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t r = w / hkv, kh = w % hkv;
  uint32_t acc = 0;
  if (r < ranges) {
    const int64_t b0 = r * nlisted / ranges, b1 = (r + 1) * nlisted / ranges;
    const int64_t row = (int64_t)hkv * 256;                   // bytes per token row
    for (int64_t b = b0; b < b1; b += UT) {
      u32x4 kv[UT][4], vv[UT][4];
#pragma unroll
      for (int t = 0; t < UT; ++t) {
        const int64_t bb = b + t < b1 ? b + t : b1 - 1;
        const int64_t base = (int64_t)blocks[bb] * 16 * row + kh * 256;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t o = base + lane_offset<MAP>(lane, u, row);
          kv[t][u] = __builtin_nontemporal_load((const u32x4*)(kp + o));
          vv[t][u] = __builtin_nontemporal_load((const u32x4*)(vp + o));
        }
      }
#pragma unroll
      for (int t = 0; t < UT; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= kv[t][u].x ^ vv[t][u].w;
    }
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int MAP>
int launch_gather(const char* k, const char* v, const int32_t* blocks, int64_t nlisted,
                  int32_t hkv, int64_t ranges, int32_t ut, uint32_t* sink, hipStream_t stream) {
  const int64_t waves = (ranges * hkv + 3) / 4 * 4;
  const dim3 grid((uint32_t)(waves / 4)), block(256);
  if (ut == 1)
    hipLaunchKernelGGL((tile_gather_kernel<1, MAP>), grid, block, 0, stream, k, v, blocks, nlisted, hkv, ranges, sink);
  else if (ut == 2)
    hipLaunchKernelGGL((tile_gather_kernel<2, MAP>), grid, block, 0, stream, k, v, blocks, nlisted, hkv, ranges, sink);
  else if (ut == 4)
    hipLaunchKernelGGL((tile_gather_kernel<4, MAP>), grid, block, 0, stream, k, v, blocks, nlisted, hkv, ranges, sink);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
}  // namespace

extern "C" {
// waves = ranges * hkv rounded up to a multiple of 4; sink holds waves * 64
// words.  Every id in blocks[0 .. nlisted) must be a valid block of both pools.
int pa_probe_tile_gather(const void* k_pool, const void* v_pool, const int32_t* blocks,
                         int64_t nlisted, int32_t hkv, int64_t ranges, int32_t tiles_in_flight,
                         int32_t lane_map, uint32_t* sink, hipStream_t stream) {
  if (nlisted <= 0 || hkv <= 0 || ranges <= 0 || ranges > nlisted) return (int)hipErrorInvalidValue;
  const char* k = (const char*)k_pool;
  const char* v = (const char*)v_pool;
  switch (lane_map) {
    case 0: return launch_gather<0>(k, v, blocks, nlisted, hkv, ranges, tiles_in_flight, sink, stream);
    case 1: return launch_gather<1>(k, v, blocks, nlisted, hkv, ranges, tiles_in_flight, sink, stream);
    case 2: return launch_gather<2>(k, v, blocks, nlisted, hkv, ranges, tiles_in_flight, sink, stream);
    default: return (int)hipErrorInvalidValue;
  }
}
}
