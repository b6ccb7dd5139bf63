// pa_cache.hip -- the write side of the paged KV cache on gfx950.
//
//   rc_scatter   : slot_mapping write of new tokens ("vLLM intro part 2",
//                  section 3.2: every new token has an absolute pool slot
//                  block * block_size + offset; decode appends one per step).
//   copy_blocks  : whole-block copy for copy-on-write ("GPU memory & KV cache",
//                  copy_blocks(blk, new) before the table is retargeted).
//
// Both are pure data movement: a token row (num_kv_heads * head_dim elements)
// is contiguous in k_new and in its pool slot, and a block is contiguous in the
// pool, so every lane moves 16 bytes per access and a wavefront covers 1 KiB.
#include "pa_internal.h"

namespace pa {
namespace {

// fp32 -> OCP e4m3fn by field arithmetic on the fp32 bits: round to nearest
// even, saturate to +-448 (infinities included), keep NaN as S.1111.111.
__device__ __forceinline__ uint32_t e4m3fn_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;        // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;       // |y| >= 448: largest finite
  if (a < 0x3C800000u) {                           // |y| < 2^-6: steps of 2^-9
    const float n = rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE
    return sign | (uint32_t)n;                     // 8 lands on the smallest normal
  }
  uint32_t code = (a >> 20) - (120u << 3);         // rebias exponent, keep 3 mantissa bits
  const uint32_t rest = a & 0xFFFFFu;
  code += (rest > 0x80000u) || (rest == 0x80000u && (code & 1u));
  return sign | code;
}

// fp32 -> OCP e5m2 the same way: round to nearest even, saturate to +-57344
// (infinities included), keep NaN as S.11111.11.
__device__ __forceinline__ uint32_t e5m2_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;        // NaN
  if (a >= 0x47600000u) return sign | 0x7Bu;       // |y| >= 57344: largest finite
  if (a < 0x38800000u) {                           // |y| < 2^-14: steps of 2^-16
    const float n = rintf(__uint_as_float(a) * 65536.0f);  // exact scaling, RNE
    return sign | (uint32_t)n;                     // 4 lands on the smallest normal
  }
  uint32_t code = (a >> 21) - (112u << 2);         // rebias exponent, keep 2 mantissa bits
  const uint32_t rest = a & 0x1FFFFFu;
  code += (rest > 0x100000u) || (rest == 0x100000u && (code & 1u));
  return sign | code;
}

// One workgroup per token.  Threads [0, n16) move K, [n16, 2*n16) move V, where
// n16 = row bytes / 16 of the binary16 source.
__global__ __launch_bounds__(256) void rc_scatter_f16(PoolGeom g, const uint4* __restrict__ k_new,
                                                      const uint4* __restrict__ v_new,
                                                      const int64_t* __restrict__ slots,
                                                      int32_t n16) {
  const int64_t i = blockIdx.x;
  const int64_t slot = slots[i];
  const int64_t cap = g.num_blocks * g.block_size;
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / g.block_size;
  const int32_t off = (int32_t)(slot - blk * g.block_size);
  const int64_t dst_off = blk * g.block_stride + (int64_t)off * g.row_stride;
  for (int t = threadIdx.x; t < 2 * n16; t += blockDim.x) {
    const bool is_v = t >= n16;
    const int c = is_v ? t - n16 : t;
    const uint4* src = (is_v ? v_new : k_new) + i * n16 + c;
    uint4* dst = (uint4*)((is_v ? g.v : g.k) + dst_off) + c;
    *dst = *src;
  }
}

// fp8 pools: each thread reads 8 binary16 values (16 B) and writes 8 bytes.
template <bool E5M2>
__global__ __launch_bounds__(256) void rc_scatter_fp8(PoolGeom g, const uint4* __restrict__ k_new,
                                                      const uint4* __restrict__ v_new,
                                                      const int64_t* __restrict__ slots,
                                                      int32_t n16) {
  const int64_t i = blockIdx.x;
  const int64_t slot = slots[i];
  const int64_t cap = g.num_blocks * g.block_size;
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / g.block_size;
  const int32_t off = (int32_t)(slot - blk * g.block_size);
  const int64_t dst_off = blk * g.block_stride + (int64_t)off * g.row_stride;
  for (int t = threadIdx.x; t < 2 * n16; t += blockDim.x) {
    const bool is_v = t >= n16;
    const int c = is_v ? t - n16 : t;
    const int head = c / (g.head_dim / 8);        // chunk c holds elements 8c .. 8c + 7
    const float scale = is_v ? (g.v_hs ? g.v_hs[head] : g.v_scale)
                             : (g.k_hs ? g.k_hs[head] : g.k_scale);
    const uint4 x = ((is_v ? v_new : k_new) + i * n16)[c];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t hb = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
      const float xf = (float)__builtin_bit_cast(_Float16, hb);
      const uint32_t code = E5M2 ? e5m2_from_f32(xf / scale) : e4m3fn_from_f32(xf / scale);
      packed[j >> 2] |= code << (8 * (j & 3));
    }
    uint2* dst = (uint2*)((is_v ? g.v : g.k) + dst_off) + c;
    *dst = make_uint2(packed[0], packed[1]);
  }
}

// fp8 byte -> its exact fp32 value, from the fields (no hardware converter).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
  if (e == 15u && m == 7u) return __uint_as_float(sign | 0x7FC00000u);   // NaN
  if (e == 0u) {                                                          // m * 2^-9
    const float v = (float)m * 0.001953125f;
    return sign ? -v : v;
  }
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}
__device__ __forceinline__ float e5m2_to_f32(uint32_t b) {
  // e5m2 is binary16 with the low 8 mantissa bits dropped
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b << 8));
}

// fp8 pools with one scale per (block, KV head), kept beside the pools and
// written here.  One workgroup per token; the token that starts a run (the
// consecutive tokens of slots that lie in one block) handles the whole run,
// the others return.  Per KV head, and for K and V separately, in fp32:
// c = max(a / m, smallest normal), a the largest finite |x| of the run and m
// the format's largest finite value; the block's new scale is c when the run
// writes slot 0, else max(old, c); when the run does not write slot 0 and the
// scale grows, every slot the run does not write is re-encoded as
// enc((value * old) / new); then the run's rows are stored as enc(x / new).
// Dynamic LDS: 6 * Hkv floats (the two pools' amax, old and new scales).
template <bool E5M2>
__global__ __launch_bounds__(256) void rc_scatter_fp8_block(PoolGeom g,
                                                            const uint4* __restrict__ k_new,
                                                            const uint4* __restrict__ v_new,
                                                            const int64_t* __restrict__ slots,
                                                            int64_t T, int32_t n16) {
  extern __shared__ float sm_f[];
  __shared__ uint32_t sm_written[4];              // bit o: the run writes slot o (block_size <= 128)
  const int64_t i = blockIdx.x;
  const int64_t cap = g.num_blocks * g.block_size;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= cap) return;
  const int64_t blk = slot / g.block_size;
  if (i > 0) {                                    // not the first token of its run
    const int64_t ps = slots[i - 1];
    if (ps >= 0 && ps < cap && ps / g.block_size == blk) return;
  }
  int64_t j = i + 1;                              // the run is [i, j), at most block_size tokens
  while (j < T && j < i + g.block_size) {
    const int64_t sj = slots[j];
    if (sj < 0 || sj >= cap || sj / g.block_size != blk) break;
    ++j;
  }
  const int H = g.num_kv_heads, dh8 = g.head_dim / 8;
  uint32_t* amax = (uint32_t*)sm_f;               // [2][H] bits of non-negative floats
  float* s_old = sm_f + 2 * H;                    // [2][H]
  float* s_new = sm_f + 4 * H;                    // [2][H]
  const float fmax_fmt = E5M2 ? 57344.0f : 448.0f;
  for (int t = threadIdx.x; t < 2 * H; t += blockDim.x) amax[t] = 0u;
  if (threadIdx.x < 4) sm_written[threadIdx.x] = 0u;
  __syncthreads();
  // which slots the run writes, and the largest finite |x| per (pool, head)
  for (int64_t t = i + threadIdx.x; t < j; t += blockDim.x) {
    const int o = (int)(slots[t] - blk * g.block_size);
    atomicOr(&sm_written[o >> 5], 1u << (o & 31));
  }
  const int64_t run = j - i;
  for (int64_t e = threadIdx.x; e < run * 2 * n16; e += blockDim.x) {
    const int64_t t = i + e / (2 * n16);
    const int c2 = (int)(e % (2 * n16));
    const bool is_v = c2 >= n16;
    const int c = is_v ? c2 - n16 : c2;
    const uint4 x = ((is_v ? v_new : k_new) + t * n16)[c];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float xf = fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[q >> 1] >> (16 * (q & 1)))));
      a = xf <= 3.4028235e38f ? fmaxf(a, xf) : a;  // finite values only
    }
    atomicMax(&amax[(is_v ? H : 0) + c / dh8], __float_as_uint(a));
  }
  __syncthreads();
  const bool fresh = sm_written[0] & 1u;
  for (int t = threadIdx.x; t < 2 * H; t += blockDim.x) {
    const float* arr = t < H ? g.k_bs : g.v_bs;
    const int h = t < H ? t : t - H;
    const float c = fmaxf(__uint_as_float(amax[t]) / fmax_fmt, 1.17549435e-38f);
    const float old = arr[blk * H + h];
    s_old[t] = old;
    s_new[t] = fresh ? c : fmaxf(old, c);
  }
  __syncthreads();
  // re-encode the slots the run does not write, where the scale grew
  if (!fresh) {
    const int64_t nch = (int64_t)g.block_size * 2 * H * dh8;   // 8-byte chunks of the block
    for (int64_t e = threadIdx.x; e < nch; e += blockDim.x) {
      const int o = (int)(e / (2 * H * dh8));
      const int r2 = (int)(e % (2 * H * dh8));
      const bool is_v = r2 >= H * dh8;
      const int c = is_v ? r2 - H * dh8 : r2;
      const int sidx = (is_v ? H : 0) + c / dh8;
      const float old = s_old[sidx], nw = s_new[sidx];
      if ((sm_written[o >> 5] >> (o & 31)) & 1u) continue;
      if (!(nw > old)) continue;
      uint2* p = (uint2*)((is_v ? g.v : g.k) + blk * g.block_stride + (int64_t)o * g.row_stride) + c;
      const uint2 b = *p;
      const uint32_t w[2] = {b.x, b.y};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t byte = (w[q >> 2] >> (8 * (q & 3))) & 0xFFu;
        const float v = E5M2 ? e5m2_to_f32(byte) : e4m3fn_to_f32(byte);
        const float y = (v * old) / nw;
        out[q >> 2] |= (E5M2 ? e5m2_from_f32(y) : e4m3fn_from_f32(y)) << (8 * (q & 3));
      }
      *p = make_uint2(out[0], out[1]);
    }
  }
  // the run's rows at the new scales
  for (int64_t e = threadIdx.x; e < run * 2 * n16; e += blockDim.x) {
    const int64_t t = i + e / (2 * n16);
    const int c2 = (int)(e % (2 * n16));
    const bool is_v = c2 >= n16;
    const int c = is_v ? c2 - n16 : c2;
    const float scale = s_new[(is_v ? H : 0) + c / dh8];
    const uint4 x = ((is_v ? v_new : k_new) + t * n16)[c];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float xf = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[q >> 1] >> (16 * (q & 1))));
      const uint32_t code = E5M2 ? e5m2_from_f32(xf / scale) : e4m3fn_from_f32(xf / scale);
      packed[q >> 2] |= code << (8 * (q & 3));
    }
    const int o = (int)(slots[t] - blk * g.block_size);
    uint2* dst = (uint2*)((is_v ? g.v : g.k) + blk * g.block_stride + (int64_t)o * g.row_stride) + c;
    *dst = make_uint2(packed[0], packed[1]);
  }
  for (int t = threadIdx.x; t < 2 * H; t += blockDim.x)
    (t < H ? g.k_bs : g.v_bs)[blk * H + (t < H ? t : t - H)] = s_new[t];
}

// Grid: (pairs, 2 pools, chunks of 4 KiB); 256 threads x 16 B per chunk.
__global__ __launch_bounds__(256) void copy_blocks_kernel(PoolGeom g,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_bytes) {
  const int64_t p = blockIdx.x;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || dst < 0 || src >= g.num_blocks || dst >= g.num_blocks) return;
  char* base = blockIdx.y ? g.v : g.k;
  const uint4* s = (const uint4*)(base + src * g.block_stride);
  uint4* d = (uint4*)(base + dst * g.block_stride);
  const int64_t n16 = block_bytes / 16;
  for (int64_t c = (int64_t)blockIdx.z * blockDim.x + threadIdx.x; c < n16;
       c += (int64_t)gridDim.z * blockDim.x)
    d[c] = s[c];
  if (g.k_bs && blockIdx.z == 0) {                // per-block scales travel with the block
    float* sc = blockIdx.y ? g.v_bs : g.k_bs;
    for (int h = threadIdx.x; h < g.num_kv_heads; h += blockDim.x)
      sc[dst * g.num_kv_heads + h] = sc[src * g.num_kv_heads + h];
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const PoolGeom& g, const _Float16* k_new,
                                    const _Float16* v_new, const int64_t* slots, int64_t T,
                                    hipStream_t stream) {
  const int32_t n16 = g.num_kv_heads * g.head_dim * 2 / 16;   // 16-B chunks per source row
  const int threads = 2 * n16 < 256 ? ((2 * n16 + 63) / 64) * 64 : 256;
  if (g.k_bs) {
    const size_t lds = sizeof(float) * 6 * (size_t)g.num_kv_heads;
    if (g.fp8_e5m2)
      hipLaunchKernelGGL(rc_scatter_fp8_block<true>, dim3((uint32_t)T), dim3(256), lds, stream, g,
                         (const uint4*)k_new, (const uint4*)v_new, slots, T, n16);
    else
      hipLaunchKernelGGL(rc_scatter_fp8_block<false>, dim3((uint32_t)T), dim3(256), lds, stream,
                         g, (const uint4*)k_new, (const uint4*)v_new, slots, T, n16);
    return hipGetLastError();
  }
  if (g.elem_bytes == 2)
    hipLaunchKernelGGL(rc_scatter_f16, dim3((uint32_t)T), dim3(threads), 0, stream, g,
                       (const uint4*)k_new, (const uint4*)v_new, slots, n16);
  else if (g.fp8_e5m2)
    hipLaunchKernelGGL(rc_scatter_fp8<true>, dim3((uint32_t)T), dim3(threads), 0, stream, g,
                       (const uint4*)k_new, (const uint4*)v_new, slots, n16);
  else
    hipLaunchKernelGGL(rc_scatter_fp8<false>, dim3((uint32_t)T), dim3(threads), 0, stream, g,
                       (const uint4*)k_new, (const uint4*)v_new, slots, n16);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const PoolGeom& g, const int64_t* pairs, int64_t n,
                              hipStream_t stream) {
  const int64_t block_bytes =
      (int64_t)g.block_size * g.num_kv_heads * g.head_dim * g.elem_bytes;
  const int64_t chunks = (block_bytes + 4095) / 4096;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)n, 2, (uint32_t)chunks), dim3(256), 0,
                     stream, g, pairs, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
