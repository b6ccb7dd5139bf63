// pa_decode.hip -- paged-attention decode on gfx950 (CDNA4).
//
// What is computed (the pages' definition): for sequence s and query head h,
// with KV head kh = h / gqa, walk the logical blocks of block_table[s]; every
// valid token t scores x_t = scale * q_h . k_t, and the output is
// sum_t e^{x_t - max} v_t / sum_t e^{x_t - max} ("KV Cache memory core",
// section 3 read path; "vLLM intro part 2", section 4.2 formulas).  Blocks are
// merged one after another with the online-softmax rule ("PagedAttention &
// vLLM", PagedAttention kernel: merge across blocks as FlashAttention does).
//
// How it maps to CDNA4:
//   * One workgroup serves one (sequence, KV head[, partition]) and ALL of the
//     gqa query heads that share that KV head, so every K/V byte is read from
//     HBM once.  Its waves take 16-token tiles round-robin.
//   * A tile's scores S[16 tokens x 16 heads] come from one 16x16x16 f16 MFMA
//     per 16 head dims: lane (row r, column c) loads 16 contiguous bytes of
//     token c's key (the A operand) and holds the same 16 bytes of query head
//     c (the B operand), so K feeds the matrix core straight from its 128-bit
//     load with no LDS staging.  Heads beyond gqa are zero columns.
//   * The MFMA result leaves lane (r, c) with the scores of tokens 4r..4r+3 for
//     head c -- exactly the A-operand layout P[head][token] of the next MFMA,
//     P.V.  V is loaded as 4 rows of D/16 contiguous elements per lane (token
//     4r+k, dims c*D/16..), then transposed inside the lane into B operands
//     V[4r..4r+3][dim] with byte permutes; D/16 MFMAs give the whole P.V.
//     P goes to the matrix core in binary16, V in binary16 (fp8 pools are
//     widened exactly first); accumulation is fp32.
//   * Softmax state per head: running max m (log2 units), per-lane partial
//     sums l, and the P.V accumulators.  The max is only moved (and l, acc
//     rescaled) when a tile's max exceeds it by more than 2^8, so P <= 256 always
//     fits binary16 and most tiles skip the rescale.
//   * Masked tokens (past the sequence or the partition) get score -inf by a
//     select and their V rows are zeroed by a select, so NaN in unused slots
//     never reaches a valid output.
//   * Split pass: each partition writes (m, l, o = acc / l) per head to the
//     workspace; lse_reduce merges them with weights l_p * 2^(m_p - M).
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for the running max
constexpr float kLazy = 8.0f;         // rescale only when the max grows by > 2^8

template <int BYTES> struct Vec;
template <> struct Vec<16> { typedef uint4 T; };
template <> struct Vec<8> { typedef uint2 T; };
template <> struct Vec<4> { typedef uint32_t T; };

template <int BYTES>
__device__ __forceinline__ void vec_words(const typename Vec<BYTES>::T& v, uint32_t* w) {
  if constexpr (BYTES == 16) { w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; }
  else if constexpr (BYTES == 8) { w[0] = v.x; w[1] = v.y; }
  else { w[0] = v; }
}

template <int BYTES>
__device__ __forceinline__ typename Vec<BYTES>::T vec_zero() {
  if constexpr (BYTES == 16) return make_uint4(0, 0, 0, 0);
  else if constexpr (BYTES == 8) return make_uint2(0, 0);
  else return 0u;
}

__device__ __forceinline__ half4_t halves_of(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(half4_t, make_uint2(lo, hi));
}

// 4 e4m3fn bytes -> 4 binary16 values (exact: every e4m3fn value is a binary16 value).
__device__ __forceinline__ half4_t fp8x4_to_half4(uint32_t w) {
  const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  const float4_t f = {a.x, a.y, b.x, b.y};
  return __builtin_convertvector(f, half4_t);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

template <int D, int BS, bool FP8, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  constexpr int E = FP8 ? 1 : 2;          // bytes per KV element
  constexpr int KCH = 16 / E;             // elements in a lane's 16-B key load
  constexpr int NKL = D * E / 64;         // 16-B key loads per lane per tile
  constexpr int GPL = KCH / 4;            // MFMA operand groups per key load
  constexpr int NQ = D / 16;              // QK MFMAs per tile (= q operands per lane)
  constexpr int DCH = D / 16;             // value dims per lane
  constexpr int VB = DCH * E;             // bytes per lane per value row
  typedef typename Vec<VB>::T VT;

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int r = lane >> 4;                // MFMA k-group / output row group
  const int c = lane & 15;                // MFMA column: token (K load) or head

  int bid = blockIdx.x;
  int part = 0;
  if constexpr (SPLIT) { part = bid % a.num_parts; bid /= a.num_parts; }
  const int kh = bid % a.num_kv_heads;
  const int s = bid / a.num_kv_heads;
  const int g = a.gqa;

  int len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
  int t_begin = 0, t_end = len;
  if constexpr (SPLIT) {
    t_begin = part * a.part_tokens;
    if (t_begin >= len) return;               // partition past the end: nothing to do
    t_end = min(len, t_begin + a.part_tokens);
  }
  const int j_begin = t_begin >> 4;           // 16-token tiles (partition sizes are x16)
  const int j_end = (t_end + 15) >> 4;        // only the last tile can be partial
  const int nblk = (len + BS - 1) / BS;       // valid table entries of this sequence
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;

  // ---- query operands: lane (r, c) holds head c, dims (cl*4*KCH + r*KCH + 4*grp ..+3)
  half4_t qop[NQ];
  {
    const _Float16* qrow = a.q + ((int64_t)s * a.num_q_heads + (int64_t)kh * g + c) * D;
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl) {
#pragma unroll
      for (int grp = 0; grp < GPL; ++grp) {
        const int d0 = cl * 4 * KCH + r * KCH + 4 * grp;
        half4_t v = {0, 0, 0, 0};
        if (c < g) v = *(const half4_t*)(qrow + d0);
        qop[cl * GPL + grp] = v;
      }
    }
  }

  // ---- addressing.  A tile's byte base inside a pool is uniform (block id from
  // the table, read with scalar loads one tile ahead); lanes add constant 32-bit
  // offsets: key token c at dims cl*4*KCH + r*KCH, value rows 4r+k at dims c*DCH.
  const int64_t head_off = (int64_t)kh * D * E;
  const int rs = a.row_stride;
  const int nb_m1 = a.num_blocks_m1;
  auto phys = [&](int lb) -> int64_t {
    lb = lb < nblk - 1 ? lb : nblk - 1;     // never read past the valid table entries
    int id = bt[lb];
    id = id < 0 ? 0 : (id > nb_m1 ? nb_m1 : id);
    return (int64_t)id * a.block_stride + head_off;
  };
  struct Ids { int64_t lo, hi; };           // bases of the tile's two halves (same if BS >= 16)
  auto tile_ids = [&](int jj) -> Ids {
    if constexpr (BS >= 16) {
      const int t = jj * 16;
      const int64_t b = phys(t / BS) + (int64_t)(t % BS) * rs;
      return {b, b};
    } else {
      return {phys(2 * jj), phys(2 * jj + 1)};
    }
  };
  // Lane offsets are constant across tiles; a tile's base is a scalar buffer
  // descriptor covering its 16 token rows, so loads carry no 64-bit per-lane
  // address math and an offset outside the rows would read zeros.
  const uint32_t koff = (uint32_t)((BS >= 16 ? c : (c & 7)) * rs + r * 16);
  const uint32_t voff = (uint32_t)((BS >= 16 ? 4 * r : ((4 * r) & 7)) * rs + c * VB);
  const int rows_bytes = 16 * rs;
  auto rsrc = [&](const char* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, rows_bytes, 0x00020000);
  };
  auto ld_k = [&](__amdgpu_buffer_rsrc_t R, int cl) -> uint4 {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, koff + cl * 64, 0, 0));
  };
  auto ld_v = [&](__amdgpu_buffer_rsrc_t R, int k) -> VT {
    if constexpr (VB == 16)
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, voff, k * rs, 0));
    else if constexpr (VB == 8)
      return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R, voff, k * rs, 0));
    else
      return __builtin_amdgcn_raw_buffer_load_b32(R, voff, k * rs, 0);
  };

  auto issue = [&](const Ids& ids, uint4* kr, VT* vr) {
    const __amdgpu_buffer_rsrc_t klo = rsrc(a.k + ids.lo), vlo = rsrc(a.v + ids.lo);
    if constexpr (BS >= 16) {
#pragma unroll
      for (int cl = 0; cl < NKL; ++cl) kr[cl] = ld_k(klo, cl);
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[k] = ld_v(vlo, k);
    } else {   // tokens 0-7 of the tile in block 2j, tokens 8-15 in block 2j+1
      const __amdgpu_buffer_rsrc_t khi = rsrc(a.k + ids.hi), vhi = rsrc(a.v + ids.hi);
#pragma unroll
      for (int cl = 0; cl < NKL; ++cl) kr[cl] = c < 8 ? ld_k(klo, cl) : ld_k(khi, cl);
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[k] = r < 2 ? ld_v(vlo, k) : ld_v(vhi, k);
    }
  };

  float m_run = kNegBig;     // per lane: head c (identical across the 4 rows)
  float l_run = 0.0f;        // per lane partial sum over the tokens it scored
  float4_t acc[DCH];
#pragma unroll
  for (int e = 0; e < DCH; ++e) acc[e] = (float4_t){0.f, 0.f, 0.f, 0.f};

  const bool head_ok = c < g;
  const float sc = a.score_scale;

  auto compute = [&](int j, const uint4* kr, const VT* vr_in) {
    // ---- scores S[token 4r+i][head c]
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl) {
      uint32_t w[4];
      vec_words<16>(kr[cl], w);
#pragma unroll
      for (int grp = 0; grp < GPL; ++grp) {
        half4_t kop;
        if constexpr (FP8) kop = fp8x4_to_half4(w[grp]);
        else kop = halves_of(w[2 * grp], w[2 * grp + 1]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(kop, qop[cl * GPL + grp], sacc, 0, 0, 0);
      }
    }
    const bool partial = j * 16 + 16 > t_end;   // wave-uniform
    const int t0 = j * 16 + 4 * r;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (t0 + i < t_end) ? sacc[i] * sc : -INFINITY;
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const bool grow = head_ok && (tmax > m_run + kLazy);
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * r + i);     // factor of head 4r+i
#pragma unroll
        for (int e = 0; e < DCH; ++e) acc[e][i] *= ai;
      }
      m_run = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    const float4_t pf = {p[0], p[1], p[2], p[3]};
    const half4_t pop = __builtin_convertvector(pf, half4_t);

    // ---- values: zero masked rows (last tile only), transpose in-lane, P.V
    uint32_t vw[4][VB / 4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vec_words<VB>(vr_in[k], vw[k]);
    if (partial) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool ok = t0 + k < t_end;
#pragma unroll
        for (int wi = 0; wi < VB / 4; ++wi) vw[k][wi] = ok ? vw[k][wi] : 0u;
      }
    }
    if constexpr (!FP8) {
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        const int wi = e >> 1, sh = (e & 1) * 16;
        const uint32_t h0 = (vw[0][wi] >> sh) & 0xFFFFu, h1 = (vw[1][wi] >> sh) & 0xFFFFu;
        const uint32_t h2 = (vw[2][wi] >> sh) & 0xFFFFu, h3 = (vw[3][wi] >> sh) & 0xFFFFu;
        const half4_t bop = halves_of(h0 | (h1 << 16), h2 | (h3 << 16));
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, bop, acc[e], 0, 0, 0);
      }
    } else {
      float vf[4][DCH];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int wi = 0; wi < VB / 4; ++wi) {
          const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[k][wi], false);
          const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[k][wi], true);
          vf[k][4 * wi + 0] = lo.x;
          vf[k][4 * wi + 1] = lo.y;
          vf[k][4 * wi + 2] = hi.x;
          vf[k][4 * wi + 3] = hi.y;
        }
      }
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        const float4_t f = {vf[0][e], vf[1][e], vf[2][e], vf[3][e]};
        const half4_t bop = __builtin_convertvector(f, half4_t);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, bop, acc[e], 0, 0, 0);
      }
    }
  };

  // ---- software pipeline: the loads of tile j+NW and the block ids of tile
  // j+2NW are in flight while tile j is computed; two register sets alternate.
  // The next tile's loads are issued unconditionally -- past the end of the
  // range they repeat the range's last tile, which is cache-resident -- so the
  // wave always waits for exactly one tile of outstanding loads.
  uint4 kA[NKL], kB[NKL];
  VT vA[4], vB[4];
  int j = j_begin + wid;
  if (j < j_end) {
    const int j_last = j_end - 1;
    issue(tile_ids(j), kA, vA);
    Ids ids_b = tile_ids(min(j + NW, j_last));
    for (;;) {
      issue(ids_b, kB, vB);
      const Ids ids_a = tile_ids(min(j + 2 * NW, j_last));
      compute(j, kA, vA);
      j += NW;
      if (j >= j_end) break;
      issue(ids_a, kA, vA);
      ids_b = tile_ids(min(j + 2 * NW, j_last));
      compute(j, kB, vB);
      j += NW;
      if (j >= j_end) break;
    }
  }

  // ---- per-wave totals: l summed over the 4 row groups
  float l_tot = xor_sum(l_run, 16);
  l_tot = xor_sum(l_tot, 32);

  // ---- merge the waves of the workgroup in LDS, then write
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_o[NW][16][D];
  if (r == 0) {
    sm_m[wid][c] = m_run;
    sm_l[wid][c] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * r + i;
    if (h < g) {
#pragma unroll
      for (int e = 0; e < DCH; ++e) sm_o[wid][h][c * DCH + e] = acc[e][i];
    }
  }
  __syncthreads();

  const int hq0 = kh * g;
  for (int idx = threadIdx.x; idx < g * D; idx += NW * 64) {
    const int h = idx / D, d = idx - (idx / D) * D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2f(sm_m[w][h] - M);
      L += f * sm_l[w][h];
      O += f * sm_o[w][h][d];
    }
    const float o = L > 0.f ? (O / L) * a.v_scale : 0.f;
    const int64_t row = (int64_t)s * a.num_q_heads + hq0 + h;
    if constexpr (SPLIT) {
      const int64_t prow = row * a.num_parts + part;
      a.ws_o[prow * D + d] = o;
      if (d == 0) a.ws_ml[prow] = make_float2(M, L);
    } else {
      a.out[row * D + d] = (_Float16)o;
    }
  }
}

// One workgroup per (sequence, query head): merge the partitions by log-sum-exp.
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - M), M = max_p m_p.
template <int D>
__global__ __launch_bounds__(256) void lse_reduce_kernel(DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int NG = NT / D;                  // thread groups sharing the partitions
  const int row_id = blockIdx.x;
  const int s = row_id / a.num_q_heads;
  int len = a.seq_lens[s];
  len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
  const int np = (len + a.part_tokens - 1) / a.part_tokens;
  const int64_t base = (int64_t)row_id * a.num_parts;
  const float2* ml = a.ws_ml + base;

  __shared__ float red[NT / 64];
  __shared__ float sm_part[NG][D];

  // M: max over partitions
  float mx = kNegBig;
  for (int p = threadIdx.x; p < np; p += NT) mx = fmaxf(mx, ml[p].x);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  // W: total weight
  float wsum = 0.f;
  for (int p = threadIdx.x; p < np; p += NT) {
    const float2 v = ml[p];
    wsum += v.y * exp2f(v.x - M);
  }
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wsum;
  __syncthreads();
  float W = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) W += red[w];

  // weighted sum of the partial outputs, groups of D threads over strided partitions
  const int d = threadIdx.x % D, grp = threadIdx.x / D;
  const float* o = a.ws_o + base * D + d;
  float acc = 0.f;
  int p = grp;
  for (; p + 3 * NG < np; p += 4 * NG) {
    const float2 v0 = ml[p], v1 = ml[p + NG], v2 = ml[p + 2 * NG], v3 = ml[p + 3 * NG];
    const float o0 = o[(int64_t)p * D], o1 = o[(int64_t)(p + NG) * D];
    const float o2 = o[(int64_t)(p + 2 * NG) * D], o3 = o[(int64_t)(p + 3 * NG) * D];
    acc += v0.y * exp2f(v0.x - M) * o0;
    acc += v1.y * exp2f(v1.x - M) * o1;
    acc += v2.y * exp2f(v2.x - M) * o2;
    acc += v3.y * exp2f(v3.x - M) * o3;
  }
  for (; p < np; p += NG) {
    const float2 v = ml[p];
    acc += v.y * exp2f(v.x - M) * o[(int64_t)p * D];
  }
  sm_part[grp][d] = acc;
  __syncthreads();
  if (grp == 0) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) tot += sm_part[q][d];
    a.out[(int64_t)row_id * D + d] = (_Float16)(W > 0.f ? tot / W : 0.f);
  }
}

constexpr int kWaves = 4;

template <int D, int BS, bool FP8>
hipError_t launch_typed(const DecodeArgs& a, int32_t num_seqs, bool split, hipStream_t stream) {
  const uint32_t units = (uint32_t)num_seqs * (uint32_t)a.num_kv_heads;
  if (split) {
    hipLaunchKernelGGL((decode_kernel<D, BS, FP8, kWaves, true>),
                       dim3(units * (uint32_t)a.num_parts), dim3(kWaves * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((lse_reduce_kernel<D>), dim3((uint32_t)num_seqs * (uint32_t)a.num_q_heads),
                       dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, BS, FP8, kWaves, false>), dim3(units), dim3(kWaves * 64),
                       0, stream, a);
  }
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_bs(const DecodeArgs& a, int32_t num_seqs, bool fp8, bool split,
                     hipStream_t stream) {
  return fp8 ? launch_typed<D, BS, true>(a, num_seqs, split, stream)
             : launch_typed<D, BS, false>(a, num_seqs, split, stream);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int32_t num_seqs, int32_t bs, bool fp8, bool split,
                    hipStream_t stream) {
  switch (bs) {
    case 8: return launch_bs<D, 8>(a, num_seqs, fp8, split, stream);
    case 16: return launch_bs<D, 16>(a, num_seqs, fp8, split, stream);
    case 32: return launch_bs<D, 32>(a, num_seqs, fp8, split, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int32_t num_seqs, int32_t head_dim,
                         int32_t block_size, bool fp8, bool split, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(a, num_seqs, block_size, fp8, split, stream);
  if (head_dim == 64) return launch_d<64>(a, num_seqs, block_size, fp8, split, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
