// pa_prefill.hip -- prefill / chunked-prefill attention over the paged cache
// on gfx950 (CDNA4).
//
// What is computed: a prompt's new tokens are first written into their blocks
// in bulk (pa_reshape_and_cache), then each of them attends to itself and to
// every earlier position of its sequence through the block table ("vLLM intro
// part 2", section 3: prefill writes the KV in bulk, attention reads it through
// the block table).  With a prefix-cache hit only the uncached tail is new
// (same page, section 6 example), so in general sequence s brings q_len new
// tokens at positions seq_len - q_len .. seq_len - 1 and new token i sees
// positions 0 .. seq_len - q_len + i.  Scores, softmax and the weighted sum are
// the decode formula of the same pages, one query position at a time.
//
// Work decomposition and data flow:
//   * A workgroup owns one (sequence, KV head, tile of QT = floor(128 / gqa)
//     new tokens).  Its 128 query rows are (token, head) pairs, head fastest,
//     so the gqa query heads of the KV head share every K/V tile it stages.
//     4 waves x 2 groups x 16 rows.
//   * K/V tiles of 32 positions are gathered through the block table into LDS
//     by whole 16-byte row chunks (fp8 pools are widened exactly to binary16 on
//     the way).  Rows are XOR-swizzled by chunk so that the column-wise reads
//     below hit distinct banks.  The next tile's global loads are issued before
//     the current tile is computed.
//   * Scores are computed transposed, S^T = K Q^T, with the 16x16x32 f16 MFMA:
//     K rows are the A operand (from LDS), the group's 16 query rows the B
//     operand (held in registers for the whole loop).  Lane (h, n) then holds
//     the scores of query row n for key positions 4h + i and 16 + 4h + i,
//     which is directly the A-operand layout of O = P V with the key order
//     permuted; V's B operand is read from LDS at the same permuted positions
//     (8 positions x 8 dims per lane) and transposed in registers.  P V block
//     nb covers dims {8n + nb} (head_dim 128) so a lane's output dims are
//     contiguous and each row is written with one 16-byte store.
//   * Online softmax per query row in log2 units; the running max moves only
//     when a tile exceeds it by more than 2^8 (P <= 256 fits binary16).  The
//     causal mask is a select on position <= query position; positions past
//     the context are never loaded (zeros in LDS) and are masked as well.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 128;       // query rows per workgroup
constexpr int kPfKeys = 32;        // key positions per tile

template <int D, int BS, int KV>
struct PfTile {
  static constexpr int E = KV ? 1 : 2;        // bytes per stored element
  static constexpr int CPR = D / 8;           // 8-element chunks per row
  static constexpr int RB = D * 2;            // LDS bytes per row (binary16)
  static constexpr int NL = kPfKeys * CPR / (kPfWaves * 64);  // chunks per thread
  static constexpr int NST = D / 32;          // 32-dim MFMA steps of q . k
  static constexpr int NB = D / 16;           // P V column blocks
  static constexpr int VB = NB * 2;           // V bytes per lane per key row
  static constexpr int TILE = kPfKeys * RB;   // LDS bytes per K (or V) tile
  static_assert(NL >= 1, "tile smaller than the workgroup");

  // byte offset of chunk c of row r inside a tile
  __device__ static __forceinline__ int slot(int r, int c) {
    return r * RB + ((c ^ (r % CPR)) << 4);
  }
};

__device__ __forceinline__ uint4 widen8(uint2 w, int kv) {
  half4_t a, b;
  if (kv == 1) { a = e4m3x4_to_half4(w.x); b = e4m3x4_to_half4(w.y); }
  else { a = e5m2x4_to_half4(w.x); b = e5m2x4_to_half4(w.y); }
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// lo/hi 16-bit halves of two words as one word: half `sel` of x low, of y high
__device__ __forceinline__ uint32_t pick_halves(uint32_t x, uint32_t y, int sel) {
  return sel ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
}

template <int D, int BS, int KV>
__global__ __launch_bounds__(kPfWaves * 64, 2) void prefill_kernel(PrefillArgs a) {
  typedef PfTile<D, BS, KV> T;
  constexpr int E = T::E, CPR = T::CPR, NL = T::NL, NST = T::NST, NB = T::NB;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::TILE];
  lds_char* ks = (lds_char*)smem;
  lds_char* vs = ks + T::TILE;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = lane >> 4, n = lane & 15;
  const int S = a.num_seqs;
  const int s = blockIdx.x % S;
  const int qt = a.num_qt - 1 - (int)(blockIdx.x / S);   // longest tiles first
  const int kh = blockIdx.y;
  const int g = a.gqa, QT = a.tile_tokens;

  const int qs0 = a.q_start[s];
  const int cap = a.max_blocks * BS;
  const int len = clamp_len(a.seq_lens[s], cap);
  int q_len = clamp_len(a.q_start[s + 1] - qs0, a.max_q_len);
  q_len = q_len < len ? q_len : len;
  const int q0 = qt * QT;
  if (q0 >= q_len) return;                       // uniform: whole workgroup
  const int ctx = len - q_len;
  const int t_hi = q_len < q0 + QT ? q_len : q0 + QT;
  const int kv_end = ctx + t_hi;                  // positions 0 .. kv_end - 1 are read
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;

  // ---- query rows: this lane's B-operand row in each group, and its position
  half8_t qop[2][NST];
  int qpos[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 32 * wid + 16 * c + n;
    const int t = r / g, j = r - t * g;
    const int row = qs0 + q0 + t;
    const bool ok = t < QT && q0 + t < q_len && row >= 0 && row < a.total_q;
    qpos[c] = ok ? ctx + q0 + t : -1;
    const _Float16* qp = a.q + ((int64_t)(ok ? row : 0) * a.num_q_heads + kh * g + j) * D;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      uint4 w = ok ? *(const uint4*)(qp + 32 * st + 8 * h) : make_uint4(0, 0, 0, 0);
      qop[c][st] = __builtin_bit_cast(half8_t, w);
    }
  }

  // ---- tile loader: thread chunk i covers row (tid + 256 i) / CPR, chunk % CPR.
  // Raw pool bytes are held in registers while the previous tile is computed;
  // fp8 is widened only when the tile is written to LDS.
  typedef typename std::conditional<E == 2, uint4, uint2>::type Raw;
  Raw kr[NL], vr[NL];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + kPfWaves * 64 * i;
      const int key = idx / CPR, ch = idx % CPR;
      const int pos = kt + key;
      // A wave's 64 chunks are 64 / CPR consecutive positions starting at a
      // multiple of 64 / CPR (4 or 8), so they share one block for every
      // supported block size: the block id is a scalar load.
      const int pos0 = uni(kt + (kPfWaves * 64 * i + 64 * wid) / CPR);
      kr[i] = Raw{};
      vr[i] = Raw{};
      if (pos0 < kv_end) {
        int blk = bt[pos0 / BS];
        blk = blk < 0 ? 0 : (blk > a.num_blocks_m1 ? a.num_blocks_m1 : blk);
        if (pos < kv_end) {
          const int64_t off = (int64_t)blk * a.block_stride +
                              (int64_t)(pos % BS) * a.row_stride + (int64_t)kh * D * E +
                              ch * 8 * E;
          kr[i] = *(const Raw*)(a.k + off);
          vr[i] = *(const Raw*)(a.v + off);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + kPfWaves * 64 * i;
      const int key = idx / CPR, ch = idx % CPR;
      uint4 kw, vw;
      if constexpr (E == 2) {
        kw = kr[i];
        vw = vr[i];
      } else {
        kw = widen8(kr[i], KV);
        vw = widen8(vr[i], KV);
      }
      *(lds_u32x4*)(ks + T::slot(key, ch)) = __builtin_bit_cast(u32x4_t, kw);
      *(lds_u32x4*)(vs + T::slot(key, ch)) = __builtin_bit_cast(u32x4_t, vw);
    }
  };

  float4_t acc[2][NB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[c][nb] = {0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegBig, kNegBig}, l_run[2] = {0.f, 0.f};
  const float sc = a.score_scale;

  load_tile(0);
  for (int kt = 0; kt < kv_end; kt += kPfKeys) {
    __syncthreads();                 // the previous tile's LDS reads are done
    store_tile();
    __syncthreads();
    if (kt + kPfKeys < kv_end) load_tile(kt + kPfKeys);

    // scores S^T for both row groups; K operand: key 16 kb + n, dims 32 st + 8 h .. + 7
    float4_t sa[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      half8_t kop[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st)
        kop[st] = __builtin_bit_cast(
            half8_t, *(const lds_u32x4*)(ks + T::slot(16 * kb + n, 4 * st + h)));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        sa[c][kb] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NST; ++st)
          sa[c][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[st], qop[c][st], sa[c][kb], 0, 0, 0);
      }
    }
    // V operands: positions key(kk) = kk < 4 ? 4h + kk : 16 + 4h + kk - 4, the
    // lane's NB dims starting at NB * n, transposed so that operand nb holds
    // dim NB * n + nb of the 8 positions
    uint32_t vw[8][NB / 2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int key = kk < 4 ? 4 * h + kk : 12 + 4 * h + kk;
      const int byte = n * T::VB;
      const int off = key * T::RB + (((byte >> 4) ^ (key % CPR)) << 4) + (byte & 15);
      if constexpr (NB == 8) {
        const u32x4_t w = *(const lds_u32x4*)(vs + off);
        vw[kk][0] = w.x; vw[kk][1] = w.y; vw[kk][2] = w.z; vw[kk][3] = w.w;
      } else {
        const u32x2_t w = *(const lds_u32x2*)(vs + off);
        vw[kk][0] = w.x; vw[kk][1] = w.y;
      }
    }
    half8_t vop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint4 w;
      w.x = pick_halves(vw[0][nb >> 1], vw[1][nb >> 1], nb & 1);
      w.y = pick_halves(vw[2][nb >> 1], vw[3][nb >> 1], nb & 1);
      w.z = pick_halves(vw[4][nb >> 1], vw[5][nb >> 1], nb & 1);
      w.w = pick_halves(vw[6][nb >> 1], vw[7][nb >> 1], nb & 1);
      vop[nb] = __builtin_bit_cast(half8_t, w);
    }

#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[4 * kb + i] = (kt + 16 * kb + 4 * h + i <= qpos[c]) ? sa[c][kb][i] * sc : -INFINITY;
      float tmax = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
      tmax = xor_max(tmax, 16);
      tmax = xor_max(tmax, 32);
      const bool grow = tmax > m_run[c] + kLazy;
      if (__any(grow)) {
        const float m_new = fmaxf(m_run[c], tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_new);
        l_run[c] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * h + i);    // factor of row 4h + i
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[c][nb][i] *= ai;
        }
        m_run[c] = m_new;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_run[c]);
      l_run[c] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const float4_t p0 = {p[0], p[1], p[2], p[3]}, p1 = {p[4], p[5], p[6], p[7]};
      const half4_t h0 = __builtin_convertvector(p0, half4_t);
      const half4_t h1 = __builtin_convertvector(p1, half4_t);
      const half8_t pop = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, vop[nb], acc[c][nb], 0, 0, 0);
    }
  }

  // ---- epilogue: lane (h, n) holds rows 4h + i, dims NB * n .. NB * n + NB - 1
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float lt = xor_sum(l_run[c], 16);
    lt = xor_sum(lt, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(lt, 4 * h + i);
      const int r = 32 * wid + 16 * c + 4 * h + i;
      const int t = r / g, j = r - t * g;
      const int row = qs0 + q0 + t;
      if (!(t < QT && q0 + t < q_len && row >= 0 && row < a.total_q)) continue;
      const float f = a.v_scale / li;
      _Float16 o[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = (_Float16)(acc[c][nb][i] * f);
      _Float16* op = a.out + ((int64_t)row * a.num_q_heads + kh * g + j) * D + NB * n;
      if constexpr (NB == 8) {
        *(uint4*)op = __builtin_bit_cast(uint4, o);
      } else {
        *(uint2*)op = __builtin_bit_cast(uint2, o);
      }
    }
  }
}

template <int D, int BS>
hipError_t launch_pf_bs(const PrefillArgs& a, int kv, hipStream_t stream) {
  const dim3 grid((uint32_t)a.num_seqs * (uint32_t)a.num_qt, (uint32_t)a.num_kv_heads);
  const dim3 block(kPfWaves * 64);
  switch (kv) {
    case 0: hipLaunchKernelGGL((prefill_kernel<D, BS, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((prefill_kernel<D, BS, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, BS, 2>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_pf_d(const PrefillArgs& a, int bs, int kv, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_pf_bs<D, 8>(a, kv, stream);
    case 16: return launch_pf_bs<D, 16>(a, kv, stream);
    case 32: return launch_pf_bs<D, 32>(a, kv, stream);
    case 64: return launch_pf_bs<D, 64>(a, kv, stream);
    case 128: return launch_pf_bs<D, 128>(a, kv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_rows_per_workgroup() { return kPfRows; }

hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, int32_t block_size, int kv,
                          hipStream_t stream) {
  if (head_dim == 128) return launch_pf_d<128>(a, block_size, kv, stream);
  if (head_dim == 64) return launch_pf_d<64>(a, block_size, kv, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
