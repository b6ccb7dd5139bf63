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
//   * A workgroup owns one (sequence, KV head, tile of QT = floor(R / gqa)
//     new tokens); the query tiles of one (sequence, KV head) are placed on
//     one XCD so that they share its L2, and the pairs are spread over the
//     XCDs so that each gets an equal share of the work (pf_item).  Its R
//     query rows are (token, head) pairs, head fastest, so the gqa query
//     heads of the KV head share every K/V tile it stages.  R = waves x
//     groups x 16 rows: 4 x 2 x 16 = 128 at head_dim 64; at head_dim 128
//     4 x 3 x 16 = 192 on grids of several workgroups per CU, else 4 x 2 x 16
//     (prefill_plan); at head_dim 256 8 x 1 x 16 = 128, one workgroup per
//     CU (two groups per wave would not fit the registers).  A wave skips the
//     compute of every tile none of its rows can see (all positions after
//     its last row, or before its first row's window, or no row in use).
//   * K/V tiles of 32 positions are gathered through the block table into LDS
//     by whole 16-byte row chunks, XOR-swizzled by chunk so that the reads
//     below hit distinct banks.  fp16 pools (prefill_f16_kernel): straight from
//     HBM into LDS with the global-to-LDS load, three buffers deep, V kept
//     row-major and read with the LDS transpose read.  fp8 pools at head_dim
//     128 (the same kernel): the stored bytes take the same global-to-LDS
//     path into a three-slot staging ring, and each tile is widened exactly
//     into the binary16 layout one tile ahead of its compute (two buffers;
//     at head_dim 256 one buffer and two slots, widened between two barriers,
//     66 KB of LDS).
//     fp8 pools at head_dim 64 (prefill_kernel): loaded into registers one
//     tile ahead and widened on the way into LDS (two buffers), V stored
//     transposed.  One workgroup barrier per tile (two for fp8 pools at
//     head_dim 256, around the widening).
//   * Scores are computed transposed, S^T = K Q^T, with the 16x16x32 f16 MFMA:
//     K rows are the A operand (from LDS), the group's 16 query rows the B
//     operand (held in registers for the whole loop).  The K rows of a score
//     block are permuted so that lane (h, n) receives the scores of query row
//     n for positions 8h .. 8h + 7, which is the A-operand layout of O = P V
//     directly; V's B operand is read at the same positions.  Lane (h, n)
//     accumulates dims 16 nb + n of rows 4h .. 4h + 3.
//   * Online softmax per query row in log2 units; the running max moves only
//     when a tile exceeds it by more than 2^8 (P <= 256 fits binary16), which
//     a wave vote detects, so the cross-lane row max is formed only then.  The
//     causal mask is a select on position <= query position, applied only on
//     tiles that reach past the workgroup's first query position; positions
//     past the context are masked as well (their rows are finite: zeros or a
//     repeated in-context row).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#ifndef PA_PF_OCC
#define PA_PF_OCC 2           // fp16 prefill: workgroups per CU the registers are sized for
#endif
#ifndef PA_PF_NBUF
#define PA_PF_NBUF 3          // fp16 prefill: LDS tile buffers (tiles in flight + 1)
#endif
#ifndef PA_PF_W16
#define PA_PF_W16 4           // fp16 prefill at head_dim 128: waves per workgroup (4 or 8)
#endif
#ifndef PA_PF_W256
#define PA_PF_W256 8          // prefill at head_dim 256: waves per workgroup (4 or 8)
#endif
#ifndef PA_PF_F8W
#define PA_PF_F8W 1           // fp8 at head_dim 256: one binary16 buffer, two staging slots
#endif
#ifndef PA_PF_G256
#define PA_PF_G256 1          // fp16 prefill at head_dim 256: 16-row groups per wave
#endif

constexpr int kPfWaves = 4;
constexpr int kPfKeys = 32;        // key positions per tile

template <int D, int BS, int KV>
struct PfTile {
  static constexpr int E = KV ? 1 : 2;        // bytes per stored element
  static constexpr int CPR = D / 8;           // 8-element chunks per row
  static constexpr int KRB = D * 2;           // LDS bytes per K row (binary16)
  static constexpr int NL = kPfKeys * CPR / (kPfWaves * 64);  // K chunks per thread
  static constexpr int VK = NL;               // V positions per thread (same count)
  static constexpr int NST = D / 32;          // 32-dim MFMA steps of q . k
  static constexpr int NB = D / 16;           // P V column blocks
  static constexpr int TILE_K = kPfKeys * KRB;
  static constexpr int TILE_V = D * kPfKeys * 2;   // V^T: one 64-byte row per dim
  static constexpr int BUF = TILE_K + TILE_V;
  static_assert(NL >= 1 && NL <= 2, "tile and workgroup sizes");

  // K tile: row per position, 16-byte chunks XOR-swizzled by sw(key); sw maps
  // the 16 positions each score MFMA reads (see kpos) to 16 distinct values.
  __device__ static __forceinline__ int sw(int key) { return ((key >> 3) << 2) | (key & 3); }
  __device__ static __forceinline__ int kslot(int key, int c) {
    return key * KRB + ((c ^ (sw(key) & (CPR - 1))) << 4);
  }
  // V^T tile: for each chunk of 8 positions kc, a 16-byte slot per dim holding
  // those 8 positions in order.  The dim's slot is XOR-swizzled by dim / 8 so
  // that a write of one dim from 8 chunk-lanes and a read of 16 consecutive
  // dims both spread over all banks.
  __device__ static __forceinline__ int vslot(int dim, int kc) {
    return (kc * D + (dim ^ ((dim >> 3) & 7))) << 4;
  }
  // Row r of score block kb holds position kpos(kb, r); then the scores a
  // lane receives are positions 8h + 4kb + i, i.e. positions 8h .. 8h + 7 of
  // the P operand's k slots in order.
  __device__ static __forceinline__ int kpos(int kb, int r) {
    return 8 * (r >> 2) + 4 * kb + (r & 3);
  }
};

__device__ __forceinline__ uint4 widen8(uint2 w, int kv) {
  half4_t a, b;
  if (kv == 1) { a = e4m3x4_to_half4(w.x); b = e4m3x4_to_half4(w.y); }
  else { a = e5m2x4_to_half4(w.x); b = e5m2x4_to_half4(w.y); }
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// 8 fp8 bytes -> 8 binary16 values of (byte value * scale), each product
// formed in fp32 and rounded to nearest even once (fp8 pools with per-block
// scales).
__device__ __forceinline__ uint4 widen8_scaled(uint2 w, int kv, float scale) {
  float f[8];
  const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (kv == 1) {
      const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[q], false);
      const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[q], true);
      f[4 * q] = lo.x;
      f[4 * q + 1] = lo.y;
      f[4 * q + 2] = hi.x;
      f[4 * q + 3] = hi.y;
    } else {                                   // e5m2 byte b is binary16 bits b << 8
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f[4 * q + i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(((ws[q] >> (8 * i)) & 0xFFu) << 8));
    }
  }
  const float4_t a = {f[0] * scale, f[1] * scale, f[2] * scale, f[3] * scale};
  const float4_t b = {f[4] * scale, f[5] * scale, f[6] * scale, f[7] * scale};
  const uint2 ua = __builtin_bit_cast(uint2, __builtin_convertvector(a, half4_t));
  const uint2 ub = __builtin_bit_cast(uint2, __builtin_convertvector(b, half4_t));
  return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// lo/hi 16-bit halves of two words as one word: half `sel` of x low, of y high
__device__ __forceinline__ uint32_t pick_halves(uint32_t x, uint32_t y, int sel) {
  return sel ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
}

// Workgroups are dealt to the 8 XCDs round-robin.  Work items are the
// (sequence, KV head) pairs ordered by residue pair mod 8, each pair's query
// tiles longest first, and XCD x takes the x-th of 8 near-equal contiguous
// runs of that list.  An XCD thus holds whole pairs, whose query tiles share
// its L2, drawn from all sequences: with 8 KV heads XCD x runs KV head x of
// every sequence, so sequences of unequal context length load the XCDs
// equally (runs of whole sequences per XCD left the busiest XCD with 1.6x the
// mean work on a batch of chunks over mixed cached lengths).  Within a residue
// class the pairs go by descending causal work q_len (2 len - q_len), ties by
// index, so that each XCD starts its longest pairs first and ends on short
// ones; classes of more than kPfSortMax pairs keep index order.  The ranking
// is a strict total order, so any lengths give a permutation of the pairs.
constexpr int kPfSortMax = 256;

__device__ __forceinline__ void pf_item(const PrefillArgs& a, int* pair, int* qt) {
  __shared__ long long sm_work[kPfSortMax];
  __shared__ int sm_pick;
  const int wg = (int)blockIdx.x, nwg = (int)gridDim.x, num_qt = a.num_qt;
  const int num_pairs = a.num_seqs * a.num_kv_heads;
  const int xcd = wg & 7, per = nwg >> 3, rem = nwg & 7;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + (wg >> 3);
  const int rank = item / num_qt;                       // place of the pair in the list
  *qt = num_qt - 1 - (item - rank * num_qt);
  // the ceil((num_pairs - c) / 8) pairs of residue c follow those of residues < c
  int c = 0, base = 0;
  for (; c < 7; ++c) {
    const int n = (num_pairs - c + 7) >> 3;
    if (rank < base + n) break;
    base += n;
  }
  const int n_c = (num_pairs - c + 7) >> 3;             // pairs of residue c
  int j = rank - base;                                  // place within the class
  if (n_c <= kPfSortMax) {                              // uniform
    for (int t = threadIdx.x; t < n_c; t += blockDim.x) {
      const int s = (c + 8 * t) / a.num_kv_heads;
      const int len = a.seq_lens[s] > 0 ? a.seq_lens[s] : 0;
      int ql = a.q_start[s + 1] - a.q_start[s];
      ql = ql < 0 ? 0 : (ql < len ? ql : len);
      sm_work[t] = (long long)ql * (2LL * len - ql);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < n_c; t += blockDim.x) {
      const long long wt = sm_work[t];
      int r = 0;
      for (int i = 0; i < n_c; ++i) {
        const long long wi = sm_work[i];
        r += (wi > wt) | ((wi == wt) & (i < t));
      }
      if (r == j) sm_pick = t;
    }
    __syncthreads();
    j = sm_pick;
  }
  *pair = c + 8 * j;
}

template <int D, int BS, int KV>
__global__ __launch_bounds__(kPfWaves * 64, 2) void prefill_kernel(PrefillArgs a) {
  typedef PfTile<D, BS, KV> T;
  constexpr int E = T::E, CPR = T::CPR, NL = T::NL, VK = T::VK, NST = T::NST, NB = T::NB;
  // two buffers, each a K tile then a V^T tile
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BUF];
  lds_char* const lds0 = (lds_char*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = lane >> 4, n = lane & 15;
  int pair, qt;
  pf_item(a, &pair, &qt);
  const int s = pair / a.num_kv_heads;
  const int kh = pair - s * a.num_kv_heads;
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
  const int kv_end = ctx + t_hi;                  // positions kstart .. kv_end - 1 are read
  // sliding window: the workgroup's first row sees nothing before
  // ctx + q0 - window + 1; tiles start at that position's tile
  const int lo = a.window > 0 ? ctx + q0 - a.window + 1 : 0;
  const int kstart = lo > 0 ? (lo / kPfKeys) * kPfKeys : 0;
  const int kstart_pos = lo > 0 ? lo : 0;         // first position any row sees
  const uint32_t wu = a.window > 0 ? (uint32_t)a.window : 0x7FFFFFFFu;
  // tiles at kt need the mask when they reach past the first row (causal) or
  // begin before the last row's window
  auto needs_mask = [&](int kt) {
    return kt + kPfKeys - 1 > ctx + q0 || (a.window > 0 && kt < ctx + t_hi - a.window);
  };
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

  // ---- tile loader.  K: chunk i of a thread is row (tid + 256 i) / CPR,
  // chunk (tid + 256 i) % CPR.  V: positions VK * (tid / CPR) + u, chunk
  // tid % CPR, written transposed.  A wave's positions (4 or 8 consecutive,
  // aligned) lie in one block for every supported block size, so block ids are
  // scalar loads.  Raw bytes wait in registers while the previous tile is
  // computed; fp8 is widened when written to LDS.
  typedef typename std::conditional<E == 2, uint4, uint2>::type Raw;
  Raw kr[NL], vr[VK];
  const int64_t head_off = (int64_t)kh * D * E;
  // V loader lanes: wave w covers positions 8w .. 8w + 7 of the tile; lane
  // bits 0-1 (and bit 2 when VK == 1) pick the position, the rest the chunk.
  const int vkey = VK == 2 ? 8 * wid + 2 * (tid & 3) : 8 * wid + (tid & 7);
  const int vch = VK == 2 ? (lane >> 2) : (lane >> 3);
  // Positions below the window (their blocks may be released) or at or past
  // kv_end are not loaded: they stay zero in LDS and are masked.  A wave's
  // positions form one aligned group of G (4 or 8) inside one block.
  // G: the wave's group size (4 or 8 positions for K, 8 for V)
  auto row_addr = [&](int pos, int pos0, int G, int ch, bool& ok) -> int64_t {
    ok = false;
    if (pos0 >= kv_end || pos0 + G - 1 < kstart_pos) return 0;
    int blk = bt[(pos0 > kstart_pos ? pos0 : kstart_pos) / BS];
    blk = blk < 0 ? 0 : (blk > a.num_blocks_m1 ? a.num_blocks_m1 : blk);
    ok = pos >= kstart_pos && pos < kv_end;
    return (int64_t)blk * a.block_stride + (int64_t)(pos % BS) * a.row_stride + head_off +
           ch * 8 * E;
  };
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + kPfWaves * 64 * i;
      const int pos = kt + idx / CPR;
      const int pos0 = uni(kt + (kPfWaves * 64 * i + 64 * wid) / CPR);
      bool ok;
      const int64_t off = row_addr(pos, pos0, 64 / CPR, idx % CPR, ok);
      kr[i] = ok ? *(const Raw*)(a.k + off) : Raw{};
    }
    const int vbase = kt + vkey;
    const int vpos0 = uni(kt + 8 * wid);
#pragma unroll
    for (int u = 0; u < VK; ++u) {
      bool ok;
      const int64_t off = row_addr(vbase + u, vpos0, 8, vch, ok);
      vr[u] = ok ? *(const Raw*)(a.v + off) : Raw{};
    }
  };
  auto widen = [&](const Raw& r) -> uint4 {
    if constexpr (E == 2) return r;
    else return widen8(r, KV);
  };
  auto store_tile = [&](lds_char* ks) {
    lds_char* vs = ks + T::TILE_K;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + kPfWaves * 64 * i;
      *(lds_u32x4*)(ks + T::kslot(idx / CPR, idx % CPR)) = __builtin_bit_cast(u32x4_t, widen(kr[i]));
    }
    const int ch = vch;
    uint4 vw[VK];
#pragma unroll
    for (int u = 0; u < VK; ++u) vw[u] = widen(vr[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = T::vslot(8 * ch + e, vkey >> 3) + (vkey & 7) * 2;
      if constexpr (VK == 2) {
        *(__attribute__((address_space(3))) uint32_t*)(vs + off) =
            pick_halves(word_of(vw[0], e >> 1), word_of(vw[1], e >> 1), e & 1);
      } else {
        const uint32_t wv = word_of(vw[0], e >> 1);
        *(__attribute__((address_space(3))) uint16_t*)(vs + off) =
            (uint16_t)((e & 1) ? (wv >> 16) : (wv & 0xFFFFu));
      }
    }
  };

  float4_t acc[2][NB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[c][nb] = {0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegBig, kNegBig}, l_run[2] = {0.f, 0.f};
  const float sc = a.k_hs ? a.score_scale * a.k_hs[kh] : a.score_scale;
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;

  // One tile of math on LDS buffer (ks, vs) for positions kt .. kt + 31.
  auto compute = [&](const lds_char* ks, const lds_char* vs, int kt, bool mask) {
    // scores S^T for both row groups; block kb row r is position kpos(kb, r)
    float4_t sa[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      half8_t kop[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st)
        kop[st] = __builtin_bit_cast(
            half8_t, *(const lds_u32x4*)(ks + T::kslot(T::kpos(kb, n), 4 * st + h)));
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        sa[c][kb] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NST; ++st)
          sa[c][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[st], qop[c][st], sa[c][kb], 0, 0, 0);
      }
    }
    // V^T operands: block nb column n is dim 16 nb + n, k slots are positions 8h .. 8h + 7
    half8_t vop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      vop[nb] = __builtin_bit_cast(half8_t, *(const lds_u32x4*)(vs + T::vslot(16 * nb + n, h)));

#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // raw scores of positions kt + 8h + k; the scale (> 0) is applied in the exponent's fma
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * kb + i] = sa[c][kb][i];
      if (mask) {            // uniform branch: only edge tiles pay for the mask
        // position kt + 8h + k counts when 0 <= qpos - position < window
        const int base = qpos[c] - kt - 8 * h;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = (uint32_t)(base - k) < wu ? x[k] : -INFINITY;
      }
      // The running max only has to move when some score exceeds it by more
      // than 2^8, so each lane tests its own 8 scores and the wave votes; the
      // row max across the 4 lanes of a row is formed only when it moves.
      float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))) * sc;
      if (__any(tmax > m_run[c] + kLazy)) {
        tmax = xor_max(tmax, 16);
        tmax = xor_max(tmax, 32);
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
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sc, -m_run[c]));
      l_run[c] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const float4_t p0 = {p[0], p[1], p[2], p[3]}, p1 = {p[4], p[5], p[6], p[7]};
      const half4_t h0 = __builtin_convertvector(p0, half4_t);
      const half4_t h1 = __builtin_convertvector(p1, half4_t);
      const half8_t pop = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, vop[nb], acc[c][nb], 0, 0, 0);
    }
  };

  load_tile(kstart);
  store_tile(lds0);
  __syncthreads();
  int buf = 0;
  for (int kt = kstart; kt < kv_end; kt += kPfKeys) {
    // One barrier per tile: the next tile goes to the other buffer, whose last
    // readers finished before the barrier that ended the previous iteration.
    const bool more = kt + kPfKeys < kv_end;
    if (more) load_tile(kt + kPfKeys);
    const lds_char* ks = lds0 + buf * T::BUF;
    compute(ks, ks + T::TILE_K, kt, needs_mask(kt));
    if (more) store_tile(lds0 + (buf ^ 1) * T::BUF);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: lane (h, n) holds rows 4h + i, dims 16 nb + n
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
      const float f = v_scale / li;
      _Float16* op = a.out + ((int64_t)row * a.num_q_heads + kh * g + j) * D + n;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) op[16 * nb] = (_Float16)(acc[c][nb][i] * f);
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 pools: K/V tiles go from HBM straight into LDS (the 16-byte
// global-to-LDS load, lane i filling bytes 16 i .. 16 i + 15 of a wave's 1 KB),
// three LDS buffers deep, so two tiles are in flight while one is computed and
// no registers hold staged data.  V stays row-major in LDS and the P V operand
// is read with the LDS transpose read (within each 16-lane group, result lane
// l, element k is halfword l % 4 of what source lane 4k + l / 4 points at), so
// nothing is transposed by hand.  LDS reads are issued as inline asm: the
// compiler would otherwise drain every outstanding global-to-LDS load before
// each LDS read; here the waits are explicit, and only for the tile in use.

typedef short short4_t __attribute__((ext_vector_type(4)));

// waves per workgroup of prefill_f16_kernel at head_dim d for pool code kvc:
// eight at head_dim 256 (every pool format), four at head_dim 64 and for fp8
// pools at head_dim 128 (whose 4 KiB byte tiles fill four waves' loads)
constexpr int pf_waves(int d, int kvc) {
  return d > 128 ? PA_PF_W256 : (kvc == 0 && d == 128 ? PA_PF_W16 : kPfWaves);
}

template <int D, int W = kPfWaves, int GG = 2>
struct PfDma {
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int RB = 2 * D;                        // bytes per row
  static constexpr int RPI = 1024 / RB;                   // rows per wave load
  static constexpr int NI = kPfKeys / RPI / W;            // loads per wave per tile, each of K and V
  static constexpr int TILE = kPfKeys * RB;
  static constexpr int BUF = 2 * TILE;                    // K tile then V tile
  static constexpr int DPT = 2 * NI;                      // loads per thread per tile
  // 16-row query groups per wave and workgroups per CU: two waves per SIMD
  // (registers for 2 or 3 groups at head_dim 128: 185 and 244 VGPRs; at head_dim
  // 256 one group per wave keeps head_dim 128's count, two would need 452
  // registers per lane and one wave per SIMD)
  static constexpr int G = D > 128 ? PA_PF_G256 : GG;
  static constexpr int OCC = (D > 128 && G > 1) || W >= 8 ? 1 : PA_PF_OCC;
  static constexpr bool SHARED_SIMD = W * OCC >= 8;       // two or more waves per SIMD
  // head_dim 256: two buffers of 32 KiB
  static constexpr int NBUF = D > 128 ? 2 : PA_PF_NBUF;
  static constexpr int NST = D / 32;
  static constexpr int NB = D / 16;
  static_assert(NI >= 1 && NBUF >= 2 && NBUF <= 4 && NBUF * BUF <= 65536, "tile shape");
  // K rows: chunk swizzle that gives the 16 rows one score MFMA reads
  // (positions 8 (n / 4) + 4 kb + n % 4, n = 0..15) distinct chunks.
  __device__ static __forceinline__ int ksw(int key) {
    return (((key >> 3) << 2) | (key & 3)) & (CPR - 1);
  }
  // V rows: the 4 rows one transpose read spans (positions differing in
  // bits 0-1) start their 32-byte dim windows on different banks, and rows
  // 8 apart (lanes 16-31 against lanes 0-15 of the same read) use the other
  // half of a 256-byte bank row.
  __device__ static __forceinline__ int vsw(int key) {
    return (2 * (key & 3) + 8 * ((key >> 3) & 1)) & (CPR - 1);
  }
};

template <int OFF>
__device__ __forceinline__ half8_t lds_b128(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return __builtin_bit_cast(half8_t, v);
}

template <int OFF>
__device__ __forceinline__ half4_t lds_tr16(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
  return __builtin_bit_cast(half4_t, v);
}

// Wait until at most N LDS / scalar-memory operations are outstanding, and
// make the values read so far depend on that wait.
template <int N, typename V>
__device__ __forceinline__ void lgkm_wait(V& v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "i"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait_all_regs() {
  asm volatile("s_waitcnt lgkmcnt(%0)" : : "i"(N) : "memory");
}

// Maxima of scores without the quieting of signalling NaNs that fmaxf adds
// to each MFMA result (one extra instruction per input); the scores here are
// never NaN (masked entries are -inf, loaded rows are finite).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int OFF>
__device__ __forceinline__ void lds_w128(uint32_t addr, uint4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2"
               : : "v"(addr), "v"(__builtin_bit_cast(u32x4_t, v)), "i"(OFF) : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  // vmcnt(N), expcnt and lgkmcnt unchanged (gfx9 encoding: vmcnt low bits
  // 3:0 and high bits 15:14, expcnt 6:4, lgkmcnt 11:8)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// KVC: pool format, 0 binary16; 1 e4m3fn or 2 e5m2 (head_dim 128, 256); 3, 4:
// e4m3fn, e5m2 with one scale per (block, KV head), applied as the tile is
// widened (the scales of the tile's blocks are read with scalar loads one
// tile ahead).  fp8 tiles
// go by the global-to-LDS load into a three-slot staging ring as stored
// (row-major bytes), and each is widened exactly into the binary16 tile layout
// below one tile ahead of its compute, two binary16 buffers deep; the math is
// the same for every format.
template <int D, int BS, int KVC, int GG>
__global__ __launch_bounds__(pf_waves(D, KVC) * 64, (PfDma<D, pf_waves(D, KVC), GG>::OCC)) void prefill_f16_kernel(
    PrefillArgs a, const int32_t* __restrict__ tables, const float* __restrict__ kbs,
    const float* __restrict__ vbs) {
  constexpr int KV = KVC >= 3 ? KVC - 2 : KVC;  // element format
  constexpr bool BSC = KVC >= 3;                // per-block scales
  constexpr int NW = pf_waves(D, KVC);
  typedef PfDma<D, NW, GG> T;
  constexpr int RB = T::RB, NST = T::NST, NB = T::NB, G = T::G;
  // raised issue priority for the score MFMAs where two waves share a SIMD,
  // except for binary16 pools at head_dim 256 (measured 2% slower with it;
  // fp8 pools there 5% faster)
  constexpr bool kPrio = T::SHARED_SIMD && (D <= 128 || KV != 0);
  static_assert(KV == 0 || D >= 128, "fp8 tiles are staged for head_dim 128 and 256");
  // fp8 at head_dim 256: one binary16 buffer and two staging slots (66 KB;
  // measured faster than two buffers and three slots)
  constexpr bool F8W = KV != 0 && D > 128 && PA_PF_F8W;
  constexpr int NBUF = KV ? (F8W ? 1 : 2) : T::NBUF;   // binary16 tile buffers
  constexpr int E = KV ? 1 : 2;                 // bytes per stored element
  constexpr int SRB = D * E;                    // stored bytes per row
  constexpr int SCPR = SRB / 16;                // 16-byte chunks per stored row
  constexpr int SRPI = 1024 / SRB;              // rows per wave load
  constexpr int NI = kPfKeys / SRPI / NW;       // loads per wave per tile, each of K and V
  constexpr int STILE = kPfKeys * SRB;          // fp8 staging: K tile then V tile per slot
  constexpr int NRAW = KV ? (F8W ? 2 : 3) : 0;
  // stored 16-byte chunks of the K tile (and of the V tile) each thread widens
  constexpr int WCH = KV ? kPfKeys * SCPR / (NW * 64) : 1;
  static_assert(NI >= 1 && (KV == 0 || WCH * NW * 64 == kPfKeys * SCPR), "load shape");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * T::BUF + NRAW * 2 * STILE];
  lds_char* const lds0 = (lds_char*)smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds0;

  const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
  const int h = lane >> 4, n = lane & 15;
  int pair, qt;
  pf_item(a, &pair, &qt);
  const int s = pair / a.num_kv_heads;
  const int kh = pair - s * a.num_kv_heads;
  const int g = a.gqa, QT = a.tile_tokens;

  const int qs0 = a.q_start[s];
  const int cap = a.max_blocks * BS;
  const int len = clamp_len(a.seq_lens[s], cap);
  int q_len = clamp_len(a.q_start[s + 1] - qs0, a.max_q_len);
  q_len = q_len < len ? q_len : len;
  const int q0 = qt * QT;
  if (q0 >= q_len) return;
  const int ctx = len - q_len;
  const int t_hi = q_len < q0 + QT ? q_len : q0 + QT;
  const int kv_end = ctx + t_hi;
  const int ntiles = (kv_end + kPfKeys - 1) / kPfKeys;
  const int lo = a.window > 0 ? ctx + q0 - a.window + 1 : 0;
  const int t0 = lo > 0 ? lo / kPfKeys : 0;     // first tile the sliding window reaches
  const int lo_c = lo > 0 ? lo : 0;             // first position any row sees
  const uint32_t wu = a.window > 0 ? (uint32_t)a.window : 0x7FFFFFFFu;
  auto needs_mask = [&](int kt) {
    return kt + kPfKeys - 1 > ctx + q0 || (a.window > 0 && kt < ctx + t_hi - a.window);
  };
  const int32_t* bt = tables + (int64_t)s * a.max_blocks;
  // Positions of this wave's first and last query rows in use.  A tile whose
  // positions all follow the last (causal mask) or all precede the first
  // one's window is skipped by the wave: its weights would all be exact
  // zeros.  A wave with no row in use (a partial last query tile) skips
  // every tile; it still takes part in the loads and barriers.
  int w_first, w_last;
  {
    const int tf = (16 * G * wid) / g;
    int tl = (16 * G * (wid + 1) - 1) / g;
    tl = tl < QT - 1 ? tl : QT - 1;
    tl = tl < q_len - q0 - 1 ? tl : q_len - q0 - 1;
    w_first = uni(ctx + q0 + tf);
    w_last = uni(tf <= tl ? ctx + q0 + tl : -1);
  }
  auto wave_sees = [&](int kt) {
    return kt <= w_last && (a.window <= 0 || kt + kPfKeys - 1 >= w_first - a.window + 1);
  };

  half8_t qop[G][NST];
  int qpos[G];
#pragma unroll
  for (int c = 0; c < G; ++c) {
    const int r = 16 * G * wid + 16 * c + n;
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

  // ---- loads of tile t into buffer t % 3: wave w fills rows (w NI + i) RPI ..
  // of K and of V; lane -> row r0 + lane / CPR, LDS chunk lane % CPR, which
  // holds the row's chunk (lane % CPR) ^ swizzle.  Positions at or past kv_end
  // repeat position kv_end - 1, positions before the sliding window repeat its
  // first position (finite data; masked out of every score).
  const char* const kbase = a.k + (int64_t)kh * D * E;
  const char* const vbase = a.v + (int64_t)kh * D * E;
  // Block ids of the NI load groups of the next tile to issue, read one tile
  // ahead (and range-clamped only when used) so that the scalar loads'
  // latency passes behind a tile's compute.  A group's RPI rows lie in one
  // block (RPI divides block_size), also when its positions are clamped.
  auto group_block = [&](int t, int i) {
    const int r0 = (wid * NI + i) * SRPI;
    const int pr0 = t * kPfKeys + r0 < lo_c ? lo_c : t * kPfKeys + r0;
    const int pu = uni(pr0 < kv_end ? pr0 : kv_end - 1);
    return bt[(uint32_t)pu / BS];
  };
  int next_blk[NI];
  // In-block byte offsets of this lane's K and V chunks for a tile with no
  // clamped position (tile start a multiple of 32, so the row in the block is
  // r mod block_size, plus the tile's offset in the block when blocks hold
  // more than one tile).
  // (Staged fp8 rows are not swizzled: the widening places the chunks.)
  auto chunk_of = [&](int r, int pch, bool v) {
    return KV ? pch : (pch ^ (v ? T::vsw(r) : T::ksw(r)));
  };
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = (wid * NI + i) * SRPI + lane / SCPR, pch = lane % SCPR;
    const uint32_t in_blk = ((uint32_t)r & (BS - 1)) * (uint32_t)a.row_stride;
    koff[i] = in_blk + ((uint32_t)chunk_of(r, pch, false) << 4);
    voff[i] = in_blk + ((uint32_t)chunk_of(r, pch, true) << 4);
  }
  auto issue = [&](int t, int b) {
    const int kt = t * kPfKeys;
    const bool whole = kt >= lo_c && kt + kPfKeys <= kv_end;      // uniform
    const int64_t tile_in_blk = BS > kPfKeys ? (int64_t)(kt & (BS - 1)) * a.row_stride : 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = (wid * NI + i) * SRPI;
      const int raw = next_blk[i];
      const int blk = raw < 0 ? 0 : (raw > a.num_blocks_m1 ? a.num_blocks_m1 : raw);
      // block base (uniform) plus a 32-bit per-lane offset inside the block
      const int64_t blk_off = (int64_t)blk * a.block_stride;
      uint32_t ko = koff[i], vo = voff[i];
      int64_t base = blk_off + tile_in_blk;
      if (!whole) {
        // positions are clamped into [lo_c, kv_end - 1]: outside rows repeat
        // an in-window row (finite data, masked), never a released block
        const int r = r0 + lane / SCPR, pch = lane % SCPR;
        const int pr = kt + r < lo_c ? lo_c : kt + r;
        const int pos = pr < kv_end ? pr : kv_end - 1;
        const uint32_t in_blk = ((uint32_t)pos & (BS - 1)) * (uint32_t)a.row_stride;
        ko = in_blk + ((uint32_t)chunk_of(r, pch, false) << 4);
        vo = in_blk + ((uint32_t)chunk_of(r, pch, true) << 4);
        base = blk_off;
      }
      // binary16: tile buffer b; fp8: staging slot b
      lds_char* kdst = KV ? lds0 + NBUF * T::BUF + b * 2 * STILE + r0 * SRB
                          : lds0 + b * T::BUF + r0 * RB;
      lds_char* vdst = kdst + (KV ? STILE : T::TILE);
      __builtin_amdgcn_global_load_lds((const void*)(kbase + base + ko),
                                       (__attribute__((address_space(3))) void*)kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + base + vo),
                                       (__attribute__((address_space(3))) void*)vdst, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) next_blk[i] = group_block(t + 1, i);
  };

  // fp8: widen staging slot `slot` (tile t) into binary16 buffer `fb`.  Thread
  // tid takes stored chunks ch = tid + 256 w of the K tile and of the V tile
  // (row ch / SCPR, dims 16 (ch % SCPR) .. + 15, as the global-to-LDS load laid
  // them out) and writes binary16 chunks 2c and 2c + 1 of that row at their
  // swizzled slots.
  // Rows of positions outside [lo_c, kv_end) (loaded as repeats of an
  // in-range row) are written as zeros, so that a repeated V row holding an
  // infinity (e5m2 has them) meets its zero weight as 0 * 0, not 0 * inf.
  // per-block scales of tile t's blocks (at most 4: block_size >= 8), for K
  // and V; positions outside the rows in use read an in-use block's entry
  constexpr int NBT = BS >= kPfKeys ? 1 : kPfKeys / BS;
  struct TSc { float k[NBT], v[NBT]; };
  auto tile_scales = [&](int t) {
    TSc r;
    if constexpr (BSC) {
      const int lb_lo = lo_c / BS, lb_hi = (kv_end - 1) / BS;
#pragma unroll
      for (int i = 0; i < NBT; ++i) {
        int lb = (t * kPfKeys) / BS + i;
        lb = lb < lb_lo ? lb_lo : (lb > lb_hi ? lb_hi : lb);
        int id = bt[lb];
        id = id < 0 ? 0 : (id > a.num_blocks_m1 ? a.num_blocks_m1 : id);
        r.k[i] = kbs[(int64_t)id * a.num_kv_heads + kh];
        r.v[i] = vbs[(int64_t)id * a.num_kv_heads + kh];
      }
    }
    return r;
  };
  auto widen_tile = [&](int slot, int fb, int t, const TSc& ts) {
    if constexpr (KV != 0) {
#pragma unroll
     for (int w = 0; w < WCH; ++w) {
      const int ch = tid + NW * 64 * w;
      const uint32_t src = lds_base + NBUF * T::BUF + slot * 2 * STILE + ch * 16;
      const int key = ch / SCPR, c = ch % SCPR;
      const int pos = t * kPfKeys + key;
      const bool in_range = pos >= lo_c && pos < kv_end;
      half8_t rk = lds_b128<0>(src), rv = lds_b128<STILE>(src);
      lgkm_wait<0>(rk);
      lgkm_wait<0>(rv);
      const uint4 rw[2] = {__builtin_bit_cast(uint4, rk), __builtin_bit_cast(uint4, rv)};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        uint4 lo, hi;
        if constexpr (BSC) {
          float sc = q ? ts.v[0] : ts.k[0];
#pragma unroll
          for (int i = 1; i < NBT; ++i) sc = key >= i * BS ? (q ? ts.v[i] : ts.k[i]) : sc;
          lo = in_range ? widen8_scaled(make_uint2(rw[q].x, rw[q].y), KV, sc) : z;
          hi = in_range ? widen8_scaled(make_uint2(rw[q].z, rw[q].w), KV, sc) : z;
        } else {
          lo = in_range ? widen8(make_uint2(rw[q].x, rw[q].y), KV) : z;
          hi = in_range ? widen8(make_uint2(rw[q].z, rw[q].w), KV) : z;
        }
        const int sw = q ? T::vsw(key) : T::ksw(key);
        const uint32_t row = lds_base + fb * T::BUF + q * T::TILE + key * RB;
        lds_w128<0>(row + (((2 * c) ^ sw) << 4), lo);
        lds_w128<0>(row + (((2 * c + 1) ^ sw) << 4), hi);
      }
     }
    }
  };

  // ---- per-lane LDS read addresses (buffer 0; buffers differ by an immediate)
  // K: position kpos(0, n) = 8 (n / 4) + (n % 4), chunk (4 st + h) ^ ksw = (4 st + h) ^ n
  uint32_t kaddr[NST];
  {
    const int key = 8 * (n >> 2) + (n & 3);
#pragma unroll
    for (int st = 0; st < NST; ++st)
      kaddr[st] = lds_base + key * RB + (((4 * st + h) ^ T::ksw(key)) << 4);
  }
  // V (transpose read): source lane n = 4k + m reads position 8h + k (+4 for the
  // second half), dims 16 nb + 4m .. +3
  uint32_t vaddr[NB];
  {
    const int k = n >> 2, m = n & 3;
    const int key = 8 * h + k;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      vaddr[nb] = lds_base + T::TILE + key * RB + (((2 * nb + (m >> 1)) ^ T::vsw(key)) << 4) +
                  8 * (m & 1);
  }

  float4_t acc[G][NB];
#pragma unroll
  for (int c = 0; c < G; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[c][nb] = {0.f, 0.f, 0.f, 0.f};
  // Row sums: one more 16x16x32 MFMA per group and tile forms P times a
  // column of ones, the binary16 weights the P V product uses, summed in fp32
  // and laid out like the accumulators (rows 4h .. 4h + 3 of lane (h, n)).
  float m_run[G];
  float4_t l_acc[G];
#pragma unroll
  for (int c = 0; c < G; ++c) {
    m_run[c] = kNegBig;
    l_acc[c] = {0.f, 0.f, 0.f, 0.f};
  }
  const float sc = a.k_hs ? a.score_scale * a.k_hs[kh] : a.score_scale;
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;

  auto compute = [&](uint32_t bo, int kt, bool mask) {
    half8_t kop[2][NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      kop[0][st] = lds_b128<0>(kaddr[st] + bo);
      kop[1][st] = lds_b128<4 * RB>(kaddr[st] + bo);
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      lgkm_wait<0>(kop[0][st]);
      lgkm_wait<0>(kop[1][st]);
    }
    // Two waves share each SIMD.  The wave issuing its score MFMAs takes
    // issue priority over the other wave (usually in its softmax), so the
    // matrix core is kept fed and the VALU work fills in behind it (measured
    // 1.5-3.5% faster at head_dim 128; see kPrio for head_dim 256).
    float4_t sa[G][2];
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < G; ++c) {
        sa[c][kb] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NST; ++st)
          sa[c][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][st], qop[c][st], sa[c][kb], 0, 0, 0);
      }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    // V reads go out after the score MFMAs (the K operands are dead by then)
    // and land while the first group's softmax runs
    half4_t vh[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      vh[nb][0] = lds_tr16<0>(vaddr[nb] + bo);
      vh[nb][1] = lds_tr16<4 * RB>(vaddr[nb] + bo);
    }
    half8_t vop[NB];
#pragma unroll
    for (int c = 0; c < G; ++c) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * kb + i] = sa[c][kb][i];
      if (mask) {
        const int base = qpos[c] - kt - 8 * h;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = (uint32_t)(base - k) < wu ? x[k] : -INFINITY;
      }
      float tmax = max3_raw(max3_raw(x[0], x[1], x[2]), max3_raw(x[3], x[4], x[5]),
                            max3_raw(x[6], x[7], x[7])) * sc;
      if (__any(tmax > m_run[c] + kLazy)) {
        tmax = xor_max(tmax, 16);
        tmax = xor_max(tmax, 32);
        const float m_new = fmaxf(m_run[c], tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_new);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * h + i);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[c][nb][i] *= ai;
          l_acc[c][i] *= ai;
        }
        m_run[c] = m_new;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sc, -m_run[c]));
      const float4_t p0 = {p[0], p[1], p[2], p[3]}, p1 = {p[4], p[5], p[6], p[7]};
      const half4_t h0 = __builtin_convertvector(p0, half4_t);
      const half4_t h1 = __builtin_convertvector(p1, half4_t);
      const half8_t pop = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      if (c == 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          lgkm_wait<0>(vh[nb][0]);
          lgkm_wait<0>(vh[nb][1]);
          vop[nb] = {vh[nb][0][0], vh[nb][0][1], vh[nb][0][2], vh[nb][0][3],
                     vh[nb][1][0], vh[nb][1][1], vh[nb][1][2], vh[nb][1][3]};
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, vop[nb], acc[c][nb], 0, 0, 0);
      {
        const _Float16 o = (_Float16)1.f;
        const half8_t ones = {o, o, o, o, o, o, o, o};
        l_acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, ones, l_acc[c], 0, 0, 0);
      }
    }
  };

  // tile t (buffer b = t % 3): wait for its loads (tile t + 1 may still be in
  // flight), barrier (every wave's loads of tile t have landed and every wave
  // is done with tile t - 1, whose buffer tile t + 2 reuses), issue tile t + 2,
  // compute tile t.
#pragma unroll
  for (int i = 0; i < NI; ++i) next_blk[i] = group_block(t0, i);
  if constexpr (F8W) {
    // fp8, head_dim 256: staging slot of tile t is (t - t0) % 2, one binary16
    // buffer.  At tile t: wait for its bytes (tile t + 1's may stay in
    // flight), barrier (every wave is done computing tile t - 1), widen it,
    // barrier (every wave is done widening: its slot is free), issue tile
    // t + 2 into that slot, compute tile t.
    constexpr int DPT = 2 * NI;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (t0 + u < ntiles) issue(t0 + u, u);
    int rs = 0;
    TSc ts_next = tile_scales(t0);
    for (int t = t0; t < ntiles; ++t) {
      const TSc ts = ts_next;
      if (BSC && t + 1 < ntiles) ts_next = tile_scales(t + 1);
      if (ntiles - 1 - t >= 1) vm_wait<DPT>();
      else vm_wait<0>();
      lgkm_wait_all_regs<0>();
      __builtin_amdgcn_s_barrier();
      widen_tile(rs, 0, t, ts);
      lgkm_wait_all_regs<0>();
      __builtin_amdgcn_s_barrier();
      if (t + 2 < ntiles) issue(t + 2, rs);
      const int kt = t * kPfKeys;
      if (wave_sees(kt)) compute(0u, kt, needs_mask(kt));
      rs ^= 1;
    }
  } else if constexpr (KV != 0) {
    // fp8: staging slot of tile t is (t - t0) % 3, binary16 buffer (t - t0) % 2.
    // At tile t: wait for tile t + 1's bytes (t + 2's may stay in flight),
    // barrier (tile t is widened, every wave is done with tile t - 1's buffer
    // and with tile t's staging slot), issue tile t + 3 into that slot, widen
    // tile t + 1, compute tile t.
    constexpr int DPT = 2 * NI;
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (t0 + u < ntiles) issue(t0 + u, u);
    if (ntiles - t0 >= 3) vm_wait<2 * DPT>();
    else if (ntiles - t0 == 2) vm_wait<DPT>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    widen_tile(0, 0, t0, tile_scales(t0));
    TSc ts_next = tile_scales(t0 + 1 < ntiles ? t0 + 1 : t0);
    int rs = 0, fb = 0;
    for (int t = t0; t < ntiles; ++t) {
      const TSc ts = ts_next;
      if (BSC && t + 2 < ntiles) ts_next = tile_scales(t + 2);
      if (ntiles - 1 - t >= 2) vm_wait<DPT>();
      else vm_wait<0>();
      lgkm_wait_all_regs<0>();
      __builtin_amdgcn_s_barrier();
      if (t + 3 < ntiles) issue(t + 3, rs);
      const int rn = rs == 2 ? 0 : rs + 1;
      if (t + 1 < ntiles) widen_tile(rn, fb ^ 1, t + 1, ts);
      const int kt = t * kPfKeys;
      if (wave_sees(kt)) compute((uint32_t)(fb * T::BUF), kt, needs_mask(kt));
      rs = rn;
      fb ^= 1;
    }
  }
  constexpr int NB_ = NBUF;
  if constexpr (KV == 0) {
#pragma unroll
  for (int u = 0; u < NB_ - 1; ++u)
    if (t0 + u < ntiles) issue(t0 + u, u);
  int b = 0;
  for (int t = t0; t < ntiles; ++t) {
    // tiles t + 1 .. t + NBUF - 2 may stay in flight
    const int later = ntiles - 1 - t;
    if (NB_ >= 4 && later >= 2) vm_wait<(NB_ >= 4 ? 2 : 1) * T::DPT>();
    else if (NB_ >= 3 && later >= 1) vm_wait<T::DPT>();
    else vm_wait<0>();
    lgkm_wait_all_regs<0>();
    __builtin_amdgcn_s_barrier();
    if (t + NB_ - 1 < ntiles) issue(t + NB_ - 1, b == 0 ? NB_ - 1 : b - 1);
    const int kt = t * kPfKeys;
    if (wave_sees(kt)) compute((uint32_t)(b * T::BUF), kt, needs_mask(kt));
    b = b == NB_ - 1 ? 0 : b + 1;
  }
  }

#pragma unroll
  for (int c = 0; c < G; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = l_acc[c][i];
      const int r = 16 * G * wid + 16 * c + 4 * h + i;
      const int t = r / g, j = r - t * g;
      const int row = qs0 + q0 + t;
      if (!(t < QT && q0 + t < q_len && row >= 0 && row < a.total_q)) continue;
      const float f = v_scale / li;
      _Float16* op = a.out + ((int64_t)row * a.num_q_heads + kh * g + j) * D + n;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) op[16 * nb] = (_Float16)(acc[c][nb][i] * f);
    }
  }
}

template <int D, int BS, int GG>
hipError_t launch_pf_g(const PrefillArgs& a, int kv, hipStream_t stream) {
  const dim3 grid((uint32_t)a.num_seqs * (uint32_t)a.num_kv_heads * (uint32_t)a.num_qt);
  const dim3 block(kPfWaves * 64);
  if (kv == 0) {
    hipLaunchKernelGGL((prefill_f16_kernel<D, BS, 0, GG>), grid, dim3(pf_waves(D, 0) * 64), 0,
                       stream, a, a.block_tables, a.k_bs, a.v_bs);
    return hipGetLastError();
  }
  if constexpr (D >= 128) {             // fp8 pools at head_dim 128, 256: staged bytes, widened in LDS
#define PA_PF_KV(C)                                                                            \
  if (kv == C)                                                                                 \
    hipLaunchKernelGGL((prefill_f16_kernel<D, BS, C, GG>), grid, dim3(pf_waves(D, C) * 64), 0, \
                       stream, a, a.block_tables, a.k_bs, a.v_bs);
    PA_PF_KV(1) else PA_PF_KV(2) else PA_PF_KV(3) else PA_PF_KV(4) else return hipErrorInvalidValue;
#undef PA_PF_KV
    return hipGetLastError();
  }
  if constexpr (D == 64) {              // fp8 pools at head_dim 64: register-staged kernel
    if (kv == 1) hipLaunchKernelGGL((prefill_kernel<D, BS, 1>), grid, block, 0, stream, a);
    else if (kv == 2) hipLaunchKernelGGL((prefill_kernel<D, BS, 2>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <int D, int BS>
hipError_t launch_pf_bs(const PrefillArgs& a, int kv, hipStream_t stream) {
  if constexpr (D == 128) {
    if (a.groups == 3) return launch_pf_g<D, BS, 3>(a, kv, stream);
    if (a.groups == 2) return launch_pf_g<D, BS, 2>(a, kv, stream);
    return hipErrorInvalidValue;
  } else {
    constexpr int G = D > 128 ? PfDma<256>::G : 2;
    if (a.groups != G) return hipErrorInvalidValue;
    return launch_pf_g<D, BS, G>(a, kv, stream);
  }
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

// Three 16-row groups per wave at head_dim 128 (192 rows per workgroup) read
// each staged K/V tile for 1.5x the rows of two, which measured 5% faster on
// fp16 pools and 13% on fp8 ones when the grid holds several workgroups per
// CU; a grid that fits the CUs about once (a batch of short chunks) ends with
// the length of its longest workgroup, where two groups per wave are faster
// (22% on 32 prompts of 50 new tokens over a 2,000-token cached prefix).  The
// host sees only the largest new-token count, so the choice is: three groups
// when that grid has at least four workgroups per CU and pads the largest
// sequence's new tokens by at most 1/16 more than two groups would.
PrefillPlan prefill_plan(int head_dim, int kv_code, int gqa, int64_t pairs, int max_q_len,
                         int force) {
  constexpr int64_t kWorkgroupsPerPass = 256 * 2;   // MI355X: 256 CUs, two workgroups each
  const int w = pf_waves(head_dim, kv_code);
  PrefillPlan p;
  if (head_dim != 128) {
    p.groups = head_dim > 128 ? PfDma<256>::G : 2;
  } else {
    const int64_t t2 = w * 32 / gqa, t3 = w * 48 / gqa;
    const int64_t n3 = (max_q_len + t3 - 1) / t3, n2 = (max_q_len + t2 - 1) / t2;
    const bool many = pairs * n3 >= 2 * kWorkgroupsPerPass;
    p.groups = force == 2 || force == 3 ? force
                                        : (many && 16 * n3 * t3 <= 17 * n2 * t2 ? 3 : 2);
  }
  p.tile_tokens = w * 16 * p.groups / gqa;
  return p;
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t head_dim, int32_t block_size, int kv,
                          hipStream_t stream) {
  if (head_dim == 128) return launch_pf_d<128>(a, block_size, kv, stream);
  if (head_dim == 64) return launch_pf_d<64>(a, block_size, kv, stream);
  if (head_dim == 256) return launch_pf_d<256>(a, block_size, kv, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
