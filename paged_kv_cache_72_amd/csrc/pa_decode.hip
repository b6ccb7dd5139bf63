// pa_decode.hip -- paged-attention decode on gfx950 (CDNA4).
//
// What is computed (the pages' definition): for sequence s and query head h,
// with KV head kh = h / gqa, walk the logical blocks of block_table[s]; every
// valid token t scores x_t = scale * q_h . k_t, and the output is
// sum_t e^{x_t - max} v_t / sum_t e^{x_t - max} ("KV Cache memory core",
// section 3 read path; "vLLM intro part 2", section 4.2 formulas).  Blocks are
// merged one after another with the online-softmax rule ("PagedAttention &
// vLLM", PagedAttention kernel: merge across blocks as FlashAttention does),
// and separately computed pieces of one context are merged by the same rule
// in log-sum-exp form.
//
// The tile engine (one copy of the math, used by every schedule):
//   * Work unit: 16 consecutive tokens of one (sequence, KV head) pair, for
//     ALL gqa query heads of that KV head, so every K/V byte leaves HBM once.
//   * Loads: every K and V load instruction covers whole token rows of the
//     head (64 lanes x 16 B = four 256-byte rows for fp16 head_dim 128), which
//     the memory system serves far better than pieces of many rows.  A tile's
//     base is a scalar buffer descriptor over its 16 rows; lanes add constant
//     offsets.  Block ids are read with scalar loads one tile ahead, and the
//     next tile's loads are always in flight while the current one is computed.
//     Single-reader pools are read with the streaming cache policy.
//   * Scores S[16 tokens x 16 heads]: one 16x16x16 f16 MFMA per 16 head dims
//     with K as the A operand (one token per lane) and the query heads as B
//     (heads beyond gqa are zero columns).  The row-wise K tile goes through a
//     per-wave, XOR-swizzled LDS buffer to reach that layout; the token order
//     is permuted so that score lane (r, c) holds tokens r, r+4, r+8, r+12 of
//     head c -- the A-operand layout of the P.V MFMA and the rows that value
//     load k = 0..3 gave the same lane.  V is transposed inside the lane into
//     B operands; D/16 MFMAs give P.V.  P and V enter the matrix core as
//     binary16 (fp8 pools are widened exactly first: e4m3fn through the fp32
//     converter, e5m2 by placing the byte above 8 zero bits), accumulation is
//     fp32.
//   * Softmax state per head: running max m (log2 units), per-lane partial sum
//     l and the P.V accumulators.  The max moves (and l, acc are rescaled) only
//     when a tile's max exceeds it by more than 2^8, so P <= 256 fits binary16.
//   * Masked tokens get score -inf by a select and their V rows are zeroed by a
//     select, so NaN in unused slots never reaches a valid output.
//
// Schedules:
//   * single pass   -- one workgroup per (sequence, KV head); its waves take
//                      tiles round-robin and merge in LDS.
//   * split pass    -- one workgroup per (sequence, KV head, partition) writing
//                      (m, l, o) partials, then lse_reduce_kernel.
//   * flat (default)-- the list of all (sequence, 16-token tile) units is cut
//                      into equal ranges; each range is walked by one wave per
//                      KV head, side by side, so long and short contexts cost
//                      the same per wave and the heads of a block are read
//                      together.  Sequences inside one range are written
//                      directly; a sequence cut by range boundaries leaves one
//                      partial per range, merged by flat_merge_heads_kernel in
//                      range order (deterministic).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Tuning knobs (compile time): waves per decode workgroup, and the occupancy
// the register allocator is asked to reach (waves per SIMD).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 3
#endif
#ifndef PA_FLAT_WAVES
#define PA_FLAT_WAVES PA_DECODE_WAVES
#endif
#ifndef PA_FLAT_WAVES_PER_EU
#define PA_FLAT_WAVES_PER_EU 2
#endif
#ifndef PA_VMEM_TABLES
#define PA_VMEM_TABLES 0      // block-table entries by vector loads (1) or scalar loads (0)
#endif
#ifndef PA_GROUP_WAVES_PER_EU
#define PA_GROUP_WAVES_PER_EU 2
#endif
#ifndef PA_GROUP_WAVES
#define PA_GROUP_WAVES 4      // grouped schedule: waves per workgroup
#endif
#ifndef PA_GROUP_NT
#define PA_GROUP_NT 1         // grouped schedule: streaming K/V loads whatever the pool flag
#endif
#ifndef PA_GROUP_EXTRA_LDS
#define PA_GROUP_EXTRA_LDS 0  // bytes of dynamic LDS per workgroup (limits residency)
#endif
#ifndef PA_FLAT_STAGES
#define PA_FLAT_STAGES 2      // flat schedule: tiles in flight per wave, plus one
#endif

template <int BYTES> struct Vec;
template <> struct Vec<16> { typedef uint4 T; };
struct u32x8 { uint4 lo, hi; };               // a lane's 32-byte value row (head_dim 256)
template <> struct Vec<32> { typedef u32x8 T; };
template <> struct Vec<8> { typedef uint2 T; };
template <> struct Vec<4> { typedef uint32_t T; };

template <int BYTES>
__device__ __forceinline__ void vec_words(const typename Vec<BYTES>::T& v, uint32_t* w) {
  if constexpr (BYTES == 32) {
    w[0] = v.lo.x; w[1] = v.lo.y; w[2] = v.lo.z; w[3] = v.lo.w;
    w[4] = v.hi.x; w[5] = v.hi.y; w[6] = v.hi.z; w[7] = v.hi.w;
  } else if constexpr (BYTES == 16) { w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; }
  else if constexpr (BYTES == 8) { w[0] = v.x; w[1] = v.y; }
  else { w[0] = v; }
}

// Byte b of words w0, w1 as two binary16 values (e5m2 widening of one value
// dim for two tokens): low half from w0, high half from w1.
__device__ __forceinline__ uint32_t e5m2_pair(uint32_t w0, uint32_t w1, int b) {
  return (((w0 >> (8 * b)) & 0xFFu) << 8) | (((w1 >> (8 * b)) & 0xFFu) << 24);
}

// First position the query of a length-len context sees (sliding window).
__device__ __forceinline__ int win_start(int len, int window) {
  return (window > 0 && len > window) ? len - window : 0;
}

// Byte bases, inside the pools, of a tile's two halves (equal when block_size >= 16).
// live = 0 marks a tile past the end of what a wave computes: its loads are
// still issued (the same instruction stream every iteration keeps the
// compiler's wait counts tight) but through an empty buffer descriptor, so
// they return zeros without touching memory.
struct Ids {
  int64_t lo, hi;
  int live;
  float ks0, ks1, vs0, vs1;   // per-block scales of the two halves (formats 3, 4)
};

// One (sequence, KV head) pair as the loads see it.
struct PairRef {
  const int32_t* bt;   // block table row
  int nblk;            // valid table entries
  int len;             // context length
  int64_t head_off;    // byte offset of the KV head inside a token row
};

// NT: K/V tiles are read with the streaming (non-temporal) cache policy, for
// pools whose blocks each belong to one sequence; blocks shared by several
// sequences of the batch are read with the default policy so that they stay
// cached for the other readers.  KV: element format of the pools, 0 binary16,
// 1 e4m3fn, 2 e5m2; 3 and 4: e4m3fn and e5m2 with one scale per (block, KV
// head), read with the block ids one tile ahead: the key scale multiplies the
// tile's scores (per half tile at block_size 8) in fp32, and the values are
// widened to fp32, scaled and rounded to binary16 for the P.V product.
template <int D, int BS, int KV, bool NT>
struct Engine {
  static constexpr int FMT = KV >= 3 ? KV - 2 : KV;   // 0 binary16, 1 e4m3fn, 2 e5m2
  static constexpr bool BSC = KV >= 3;         // scales per (block, KV head)
  static constexpr int CPOL = NT ? 2 : 0;      // cache-policy operand of the tile loads
  static constexpr int E = FMT ? 1 : 2;        // bytes per KV element
  static constexpr int KCH = 16 / E;           // elements in a 16-B key chunk
  static constexpr int NKL = D * E / 64;       // 16-B key loads per lane per tile
  static constexpr int GPL = KCH / 4;          // MFMA operand groups per key chunk
  static constexpr int NQ = D / 16;            // QK MFMAs per tile (q operands per lane)
  static constexpr int DCH = D / 16;           // value dims per lane
  static constexpr int VB = DCH * E;           // bytes per lane per value row
  static constexpr int RB = D * E;             // bytes of one KV head's row of one token
  static constexpr int CPR = RB / 16;          // 16-B chunks per row
  static constexpr int RPI = 64 / CPR;         // whole rows covered by one 64-lane key load
  static constexpr int PER = RB >= 256 ? 1 : 256 / RB;   // rows per 256-B LDS bank period
  static constexpr int KST = 16 * RB;          // bytes of one key tile staged in LDS
  typedef typename Vec<VB>::T VT;

  int r, c, g, rs, nb_m1;
  int t0, ch;                                  // this lane's row and chunk in a key load
  uint32_t koff, voff;
  int64_t block_stride;
  const char* kp;
  const char* vp;
  lds_char* kst;                               // this wave's key tile in LDS
  float sc;
  const float* kbs;                            // per-block scales of this wave's KV head
  const float* vbs;                            //   (stride hkv), formats 3 and 4
  int hkv;

  half4_t qop[NQ];
  float m_run, l_run;
  float4_t acc[DCH];

  // kstage: KST bytes of LDS owned by this wave alone.
  __device__ __forceinline__ void init(const DecodeArgs& a, int lane, lds_char* kstage) {
    r = lane >> 4;
    c = lane & 15;
    g = a.gqa;
    rs = a.row_stride;
    nb_m1 = a.num_blocks_m1;
    block_stride = a.block_stride;
    kp = a.k;
    vp = a.v;
    kst = kstage;
    sc = a.score_scale;
    kbs = vbs = nullptr;
    hkv = a.num_kv_heads;
    t0 = lane / CPR;
    ch = lane % CPR;
    koff = (uint32_t)((BS >= 16 || RPI <= 8 ? t0 : (t0 & 7)) * rs + ch * 16);
    voff = (uint32_t)(r * rs + c * VB);
  }

  // The per-block scale arrays ([num_blocks][Hkv]; kernel arguments, so that
  // their entries are read with scalar loads) at KV head kh.
  __device__ __forceinline__ void set_block_scales(const float* k, const float* v, int kh) {
    if constexpr (BSC) {
      kbs = k + kh;
      vbs = v + kh;
    }
  }

  // LDS chunk slot of chunk `k` of token row t: XOR-swizzled so that both the
  // row-wise writes and the column-wise operand reads hit distinct banks.
  __device__ __forceinline__ static int kslot(int t, int k) {
    return t * RB + ((k ^ ((t / PER) % CPR)) << 4);
  }

  __device__ __forceinline__ void reset() {
    m_run = kNegBig;
    l_run = 0.0f;
#pragma unroll
    for (int e = 0; e < DCH; ++e) acc[e] = (float4_t){0.f, 0.f, 0.f, 0.f};
  }

  // q rows of the pair's gqa heads, starting at head 0 of the group.
  // Lane (r, c) holds head c at dims cl*4*KCH + r*KCH + 4*grp .. +3.  The
  // rows are read through a buffer descriptor sized to the group, so lanes of
  // heads c >= gqa read zeros and the address stays in scalar registers.
  __device__ __forceinline__ void load_q_into(half4_t* dst, const _Float16* qrow0) const {
    const __amdgpu_buffer_rsrc_t R =
        __builtin_amdgcn_make_buffer_rsrc((void*)qrow0, (short)0, g * D * 2, 0x00020000);
    const uint32_t qoff = (uint32_t)((c * D + r * KCH) * 2);
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl) {
#pragma unroll
      for (int grp = 0; grp < GPL; ++grp)
        dst[cl * GPL + grp] = __builtin_bit_cast(
            half4_t, __builtin_amdgcn_raw_buffer_load_b64(R, qoff, (cl * 4 * KCH + 4 * grp) * 2, 0));
    }
  }
  __device__ __forceinline__ void load_q(const _Float16* qrow0) { load_q_into(qop, qrow0); }
  // Query operands when every column has its own row: lane (r, c) reads
  // qrow, the row of column c (nullptr: a padding column, zeros), at the
  // dims load_q_into gives it.
  __device__ __forceinline__ void load_q_rows_into(half4_t* dst, const _Float16* qrow) const {
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl) {
#pragma unroll
      for (int grp = 0; grp < GPL; ++grp)
        dst[cl * GPL + grp] =
            qrow ? *(const half4_t*)(qrow + cl * 4 * KCH + r * KCH + 4 * grp) : (half4_t){};
    }
  }
  __device__ __forceinline__ void load_q_rows(const _Float16* qrow) { load_q_rows_into(qop, qrow); }
  __device__ __forceinline__ void take_q(const half4_t* src) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) qop[i] = src[i];
  }

  __device__ __forceinline__ int64_t phys(const PairRef& p, int lb) const {
    return (int64_t)id_of(p, lb) * block_stride + p.head_off;
  }

  __device__ __forceinline__ int id_of(const PairRef& p, int lb) const {
    lb = lb < p.nblk - 1 ? lb : p.nblk - 1;      // never past the valid table entries
#if PA_VMEM_TABLES
    // a vector load (all lanes the same address): its wait counts with the
    // K/V loads, so LDS accesses in between do not wait for it
    const __amdgpu_buffer_rsrc_t R =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.bt, (short)0, p.nblk * 4, 0x00020000);
    int id = uni((int)__builtin_amdgcn_raw_buffer_load_b32(R, lb * 4, 0, 0));
#else
    int id = p.bt[lb];
#endif
    return id < 0 ? 0 : (id > nb_m1 ? nb_m1 : id);
  }

  __device__ __forceinline__ Ids tile_ids(const PairRef& p, int j, bool live = true) const {
    if constexpr (BS >= 16) {
      const int t = j * 16;
      const int id = id_of(p, t / BS);
      const int64_t b = (int64_t)id * block_stride + p.head_off + (int64_t)(t % BS) * rs;
      Ids r{b, b, live, 1.f, 1.f, 1.f, 1.f};
      if constexpr (BSC) {
        r.ks0 = r.ks1 = kbs[(int64_t)id * hkv];
        r.vs0 = r.vs1 = vbs[(int64_t)id * hkv];
      }
      return r;
    } else {
      const int i0 = id_of(p, 2 * j), i1 = id_of(p, 2 * j + 1);
      Ids r{(int64_t)i0 * block_stride + p.head_off, (int64_t)i1 * block_stride + p.head_off,
            live, 1.f, 1.f, 1.f, 1.f};
      if constexpr (BSC) {
        r.ks0 = kbs[(int64_t)i0 * hkv];
        r.ks1 = kbs[(int64_t)i1 * hkv];
        r.vs0 = vbs[(int64_t)i0 * hkv];
        r.vs1 = vbs[(int64_t)i1 * hkv];
      }
      return r;
    }
  }

  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* p, int live) const {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, live ? 16 * rs : 0, 0x00020000);
  }
  __device__ __forceinline__ uint4 ld_k(__amdgpu_buffer_rsrc_t R, int soff) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, koff, soff, CPOL));
  }
  __device__ __forceinline__ VT ld_v(__amdgpu_buffer_rsrc_t R, int k) const {
    // value load k: rows 4k .. 4k+3 of the tile (lane: row 4k + r, chunk c)
    const int so = (BS >= 16 ? 4 * k : ((4 * k) & 7)) * rs;
    if constexpr (VB == 32)
      return u32x8{__builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, voff, so, CPOL)),
                   __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, voff, so + 16, CPOL))};
    else if constexpr (VB == 16)
      return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(R, voff, so, CPOL));
    else if constexpr (VB == 8)
      return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R, voff, so, CPOL));
    else
      return __builtin_amdgcn_raw_buffer_load_b32(R, voff, so, CPOL);
  }

  // ts: where the tile's per-block scales (keys of its two halves, values of
  // its two halves) go, for compute (formats 3 and 4).
  __device__ __forceinline__ void issue(const Ids& ids, uint4* kr, VT* vr,
                                        float4* ts = nullptr) const {
    if constexpr (BSC) {
      if (ts) *ts = make_float4(ids.ks0, ids.ks1, ids.vs0, ids.vs1);
    }
    const __amdgpu_buffer_rsrc_t klo = rsrc(kp + ids.lo, ids.live);
    const __amdgpu_buffer_rsrc_t vlo = rsrc(vp + ids.lo, ids.live);
    // Key load u reads whole rows u*RPI .. u*RPI+RPI-1 of the tile (lane: row
    // t0, chunk ch), so each load instruction covers contiguous 256-B runs.
    if constexpr (BS >= 16) {
#pragma unroll
      for (int u = 0; u < NKL; ++u) kr[u] = ld_k(klo, u * RPI * rs);
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[k] = ld_v(vlo, k);
    } else {   // tokens 0-7 of the tile in block 2j, tokens 8-15 in block 2j+1
      const __amdgpu_buffer_rsrc_t khi = rsrc(kp + ids.hi, ids.live);
      const __amdgpu_buffer_rsrc_t vhi = rsrc(vp + ids.hi, ids.live);
#pragma unroll
      for (int u = 0; u < NKL; ++u) {
        if constexpr (RPI <= 8) kr[u] = ld_k(u * RPI >= 8 ? khi : klo, ((u * RPI) & 7) * rs);
        else kr[u] = t0 < 8 ? ld_k(klo, 0) : ld_k(khi, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[k] = ld_v(k < 2 ? vlo : vhi, k);
    }
  }

  // Fold tile j (tokens 16j..16j+15) into the running state.  Tokens
  // t_begin .. t_end - 1 of tile j count; the others are masked.  With
  // COLS, only query columns col_lo .. col_hi - 1 take this tile (the other
  // columns' scores are masked, so their state is untouched): the grouped
  // schedule's columns belong to several sequences.
  template <bool COLS = false>
  __device__ __forceinline__ void compute(int j, int t_begin, int t_end, const uint4* kr,
                                          const VT* vr_in, int col_lo = 0, int col_hi = 16,
                                          float4 ts = float4{1.f, 1.f, 1.f, 1.f}) {
    // Loads issued before this point stay before it: otherwise the scheduler
    // hoists the waits for this tile above the next tile's loads.
    __builtin_amdgcn_sched_barrier(0);
    // Keys arrive row-wise; the QK MFMA wants one token per lane.  Regroup
    // through this wave's LDS tile: lane (r, c) reads chunks cl*4 + r of row
    // (c >> 2) + 4 (c & 3), so that score lane (r, c) ends up holding tokens
    // r, r+4, r+8, r+12 -- the rows value load k = 0..3 gives that lane.
#pragma unroll
    for (int u = 0; u < NKL; ++u)
      *(lds_u32x4*)(kst + kslot(u * RPI + t0, ch)) = __builtin_bit_cast(u32x4_t, kr[u]);
    uint4 kc[NKL];
    const int krow = (c >> 2) + 4 * (c & 3);
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl)
      kc[cl] = __builtin_bit_cast(uint4, *(const lds_u32x4*)(kst + kslot(krow, cl * 4 + r)));
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cl = 0; cl < NKL; ++cl) {
      uint32_t w[4];
      vec_words<16>(kc[cl], w);
#pragma unroll
      for (int grp = 0; grp < GPL; ++grp) {
        half4_t kop;
        if constexpr (FMT == 1) kop = e4m3x4_to_half4(w[grp]);
        else if constexpr (FMT == 2) kop = e5m2x4_to_half4(w[grp]);
        else kop = halves_of(w[2 * grp], w[2 * grp + 1]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(kop, qop[cl * GPL + grp], sacc, 0, 0, 0);
      }
    }
    const bool partial = j * 16 + 16 > t_end || j * 16 < t_begin;   // wave-uniform
    const uint32_t span = (uint32_t)(t_end - t_begin);
    const int tb = j * 16 + r;                  // token of score i: tb + 4 i
    float x[4];
    const bool col_ok = !COLS || (uint32_t)(c - col_lo) < (uint32_t)(col_hi - col_lo);
    // the key scale of each score's block: scores 0, 1 are tokens r, r + 4 (the
    // first half tile), 2, 3 tokens r + 8, r + 12
    const float sc_lo = BSC ? sc * ts.x : sc, sc_hi = BSC ? sc * (BS >= 16 ? ts.x : ts.y) : sc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = (col_ok && (uint32_t)(tb + 4 * i - t_begin) < span)
                 ? sacc[i] * (i < 2 ? sc_lo : sc_hi) : -INFINITY;
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const bool grow = (COLS ? col_ok : (c < g)) && (tmax > m_run + kLazy);
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

    uint32_t vw[4][VB / 4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vec_words<VB>(vr_in[k], vw[k]);
    if (partial) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool ok = (uint32_t)(tb + 4 * k - t_begin) < span;
#pragma unroll
        for (int wi = 0; wi < VB / 4; ++wi) vw[k][wi] = ok ? vw[k][wi] : 0u;
      }
    }
    if constexpr (FMT == 0) {
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        const int wi = e >> 1, sh = (e & 1) * 16;
        const uint32_t h0 = (vw[0][wi] >> sh) & 0xFFFFu, h1 = (vw[1][wi] >> sh) & 0xFFFFu;
        const uint32_t h2 = (vw[2][wi] >> sh) & 0xFFFFu, h3 = (vw[3][wi] >> sh) & 0xFFFFu;
        const half4_t bop = halves_of(h0 | (h1 << 16), h2 | (h3 << 16));
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, bop, acc[e], 0, 0, 0);
      }
    } else if constexpr (FMT == 2 && !BSC) {
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        const int wi = e >> 2, b = e & 3;
        const half4_t bop = halves_of(e5m2_pair(vw[0][wi], vw[1][wi], b),
                                      e5m2_pair(vw[2][wi], vw[3][wi], b));
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, bop, acc[e], 0, 0, 0);
      }
    } else {
      // e4m3fn (and e5m2 with per-block scales): fp32 values, times the
      // block's value scale (value load k holds rows 4k .. 4k + 3: the first
      // half tile for k < 2)
      float vf[4][DCH];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int wi = 0; wi < VB / 4; ++wi) {
          if constexpr (FMT == 1) {
            const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[k][wi], false);
            const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)vw[k][wi], true);
            vf[k][4 * wi + 0] = lo.x;
            vf[k][4 * wi + 1] = lo.y;
            vf[k][4 * wi + 2] = hi.x;
            vf[k][4 * wi + 3] = hi.y;
          } else {                             // e5m2 byte b is binary16 bits b << 8
#pragma unroll
            for (int q = 0; q < 4; ++q)
              vf[k][4 * wi + q] = (float)__builtin_bit_cast(
                  _Float16, (uint16_t)(((vw[k][wi] >> (8 * q)) & 0xFFu) << 8));
          }
        }
        if constexpr (BSC) {
          const float vsk = (BS >= 16 || k < 2) ? ts.z : ts.w;
#pragma unroll
          for (int e = 0; e < DCH; ++e) vf[k][e] *= vsk;
        }
      }
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        const float4_t f = {vf[0][e], vf[1][e], vf[2][e], vf[3][e]};
        const half4_t bop = __builtin_convertvector(f, half4_t);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, bop, acc[e], 0, 0, 0);
      }
    }
  }

  // Sum of l over the 4 row groups: lane (any r, c) then holds head c's total.
  __device__ __forceinline__ float l_total() const {
    return xor_sum(xor_sum(l_run, 16), 32);
  }

  // Write acc / l (times v_scale) for the gqa heads of a pair.  dst points at
  // head 0 of the group; rows are D elements apart.
  __device__ __forceinline__ void store_out(_Float16* dst, float lt, float v_scale) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r + i;
      const float lh = __shfl(lt, h);
      if (h < g) {
        const float inv = lh > 0.f ? v_scale / lh : 0.f;
        _Float16 o[DCH];
#pragma unroll
        for (int e = 0; e < DCH; ++e) o[e] = (_Float16)(acc[e][i] * inv);
        if constexpr (DCH == 16) {
          uint4* d16 = (uint4*)(dst + (int64_t)h * D + c * DCH);
          const u32x8 w = __builtin_bit_cast(u32x8, o);
          d16[0] = w.lo;
          d16[1] = w.hi;
        } else if constexpr (DCH == 8) {
          *(uint4*)(dst + (int64_t)h * D + c * DCH) = __builtin_bit_cast(uint4, o);
        } else {
          *(uint2*)(dst + (int64_t)h * D + c * DCH) = __builtin_bit_cast(uint2, o);
        }
      }
    }
  }

  // Write acc / l (times v_scale) for columns 0 .. ncols - 1, column h to the
  // row dst(h) (a grouped segment: the columns belong to several sequences).
  template <class RowOf>
  __device__ __forceinline__ void store_out_cols(const RowOf& dst, int ncols, float lt,
                                                 float v_scale) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r + i;
      const float lh = __shfl(lt, h);
      if (h < ncols) {
        const float inv = lh > 0.f ? v_scale / lh : 0.f;
        _Float16 o[DCH];
#pragma unroll
        for (int e = 0; e < DCH; ++e) o[e] = (_Float16)(acc[e][i] * inv);
        _Float16* row = dst(h) + c * DCH;
        if constexpr (DCH == 16) {
          const u32x8 w = __builtin_bit_cast(u32x8, o);
          ((uint4*)row)[0] = w.lo;
          ((uint4*)row)[1] = w.hi;
        } else if constexpr (DCH == 8) {
          *(uint4*)row = __builtin_bit_cast(uint4, o);
        } else {
          *(uint2*)row = __builtin_bit_cast(uint2, o);
        }
      }
    }
  }

  // A 16-column partial record: o[h][d] (fp32, normalised, times v_scale) for
  // h < 16, then (m, l) per column; columns >= ncols are written as empty.
  __device__ __forceinline__ void store_partial16(float* rec, int ncols, float lt,
                                                  float v_scale) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r + i;
      const float lh = __shfl(lt, h);
      if (h < ncols) {
        const float inv = lh > 0.f ? v_scale / lh : 0.f;
        float4* d4 = (float4*)(rec + (int64_t)h * D + c * DCH);
#pragma unroll
        for (int q = 0; q < DCH / 4; ++q)
          d4[q] = make_float4(acc[4 * q][i] * inv, acc[4 * q + 1][i] * inv,
                              acc[4 * q + 2][i] * inv, acc[4 * q + 3][i] * inv);
      }
    }
    if (r == 0)
      ((float2*)(rec + 16 * D))[c] = c < ncols ? make_float2(m_run, lt) : make_float2(kNegBig, 0.f);
  }

  // Write a partial: o[h][d] = acc / l * v_scale (fp32) then (m, l) per head.
  __device__ __forceinline__ void store_partial(float* rec, float lt, float v_scale) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r + i;
      const float lh = __shfl(lt, h);
      if (h < g) {
        const float inv = lh > 0.f ? v_scale / lh : 0.f;
        float4* d4 = (float4*)(rec + (int64_t)h * D + c * DCH);
#pragma unroll
        for (int q = 0; q < DCH / 4; ++q)
          d4[q] = make_float4(acc[4 * q][i] * inv, acc[4 * q + 1][i] * inv,
                              acc[4 * q + 2][i] * inv, acc[4 * q + 3][i] * inv);
      }
    }
    if (r == 0 && c < g) ((float2*)(rec + g * D))[c] = make_float2(m_run, lt);
  }
};

// ---------------------------------------------------------------- workgroup merge

// The NW waves of a workgroup each hold softmax state (m, l, unnormalised
// acc) for up to 16 rows; the workgroup's result per row is the log-sum-exp
// merge of the waves' states.  The states go to LDS (acc as float4 rows);
// one thread per row then forms the row's (M, L) and one weight per wave,
// f_w = 2^(m_w - M) * v_scale / L, and every thread finishes four dims of a
// row at a time as sum_w f_w * acc_w.  The per-row exponentials are formed
// once per row instead of once per output element.
template <int D, int NW>
struct WgMergeLds {
  float m[NW][16];
  float l[NW][16];
  float f[NW][16];
  float2 ml[16];
  float o[NW][16][D];
};

template <int D, int NW, int DCH>
__device__ __forceinline__ void wg_merge_put(WgMergeLds<D, NW>& sm, int wid, int lane,
                                             const float4_t* acc, float m_run, float l_tot,
                                             int nrows) {
  const int r = lane >> 4, c = lane & 15;
  if (r == 0) {
    sm.m[wid][c] = m_run;
    sm.l[wid][c] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * r + i;
    if (h < nrows) {
#pragma unroll
      for (int q = 0; q < DCH / 4; ++q)
        *(float4*)&sm.o[wid][h][c * DCH + 4 * q] =
            make_float4(acc[4 * q][i], acc[4 * q + 1][i], acc[4 * q + 2][i], acc[4 * q + 3][i]);
    }
  }
}

// After wg_merge_put by every wave and a barrier: calls put(h, d, o4, M, L)
// for every row h < nrows and every fourth dim d, o4 = dims d .. d + 3 of the
// merged, normalised row (times v_scale; zeros for an empty row).
template <int D, int NW, class Put>
__device__ __forceinline__ void wg_merge_finish(WgMergeLds<D, NW>& sm, int nrows, float v_scale,
                                                const Put& put) {
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = sm.m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
    float e[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      e[w] = exp2f(sm.m[w][h] - M);
      L += e[w] * sm.l[w][h];
    }
    const float inv = L > 0.f ? v_scale / L : 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sm.f[w][h] = e[w] * inv;
    sm.ml[h] = make_float2(M, L);
  }
  __syncthreads();
  constexpr int Q = D / 4;
  for (int idx = threadIdx.x; idx < nrows * Q; idx += NW * 64) {
    const int h = idx / Q, d = (idx - (idx / Q) * Q) * 4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = sm.f[w][h];
      const float4 a = *(const float4*)&sm.o[w][h][d];
      o.x += f * a.x;
      o.y += f * a.y;
      o.z += f * a.z;
      o.w += f * a.w;
    }
    put(h, d, o, sm.ml[h].x, sm.ml[h].y);
  }
}

__device__ __forceinline__ void store_half4(_Float16* dst, float4 o) {
  *(half4_t*)dst = (half4_t){(_Float16)o.x, (_Float16)o.y, (_Float16)o.z, (_Float16)o.w};
}

// ---------------------------------------------------------------- single / split

template <int D, int BS, int KV, int NW, bool SPLIT, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : PA_WAVES_PER_EU, 8)))
void decode_kernel(DecodeArgs a, const int32_t* __restrict__ tables,
                   const int32_t* __restrict__ lens, const float* __restrict__ kbs,
                   const float* __restrict__ vbs) {
  // The tables arrive as restrict arguments so that their uniform reads stay
  // scalar loads (as in decode_flat_kernel).
  typedef Engine<D, BS, KV, NT> En;
  typedef typename En::VT VT;
  const int lane = threadIdx.x & 63;
  const int wid = uni(threadIdx.x >> 6);

  int bid = blockIdx.x;
  int part = 0;
  if constexpr (SPLIT) { part = bid % a.num_parts; bid /= a.num_parts; }
  const int kh = bid % a.num_kv_heads;
  const int s = bid / a.num_kv_heads;
  const int g = a.gqa;

  // The first two tiles' block ids are read together with the length (their
  // logical blocks clamped to the table row, which the host bounds, rather
  // than to the length), so the first K/V loads wait on one round trip.
  const int j0 = (SPLIT ? part * a.part_tokens : 0) / 16 + wid;
  const int64_t head_off = (int64_t)kh * D * Engine<D, BS, KV, NT>::E;
  const PairRef row{tables + (int64_t)s * a.max_blocks, a.max_blocks, 0, head_off};
  const int len = clamp_len(lens[s], a.len_cap);
  const int w0 = win_start(len, a.window);    // first position the query sees
  int t_begin = w0, t_end = len;
  if constexpr (SPLIT) {
    t_begin = part * a.part_tokens;
    if (t_begin >= len) return;               // partition past the end: nothing to do
    t_end = min(len, t_begin + a.part_tokens);
    if (t_end <= w0) return;                  // partition before the window: not read
    t_begin = max(t_begin, w0);               // (the reduce skips such partitions)
  }
  const int j_begin = t_begin >> 4;
  const int j_end = (t_end + 15) >> 4;

  __shared__ __attribute__((aligned(16))) char kstage[NW][En::KST];
  En en;
  en.init(a, lane, (lds_char*)kstage[wid]);
  if (a.k_hs) en.sc *= a.k_hs[kh];
  en.set_block_scales(kbs, vbs, kh);
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;
  en.load_q(a.q + ((int64_t)s * a.num_q_heads + (int64_t)kh * g) * D);
  en.reset();
  const PairRef pr{tables + (int64_t)s * a.max_blocks, (len + BS - 1) / BS, len, head_off};
  Ids ids0 = en.tile_ids(row, j0), ids1 = en.tile_ids(row, j0 + NW);
  if (j_begin + wid != j0) {                  // window start: the speculation missed
    ids0 = en.tile_ids(row, j_begin + wid);
    ids1 = en.tile_ids(row, j_begin + wid + NW);
  }

  // The loads of tile j+NW and the block ids of tile j+2NW are in flight while
  // tile j is computed; two register sets alternate.  Tiles past the wave's
  // last one are dead (their loads fetch nothing).
  uint4 kA[En::NKL], kB[En::NKL];
  VT vA[4], vB[4];
  float4 tsA = float4{1.f, 1.f, 1.f, 1.f}, tsB = tsA;
  int j = j_begin + wid;
  if (j < j_end) {
    const int j_last = j_end - 1;
    en.issue(ids0, kA, vA, &tsA);
    Ids ids_b = ids1;
    ids_b.live = j + NW <= j_last;
    for (;;) {
      // the block ids two tiles ahead are read before the next tile's loads
      // are issued, so waiting for them never waits for those loads
      const Ids ids_a = en.tile_ids(pr, min(j + 2 * NW, j_last), j + 2 * NW <= j_last);
      en.issue(ids_b, kB, vB, &tsB);
      en.compute(j, t_begin, t_end, kA, vA, 0, 16, tsA);
      j += NW;
      if (j >= j_end) break;
      ids_b = en.tile_ids(pr, min(j + 2 * NW, j_last), j + 2 * NW <= j_last);
      en.issue(ids_a, kA, vA, &tsA);
      en.compute(j, t_begin, t_end, kB, vB, 0, 16, tsB);
      j += NW;
      if (j >= j_end) break;
    }
  }
  const float l_tot = en.l_total();

  // ---- merge the waves of the workgroup in LDS, then write
  __shared__ WgMergeLds<D, NW> sm;
  wg_merge_put<D, NW, En::DCH>(sm, wid, lane, en.acc, en.m_run, l_tot, g);
  __syncthreads();
  const int64_t row0 = (int64_t)s * a.num_q_heads + (int64_t)kh * g;
  wg_merge_finish<D, NW>(sm, g, v_scale, [&](int h, int d, float4 o, float M, float L) {
    if constexpr (SPLIT) {
      const int64_t prow = (row0 + h) * a.num_parts + part;
      *(float4*)&a.ws_o[prow * D + d] = o;
      if (d == 0) a.ws_ml[prow] = make_float2(M, L);
    } else {
      store_half4(a.out + (row0 + h) * D + d, o);
    }
  });
}

// ---------------------------------------------------------------- grouped

// One workgroup per (group, KV head).  A group is up to 16 / gqa sequences
// listed in an order where each member shares its first positions with the
// member before it: member i's table lists the same physical blocks as member
// i - 1's for its first dep_i whole 16-token tiles (forks, prefix-cache hits:
// "PagedAttention & vLLM", memory sharing).  Query column c is (member
// c / gqa, head c % gqa), so one 16x16 MFMA scores a K tile for several
// members at once.  Units: member i's tiles dep_i .. end_i - 1 (dep_0 = 0);
// tile t of member i is also the tile t of members i + 1 .. j as long as
// each of them shares more than t tiles with its predecessor, so the unit
// feeds the columns of members i .. j and every distinct (tile, block) of
// the group leaves HBM once.  The waves take units round-robin, one tile in
// flight ahead of the one computed, and merge in LDS.
template <int D, int BS, int KV, int NW, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : PA_GROUP_WAVES_PER_EU, 8)))
void decode_group_kernel(DecodeArgs a, GroupArgs gp, const int32_t* __restrict__ tables,
                         const int32_t* __restrict__ lens, const float* __restrict__ kbs,
                         const float* __restrict__ vbs) {
  typedef Engine<D, BS, KV, NT> En;
  typedef typename En::VT VT;
  const int lane = threadIdx.x & 63;
  const int wid = uni(threadIdx.x >> 6);
  const int kh = blockIdx.x % a.num_kv_heads;
  const int grp = blockIdx.x / a.num_kv_heads;
  const int g = a.gqa;

  // ---- members, clamped into the arrays (device contents are not validated),
  // read by the lanes of wave 0 in parallel: one member per lane
  __shared__ int sm_seq[16], sm_len[16], sm_dep[16], sm_pre[17], sm_nm;
  if (wid == 0) {
    int m0 = gp.member_start[grp], m1 = gp.member_start[grp + 1];
    m0 = m0 < 0 ? 0 : (m0 > gp.num_members ? gp.num_members : m0);
    m1 = m1 < m0 ? m0 : (m1 > gp.num_members ? gp.num_members : m1);
    const int nm = m1 - m0 < 16 / g ? m1 - m0 : 16 / g;
    int sq = 0, ln = 0, sh = 0;
    if (lane < nm) {
      sq = gp.members[m0 + lane];
      sq = sq < 0 ? 0 : (sq >= gp.num_seqs ? gp.num_seqs - 1 : sq);
      ln = clamp_len(lens[sq], a.len_cap);
      sh = gp.member_shared[m0 + lane];
    }
    const int prev = __shfl_up(ln, 1);        // the previous member's length
    int dep = 0;                              // whole tiles shared with it
    if (lane > 0 && lane < nm) dep = (sh < 0 ? 0 : min(sh, min(ln, prev))) >> 4;
    int x = lane < nm ? ((ln + 15) >> 4) - dep : 0;   // the member's units
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {        // inclusive scan over lanes 0..15
      const int y = __shfl_up(x, o);
      if ((lane & 15) >= o) x += y;
    }
    if (lane < nm) {
      sm_seq[lane] = sq;
      sm_len[lane] = ln;
      sm_dep[lane] = dep;
    }
    if (lane < 16) sm_pre[lane + 1] = x;
    if (lane == 0) {
      sm_pre[0] = 0;
      sm_nm = nm;
    }
  }
  __syncthreads();
  const int nm = uni(sm_nm);
  const int U = uni(sm_pre[nm]);              // units of the workgroup
  const int ncols = nm * g;

  __shared__ __attribute__((aligned(16))) char kstage[NW][En::KST];
  En en;
  en.init(a, lane, (lds_char*)kstage[wid]);
  if (a.k_hs) en.sc *= a.k_hs[kh];
  en.set_block_scales(kbs, vbs, kh);
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;
  const int64_t head_off = (int64_t)kh * D * En::E;
  {
    const int c = lane & 15;
    const _Float16* qrow = nullptr;
    if (c < ncols)
      qrow = a.q + ((int64_t)sm_seq[c / g] * a.num_q_heads + (int64_t)kh * g + c % g) * D;
    en.load_q_rows(qrow);
  }
  en.reset();

  // unit u -> (member i, tile t, last member j taking it)
  struct Unit { int i, t, j; };
  auto unit_of = [&](int u) -> Unit {
    int i = 0;
    while (i + 1 < nm && sm_pre[i + 1] <= u) ++i;
    i = uni(i);
    const int t = uni(sm_dep[i]) + u - uni(sm_pre[i]);
    int j = i;
    while (j + 1 < nm && sm_dep[j + 1] > t) ++j;
    return {i, t, uni(j)};
  };
  auto ids_of = [&](int u) -> Ids {
    const Unit un = unit_of(u);
    const int ln = uni(sm_len[un.i]);
    const PairRef p{tables + (int64_t)uni(sm_seq[un.i]) * a.max_blocks,
                    ln > 0 ? (ln + BS - 1) / BS : 1, ln, head_off};
    return en.tile_ids(p, un.t);
  };
  auto run = [&](int u, const uint4* kr, const VT* vr, float4 ts) {
    const Unit un = unit_of(u);
    en.template compute<true>(un.t, 0, uni(sm_len[un.i]), kr, vr, un.i * g, (un.j + 1) * g, ts);
  };

  uint4 kA[En::NKL], kB[En::NKL];
  VT vA[4], vB[4];
  float4 tsA = float4{1.f, 1.f, 1.f, 1.f}, tsB = tsA;
  int u = wid;
  if (u < U) {
    const int u_last = U - 1;
    auto ids_ahead = [&](int v) {             // dead past the wave's last unit
      Ids x = ids_of(min(v, u_last));
      x.live = v <= u_last;
      return x;
    };
    en.issue(ids_of(u), kA, vA, &tsA);
    Ids ids_b = ids_ahead(u + NW);
    for (;;) {
      const Ids ids_a = ids_ahead(u + 2 * NW);
      en.issue(ids_b, kB, vB, &tsB);
      run(u, kA, vA, tsA);
      u += NW;
      if (u >= U) break;
      ids_b = ids_ahead(u + 2 * NW);
      en.issue(ids_a, kA, vA, &tsA);
      run(u, kB, vB, tsB);
      u += NW;
      if (u >= U) break;
    }
  }
  const float l_tot = en.l_total();

  // ---- merge the waves of the workgroup in LDS, then write every column
  __shared__ WgMergeLds<D, NW> sm;
  wg_merge_put<D, NW, En::DCH>(sm, wid, lane, en.acc, en.m_run, l_tot, ncols);
  __syncthreads();
  wg_merge_finish<D, NW>(sm, ncols, v_scale, [&](int h, int d, float4 o, float, float) {
    const int64_t row = (int64_t)sm_seq[h / g] * a.num_q_heads + (int64_t)kh * g + h % g;
    store_half4(a.out + row * D + d, o);
  });
}

// One workgroup per (sequence, query head): merge the partitions by log-sum-exp.
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - M), M = max_p m_p.
template <int D>
__global__ __launch_bounds__(256) void lse_reduce_kernel(DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int NG = NT / D;                  // thread groups sharing the partitions
  const int row_id = blockIdx.x;
  const int s = row_id / a.num_q_heads;
  const int len = clamp_len(a.seq_lens[s], a.len_cap);
  // partitions before the sliding window wrote nothing: start at the window's
  const int p0 = win_start(len, a.window) / a.part_tokens;
  const int np = (len + a.part_tokens - 1) / a.part_tokens - p0;
  const int64_t base = (int64_t)row_id * a.num_parts + p0;
  const float2* ml = a.ws_ml + base;

  __shared__ float red[NT / 64];
  __shared__ float sm_part[NG][D];

  float mx = kNegBig;
  for (int p = threadIdx.x; p < np; p += NT) mx = fmaxf(mx, ml[p].x);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

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

// ---------------------------------------------------------------- flat schedule

// Range that owns unit t when T units are cut into NR ranges
// [floor(r*T/NR), floor((r+1)*T/NR)).
__device__ __forceinline__ int range_of(int64_t t, int64_t T, int64_t NR) {
  return (int)(((t + 1) * NR - 1) / T);
}

// True when range r owns no unit (more ranges than units this call: the host
// sizes the ranges from max_seq_len, and windows shorten what is read).  Its
// waves return at once, so the merge must not read its record slots, which
// hold whatever an earlier call left there.
__device__ __forceinline__ bool range_empty(int64_t r, int64_t T, int64_t NR) {
  return r * T / NR == (r + 1) * T / NR;
}

// Units are (sequence, 16-token tile) pairs in sequence order.  Range r is
// walked by the Hkv consecutive waves r*Hkv + kh, one per KV head, so the heads
// of a block are read together.  A sequence that lies inside one range is
// written directly; one cut by range boundaries leaves a partial record per
// range (slot 0: the range's first sequence, slot 1: its last), merged by
// flat_merge_heads_kernel.
template <int D, int BS, int KV, int NW, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : PA_FLAT_WAVES_PER_EU, 8)))
void decode_flat_kernel(DecodeArgs a, FlatArgs f, const int32_t* __restrict__ tables,
                        const int32_t* __restrict__ lens, const _Float16* __restrict__ qs,
                        _Float16* __restrict__ outs, float* __restrict__ slots,
                        int32_t* __restrict__ prefix, const float* __restrict__ kbs,
                        const float* __restrict__ vbs) {
  // The read-only arrays arrive as separate restrict arguments: stores to the
  // outputs inside the loop then provably leave the block table alone, so its
  // entries can be read with scalar loads.
  typedef Engine<D, BS, KV, NT> En;
  typedef typename En::VT VT;
  extern __shared__ int sm[];                 // [S + 1] tiles before sequence s, then [S] lengths
  const int S = f.num_seqs, Hkv = a.num_kv_heads, g = a.gqa;
  int* sm_pre = sm;
  int* sm_len = sm + S + 1;
  const int lane = threadIdx.x & 63;
  const int wid = uni(threadIdx.x >> 6);

  // ---- lengths and exclusive prefix of per-sequence tile counts in LDS
  // (workgroup 0 also stores the prefix for the merge), and zero rows of
  // empty sequences.  Every thread loads lengths; the scan is workgroup-wide:
  // thread t sums its run of `per` counts, the run sums are scanned across
  // waves, then each thread writes its run's prefixes.
  constexpr int NTH = NW * 64;
  __shared__ int sm_wsum[NW];
  for (int i = threadIdx.x; i < S; i += NTH) {
    const int len = clamp_len(lens[i], a.len_cap);
    sm_len[i] = len;
    sm_pre[i + 1] = ((len + 15) >> 4) - (win_start(len, a.window) >> 4);   // tiles it reads
  }
  __syncthreads();
  {
    const int per = (S + NTH - 1) / NTH;
    const int b0 = min(S, (int)threadIdx.x * per), b1 = min(S, b0 + per);
    int sum = 0;
    for (int i = b0; i < b1; ++i) sum += sm_pre[i + 1];
    int x = sum;                               // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) sm_wsum[wid] = x;
    __syncthreads();
    int run = x - sum;
    for (int w = 0; w < wid; ++w) run += sm_wsum[w];
    for (int i = b0; i < b1; ++i) {
      run += sm_pre[i + 1];
      sm_pre[i + 1] = run;
    }
    if (threadIdx.x == 0) sm_pre[0] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= S; i += NTH) prefix[i] = sm_pre[i];
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    if (sm_len[s] == 0) {
      _Float16* o = outs + (int64_t)s * a.num_q_heads * D;
      for (int i = threadIdx.x; i < a.num_q_heads * D; i += NTH) o[i] = (_Float16)0.f;
    }
  }

  const int64_t T = sm_pre[S];
  const int64_t NR = f.num_ranges;
  const int gw = blockIdx.x * NW + wid;
  const int rg = gw / Hkv, kh = gw - (gw / Hkv) * Hkv;
  if (rg >= NR) return;                        // no barrier follows
  const int g0 = (int)((int64_t)rg * T / NR), g1 = (int)((int64_t)(rg + 1) * T / NR);
  if (g0 >= g1) return;

  // ---- cursors over (sequence, tile) units; all wave-uniform.  cur[0] is the
  // unit being computed, cur[k] the k-th after it (clamped to the range's
  // last unit; the loads of such a cursor are dead).
  auto ntiles = [&](int ss) { return uni(sm_pre[ss + 1] - sm_pre[ss]); };
  struct Cur { int s, j; };
  auto advance = [&](Cur c) -> Cur {           // the next unit (callers know one exists)
    if (c.j + 1 < ntiles(c.s)) return {c.s, c.j + 1};
    int ns = c.s;
    do { ++ns; } while (ntiles(ns) == 0);
    return {uni(ns), 0};
  };
  int lo = 0, hi = S;                          // sequence with pre[s] <= g0 < pre[s+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sm_pre[mid] <= g0) lo = mid; else hi = mid;
  }
  constexpr int ST = PA_FLAT_STAGES;           // tiles in flight per wave, plus one
  static_assert(ST >= 2, "at least one tile in flight");
  Cur cur[ST + 1];
  cur[0] = {uni(lo), uni(g0 - sm_pre[lo])};
#pragma unroll
  for (int k = 1; k <= ST; ++k) cur[k] = g0 + k < g1 ? advance(cur[k - 1]) : cur[k - 1];

  __shared__ __attribute__((aligned(16))) char kstage[NW][En::KST];
  En en;
  en.init(a, lane, (lds_char*)kstage[wid]);
  if (a.k_hs) en.sc *= a.k_hs[kh];
  en.set_block_scales(kbs, vbs, kh);
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;
  const int64_t head_off = (int64_t)kh * D * En::E;
  // unit j of a sequence is its tile j + (window start >> 4)
  auto ids_of = [&](Cur c) -> Ids {
    const int len = uni(sm_len[c.s]);
    const PairRef p{tables + (int64_t)c.s * a.max_blocks, (len + BS - 1) / BS, len, head_off};
    return en.tile_ids(p, c.j + (win_start(len, a.window) >> 4));
  };
  auto q_of = [&](int cs) { return qs + ((int64_t)cs * a.num_q_heads + (int64_t)kh * g) * D; };
  float* rec_base = slots + (int64_t)gw * 2 * g * (D + 2);

  en.load_q(q_of(cur[0].s));
  en.reset();
  // The query rows of a sequence are loaded into qpre when its first tile is
  // issued, so switching sequences waits on nothing that a tile load does not
  // already wait on.  One set is held (tagged with its sequence); a sequence
  // that starts while another's rows are pending loads its rows on switching.
  half4_t qpre[En::NQ];
  int q_seq = -1;
  bool seg_from_start = cur[0].j == 0;         // the current segment began at tile 0
  int seg_start = g0;                          // unit index where the current segment began
  int gt = g0;

  // After folding unit cur[0]: when it ends its sequence or the range, write
  // the segment and, if the range goes on, switch to the next sequence.
  auto finish = [&]() {
    const bool seq_end = cur[0].j + 1 == ntiles(cur[0].s);
    if (!(seq_end || gt + 1 == g1)) return;
    const float lt = en.l_total();
    if (seg_from_start && seq_end) {
      en.store_out(outs + ((int64_t)cur[0].s * a.num_q_heads + (int64_t)kh * g) * D, lt,
                   v_scale);
    } else {                                   // slot 0: the range's first segment
      en.store_partial(rec_base + (seg_start == g0 ? 0 : 1) * g * (D + 2), lt, v_scale);
    }
    if (gt + 1 < g1) {                         // next sequence: new query rows, fresh state
      if (q_seq == cur[1].s) en.take_q(qpre); else en.load_q(q_of(cur[1].s));
      q_seq = -1;
      en.reset();
      seg_from_start = true;
      seg_start = gt + 1;
    }
  };

  // ST register sets rotate: while unit gt is computed, units gt+1 .. gt+ST-1
  // are in flight.
  uint4 kb[ST][En::NKL];
  VT vb[ST][4];
  float4 tsc[ST];
#pragma unroll
  for (int k = 0; k < ST - 1; ++k) {
    if (k > 0 && cur[k].j == 0 && g0 + k < g1 && q_seq < 0) {   // a sequence starts early
      en.load_q_into(qpre, q_of(cur[k].s));
      q_seq = cur[k].s;
    }
    Ids ik = ids_of(cur[k]);
    ik.live = g0 + k < g1;
    en.issue(ik, kb[k], vb[k], &tsc[k]);
  }
  Ids ids_next = ids_of(cur[ST - 1]);
  ids_next.live = g0 + ST - 1 < g1;
  for (;;) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      if (cur[ST - 1].j == 0 && gt + ST - 1 < g1 && q_seq < 0) {
        en.load_q_into(qpre, q_of(cur[ST - 1].s));
        q_seq = cur[ST - 1].s;
      }
      {
        // the block ids are read before the loads below are issued; the
        // loads of a unit past the range are dead (a branch around the issue
        // instead cost 8-13%: the waits after it then drain every load)
        Ids ids_new = ids_of(cur[ST]);
        ids_new.live = gt + ST < g1;
        en.issue(ids_next, kb[(st + ST - 1) % ST], vb[(st + ST - 1) % ST], &tsc[(st + ST - 1) % ST]);
        ids_next = ids_new;
      }
      {
        const int len = uni(sm_len[cur[0].s]), w0 = win_start(len, a.window);
        en.compute(cur[0].j + (w0 >> 4), w0, len, kb[st], vb[st], 0, 16, tsc[st]);
      }
      finish();
      if (++gt == g1) return;
#pragma unroll
      for (int k = 0; k < ST; ++k) cur[k] = cur[k + 1];
      if (gt + ST < g1) cur[ST] = advance(cur[ST]);
    }
  }
}

// One workgroup per (sequence, KV head), for sequences cut by range
// boundaries: the log-sum-exp merge of the sequence's records, all gqa rows at
// once.  Thread t covers output float4 q = t mod F4 (F4 = gqa * D / 4) and
// folds every K-th record from record t div F4 (K = the power of two that
// fits the workgroup), so the records' loads are in flight together; the K
// partial states of an output are then combined in LDS in a fixed order
// (deterministic).  Records of ranges that own no unit hold an earlier call's
// bytes and are replaced by an empty state by a select.
template <int D>
__global__ __launch_bounds__(1024) void flat_merge_heads_kernel(DecodeArgs a, FlatArgs f) {
  const int Hkv = a.num_kv_heads;
  const int s = blockIdx.x / Hkv, kh = blockIdx.x - s * Hkv;
  const int64_t T = f.prefix[f.num_seqs];
  const int pre = f.prefix[s], end = f.prefix[s + 1];
  if (end == pre) return;
  const int64_t NR = f.num_ranges;
  const int r_first = range_of(pre, T, NR), r_last = range_of(end - 1, T, NR);
  if (r_first == r_last) return;               // written by the decode kernel
  const bool first_is_last_slot = (int64_t)r_first * T / NR < pre;
  const bool some_empty = T < NR;              // else every range owns a unit
  const int g = a.gqa, F4 = g * D / 4;
  const int64_t rec = (int64_t)g * (D + 2);
  int K = 1;
  while (2 * K * F4 <= (int)blockDim.x) K *= 2;
  const int t = threadIdx.x, k = t / F4, q = t - k * F4, h = 4 * q / D;
  float M = kNegBig, L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  // Records r_first + k, + K, ... of this thread are loaded RB at a time
  // before any is folded, so their loads are in flight together (RB: the
  // power of two, at most 8, that covers the records per thread).  Places
  // past the last record load the last one again and fold an empty state,
  // which leaves M, L and O bit for bit unchanged.
  auto fold = [&](auto rb) {
    constexpr int RB = decltype(rb)::value;
    for (int r0 = r_first + k; r0 <= r_last; r0 += RB * K) {
      float2 ml[RB];
      float4 ov[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int r = r0 + i * K;
        const int rr = r <= r_last ? r : r_last;
        const bool empty = r > r_last || (some_empty && range_empty(rr, T, NR));
        const int slot = (rr == r_first && first_is_last_slot) ? 1 : 0;
        const float* p = f.slots + ((int64_t)(rr * Hkv + kh) * 2 + slot) * rec;
        const float2 ml0 = ((const float2*)(p + g * D))[h];
        const float4 ov0 = ((const float4*)p)[q];
        ml[i] = empty ? make_float2(kNegBig, 0.f) : ml0;
        ov[i] = empty ? make_float4(0.f, 0.f, 0.f, 0.f) : ov0;
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const float mn = fmaxf(M, ml[i].x);
        const float sa = __builtin_amdgcn_exp2f(M - mn);
        const float sb = ml[i].y * __builtin_amdgcn_exp2f(ml[i].x - mn);
        L = L * sa + sb;
        O.x = O.x * sa + sb * ov[i].x;
        O.y = O.y * sa + sb * ov[i].y;
        O.z = O.z * sa + sb * ov[i].z;
        O.w = O.w * sa + sb * ov[i].w;
        M = mn;
      }
    }
  };
  if (k < K) {
    const int per = (r_last - r_first + K) / K;          // records per thread, at most
    if (per <= 1) fold(std::integral_constant<int, 1>());
    else if (per <= 2) fold(std::integral_constant<int, 2>());
    else if (per <= 4) fold(std::integral_constant<int, 4>());
    else fold(std::integral_constant<int, 8>());
  }
  __shared__ float4 sm_o[1024];
  __shared__ float2 sm_ml[1024];
  sm_o[t] = O;
  sm_ml[t] = make_float2(M, L);
  __syncthreads();
  if (k != 0) return;
  float Mt = sm_ml[q].x;
  for (int j = 1; j < K; ++j) Mt = fmaxf(Mt, sm_ml[j * F4 + q].x);
  float Lt = 0.f;
  float4 Ot = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < K; ++j) {
    const float2 ml = sm_ml[j * F4 + q];
    const float4 o = sm_o[j * F4 + q];
    const float w = __builtin_amdgcn_exp2f(ml.x - Mt);
    Lt += ml.y * w;
    Ot.x += o.x * w;
    Ot.y += o.y * w;
    Ot.z += o.z * w;
    Ot.w += o.w * w;
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  store_half4(a.out + ((int64_t)s * a.num_q_heads + (int64_t)kh * g) * D + 4 * q,
              make_float4(Ot.x * inv, Ot.y * inv, Ot.z * inv, Ot.w * inv));
}

// ---------------------------------------------------------------- flat schedule over groups

// The grouped schedule's work laid out as the flat schedule lays out
// sequences: the units of each group (member i's tiles dep_i .. end_i - 1, as
// in decode_group_kernel) are listed group after group and cut into equal
// ranges, walked by one wave per KV head.  A group inside one range is
// written directly; a group cut by range boundaries leaves one 16-column
// partial record per range (slot 0: the range's first segment, slot 1: its
// last), merged by flat_group_merge_kernel.  Query column c of a group is
// (member c / gqa, head c % gqa).
template <int D, int BS, int KV, int NW, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : PA_FLAT_WAVES_PER_EU, 8)))
void decode_flat_group_kernel(DecodeArgs a, FlatArgs f, GroupArgs gp,
                              const int32_t* __restrict__ tables,
                              const int32_t* __restrict__ lens, const _Float16* __restrict__ qs,
                              _Float16* __restrict__ outs, float* __restrict__ slots,
                              int32_t* __restrict__ prefix, const float* __restrict__ kbs,
                              const float* __restrict__ vbs) {
  typedef Engine<D, BS, KV, NT> En;
  typedef typename En::VT VT;
  const int G = gp.num_groups, M = gp.num_members, Hkv = a.num_kv_heads, g = a.gqa;
  const int cap = 16 / g;
  extern __shared__ int sm[];
  int* sm_pre = sm;                            // [G + 1] units before group i
  int* sm_ms = sm_pre + G + 1;                 // [G + 1] first member of group i
  int* sm_seq = sm_ms + G + 1;                 // [M] sequence of member p
  int* sm_len = sm_seq + M;                    // [M] its context length
  int* sm_dep = sm_len + M;                    // [M] tiles it shares with member p - 1
  int* sm_mpre = sm_dep + M;                   // [M] units of the members before p in its group
  const int lane = threadIdx.x & 63;
  const int wid = uni(threadIdx.x >> 6);
  constexpr int NTH = NW * 64;

  // ---- group and member tables in LDS, clamped into the arrays (device
  // contents are not validated); per-group unit counts, then their scan
  for (int i = threadIdx.x; i <= G; i += NTH) {
    const int v = gp.member_start[i];
    sm_ms[i] = v < 0 ? 0 : (v > M ? M : v);
  }
  for (int p = threadIdx.x; p < M; p += NTH) {
    int sq = gp.members[p];
    sq = sq < 0 ? 0 : (sq >= gp.num_seqs ? gp.num_seqs - 1 : sq);
    sm_seq[p] = sq;
    sm_len[p] = clamp_len(lens[sq], a.len_cap);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G; i += NTH) {
    const int m0 = sm_ms[i], m1 = sm_ms[i + 1] > m0 ? sm_ms[i + 1] : m0;
    const int nm = m1 - m0 < cap ? m1 - m0 : cap;
    int units = 0;
    for (int p = m0; p < m0 + nm; ++p) {
      int dep = 0;
      if (p > m0) {
        const int sh = gp.member_shared[p], lim = min(sm_len[p], sm_len[p - 1]);
        dep = (sh < 0 ? 0 : min(sh, lim)) >> 4;
      }
      sm_dep[p] = dep;
      sm_mpre[p] = units;
      units += ((sm_len[p] + 15) >> 4) - dep;
    }
    sm_pre[i + 1] = units;
  }
  __syncthreads();
  __shared__ int sm_wsum[NW];
  {
    const int per = (G + NTH - 1) / NTH;
    const int b0 = min(G, (int)threadIdx.x * per), b1 = min(G, b0 + per);
    int sum = 0;
    for (int i = b0; i < b1; ++i) sum += sm_pre[i + 1];
    int x = sum;                               // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) sm_wsum[wid] = x;
    __syncthreads();
    int run = x - sum;
    for (int w = 0; w < wid; ++w) run += sm_wsum[w];
    for (int i = b0; i < b1; ++i) {
      run += sm_pre[i + 1];
      sm_pre[i + 1] = run;
    }
    if (threadIdx.x == 0) sm_pre[0] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= G; i += NTH) prefix[i] = sm_pre[i];
  // groups without any unit (every member empty) get all-zero rows here
  for (int i = blockIdx.x; i < G; i += gridDim.x) {
    if (sm_pre[i + 1] != sm_pre[i]) continue;
    const int m0 = sm_ms[i], m1 = sm_ms[i + 1] > m0 ? sm_ms[i + 1] : m0;
    const int nm = m1 - m0 < cap ? m1 - m0 : cap;
    for (int p = m0; p < m0 + nm; ++p) {
      _Float16* o = outs + (int64_t)sm_seq[p] * a.num_q_heads * D;
      for (int k = threadIdx.x; k < a.num_q_heads * D; k += NTH) o[k] = (_Float16)0.f;
    }
  }

  const int64_t T = sm_pre[G];
  const int64_t NR = f.num_ranges;
  const int gw = blockIdx.x * NW + wid;
  const int rg = gw / Hkv, kh = gw - (gw / Hkv) * Hkv;
  if (rg >= NR) return;                        // no barrier follows
  const int g0 = (int)((int64_t)rg * T / NR), g1 = (int)((int64_t)(rg + 1) * T / NR);
  if (g0 >= g1) return;

  // ---- cursors over (group, unit) pairs, all wave-uniform.  Besides the
  // group s and the unit j, a cursor carries the member p whose tile t the
  // unit is, that member's sequence and length, and the last member hi that
  // takes the tile too, so stepping to the next unit reads LDS only for the
  // sharing span and when the member or the group changes.
  // nt caches the group's unit count and drop the tile from which the span
  // hi shrinks (the smallest shared depth among members p + 1 .. hi), so the
  // common step -- the member's next tile -- reads no LDS at all.
  struct Cur { int s, j, p, t, seq, len, m0, nm, hi, drop, nt; };
  auto ntiles = [&](int gi) { return uni(sm_pre[gi + 1] - sm_pre[gi]); };
  auto set_span = [&](Cur& c) {               // drop: the smallest depth in the span
    int q = c.p, mn = INT32_MAX;
    while (q + 1 < c.m0 + c.nm && sm_dep[q + 1] > c.t) {
      ++q;
      mn = min(mn, (int)sm_dep[q]);
    }
    c.hi = uni(q);
    c.drop = uni(mn);
  };
  auto enter_member = [&](Cur c, int p) -> Cur {
    c.p = p;
    c.t = uni(sm_dep[p]);
    c.seq = uni(sm_seq[p]);
    c.len = uni(sm_len[p]);
    set_span(c);
    return c;
  };
  auto at_unit = [&](int gi, int j) -> Cur {   // unit j of group gi, from scratch
    Cur c;
    c.s = gi;
    c.j = j;
    c.nt = ntiles(gi);
    c.m0 = uni(sm_ms[gi]);
    const int m1 = uni(sm_ms[gi + 1]);
    c.nm = m1 > c.m0 ? (m1 - c.m0 < cap ? m1 - c.m0 : cap) : 0;
    int p = c.m0;
    while (p + 1 < c.m0 + c.nm && sm_mpre[p + 1] <= j) ++p;
    c = enter_member(c, uni(p));
    c.t += j - uni(sm_mpre[c.p]);
    set_span(c);
    return c;
  };
  auto advance = [&](Cur c) -> Cur {           // the next unit (callers know one exists)
    if (c.j + 1 < c.nt) {
      ++c.j;
      if (c.t + 1 < ((c.len + 15) >> 4)) {
        ++c.t;
        if (c.t >= c.drop) set_span(c);
        return c;
      }
      int p = c.p + 1;                         // the next member with units of its own
      while (((sm_len[p] + 15) >> 4) == sm_dep[p]) ++p;
      return enter_member(c, uni(p));
    }
    int ns = c.s;
    do { ++ns; } while (ntiles(ns) == 0);
    return at_unit(uni(ns), 0);
  };
  int lo = 0, hi = G;                          // group with pre[i] <= g0 < pre[i+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sm_pre[mid] <= g0) lo = mid; else hi = mid;
  }
  constexpr int ST = PA_FLAT_STAGES;
  Cur cur[ST + 1];
  cur[0] = at_unit(uni(lo), uni(g0 - sm_pre[lo]));
#pragma unroll
  for (int k = 1; k <= ST; ++k) cur[k] = g0 + k < g1 ? advance(cur[k - 1]) : cur[k - 1];

  __shared__ __attribute__((aligned(16))) char kstage[NW][En::KST];
  En en;
  en.init(a, lane, (lds_char*)kstage[wid]);
  if (a.k_hs) en.sc *= a.k_hs[kh];
  en.set_block_scales(kbs, vbs, kh);
  const float v_scale = a.v_hs ? a.v_hs[kh] : a.v_scale;
  const int64_t head_off = (int64_t)kh * D * En::E;
  auto ids_of = [&](const Cur& c) -> Ids {
    const PairRef pr{tables + (int64_t)c.seq * a.max_blocks,
                     c.len > 0 ? (c.len + BS - 1) / BS : 1, c.len, head_off};
    return en.tile_ids(pr, c.t);
  };
  // this lane's query row in a group (column lane & 15), or nullptr
  auto qrow_of = [&](const Cur& c) -> const _Float16* {
    const int col = lane & 15;
    if (col >= c.nm * g) return nullptr;
    return qs + ((int64_t)sm_seq[c.m0 + col / g] * a.num_q_heads + (int64_t)kh * g + col % g) * D;
  };
  float* rec_base = slots + (int64_t)gw * 2 * 16 * (D + 2);

  en.load_q_rows(qrow_of(cur[0]));
  en.reset();
  half4_t qpre[En::NQ];
  int q_grp = -1;
  bool seg_from_start = cur[0].j == 0;
  int seg_start = g0;
  int gt = g0;

  auto finish = [&]() {
    const bool grp_end = cur[0].j + 1 == cur[0].nt;
    if (!(grp_end || gt + 1 == g1)) return;
    const float lt = en.l_total();
    const int m0 = cur[0].m0, ncols = cur[0].nm * g;
    if (seg_from_start && grp_end) {
      en.store_out_cols(
          [&](int h) {
            return outs + ((int64_t)sm_seq[m0 + h / g] * a.num_q_heads + (int64_t)kh * g +
                           h % g) * D;
          },
          ncols, lt, v_scale);
    } else {
      en.store_partial16(rec_base + (seg_start == g0 ? 0 : 1) * 16 * (D + 2), ncols, lt,
                         v_scale);
    }
    if (gt + 1 < g1) {
      if (q_grp == cur[1].s) en.take_q(qpre); else en.load_q_rows(qrow_of(cur[1]));
      q_grp = -1;
      en.reset();
      seg_from_start = true;
      seg_start = gt + 1;
    }
  };

  uint4 kb[ST][En::NKL];
  VT vb[ST][4];
  float4 tsc[ST];
#pragma unroll
  for (int k = 0; k < ST - 1; ++k) {
    if (k > 0 && cur[k].j == 0 && g0 + k < g1 && q_grp < 0) {
      en.load_q_rows_into(qpre, qrow_of(cur[k]));
      q_grp = cur[k].s;
    }
    Ids ik = ids_of(cur[k]);
    ik.live = g0 + k < g1;
    en.issue(ik, kb[k], vb[k], &tsc[k]);
  }
  Ids ids_next = ids_of(cur[ST - 1]);
  ids_next.live = g0 + ST - 1 < g1;
  for (;;) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      if (cur[ST - 1].j == 0 && gt + ST - 1 < g1 && q_grp < 0) {
        en.load_q_rows_into(qpre, qrow_of(cur[ST - 1]));
        q_grp = cur[ST - 1].s;
      }
      {
        // the block ids are read before the loads below are issued; the
        // loads of a unit past the range are dead (a branch around the issue
        // instead cost 8-13%: the waits after it then drain every load)
        Ids ids_new = ids_of(cur[ST]);
        ids_new.live = gt + ST < g1;
        en.issue(ids_next, kb[(st + ST - 1) % ST], vb[(st + ST - 1) % ST], &tsc[(st + ST - 1) % ST]);
        ids_next = ids_new;
      }
      {
        const Cur& c = cur[0];                 // members p .. hi take the tile
        en.template compute<true>(c.t, 0, c.len, kb[st], vb[st], (c.p - c.m0) * g,
                                  (c.hi - c.m0 + 1) * g, tsc[st]);
      }
      finish();
      if (++gt == g1) return;
#pragma unroll
      for (int k = 0; k < ST; ++k) cur[k] = cur[k + 1];
      if (gt + ST < g1) cur[ST] = advance(cur[ST]);
    }
  }
}

// One workgroup per (group, KV head): if the group was cut by range
// boundaries, merge its per-range 16-column records by log-sum-exp, in range
// order (deterministic), and write every member's rows.
template <int D>
__global__ __launch_bounds__(256) void flat_group_merge_kernel(DecodeArgs a, FlatArgs f,
                                                               GroupArgs gp) {
  const int kh = blockIdx.x % a.num_kv_heads, gi = blockIdx.x / a.num_kv_heads;
  const int g = a.gqa, cap = 16 / g, G = gp.num_groups;
  const int64_t T = f.prefix[G];
  const int pre = f.prefix[gi], end = f.prefix[gi + 1];
  if (end == pre) return;
  const int64_t NR = f.num_ranges;
  const int r_first = range_of(pre, T, NR), r_last = range_of(end - 1, T, NR);
  if (r_first == r_last) return;               // written by the decode kernel
  const bool first_is_last_slot = (int64_t)r_first * T / NR < pre;
  const bool some_empty = T < NR;              // else every range owns a unit
  int m0 = gp.member_start[gi], m1 = gp.member_start[gi + 1];
  m0 = m0 < 0 ? 0 : (m0 > gp.num_members ? gp.num_members : m0);
  m1 = m1 < m0 ? m0 : (m1 > gp.num_members ? gp.num_members : m1);
  const int ncols = (m1 - m0 < cap ? m1 - m0 : cap) * g;
  constexpr int Q = D / 4;
  for (int idx = threadIdx.x; idx < ncols * Q; idx += 256) {
    const int h = idx / Q, d = (idx - (idx / Q) * Q) * 4;
    float M = kNegBig, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    // records are loaded whether or not their range owns units (every slot
    // lies inside the workspace); an empty range's record counts as empty,
    // so the loads of several records can be in flight together
#pragma unroll 4
    for (int r = r_first; r <= r_last; ++r) {
      const bool empty = some_empty && range_empty(r, T, NR);
      const int slot = (r == r_first && first_is_last_slot) ? 1 : 0;
      const float* p = f.slots + ((int64_t)(r * a.num_kv_heads + kh) * 2 + slot) * 16 * (D + 2);
      float2 ml = ((const float2*)(p + 16 * D))[h];
      float4 ov = *(const float4*)(p + h * D + d);
      if (empty) {
        ml = make_float2(kNegBig, 0.f);
        ov = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const float mn = fmaxf(M, ml.x);
      const float sa = __builtin_amdgcn_exp2f(M - mn), sb = ml.y * __builtin_amdgcn_exp2f(ml.x - mn);
      L = L * sa + sb;
      O.x = O.x * sa + sb * ov.x;
      O.y = O.y * sa + sb * ov.y;
      O.z = O.z * sa + sb * ov.z;
      O.w = O.w * sa + sb * ov.w;
      M = mn;
    }
    int sq = gp.members[m0 + h / g];
    sq = sq < 0 ? 0 : (sq >= gp.num_seqs ? gp.num_seqs - 1 : sq);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    store_half4(a.out + ((int64_t)sq * a.num_q_heads + (int64_t)kh * g + h % g) * D + d,
                make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv));
  }
}

// ---------------------------------------------------------------- launchers

constexpr int kWaves = PA_DECODE_WAVES;

template <int D, int BS, int KV, bool NT>
hipError_t launch_typed(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                        int32_t num_seqs, int mode, hipStream_t stream) {
  const uint32_t units = (uint32_t)num_seqs * (uint32_t)a.num_kv_heads;
  if (mode == kModeFlat) {
    const size_t lds = sizeof(int) * (2 * (size_t)num_seqs + 1);
    const int64_t waves = (int64_t)f->num_ranges * a.num_kv_heads;
    constexpr int FW = PA_FLAT_WAVES;
    hipLaunchKernelGGL((decode_flat_kernel<D, BS, KV, FW, NT>),
                       dim3((uint32_t)((waves + FW - 1) / FW)), dim3(FW * 64), lds,
                       stream, a, *f, a.block_tables, a.seq_lens, a.q, a.out, f->slots,
                       f->prefix, a.k_bs, a.v_bs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // records per cut sequence ~ ranges / sequences + 1: a power of two of
    // thread sets, each the gqa * D / 4 threads of one (sequence, KV head)
    const int f4 = a.gqa * D / 4;
    const int64_t per_seq = (num_seqs > 0 ? f->num_ranges / num_seqs : 0) + 2;
    int sets = 1;
    while (sets < per_seq && 2 * sets * f4 <= 1024) sets *= 2;
    hipLaunchKernelGGL((flat_merge_heads_kernel<D>), dim3((uint32_t)num_seqs * a.num_kv_heads),
                       dim3((sets * f4 + 63) / 64 * 64), 0, stream, a, *f);
  } else if (mode == kModeFlatGroup) {
    const size_t lds = sizeof(int) * (2 * (size_t)gr->num_groups + 2 + 4 * (size_t)gr->num_members);
    const int64_t waves = (int64_t)f->num_ranges * a.num_kv_heads;
    constexpr int FW = PA_FLAT_WAVES;
    hipLaunchKernelGGL((decode_flat_group_kernel<D, BS, KV, FW, PA_GROUP_NT || NT>),
                       dim3((uint32_t)((waves + FW - 1) / FW)), dim3(FW * 64), lds, stream, a,
                       *f, *gr, a.block_tables, a.seq_lens, a.q, a.out, f->slots, f->prefix,
                       a.k_bs, a.v_bs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((flat_group_merge_kernel<D>),
                       dim3((uint32_t)gr->num_groups * (uint32_t)a.num_kv_heads), dim3(256), 0,
                       stream, a, *f, *gr);
  } else if (mode == kModeGroup) {
    // every tile is read by one wave of one group: streaming loads (a member's
    // own tiles may sit in blocks other members also list past the shared
    // length; those few re-reads go to HBM again)
    hipLaunchKernelGGL((decode_group_kernel<D, BS, KV, PA_GROUP_WAVES, PA_GROUP_NT || NT>),
                       dim3((uint32_t)gr->num_groups * (uint32_t)a.num_kv_heads),
                       dim3(PA_GROUP_WAVES * 64), PA_GROUP_EXTRA_LDS, stream, a, *gr,
                       a.block_tables, a.seq_lens, a.k_bs, a.v_bs);
  } else if (mode == kModeSplit) {
    hipLaunchKernelGGL((decode_kernel<D, BS, KV, kWaves, true, NT>),
                       dim3(units * (uint32_t)a.num_parts), dim3(kWaves * 64), 0, stream, a,
                       a.block_tables, a.seq_lens, a.k_bs, a.v_bs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((lse_reduce_kernel<D>), dim3((uint32_t)num_seqs * (uint32_t)a.num_q_heads),
                       dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, BS, KV, kWaves, false, NT>), dim3(units),
                       dim3(kWaves * 64), 0, stream, a, a.block_tables, a.seq_lens, a.k_bs,
                       a.v_bs);
  }
  return hipGetLastError();
}

template <int D, int BS, int KV>
hipError_t launch_nt(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                     int32_t num_seqs, bool stream_kv, int mode, hipStream_t stream) {
  return stream_kv ? launch_typed<D, BS, KV, true>(a, f, gr, num_seqs, mode, stream)
                   : launch_typed<D, BS, KV, false>(a, f, gr, num_seqs, mode, stream);
}

}  // namespace

// Launchers of one (head_dim, KV format) pair over every block size.  Each
// pair is explicitly instantiated below; the build compiles this file once per
// pair (PA_DECODE_SLICE_D / PA_DECODE_SLICE_KV) so the slices compile in
// parallel, and a plain compile instantiates all of them.
template <int D, int KV>
hipError_t launch_decode_dk(const DecodeArgs& a, const FlatArgs* f, const GroupArgs* gr,
                            int32_t num_seqs, int32_t bs, bool stream_kv, int mode,
                            hipStream_t stream) {
  switch (bs) {
    case 8: return launch_nt<D, 8, KV>(a, f, gr, num_seqs, stream_kv, mode, stream);
    case 16: return launch_nt<D, 16, KV>(a, f, gr, num_seqs, stream_kv, mode, stream);
    case 32: return launch_nt<D, 32, KV>(a, f, gr, num_seqs, stream_kv, mode, stream);
    case 64: return launch_nt<D, 64, KV>(a, f, gr, num_seqs, stream_kv, mode, stream);
    case 128: return launch_nt<D, 128, KV>(a, f, gr, num_seqs, stream_kv, mode, stream);
  }
  return hipErrorInvalidValue;
}

#define PA_DECODE_INSTANTIATE(D, KV)                                                         \
  template hipError_t launch_decode_dk<D, KV>(const DecodeArgs&, const FlatArgs*,            \
                                              const GroupArgs*, int32_t, int32_t, bool, int, \
                                              hipStream_t);
#if defined(PA_DECODE_SLICE_D) && defined(PA_DECODE_SLICE_KV)
PA_DECODE_INSTANTIATE(PA_DECODE_SLICE_D, PA_DECODE_SLICE_KV)
#else
PA_DECODE_INSTANTIATE(64, 0)
PA_DECODE_INSTANTIATE(64, 1)
PA_DECODE_INSTANTIATE(64, 2)
PA_DECODE_INSTANTIATE(128, 0)
PA_DECODE_INSTANTIATE(128, 1)
PA_DECODE_INSTANTIATE(128, 2)
PA_DECODE_INSTANTIATE(256, 0)
PA_DECODE_INSTANTIATE(256, 1)
PA_DECODE_INSTANTIATE(256, 2)
#endif

}  // namespace pa
