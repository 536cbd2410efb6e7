// Segment-causal, action-aware attention forward over an INT8 KV cache (gfx950).
//
// One softmax over the union of visible keys of a video query
// ("Hy-Nomas 拆解" teardown, section "架构": segment-causal plus action-aware
// causal attention); history keys/values are INT8 with fp32 scales and the
// arithmetic is BF16 (same page, "单卡 4090 怎么做到的", first technique).
//
// Work decomposition (template <NW, QB, KT>)
//   block  = one (head, query tile of 32*QB*NW rows); NW waves, each owning
//            QB blocks of 32 query rows.  Every K/V operand a wave reads from
//            LDS feeds QB MFMAs, so QB = 2 halves the LDS traffic per flop.
//   tile   = KT keys of one span of the tile plan, staged in LDS as bf16:
//            K as [key][d] (row pitch 136 elements) and V transposed as
//            [d][key] (row pitch KT+8 elements).  The transposed writes are
//            conflict-free because the 16 lanes that write together hold 16
//            different 4-key groups of the same 8 d values.
//            Global loads are raw buffer loads: per-thread offsets are fixed
//            for the block, each tile adds a scalar offset, and the buffer
//            bound returns 0 past a source's end (no clamping, no branches).
//            INT8 tiles are read from HBM as int8 (half the bytes), converted
//            to bf16 in registers on their way into LDS (int8 -> bf16 is exact),
//            and their fp32 scales are applied after the MFMA: the key scale to
//            the score column, the value scale to the probability.
//   math   = S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (each lane then holds
//            the tile's keys for one query, so the row max/sum are in-lane plus
//            one v_permlane32_swap with lane^32); online softmax in the log2
//            domain with the score scale folded into the exp2 argument; the
//            probabilities are packed to bf16 in registers and used directly
//            as the B operand of O^T = V^T P^T, whose accumulator keeps each
//            query's 128 outputs in its own lane pair.
//   rescale= lazy: the running max only moves (and O, l are rescaled) when a
//            row's tile max exceeds it by more than 8 in log2 units, so
//            probabilities stay <= 2^8 and the rescale is rare after the
//            first tiles.  The result is exact algebra (same max in O and l).
//   masks  = only partial tiles pay for masking: ragged tile ends and action
//            tails whose row range does not cover all of a wave's rows.  Full
//            bf16 tiles take a lean path; INT8 and partial tiles share one
//            general path (bf16 tiles carry unit scales in LDS for it).
//   order  = the plan's span order, KT keys at a time, double-buffered: global
//            loads of tile n+1 are in flight while tile n is computed.
//   grid   = XCD-aware: block b runs on XCD b % 8, and each XCD gets a
//            contiguous range of (head, tile) tasks, so one head's keys and
//            values stay in one XCD's L2.
#include <climits>

#include "hn_internal.h"

namespace hn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float RESCALE_SLACK = 8.0f;  // log2 units the running max may lag
constexpr int KP = D + 8;              // LDS pitch of a K row (bf16 elements)

template <int NW_, int QB_, int KT_>
struct Cfg {
  static constexpr int NW = NW_, QB = QB_, KT = KT_;
  static constexpr int T = 64 * NW;            // threads per block
  static constexpr int ROWS = 32 * QB * NW;    // query rows per block
  static constexpr int KB = KT / 32;           // 32-key blocks per tile
  static constexpr int NT = KT / 16;           // PV MFMAs per d-block
  static constexpr int VP = KT + 8;            // LDS pitch of a V^T row
  static constexpr int NKQ = KT / 4;           // 4-key groups per tile
  static constexpr int VU = NKQ * 16;          // V transpose units (4 keys x 8 d)
  static constexpr int KCH = 16 * KT / T;      // bf16 K 16-byte chunks per thread
  static constexpr int KCH8 = 8 * KT / T;      // INT8 K 16-byte chunks per thread
  static constexpr int VPT = VU >= T ? VU / T : 1;  // V units per thread
  static_assert(KT % 32 == 0 && KCH >= 1 && KCH8 >= 1, "tile shape");
  static_assert(VU % T == 0 || T % VU == 0, "V units");
  static_assert(T % NKQ == 0 || VU >= T, "V mapping");
  static_assert(2 * KT <= T, "one scale per thread");
};

template <class C>
struct Smem {
  __bf16 k[2][C::KT * KP];
  __bf16 vt[2][D * C::VP];
  float ks[2][C::KT];
  float vs[2][C::KT];
};

struct TileDesc {
  int src, kb, nk, r0, r1;
};

// Position of key `key` in a V^T row: bits 2 and 3 swapped, so the 8 keys one
// lane group feeds to a PV MFMA are contiguous.
__device__ inline int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// max / sum of a value and its lane^32 partner
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint4 ld_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline uint2 ld_b64(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}

// Two signed bytes of w (bytes b, b+1) -> packed bf16 pair (exact for |q| <= 127).
__device__ inline uint32_t i8x2_bf16(uint32_t w, int b) {
  const bf16x2 v = {(__bf16)(float)(int8_t)(w >> (8 * b)), (__bf16)(float)(int8_t)(w >> (8 * b + 8))};
  return __builtin_bit_cast(uint32_t, v);
}

template <class C>
struct Prefetch {
  uint4 k[C::KCH];
  uint4 v[C::VPT][4];
  float sc;
};

// Buffer resources of one head's key/value sources and the per-thread
// offsets of its share of a tile (both fixed for the whole block).
struct Sources {
  rsrc_t k_txt, v_txt, k_vid, v_vid;             // bf16, token-major
  rsrc_t k_heads, v_heads, ks_heads, vs_heads;   // INT8 head store + scales
  rsrc_t k_ring, v_ring, ks_ring, vs_ring;       // INT8 ring + scales
  uint32_t tok_bytes;                            // bf16 token stride = H * D * 2
  uint32_t vo_kb, vo_vb;                         // bf16 K / V thread offsets
  uint32_t vo_ki, vo_vi;                         // INT8 K / V thread offsets
  uint32_t vo_sc;                                // scale thread offset
};

// V transpose unit of thread tid (first of its VPT units): 4-key group kq and
// 8-d chunk dc; further units of the thread add T / NKQ to dc.
template <class C>
__device__ inline int v_kq(int tid) { return tid % C::NKQ; }
template <class C>
__device__ inline int v_dc(int tid) { return tid / C::NKQ; }

template <class C>
__device__ inline void init_sources(const AttnParams& p, int h, Sources& S) {
  const int tid = threadIdx.x;
  const uint32_t tb = (uint32_t)p.H * D * 2;
  S.tok_bytes = tb;
  const uint32_t hoff = (uint32_t)h * D * 2;
  const uint32_t txt_bytes = p.txt_len > 0 ? (uint32_t)p.txt_len * tb - hoff : 0u;
  S.k_txt = make_rsrc(p.k_txt + h * D, txt_bytes);
  S.v_txt = make_rsrc(p.v_txt + h * D, txt_bytes);
  S.k_vid = make_rsrc(p.k_vid + h * D, (uint32_t)p.lq * tb - hoff);
  S.v_vid = make_rsrc(p.v_vid + h * D, (uint32_t)p.lq * tb - hoff);
  S.k_heads = make_rsrc(p.heads_k + (int64_t)h * p.head_cap * D, (uint32_t)p.head_cap * D);
  S.v_heads = make_rsrc(p.heads_v + (int64_t)h * p.head_cap * D, (uint32_t)p.head_cap * D);
  S.ks_heads = make_rsrc(p.heads_ks + (int64_t)h * p.head_cap, (uint32_t)p.head_cap * 4);
  S.vs_heads = make_rsrc(p.heads_vs + (int64_t)h * p.head_cap, (uint32_t)p.head_cap * 4);
  S.k_ring = make_rsrc(p.ring_k + (int64_t)h * p.ring_cap * D, (uint32_t)p.ring_cap * D);
  S.v_ring = make_rsrc(p.ring_v + (int64_t)h * p.ring_cap * D, (uint32_t)p.ring_cap * D);
  S.ks_ring = make_rsrc(p.ring_ks + (int64_t)h * p.ring_cap, (uint32_t)p.ring_cap * 4);
  S.vs_ring = make_rsrc(p.ring_vs + (int64_t)h * p.ring_cap, (uint32_t)p.ring_cap * 4);
  const int kq = v_kq<C>(tid), dc = v_dc<C>(tid);
  S.vo_kb = (uint32_t)(tid >> 4) * tb + (tid & 15) * 16;   // key c*T/16 + tid/16, chunk tid%16
  S.vo_vb = (uint32_t)(4 * kq) * tb + dc * 16;             // key 4kq + r, d chunk dc
  S.vo_ki = (uint32_t)(tid >> 3) * D + (tid & 7) * 16;     // key c*T/8 + tid/8, 16 codes
  S.vo_vi = (uint32_t)(4 * kq) * D + dc * 8;               // key 4kq + r, 8 codes
  S.vo_sc = (uint32_t)(tid % C::KT) * 4;
}

template <class C>
__device__ inline bool v_active(int tid) { return C::VU >= C::T || tid < C::VU; }

template <class C>
__device__ inline void load_bf16(const Sources& S, rsrc_t rk, rsrc_t rv, int kb, Prefetch<C>& pf) {
  const uint32_t base = (uint32_t)kb * S.tok_bytes;
#pragma unroll
  for (int c = 0; c < C::KCH; ++c) pf.k[c] = ld_b128(rk, S.vo_kb, base + c * (C::T / 16) * S.tok_bytes);
  if (v_active<C>(threadIdx.x)) {
#pragma unroll
    for (int i = 0; i < C::VPT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pf.v[i][r] = ld_b128(rv, S.vo_vb, base + r * S.tok_bytes + i * (C::T / C::NKQ) * 16);
  }
  pf.sc = 1.0f;
}

template <class C>
__device__ inline void load_i8(const Sources& S, rsrc_t rk, rsrc_t rv, rsrc_t rks, rsrc_t rvs, int kb,
                               int nk, Prefetch<C>& pf) {
  const int tid = threadIdx.x;
  const uint32_t base = (uint32_t)kb * D;
#pragma unroll
  for (int c = 0; c < C::KCH8; ++c) pf.k[c] = ld_b128(rk, S.vo_ki, base + c * (C::T / 8) * D);
  if (v_active<C>(tid)) {
#pragma unroll
    for (int i = 0; i < C::VPT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 w = ld_b64(rv, S.vo_vi, base + r * D + i * (C::T / C::NKQ) * 8);
        pf.v[i][r] = make_uint4(w.x, w.y, 0, 0);
      }
  }
  float sc = 0.0f;
  if (tid < 2 * C::KT) {
    const float v = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(tid < C::KT ? rks : rvs, S.vo_sc, (uint32_t)kb * 4, 0));
    sc = (tid % C::KT) < nk ? v : 0.0f;
  }
  pf.sc = sc;
}

// Global -> registers for one tile.  Keys past the span end read other finite
// data (or 0 past the buffer end) and are masked by the math; their value
// scales are zeroed so that a 0 probability times the scale stays 0.
template <class C>
__device__ inline void load_tile(const Sources& S, const TileDesc& t, Prefetch<C>& pf) {
  if (t.src == SRC_VID) load_bf16<C>(S, S.k_vid, S.v_vid, t.kb, pf);
  else if (t.src == SRC_TXT) load_bf16<C>(S, S.k_txt, S.v_txt, t.kb, pf);
  else if (t.src == SRC_RING) load_i8<C>(S, S.k_ring, S.v_ring, S.ks_ring, S.vs_ring, t.kb, t.nk, pf);
  else load_i8<C>(S, S.k_heads, S.v_heads, S.ks_heads, S.vs_heads, t.kb, t.nk, pf);
}

// Registers -> LDS buffer `b` (bf16 K rows, bf16 V^T rows, scales).
template <class C>
__device__ inline void store_tile(Smem<C>& sm, int b, bool i8, const Prefetch<C>& pf) {
  const int tid = threadIdx.x;
  uint32_t rows[C::VPT][4][4];  // V rows as 4 x (8 bf16) packed words
  if (!i8) {
    // unit scales, so bf16 tiles can take the general (scaled) path too
    if (tid < 2 * C::KT) (tid < C::KT ? sm.ks[b][tid] : sm.vs[b][tid - C::KT]) = 1.0f;
#pragma unroll
    for (int c = 0; c < C::KCH; ++c) {
      const int key = c * (C::T / 16) + (tid >> 4), dch = tid & 15;
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 8]) = pf.k[c];
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rows[i][r][0] = pf.v[i][r].x; rows[i][r][1] = pf.v[i][r].y;
        rows[i][r][2] = pf.v[i][r].z; rows[i][r][3] = pf.v[i][r].w;
      }
  } else {
#pragma unroll
    for (int c = 0; c < C::KCH8; ++c) {
      const int key = c * (C::T / 8) + (tid >> 3), dch = tid & 7;
      const uint4 w = pf.k[c];
      uint4 lo, hi;
      lo.x = i8x2_bf16(w.x, 0); lo.y = i8x2_bf16(w.x, 2);
      lo.z = i8x2_bf16(w.y, 0); lo.w = i8x2_bf16(w.y, 2);
      hi.x = i8x2_bf16(w.z, 0); hi.y = i8x2_bf16(w.z, 2);
      hi.z = i8x2_bf16(w.w, 0); hi.w = i8x2_bf16(w.w, 2);
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 16]) = lo;
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 16 + 8]) = hi;
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rows[i][r][0] = i8x2_bf16(pf.v[i][r].x, 0); rows[i][r][1] = i8x2_bf16(pf.v[i][r].x, 2);
        rows[i][r][2] = i8x2_bf16(pf.v[i][r].y, 0); rows[i][r][3] = i8x2_bf16(pf.v[i][r].y, 2);
      }
    if (tid < C::KT) sm.ks[b][tid] = pf.sc;
    else if (tid < 2 * C::KT) sm.vs[b][tid - C::KT] = pf.sc;
  }
  if (!v_active<C>(tid)) return;
  // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
  const int pos = vt_pos(4 * v_kq<C>(tid));
#pragma unroll
  for (int i = 0; i < C::VPT; ++i) {
    const int dc = v_dc<C>(tid) + i * (C::T / C::NKQ);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int d0 = dc * 8 + 2 * w;
      uint2 e, o;
      e.x = __builtin_amdgcn_perm(rows[i][1][w], rows[i][0][w], 0x05040100u);
      e.y = __builtin_amdgcn_perm(rows[i][3][w], rows[i][2][w], 0x05040100u);
      o.x = __builtin_amdgcn_perm(rows[i][1][w], rows[i][0][w], 0x07060302u);
      o.y = __builtin_amdgcn_perm(rows[i][3][w], rows[i][2][w], 0x07060302u);
      *reinterpret_cast<uint2*>(&sm.vt[b][d0 * C::VP + pos]) = e;
      *reinterpret_cast<uint2*>(&sm.vt[b][(d0 + 1) * C::VP + pos]) = o;
    }
  }
}

__device__ inline bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ inline bf16x8 pack_p(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

struct RowState {
  float m;   // running max (log2 units) of this lane's query
  float l;   // this lane's partial sum of probabilities (partner holds the rest)
};

// One KT-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
//   I8   : general path: per-key scales from LDS (1 for bf16 tiles), masking
//   MASK : some keys (ragged end) or rows (tail window) of the tile are invisible
// The QK MFMAs of all 32-key blocks are issued first; then each block's
// softmax runs while the next block's MFMAs are still in flight, and its PV
// MFMAs run while the following block's softmax is computed.
template <class C, bool I8, bool MASK>
__device__ __forceinline__ void tile_math(const Smem<C>& sm, int buf, const bf16x8 (&qreg)[C::QB][8],
                                          f32x16 (&acc)[C::QB][4], RowState (&st)[C::QB],
                                          float scale_log2, int nk, const bool (&row_ok)[C::QB]) {
  constexpr int QB = C::QB, KB = C::KB;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const __bf16* kl = sm.k[buf];
  const __bf16* vl = sm.vt[buf];

  f32x16 s[QB][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int q = 0; q < QB; ++q) s[q][kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 kk = ld8(kl + (kb * 32 + l32) * KP + 16 * t + 8 * g);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        s[q][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[q][t], s[q][kb], 0, 0, 0);
    }
  }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    bf16x8 pb[QB][2];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      // scores in log2 units; element 4r+i is key kb*32 + 8r + 4g + i
      float mx;
      if (I8 || MASK) {
        mx = -INFINITY;
        const int nkg = row_ok[q] ? nk - 4 * g : INT_MIN;  // key visible iff kb*32+8r+i < nkg
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 ksc = *reinterpret_cast<const float4*>(&sm.ks[buf][kb * 32 + 8 * r + 4 * g]);
          const float cc[4] = {ksc.x * scale_log2, ksc.y * scale_log2, ksc.z * scale_log2,
                               ksc.w * scale_log2};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[q][kb][4 * r + i] * cc[i];
            if (MASK && kb * 32 + 8 * r + i >= nkg) v = -INFINITY;
            s[q][kb][4 * r + i] = v;
            mx = fmaxf(mx, v);
          }
        }
      } else {
        // every key visible and one scale: take the max of the raw scores
        float m0 = s[q][kb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m0 = fmaxf(m0, s[q][kb][i]);
        mx = m0 * scale_log2;
      }
      mx = pair_max(mx);

      // lazy rescale: move the running max only when it lags by more than the slack
      if (__any(mx > st[q].m + RESCALE_SLACK)) {
        const float m_new = fmaxf(st[q].m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st[q].m - m_new);
        st[q].m = m_new;
        st[q].l *= alpha;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[q][c] *= alpha;
      }
      const float m_use = (st[q].m == -INFINITY) ? 0.0f : st[q].m;

      float pv[16];
      if (I8 || MASK) {
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 vsc = *reinterpret_cast<const float4*>(&sm.vs[buf][kb * 32 + 8 * r + 4 * g]);
          const float vv[4] = {vsc.x, vsc.y, vsc.z, vsc.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e2 = __builtin_amdgcn_exp2f(s[q][kb][4 * r + i] - m_use);
            psum += e2;
            pv[4 * r + i] = e2 * vv[i];
          }
        }
        st[q].l += psum;
        pb[q][0] = pack_p(pv);
        pb[q][1] = pack_p(pv + 8);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][kb][i], scale_log2, -m_use));
        pb[q][0] = pack_p(pv);
        pb[q][1] = pack_p(pv + 8);
        // row sum of the bf16 probabilities the PV MFMA uses (dot with ones)
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        float l = st[q].l;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 pp = {pb[q][h2][2 * j], pb[q][h2][2 * j + 1]};
            l = __builtin_amdgcn_fdot2_f32_bf16(pp, one, l, false);
          }
        st[q].l = l;
      }
    }

    // O^T += V^T P^T for this 32-key block
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 32 * c + l32;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 vv = ld8(vl + d * C::VP + 32 * kb + 16 * t + 8 * g);
#pragma unroll
        for (int q = 0; q < QB; ++q)
          acc[q][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[q][t], acc[q][c], 0, 0, 0);
      }
    }
  }
}

template <class C, int MIN_BLOCKS>
__global__ __launch_bounds__(C::T, MIN_BLOCKS) void seg_attn_fwd_kernel(AttnParams p) {
  constexpr int QB = C::QB;
  __shared__ Smem<C> sm;
  const int task = (blockIdx.x & 7) * p.tasks_per_xcd + (blockIdx.x >> 3);
  if (task >= p.n_tasks) return;  // whole block leaves before any barrier
  const int h = task / p.n_qtiles;
  const int qt = task - h * p.n_qtiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int wrow0 = qt * C::ROWS + wave * 32 * QB;  // first row of this wave
  int row[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) row[q] = wrow0 + 32 * q + l32;

  // Q^T as the B operand: lane (q, g) holds Q[q][16t + 8g .. +8] for t = 0..7;
  // rows past the segment read as 0
  bf16x8 qreg[QB][8];
  {
    const uint32_t tb = (uint32_t)p.H * D * 2;
    const rsrc_t rq = make_rsrc(p.q + h * D, (uint32_t)p.lq * tb - (uint32_t)h * D * 2);
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qreg[q][t] = __builtin_bit_cast(bf16x8, ld_b128(rq, (uint32_t)row[q] * tb + 16 * g, 32 * t));
  }
  Sources S;
  init_sources<C>(p, h, S);

  f32x16 acc[QB][4];
  RowState st[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[q][c] = f32x16{};
    st[q].m = -INFINITY;
    st[q].l = 0.0f;
  }

  const int n_spans = p.counts[qt];
  const Span* spans = p.spans + (int64_t)qt * p.max_spans;

  // tile iterator over the spans (block-uniform)
  int e = 0;
  int kpos = n_spans > 0 ? spans[0].k0 : 0;
  auto next_tile = [&](TileDesc& t) -> bool {
    if (e >= n_spans) return false;
    const Span s = spans[e];
    t.src = s.src;
    t.kb = kpos;
    t.nk = min(C::KT, s.k1 - kpos);
    t.r0 = s.r0;
    t.r1 = s.r1;
    kpos += t.nk;
    if (kpos >= s.k1) {
      ++e;
      if (e < n_spans) kpos = spans[e].k0;
    }
    return true;
  };

  TileDesc cur, nxt;
  bool have = next_tile(cur);
  Prefetch<C> pf;
  if (have) {
    load_tile<C>(S, cur, pf);
    store_tile<C>(sm, 0, cur.src < SRC_TXT, pf);
  }
  __syncthreads();
  int buf = 0;
  while (have) {
    const bool have_next = next_tile(nxt);
    if (have_next) load_tile<C>(S, nxt, pf);

    // rows of this wave that see the tile; skip the math if none does
    const int wrows = 32 * QB;
    const bool wave_live = (cur.r0 < wrow0 + wrows) && (cur.r1 > wrow0);
    if (wave_live) {
      const bool rows_all = (cur.r0 <= wrow0) && (cur.r1 >= wrow0 + wrows);
      bool row_ok[QB];
#pragma unroll
      for (int q = 0; q < QB; ++q) row_ok[q] = row[q] >= cur.r0 && row[q] < cur.r1;
      const bool mask = (cur.nk < C::KT) || !rows_all;
      const float sl = p.scale_log2;
      // two code paths only (more would raise register pressure past two
      // waves per SIMD): unmasked bf16 tiles, and everything else
      if (cur.src < SRC_TXT || mask) tile_math<C, true, true>(sm, buf, qreg, acc, st, sl, cur.nk, row_ok);
      else tile_math<C, false, false>(sm, buf, qreg, acc, st, sl, cur.nk, row_ok);
    }

    if (have_next) store_tile<C>(sm, buf ^ 1, nxt.src < SRC_TXT, pf);
    __syncthreads();
    cur = nxt;
    have = have_next;
    buf ^= 1;
  }

  // epilogue: O = acc / l, lse = (m + log2 l) * ln 2
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const float l_tot = pair_sum(st[q].l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (row[q] < p.lq) {
      __bf16* orow = p.o + ((int64_t)row[q] * p.H + h) * D;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * c + 8 * r + 4 * g;
          const bf16x2 lo = {(__bf16)(acc[q][c][4 * r + 0] * inv), (__bf16)(acc[q][c][4 * r + 1] * inv)};
          const bf16x2 hi = {(__bf16)(acc[q][c][4 * r + 2] * inv), (__bf16)(acc[q][c][4 * r + 3] * inv)};
          *reinterpret_cast<uint2*>(orow + d0) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
      }
      if (p.lse != nullptr && g == 0) {
        p.lse[(int64_t)h * p.lq + row[q]] =
            l_tot > 0.0f ? (st[q].m + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
      }
    }
  }
}

// Dense and keep-list plans both use 128-row blocks of 4 waves x 32 rows with
// two blocks per CU (two waves per SIMD from independent blocks, which drift
// out of phase so one block's MFMAs overlap the other's softmax).  Measured
// alternatives: 8-wave 256-row blocks (c3/c4 slower), 4 waves x 64 rows at
// one wave per SIMD (much slower), 128-key tiles (spill).
#ifndef HN_DENSE_NW
#define HN_DENSE_NW 4
#endif
#ifndef HN_DENSE_QB
#define HN_DENSE_QB 1
#endif
#ifndef HN_DENSE_MINB
#define HN_DENSE_MINB 2
#endif
using DenseCfg = Cfg<HN_DENSE_NW, HN_DENSE_QB, 64>;
using SparseCfg = Cfg<4, 1, 64>;
static_assert(SparseCfg::ROWS == HN_TILE, "keep-list blocks must match the keep-list tile");

}  // namespace

int attn_dense_rows() { return DenseCfg::ROWS; }

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  if (p.n_tasks == 0) return hipSuccess;
  const int blocks = 8 * p.tasks_per_xcd;
  if (p.tile_rows == DenseCfg::ROWS) {
    hipLaunchKernelGGL((seg_attn_fwd_kernel<DenseCfg, HN_DENSE_MINB>), dim3(blocks), dim3(DenseCfg::T), 0, s, p);
  } else if (p.tile_rows == SparseCfg::ROWS) {
    hipLaunchKernelGGL((seg_attn_fwd_kernel<SparseCfg, 2>), dim3(blocks), dim3(SparseCfg::T), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hn
