// Segment-causal, action-aware attention forward over an INT8 KV cache (gfx950).
//
// One softmax over the union of visible keys of a video query
// ("Hy-Nomas 拆解" teardown, section "架构": segment-causal plus action-aware
// causal attention); history keys/values are INT8 with fp32 scales and the
// arithmetic is 16-bit (same page, "单卡 4090 怎么做到的", first technique):
// bf16 for the segment's own keys and values, fp16 for the dequantized
// history (see "tile" below).
//
// Work decomposition (template <NW, QB, KT, QL, SW>)
//   block  = one (head, query tile of 32*QB*NW rows); NW waves, each owning
//            QB blocks of 32 query rows.  Every K/V operand a wave reads from
//            LDS feeds QB MFMAs; QB = 2 would halve the LDS traffic per flop
//            but needs more than 256 VGPRs (one wave per SIMD), which measured
//            slower, so the instances below use QB = 1: for dense plans 8
//            waves x 32 rows (Q in registers) or 12 waves x 32 rows (three
//            per SIMD; Q in LDS, QL, and the first SW = 8 waves staging; the
//            bf16-only instance keeps five of a wave's eight Q chunks in
//            registers as well), one block per CU, whichever the plan chose; 4 waves x 32 rows, two
//            blocks per CU, for keep-list plans (the keep list's 128-row
//            query tile).
//   tile   = KT keys of one span of the tile plan, staged in LDS as bf16 in
//            operand-major order, so that every MFMA operand a wave reads is
//            64 consecutive slots (conflict-free); the V^T operand of the PV
//            MFMA comes from gfx950's transposing ds_read_b64_tr_b16, so V is
//            never transposed in registers.  bf16 tiles travel L2 -> LDS by
//            buffer loads that write LDS directly (no registers, no ds_write);
//            per-lane offsets are fixed for the block, each tile adds a scalar
//            offset, and the buffer bound returns 0 past a source's end.
//            INT8 tiles are read from HBM as int8 (half the bytes) with their
//            per-token fp32 scales and dequantized in registers on their way
//            into LDS, so the math never sees a scale.  They are staged and
//            multiplied in fp16, not bf16: K' = fp16(code x fp16(scale)) and
//            V' = fp16(code x 2^-7 x fp16(scale)), in packed fp16 arithmetic,
//            against an fp16 copy of Q and fp16 probabilities that carry the
//            2^7 back.  fp16 keeps 11 significant bits where bf16 keeps 8,
//            which bounds the error of the dequantized history 4x tighter (two
//            fp16 roundings against one bf16 rounding) at the same nominal
//            MFMA rate; the power-of-two shifts keep K', V' and P inside
//            fp16's range.  A tile whose scales would leave that range (|K|
//            above 65,024 or |V| above 8.3e6) falls back to bf16 K and V.
//   math   = S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (_f16 on the INT8
//            tiles; each lane then holds the tile's keys for one query, so the
//            row max/sum are in-lane plus one v_permlane32_swap with lane^32);
//            online softmax in the log2 domain with the score scale folded into
//            the exp2 argument; the probabilities are packed to bf16 (fp16 on
//            INT8 tiles) in registers and used directly as the B operand of
//            O^T = V^T P^T, whose accumulator keeps each query's 128 outputs
//            in its own lane pair.
//   rescale= lazy: the running max only moves (and O, l are rescaled) when a
//            row's tile max exceeds it by more than 8 in log2 units, so
//            probabilities stay <= 2^8 and the rescale is rare after the
//            first tiles.  The result is exact algebra (same max in O and l).
//   masks  = only partial tiles pay for masking: ragged tile ends and action
//            tails whose row range does not cover all of a wave's rows.  Full
//            tiles of any source take a lean path.
//   order  = the plan's span order, KT keys at a time, double-buffered: global
//            loads of tile n+1 are in flight while tile n is computed.
//   grid   = XCD-aware: block b runs on XCD b % 8, and each XCD gets a
//            contiguous range of (head, tile) tasks, so one head's keys and
//            values stay in one XCD's L2; with a hybrid key split, the whole
//            query tiles first and then the split pieces, on every XCD.
#include <climits>
#include <type_traits>

#include "hn_internal.h"

namespace hn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

#ifndef HN_KLOOK
#define HN_KLOOK 5
#endif
#ifndef HN_VLOOK
#define HN_VLOOK 4
#endif
// QL, bf16-only instance (384-row blocks on the segment's own keys): the
// first QRES 16-d chunks of the wave's Q stay in registers and only the rest
// are read from LDS every tile, the others QLOOK chunks ahead; K and V
// operands are read KLOOK / VLOOK MFMAs ahead.  With 166 of the 168 VGPRs
// three waves per SIMD allow, resident Q chunks trade against operand
// lookahead; on the 480x832 segment (ms per launch, two passes each, same
// run) QRES/KLOOK/VLOOK/QLOOK 0/4/3/2 1.0667, 2/4/3/2 1.0612; on another
// box 2/4/3/2 1.0484, 4/2/3/2 1.0437, 4/2/2/2 1.0433, 5/2/2/1 1.0420,
// 5/2/3/1 1.0429, 4/3/2/1 1.0439, 4/3/3/1 1.0452, 5/1/3/2 1.0567,
// 6/1/2/2 1.0537 (one K operand ahead is too few); combinations that spill
// were not run.
#ifndef HN_QL_KLOOK
#define HN_QL_KLOOK 2
#endif
#ifndef HN_QL_VLOOK
#define HN_QL_VLOOK 2
#endif
#ifndef HN_QL_QLOOK
#define HN_QL_QLOOK 1
#endif
#ifndef HN_QL_QRES
#define HN_QL_QRES 5
#endif
#ifndef HN_QLI_KLOOK
#define HN_QLI_KLOOK 4
#endif
#ifndef HN_QLI_VLOOK
#define HN_QLI_VLOOK 2
#endif
#ifndef HN_QLI_QLOOK
#define HN_QLI_QLOOK 2
#endif
constexpr float RESCALE_SLACK = 8.0f;  // log2 units the running max may lag
// fp16 staging of INT8 tiles.  Probabilities are <= 2^RESCALE_SLACK, so with
// the 2^7 shift they stay <= 2^15; codes are <= 127 in magnitude, so
// K' = code x ks fits fp16 (max 65504) for ks <= 512, and V' = code x 2^-7 x
// vs for any scale fp16 holds (vs <= 65504).
constexpr float P_SHIFT = 7.0f;
constexpr float KS_MAX_F16 = 512.0f;
constexpr float VS_MAX_F16 = 65504.0f;
// QL: Q lives in LDS (each wave's rows in a region of its own, operand-major)
// instead of registers; the first SW waves stage the tiles.
template <int NW_, int QB_, int KT_, bool QL_ = false, int SW_ = NW_>
struct Cfg {
  static constexpr int NW = NW_, QB = QB_, KT = KT_, SW = SW_;
  static constexpr bool QL = QL_;
  static constexpr int T = 64 * NW;            // threads per block
  static constexpr int ROWS = 32 * QB * NW;    // query rows per block
  static constexpr int KB = KT / 32;           // 32-key blocks per tile
  static constexpr int KBLK = KB * 8;          // 1 KB K-operand blocks per tile
  static constexpr int VBLK = 4 * KB * 2;      // 1 KB V-operand block pairs per tile
  static constexpr int CH8 = 8 * KT / (64 * SW);  // INT8 16-byte chunks per staging thread (K and V each)
  static constexpr int RG = KT / 64;           // INT8 staging: 64-row groups; wave w takes rows
                                               // 64 (w % RG) + lane, chunks of 16 codes w / RG + c SW/RG
  static_assert(KT == 64 || KT == 128, "tile shape");
  static_assert(SW <= NW && SW % 4 == 0, "staging waves: whole SIMD rounds");
  static_assert(KBLK % SW == 0 && VBLK % SW == 0 && CH8 >= 1 && SW % RG == 0, "load split");
  static_assert(2 * KT <= T, "one scale per thread");
  static_assert(!QL || QB == 1, "Q in LDS: one 32-row block per wave");
};

// LDS tiles are stored operand-major, so that every operand read of a wave is
// 64 consecutive 16-byte (K) or 8-byte (V) slots.
//   K block (kb, t), 1 KB: slot lane = 32g + q holds K[kb*32 + q][16t + 8g .. +8],
//     the A operand of the QK MFMA of 16-d chunk t for lane (q, g).
//   V blocks, 512 bytes each, indexed ((c*KB + kb)*2 + h)*2 + half: slot L
//     (16-lane group G = L/16, s = L%16, g = L/32) holds the four values
//     V[kb*32 + 16h + 8*half + 4g + s/4][32c + 16(G&1) + 4(s&3) .. +4]; one
//     ds_read_b64_tr_b16 of the block gives lane (d, g) keys 16h + 8*half + 4g
//     + {0..3} of column d, the keys its P register holds.
// One LDS stage.  The kernel keeps two stages as separate __shared__ objects
// (never one array indexed by a runtime stage number) so that the compiler can
// tell the stage being read from the stage being filled by direct-to-LDS loads
// and does not wait for those loads before reading.
template <class C>
struct Stage {
  __bf16 k[C::KT * D];
  __bf16 v[C::KT * D];
};
// Q of the block in LDS (QL): wave w's 32 rows at [w * 32 * D, ...), 16-d
// chunk t as the 1 KB B operand of the QK MFMA (slot lane = 32g + q holds
// Q[q][16t + 8g .. +8]).
template <class C>
struct QStore {
  __bf16 q[C::QL ? C::ROWS * D : 8];
};

struct TileDesc {
  int src, kb, nk, r0, r1;
  // INT8 tile staged in fp16 whose scales fit fp16's range (set when the
  // tile is stored)
  bool ok16;
};

// Maximum of two scores as gfx950's v_maximum3_f32 takes it (a NaN wins, as
// it would in any case through the exponentials): unlike fmaxf it needs no
// quieting of the MFMA results first, two instructions fewer per 16 scores.
__device__ inline float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum of a value and its lane^32 partner
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint4 ld_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16 bytes per lane straight into LDS: lane l's bytes land at dst + 16 l.
__device__ inline void ld_lds16(rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// Four INT8 codes of w times the row scale sc -> two packed bf16 pairs.
// With u = q + 128 (the codes' bytes xor 0x80), fma(u, sc, -128 sc) is the
// correctly rounded fp32 product q * sc (128 sc is exact), then rounded to
// bf16.
__device__ inline void i8x4_dequant_bf16(uint32_t w, float sc, float m128, uint32_t& p0, uint32_t& p1) {
  const uint32_t u = w ^ 0x80808080u;
  const float f0 = __builtin_fmaf((float)(u & 0xffu), sc, m128);
  const float f1 = __builtin_fmaf((float)((u >> 8) & 0xffu), sc, m128);
  const float f2 = __builtin_fmaf((float)((u >> 16) & 0xffu), sc, m128);
  const float f3 = __builtin_fmaf((float)(u >> 24), sc, m128);
  const bf16x2 a = {(__bf16)f0, (__bf16)f1};
  const bf16x2 b = {(__bf16)f2, (__bf16)f3};
  p0 = __builtin_bit_cast(uint32_t, a);
  p1 = __builtin_bit_cast(uint32_t, b);
}
// Four INT8 codes of w times the fp16 row scale s2 -> two packed fp16 pairs,
// in packed fp16 arithmetic: the byte u = q + 128 placed under the fp16
// exponent of 1024 is the fp16 value 1024 + u (ulp 1 there), so one byte
// permute makes two of them, one packed subtraction of 1152 gives q exactly
// (SHIFT: one packed fma x 2^-7 - 9 gives q x 2^-7 exactly), and one packed
// multiply gives fp16(q x s2) (x 2^-7), rounded once.  (7 VALU operations
// per 4 codes against 11 for the fp32 product and conversion.)  The shift
// goes on the exact code, not on the scale, so that scales of rows with
// |V| >= 0.0078 stay in fp16's normal range.
template <bool SHIFT>
__device__ inline void i8x4_dequant_f16(uint32_t w, f16x2 s2, uint32_t& p0, uint32_t& p1) {
  const uint32_t u = w ^ 0x80808080u;
  // bytes 4-7 of the permute's source are 0x64: codes 0, 1 -> halves of p0
  const f16x2 e0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  const f16x2 e1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
  f16x2 q0, q1;
  if constexpr (SHIFT) {
    const f16x2 sh = {(_Float16)0x1p-7f, (_Float16)0x1p-7f};
    const f16x2 nine = {(_Float16)-9.0f, (_Float16)-9.0f};
    q0 = __builtin_elementwise_fma(e0, sh, nine);  // (1024 + u) / 128 - 9 = q / 128
    q1 = __builtin_elementwise_fma(e1, sh, nine);
  } else {
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    q0 = e0 - bias;
    q1 = e1 - bias;
  }
  p0 = __builtin_bit_cast(uint32_t, q0 * s2);
  p1 = __builtin_bit_cast(uint32_t, q1 * s2);
}
// 16 INT8 codes of one row -> 16 dequantized 16-bit values (two 16-byte
// words): fp16 (F16, scale rounded to fp16 first; SHIFT: times 2^-7) or
// bf16.
template <bool F16, bool SHIFT = false>
__device__ inline void i8x16_dequant(uint4 w, float sc, uint4& lo, uint4& hi) {
  if constexpr (F16) {
    const _Float16 h = (_Float16)sc;
    const f16x2 s2 = {h, h};
    i8x4_dequant_f16<SHIFT>(w.x, s2, lo.x, lo.y);
    i8x4_dequant_f16<SHIFT>(w.y, s2, lo.z, lo.w);
    i8x4_dequant_f16<SHIFT>(w.z, s2, hi.x, hi.y);
    i8x4_dequant_f16<SHIFT>(w.w, s2, hi.z, hi.w);
  } else {
    const float m128 = -128.0f * sc;
    i8x4_dequant_bf16(w.x, sc, m128, lo.x, lo.y);
    i8x4_dequant_bf16(w.y, sc, m128, lo.z, lo.w);
    i8x4_dequant_bf16(w.z, sc, m128, hi.x, hi.y);
    i8x4_dequant_bf16(w.w, sc, m128, hi.z, hi.w);
  }
}

template <class C>
struct Prefetch {  // INT8 tiles only
  uint4 k[C::CH8];
  uint4 v[C::CH8];
  float ks, vs;  // scales of this thread's row
  bool ok;       // the row is one of the tile's valid keys
};

// Buffer resources of one head's key/value sources and the per-lane offsets
// of the operand-major loads (all fixed for the whole block).
struct Sources {
  rsrc_t k_txt, v_txt, k_vid, v_vid;             // bf16, token-major
  rsrc_t k_heads, v_heads, ks_heads, vs_heads;   // INT8 head store + scales
  rsrc_t k_ring, v_ring, ks_ring, vs_ring;       // INT8 ring + scales
  uint32_t tok_bytes;                            // bf16 token stride = H * D * 2
  uint32_t vo_k, vo_v;                           // bf16 direct-load lane offsets
  uint32_t vo_i;                                 // INT8 lane offset (row lane%64, 16 codes)
  uint32_t vo_sc;                                // scale lane offset
};

template <class C>
__device__ inline void init_sources(const AttnParams& p, int h, Sources& S) {
  const int tid = threadIdx.x, lane = tid & 63;
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
  // K block slot lane = 32g + q  <-  row q, 16-byte chunk g (of the block's 32 bytes)
  S.vo_k = (uint32_t)(lane & 31) * tb + (lane >> 5) * 16;
  // V block pair: lane i feeds slots 2(i%32), 2(i%32)+1 of block half i/32:
  //   row 8(i/32) + 4((i/16)%2) + (i/2)%4, column 16((i/8)%2) + 8(i%2)
  S.vo_v = (uint32_t)(8 * (lane >> 5) + 4 * ((lane >> 4) & 1) + ((lane >> 1) & 3)) * tb +
           (16 * ((lane >> 3) & 1) + 8 * (lane & 1)) * 2;
  S.vo_i = (uint32_t)lane * D;
  S.vo_sc = (uint32_t)(tid % C::KT) * 4;
}

// bf16 tile: every K and V byte goes straight from L2 into its LDS slot.
template <class C>
__device__ inline void load_bf16(const Sources& S, rsrc_t rk, rsrc_t rv, int kb, Stage<C>& sb) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
  const uint32_t base = (uint32_t)kb * S.tok_bytes;
#pragma unroll
  for (int j = 0; j < C::KBLK / C::SW; ++j) {
    const int blk = wave * (C::KBLK / C::SW) + j;          // (kb32, t) = (blk / 8, blk % 8)
    ld_lds16(rk, &sb.k[blk * 512], S.vo_k, base + (blk >> 3) * 32 * S.tok_bytes + (blk & 7) * 32);
  }
#pragma unroll
  for (int j = 0; j < C::VBLK / C::SW; ++j) {
    const int pr = wave * (C::VBLK / C::SW) + j;           // ((c*KB + kb32)*2 + h)
    const int c = pr / (2 * C::KB), kb32 = (pr / 2) % C::KB, h = pr & 1;
    ld_lds16(rv, &sb.v[pr * 512], S.vo_v, base + (kb32 * 32 + 16 * h) * S.tok_bytes + 64 * c);
  }
}

template <class C>
__device__ inline void load_i8(const Sources& S, rsrc_t rk, rsrc_t rv, rsrc_t rks, rsrc_t rvs, int kb,
                               int nk, Prefetch<C>& pf) {
  // wave index made scalar so that offsets and descriptors stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave % C::RG;                         // row group of this wave
  const uint32_t base = (uint32_t)(kb + 64 * rg) * D;
  if (C::SW == C::NW || wave < C::SW) {
#pragma unroll
    for (int c = 0; c < C::CH8; ++c) {
      const uint32_t dch = c * (C::SW / C::RG) + wave / C::RG;  // 16-code chunk of row 64 rg + lane
      pf.k[c] = ld_b128(rk, S.vo_i, base + dch * 16);
      pf.v[c] = ld_b128(rv, S.vo_i, base + dch * 16);
    }
  }
  // every thread dequantizes its row, so every thread needs its scales
  // (vo_sc = (tid % KT) * 4 addresses row 64 rg + lane)
  const bool ok = (int)(threadIdx.x & 63) + 64 * rg < nk;
  const float ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, S.vo_sc, (uint32_t)kb * 4, 0));
  const float vs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, S.vo_sc, (uint32_t)kb * 4, 0));
  pf.ks = ks;  // used only after the current tile's math: no wait here
  pf.vs = vs;
  pf.ok = ok;
}

// INT8 tile: convert and write the operand-major layouts (row r = 64 rg + lane,
// codes [16 dch, 16 dch + 16)), in fp16 (F16) or bf16.
template <class C, bool F16>
__device__ inline void store_i8_as(Stage<C>& sb, const Prefetch<C>& pf, float ks, float vs) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int r = (tid & 63) + 64 * (wave % C::RG);
  const int kb32 = r >> 5, q32 = r & 31;
  // V slot coordinates of row r
  const int h = (r >> 4) & 1, half = (r >> 3) & 1, g = (r >> 2) & 1, qq = r & 3;
#pragma unroll
  for (int c8 = 0; c8 < C::CH8; ++c8) {
    const int dch = c8 * (C::SW / C::RG) + wave / C::RG;
    uint4 lo, hi;
    i8x16_dequant<F16>(pf.k[c8], ks, lo, hi);
    // d chunks 2dch (g=0) and 2dch+1 (g=1) of K block (kb32, t = dch)
    __bf16* kblk = &sb.k[(kb32 * 8 + dch) * 512];
    *reinterpret_cast<uint4*>(kblk + q32 * 8) = lo;
    *reinterpret_cast<uint4*>(kblk + (32 + q32) * 8) = hi;
    i8x16_dequant<F16, F16>(pf.v[c8], vs, lo, hi);  // fp16 V carries 2^-P_SHIFT
    // columns 16 dch .. +16 -> c = dch / 2, G&1 = dch % 2, slots 16G + 4qq + {0..3}
    const int c = dch >> 1, G = 2 * g + (dch & 1);
    __bf16* vblk = &sb.v[(((c * C::KB + kb32) * 2 + h) * 2 + half) * 256];
    *reinterpret_cast<uint4*>(vblk + (16 * G + 4 * qq) * 4) = lo;
    *reinterpret_cast<uint4*>(vblk + (16 * G + 4 * qq) * 4 + 8) = hi;
  }
}
// Stages an INT8 tile: in fp16 (F16: K' = code x fp16(ks), V' = code x 2^-
// P_SHIFT x fp16(vs), products rounded to fp16; t.ok16 says whether every
// scale of the tile fits fp16's range, which every wave decides alike since
// each holds the scales of all the tile's rows), or in bf16 (code x scale
// rounded to bf16).
template <class C, bool F16>
__device__ inline void store_i8(TileDesc& t, Stage<C>& sb, const Prefetch<C>& pf) {
  static_assert(C::RG == 1, "the staging decision needs every row's scale in every wave");
  // rows past the tile's valid keys become zeros
  const float ks = pf.ok ? pf.ks : 0.0f, vs = pf.ok ? pf.vs : 0.0f;
  const bool stager = C::SW == C::NW || __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < C::SW;
  if constexpr (F16) {
    t.ok16 = !__any(!(ks <= KS_MAX_F16 && vs <= VS_MAX_F16));
    if (stager) store_i8_as<C, true>(sb, pf, ks, vs);
  } else {
    if (stager) store_i8_as<C, false>(sb, pf, ks, vs);
  }
}

// Start loading tile t into LDS buffer b: bf16 tiles land in LDS directly;
// INT8 tiles go to registers and are stored by finish_tile (I8: 0 = no INT8
// tiles, 1 = staged in fp16, 2 = staged in bf16).
template <class C, int I8>
__device__ inline void start_tile(const Sources& S, const TileDesc& t, Stage<C>& sb, Prefetch<C>& pf) {
  if (t.src >= SRC_TXT) {
    if (C::SW < C::NW && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= C::SW) return;
    if (t.src == SRC_VID) load_bf16<C>(S, S.k_vid, S.v_vid, t.kb, sb);
    else load_bf16<C>(S, S.k_txt, S.v_txt, t.kb, sb);
  } else if constexpr (I8 != 0) {
    if (t.src == SRC_RING) load_i8<C>(S, S.k_ring, S.v_ring, S.ks_ring, S.vs_ring, t.kb, t.nk, pf);
    else load_i8<C>(S, S.k_heads, S.v_heads, S.ks_heads, S.vs_heads, t.kb, t.nk, pf);
  }
}
template <class C, int I8>
__device__ inline void finish_tile(TileDesc& t, Stage<C>& sb, const Prefetch<C>& pf) {
  if constexpr (I8 != 0) {
    if (t.src < SRC_TXT) store_i8<C, I8 == 1>(t, sb, pf);
  }
}

__device__ inline bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Two ds_read_b64_tr_b16 (elements 0..3 from p0, 4..7 from p1).  Within each
// 16-lane group, output lane i element k is element (i & 3) of the 8 bytes that
// lane 4k + (i >> 2) addresses.
__device__ inline bf16x8 tr_read8(const __bf16* p0, const __bf16* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Eight probabilities as the B operand of the PV MFMA: bf16, or fp16 bits
// for the fp16 path (same register layout).
template <bool F16>
__device__ inline bf16x8 pack_p(const float* x) {
  if constexpr (F16) {
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
    return __builtin_bit_cast(bf16x8, r);
  } else {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
    return r;
  }
}

struct RowState {
  float m;   // running max (log2 units) of this lane's query
  float l;   // this lane's partial sum of probabilities (partner holds the rest)
};

// One KT-key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
//   MASK : some keys (ragged end) or rows (tail window) of the tile are invisible
//   QK16 : INT8 tile: K' is fp16 and qreg holds the fp16 copy of Q
//   PV16 : V' is fp16 carrying 2^-P_SHIFT; the probabilities are taken as
//          p * 2^P_SHIFT in fp16 (else both are bf16)
// The QK MFMAs of the whole tile are issued first, then one rescale decision
// is taken from the maxima of all its 32-key blocks, so that the exponentials
// and PV MFMAs of the blocks form one straight-line region.  The row sum adds
// the 16-bit probabilities the PV MFMA consumes, so their rounding cancels in
// O = acc / l.  scale[q] is the score scale (log2 units) of query block q.
// With Q in LDS (QL) the QK loop reads the wave's Q chunks from qw (the
// lane's slot of chunk 0), QLOOK chunks ahead, instead of qreg, except the
// first QRES chunks, which stay in qreg (bf16-only instance).  TIGHT: the
// kernel also carries INT8 staging registers in its 168 VGPRs, and takes the
// operand lookaheads that measured fastest there (a few registers spill,
// outside the MFMA loops).
template <class C, bool MASK, bool QK16, bool PV16, bool TIGHT = false>
__device__ __forceinline__ void tile_math(const Stage<C>& sb, const bf16x8 (&qreg)[C::QB][8], const __bf16* qw,
                                          f32x16 (&acc)[C::QB][4], RowState (&st)[C::QB],
                                          const float (&scale)[C::QB], int nk, const bool (&row_ok)[C::QB]) {
  constexpr int QB = C::QB, KB = C::KB;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const __bf16* kl = sb.k + lane * 8;   // slot of this lane in every K block
  const __bf16* vl = sb.v + lane * 4;   // slot of this lane in every V block

  f32x16 s[QB][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int q = 0; q < QB; ++q) s[q][kb] = f32x16{};
  // consecutive MFMAs accumulate into different 32-key blocks, so none waits
  // for the previous one's result.  MFMA i (t = i / KB, kb = i % KB) reads its
  // K operand KLOOK MFMAs ahead; a fence after each MFMA keeps that order (left
  // to itself the compiler reads one or two ahead and waits on LDS): +2% on
  // the 480x832 segment and on the 1280x704 steady state.
  {
    constexpr int NK = 8 * KB, KLOOK = TIGHT ? HN_QLI_KLOOK : (C::QL ? HN_QL_KLOOK : HN_KLOOK),
                  QLOOK = TIGHT ? HN_QLI_QLOOK : HN_QL_QLOOK, QRES = (TIGHT || !C::QL) ? 0 : HN_QL_QRES;
    bf16x8 kk[NK];
    bf16x8 qq[8];
    if constexpr (C::QL) {
#pragma unroll
      for (int t = QRES; t < QRES + QLOOK && t < 8; ++t) qq[t] = ld8(qw + t * 512);
    }
#pragma unroll
    for (int i = 0; i < KLOOK; ++i) kk[i] = ld8(kl + ((i % KB) * 8 + i / KB) * 512);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int t = i / KB, kb = i % KB;
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const bf16x8 qop = C::QL ? (t < QRES ? qreg[0][t] : qq[t]) : qreg[q][t];
        if constexpr (QK16)
          s[q][kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kk[i]),
                                                            __builtin_bit_cast(f16x8, qop), s[q][kb], 0, 0, 0);
        else
          s[q][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[i], qop, s[q][kb], 0, 0, 0);
      }
      if (i + KLOOK < NK) kk[i + KLOOK] = ld8(kl + (((i + KLOOK) % KB) * 8 + (i + KLOOK) / KB) * 512);
      if constexpr (C::QL) {
        if (kb == KB - 1 && t >= QRES && t + QLOOK < 8) qq[t + QLOOK] = ld8(qw + (t + QLOOK) * 512);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // one rescale decision per tile: maxima of every block first
  float m_use[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (MASK) {
        const int nkg = row_ok[q] ? nk - 4 * g : INT_MIN;  // key visible iff kb*32+8r+i < nkg
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[q][kb][4 * r + i] * scale[q];
            if (kb * 32 + 8 * r + i >= nkg) v = -INFINITY;
            s[q][kb][4 * r + i] = v;
            mx = smax(mx, v);
          }
      } else {
        float m0 = s[q][kb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m0 = smax(m0, s[q][kb][i]);
        mx = smax(mx, m0 * scale[q]);
      }
    }
    mx = pair_max(mx);
    if (__any(mx > st[q].m + RESCALE_SLACK)) {
      const float m_new = fmaxf(st[q].m, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(st[q].m - m_new);
      st[q].m = m_new;
      st[q].l *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[q][c] *= alpha;
    }
    m_use[q] = (st[q].m == -INFINITY) ? 0.0f : st[q].m;
    if constexpr (PV16) m_use[q] -= P_SHIFT;  // probabilities times 2^P_SHIFT
  }

  // probabilities of block kb, element i, in place of its scores (on the
  // masked path the scores are already scaled, and -inf where invisible)
  auto prob = [&](int q, int kb, int i) __attribute__((always_inline)) {
    if (MASK) s[q][kb][i] = __builtin_amdgcn_exp2f(s[q][kb][i] - m_use[q]);
    else s[q][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[q][kb][i], scale[q], -m_use[q]));
  };
  bf16x8 pb[KB][QB][2];
  // slice j (0..7) of block kb's softmax: two exponentials per query block;
  // every fourth slice packs a half and adds it to the row sum
  auto slice = [&](int kb, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      prob(q, kb, 2 * j);
      prob(q, kb, 2 * j + 1);
      if (j % 4 == 3) {
        const int h = j / 4;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[q][kb][8 * h + e];
        pb[kb][q][h] = pack_p<PV16>(pv);
        float l = st[q].l;
        if constexpr (PV16) {
          // sum of the fp16 probabilities, each times 2^-P_SHIFT (exact)
          const f16x8 ph = __builtin_bit_cast(f16x8, pb[kb][q][h]);
          const f16x2 unshift = {(_Float16)0x1p-7f, (_Float16)0x1p-7f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 pp = {ph[2 * e], ph[2 * e + 1]};
            l = __builtin_amdgcn_fdot2(pp, unshift, l, false);
          }
        } else {
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 pp = {pb[kb][q][h][2 * e], pb[kb][q][h][2 * e + 1]};
            l = __builtin_amdgcn_fdot2_f32_bf16(pp, one, l, false);
          }
        }
        st[q].l = l;
      }
    }
  };
  // PV MFMA i = (kb, t, c) = (i / 8, (i / 4) % 2, i % 4) reads its V operand
  // VLOOK MFMAs ahead, and the softmax of block kb + 1 runs in slices beside
  // the MFMAs of block kb; a fence after each MFMA keeps that order (left to
  // itself the compiler reads one or two operands ahead and waits on LDS
  // before the MFMA): +0.4-1.8% on the 480x832 segment and the 1280x704
  // history, same-run.
  constexpr int NP = 8 * KB, VLOOK = TIGHT ? HN_QLI_VLOOK : (C::QL ? HN_QL_VLOOK : HN_VLOOK);
  auto vaddr = [&](int i) __attribute__((always_inline)) {
    const int kb = i / 8, t = (i / 4) % 2, c = i % 4;
    return vl + ((c * KB + kb) * 2 + t) * 512;
  };
  bf16x8 vv[NP];
#pragma unroll
  for (int i = 0; i < VLOOK; ++i) vv[i] = tr_read8(vaddr(i), vaddr(i) + 256);
#pragma unroll
  for (int j = 0; j < 8; ++j) slice(0, j);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int kb = i / 8, t = (i / 4) % 2, c = i % 4;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if constexpr (PV16)
        acc[q][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vv[i]),
                                                           __builtin_bit_cast(f16x8, pb[kb][q][t]),
                                                           acc[q][c], 0, 0, 0);
      else
        acc[q][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[i], pb[kb][q][t], acc[q][c], 0, 0, 0);
    }
    if (i + VLOOK < NP) vv[i + VLOOK] = tr_read8(vaddr(i + VLOOK), vaddr(i + VLOOK) + 256);
    if (kb + 1 < KB) slice(kb + 1, i % 8);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// HAS_I8: the plan has INT8 history sources (description heads or ring
// frames); without them the kernel carries no INT8 or fp16 code.
//
// Every span list visits its INT8 sources (earlier heads, ring frames) before
// the bf16 ones of the current segment, so a block runs in two phases: the
// INT8 tiles with the fp16 copy of Q in qreg, then the bf16 tiles with Q
// reloaded as bf16 into the same registers.  One copy of Q is live at a time
// (both do not fit two waves per SIMD beside the rest).
template <class C, int MIN_BLOCKS, bool HAS_I8>
__global__ __launch_bounds__(C::T, MIN_BLOCKS) void seg_attn_fwd_kernel(AttnParams p) {
  constexpr int QB = C::QB;
  __shared__ __attribute__((aligned(4096))) Stage<C> stage0;
  __shared__ __attribute__((aligned(4096))) Stage<C> stage1;
  __shared__ QStore<C> qstore;
  // block b runs on XCD b % 8; its position b / 8 there picks a whole video
  // tile first, then a split piece or text tile (head-major in each class)
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  int h, vt;  // vt: virtual tile (query tile, key split), split fastest
  if (pos < p.a_per_xcd) {
    const int i = xcd * p.a_per_xcd + pos;
    if (i >= p.a_tasks) return;  // whole block leaves before any barrier
    h = i / p.n_whole;
    vt = i - h * p.n_whole;
  } else {
    const int i = xcd * p.b_per_xcd + (pos - p.a_per_xcd);
    if (i >= p.b_tasks) return;
    const int nb = p.n_tiles - p.n_whole;
    h = i / nb;
    vt = p.n_whole + (i - h * nb);
  }
  int tile, split_unused, n_split;
  vt_decode(vt, p.n_qtiles, p.n_whole, p.n_splits, p.n_splits_text, tile, split_unused, n_split);
  // plan tiles: video query tiles, then text query tiles (own head and tails)
  const bool text = tile >= p.n_qtiles;
  const int qt = text ? tile - p.n_qtiles : tile;  // tile within its query set
  const int lq = text ? p.lq_txt : p.lq;
  const __bf16* qsrc = text ? p.q_txt : p.q;
  __bf16* odst = text ? p.o_txt : p.o;
  float* lse_dst = text ? p.lse_txt : p.lse;

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
  const uint32_t q_tb = (uint32_t)p.H * D * 2;
  const rsrc_t rq = make_rsrc(qsrc + h * D, (uint32_t)lq * q_tb - (uint32_t)h * D * 2);
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qreg[q][t] = __builtin_bit_cast(bf16x8, ld_b128(rq, (uint32_t)row[q] * q_tb + 16 * g, 32 * t));
  };
  load_q();
  // QL: this wave's Q region and the lane's slot in its chunk 0; publish_q
  // writes qreg there (only this wave reads it, so no barrier is needed)
  const __bf16* qw = qstore.q + wave * 32 * D + lane * 8;
  auto publish_q = [&]() __attribute__((always_inline)) {
    if constexpr (C::QL) {
      __bf16* qd = qstore.q + wave * 32 * D + lane * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<bf16x8*>(qd + t * 512) = qreg[0][t];
    }
  };
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

  const int n_spans = p.counts[vt];
  const Span* spans = p.spans + (int64_t)vt * p.max_spans;

  // tile iterator over the spans (block-uniform).  The current span is kept in
  // registers and the next one is read when a span ends, so the read is
  // waited on one step later, behind that step's tile loads.
  int e = 0;
  Span sp{};
  if (n_spans > 0) sp = spans[0];
  int kpos = sp.k0;
  auto next_tile = [&](TileDesc& t) __attribute__((always_inline)) -> bool {
    if (e >= n_spans) return false;
    t.src = sp.src;
    t.kb = kpos;
    t.nk = min(C::KT, sp.k1 - kpos);
    t.r0 = sp.r0;
    t.r1 = sp.r1;
    t.ok16 = true;
    kpos += t.nk;
    if (kpos >= sp.k1) {
      ++e;
      if (e < n_spans) {
        sp = spans[e];
        kpos = sp.k0;
      }
    }
    return true;
  };

  TileDesc cur, nxt;
  bool have = next_tile(cur);
  // Scores of the fp16 tiles: Q * 2^-qs per row, with qs = 0 unless the row
  // holds a |Q| >= 2^15, then the least shift that brings it below 2^15 (a
  // power of two: exact, and folded back into the score scale).
  float scale_h[QB];
  auto to_f16_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float mx = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf((float)qreg[q][t][i]));
      mx = pair_max(mx);  // the row's other 64 values sit in lane ^ 32
      const int qs = mx >= 0x1p15f ? ilogbf(mx) - 14 : 0;
      const float f = ldexpf(1.0f, -qs);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f16x8 x;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (_Float16)((float)qreg[q][t][i] * f);
        qreg[q][t] = __builtin_bit_cast(bf16x8, x);
      }
      scale_h[q] = ldexpf(p.scale_log2, qs);
    }
  };
  // the math of tile `cur` from stage sc: the rows of this wave that see it,
  // full tiles on the lean path, ragged or row-cut ones on the masked path
  auto compute = [&](const Stage<C>& sc, auto f16_tag) __attribute__((always_inline)) {
    constexpr bool F16 = decltype(f16_tag)::value;
    const int wrows = 32 * QB;
    // waves whose rows all lie past the query set's end skip the math (a
    // tile's last rows; full spans carry the row range [0, INT_MAX))
    const bool wave_live = wrow0 < lq && (cur.r0 < wrow0 + wrows) && (cur.r1 > wrow0);
    if (!wave_live) return;
    const bool rows_all = (cur.r0 <= wrow0) && (cur.r1 >= wrow0 + wrows);
    bool row_ok[QB];
    float sc_t[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      row_ok[q] = row[q] >= cur.r0 && row[q] < cur.r1;
      sc_t[q] = F16 ? scale_h[q] : p.scale_log2;
    }
    const bool mask = (cur.nk < C::KT) || !rows_all;
    constexpr bool TIGHT = C::QL && HAS_I8;
    if (mask) tile_math<C, true, F16, F16, TIGHT>(sc, qreg, qw, acc, st, sc_t, cur.nk, row_ok);
    else tile_math<C, false, F16, F16, TIGHT>(sc, qreg, qw, acc, st, sc_t, cur.nk, row_ok);
  };
  // One pipeline step: compute tile `cur` from stage `sc` while tile `nxt`
  // streams into stage `sn`; the stages alternate, unrolled by two so that
  // each step's stages are distinct objects.  The prefetch registers of an
  // INT8 tile are fresh in every step (not carried around the loop), so no
  // copies of them sit between the loads and the math of the current tile.
  // I8 = 1: the INT8 phase (fp16 math; the next tile may be INT8 or the first
  // bf16 one); I8 = 2 / 0: bf16 math, INT8 tiles (if any) staged in bf16.
  auto step = [&](const Stage<C>& sc, Stage<C>& sn, auto i8_tag) __attribute__((always_inline)) {
    constexpr int I8 = decltype(i8_tag)::value;
    const bool have_next = next_tile(nxt);
    Prefetch<C> pf;
    if (have_next) start_tile<C, I8>(S, nxt, sn, pf);
    compute(sc, std::integral_constant<bool, I8 == 1>{});
    if (have_next) finish_tile<C, I8>(nxt, sn, pf);
    __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS loads of this thread have landed
    __syncthreads();
    cur = nxt;
    have = have_next;
  };
  auto first_tile = [&](auto i8_tag) __attribute__((always_inline)) {
    if (have) {
      Prefetch<C> pf;
      start_tile<C, decltype(i8_tag)::value>(S, cur, stage0, pf);
      finish_tile<C, decltype(i8_tag)::value>(cur, stage0, pf);
    }
    __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS loads of this thread have landed
    __syncthreads();
  };
  constexpr int I8_BF16 = HAS_I8 ? 2 : 0;
  bool odd = false;  // the current tile sits in stage1
  if constexpr (HAS_I8) {
    // Phase 1: the INT8 tiles in fp16.  A tile whose scales do not fit fp16's
    // range (|K| > 65,024 or |V| > 8.3e6 in the history) sends the block back
    // to the start, to take every tile in bf16.
    if (have && cur.src < SRC_TXT) {
      to_f16_q();
      publish_q();
      first_tile(std::integral_constant<int, 1>{});
      bool redo = false;
      while (have && cur.src < SRC_TXT) {
        if (!cur.ok16) { redo = true; break; }
        step(stage0, stage1, std::integral_constant<int, 1>{});
        if (!have || cur.src >= SRC_TXT) { odd = true; break; }
        if (!cur.ok16) { redo = true; odd = true; break; }
        step(stage1, stage0, std::integral_constant<int, 1>{});
      }
      // bf16 Q for what follows; every load of the last step has been waited
      // for, so this wait covers only these
      if (have || redo) {
        load_q();
        __builtin_amdgcn_s_waitcnt(0);
        publish_q();
      }
      if (redo) {
        // start over: one softmax over every tile, INT8 ones staged in bf16
#pragma unroll
        for (int q = 0; q < QB; ++q) {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[q][c] = f32x16{};
          st[q].m = -INFINITY;
          st[q].l = 0.0f;
        }
        e = 0;
        sp = spans[0];
        kpos = sp.k0;
        have = next_tile(cur);
        odd = false;
        first_tile(std::integral_constant<int, I8_BF16>{});
      }
    } else {
      publish_q();
      first_tile(std::integral_constant<int, I8_BF16>{});
    }
  } else {
    publish_q();
    first_tile(std::integral_constant<int, I8_BF16>{});
  }
  // Phase 2: the bf16 tiles (and, after a restart, every tile)
  if (have && odd) step(stage1, stage0, std::integral_constant<int, I8_BF16>{});
  while (have) {
    step(stage0, stage1, std::integral_constant<int, I8_BF16>{});
    if (!have) break;
    step(stage1, stage0, std::integral_constant<int, I8_BF16>{});
  }

  // epilogue: O = acc / l, lse = (m + log2 l) * ln 2; with key splits the
  // normalized fp32 O and the lse of this split go to the partial buffers
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const float l_tot = pair_sum(st[q].l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = l_tot > 0.0f ? (st[q].m + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    if (row[q] >= lq) continue;
    if (n_split > 1) {
      const int64_t prow = ((int64_t)h * p.n_pvt + (vt - p.part_vt0)) * C::ROWS + (row[q] - qt * C::ROWS);
      float* orow = p.part_o + prow * D;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d0 = 32 * c + 8 * r + 4 * g;
          *reinterpret_cast<float4*>(orow + d0) =
              make_float4(acc[q][c][4 * r + 0] * inv, acc[q][c][4 * r + 1] * inv,
                          acc[q][c][4 * r + 2] * inv, acc[q][c][4 * r + 3] * inv);
        }
      }
      if (g == 0) p.part_lse[prow] = lse_v;
      continue;
    }
    __bf16* orow = odst + ((int64_t)row[q] * p.H + h) * D;
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
    if (lse_dst != nullptr && g == 0) lse_dst[(int64_t)h * lq + row[q]] = lse_v;
  }
}

// Split-KV merge: for every (head, query tile) that was split, the partial results
// (normalized O in fp32, lse) of the same rows are combined exactly as one
// softmax over the union of their keys: with M = max_s lse_s and
// w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s and
// lse = M + log(sum_s w_s); rows no split saw (all lse = -inf) get O = 0.
// Block = MERGE_ROWS rows of one (head, query tile); each 32-lane group
// merges one 128-wide row with float4 loads.  With one block per whole tile,
// a launch that merges only a few split tiles (the text tiles of a joint
// launch: 80 blocks) was bound by 32 dependent load round trips per block,
// 82-89 us on the 480x832 segment.
constexpr int MERGE_ROWS = 8;
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int chunks = (p.tile_rows + MERGE_ROWS - 1) / MERGE_ROWS;
  const int ht = blockIdx.x / chunks;
  const int chunk = blockIdx.x - ht * chunks;
  const int h = ht / p.n_tiles;
  const int t = ht - h * p.n_tiles;
  const bool text = t >= p.n_qtiles;
  const int n_split = text ? p.n_splits_text : (t < p.n_whole ? 1 : p.n_splits);
  if (n_split == 1) return;  // this tile wrote its outputs directly
  const int qt = text ? t - p.n_qtiles : t;
  const int lq = text ? p.lq_txt : p.lq;
  __bf16* out = text ? p.o_txt : p.o;
  float* lse_out = text ? p.lse_txt : p.lse;
  const int d4 = threadIdx.x & 31;
  const int rl_end = min((chunk + 1) * MERGE_ROWS, p.tile_rows);
  for (int rl = chunk * MERGE_ROWS + (threadIdx.x >> 5); rl < rl_end; rl += 8) {
    const int row = qt * p.tile_rows + rl;
    if (row >= lq) break;
    const int64_t base =
        ((int64_t)h * p.n_pvt + (vt_first(t, p.n_qtiles, p.n_whole, p.n_splits, p.n_splits_text) - p.part_vt0)) *
            p.tile_rows + rl;
    float m = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp) m = fmaxf(m, p.part_lse[base + (int64_t)sp * p.tile_rows]);
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float wsum = 0.0f;
    if (m != -INFINITY) {
      for (int sp = 0; sp < n_split; ++sp) {
        const int64_t pr = base + (int64_t)sp * p.tile_rows;
        const float w = expf(p.part_lse[pr] - m);
        const float4 v = *reinterpret_cast<const float4*>(p.part_o + pr * D + 4 * d4);
        acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
        wsum += w;
      }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const bf16x2 lo = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv)};
    const bf16x2 hi = {(__bf16)(acc.z * inv), (__bf16)(acc.w * inv)};
    *reinterpret_cast<uint2*>(out + ((int64_t)row * p.H + h) * D + 4 * d4) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    if (lse_out != nullptr && d4 == 0)
      lse_out[(int64_t)h * lq + row] = wsum > 0.0f ? m + logf(wsum) : -INFINITY;
  }
}

// Dense plans use 256-row blocks of 8 waves x 32 rows, one block per CU (two
// waves per SIMD): every staged (and, for INT8, dequantized) key/value tile
// serves 256 query rows.  Measured against 128-row 4-wave blocks at two per
// CU: +3% on the 480x832 segment, +2% on the 1280x704 steady state, +13% on
// the 7th 1280x704 segment with 158k INT8 history keys.  Keep-list plans use
// 128-row blocks (the keep list's query tile).  Also measured: 4 waves x 64
// rows at one wave per SIMD (much slower), 128-key tiles (spill).
#ifndef HN_DENSE_NW
#define HN_DENSE_NW 8
#endif
#ifndef HN_DENSE_QB
#define HN_DENSE_QB 1
#endif
#ifndef HN_DENSE_MINB
#define HN_DENSE_MINB 1
#endif
#ifndef HN_DENSE_KT
#define HN_DENSE_KT 64
#endif
using DenseCfg = Cfg<HN_DENSE_NW, HN_DENSE_QB, HN_DENSE_KT>;
// 384-row blocks: 12 waves x 32 rows (three per SIMD, <= 168 VGPRs, which
// Q fits only in LDS: 96 KB beside the two 32 KB stages fills the CU's
// 160 KB); waves 0-7 stage the tiles, so every SIMD has two staging waves.
using Dense384Cfg = Cfg<12, 1, 64, true, 8>;
using SparseCfg = Cfg<4, 1, 64>;
static_assert(SparseCfg::ROWS == HN_TILE, "keep-list blocks must match the keep-list tile");

}  // namespace

bool attn_rows_supported(int rows) {
  return rows == DenseCfg::ROWS || rows == Dense384Cfg::ROWS || rows == SparseCfg::ROWS;
}

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  if (p.a_tasks + p.b_tasks == 0) return hipSuccess;
  const int blocks = 8 * (p.a_per_xcd + p.b_per_xcd);
  if (p.tile_rows == DenseCfg::ROWS) {
    if (p.has_i8)
      hipLaunchKernelGGL((seg_attn_fwd_kernel<DenseCfg, HN_DENSE_MINB, true>), dim3(blocks), dim3(DenseCfg::T),
                         0, s, p);
    else
      hipLaunchKernelGGL((seg_attn_fwd_kernel<DenseCfg, HN_DENSE_MINB, false>), dim3(blocks), dim3(DenseCfg::T),
                         0, s, p);
  } else if (p.tile_rows == Dense384Cfg::ROWS) {
    if (p.has_i8)
      hipLaunchKernelGGL((seg_attn_fwd_kernel<Dense384Cfg, 1, true>), dim3(blocks), dim3(Dense384Cfg::T), 0, s,
                         p);
    else
      hipLaunchKernelGGL((seg_attn_fwd_kernel<Dense384Cfg, 1, false>), dim3(blocks), dim3(Dense384Cfg::T), 0, s,
                         p);
  } else if (p.tile_rows == SparseCfg::ROWS) {
    if (p.has_i8)
      hipLaunchKernelGGL((seg_attn_fwd_kernel<SparseCfg, 2, true>), dim3(blocks), dim3(SparseCfg::T), 0, s, p);
    else
      hipLaunchKernelGGL((seg_attn_fwd_kernel<SparseCfg, 2, false>), dim3(blocks), dim3(SparseCfg::T), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.H * p.n_tiles * ((p.tile_rows + MERGE_ROWS - 1) / MERGE_ROWS);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hn
