// Segment-causal, action-aware attention forward over an INT8 KV cache (gfx950).
//
// One softmax over the union of visible keys of a video query
// ("Hy-Nomas 拆解" teardown, section "架构": segment-causal plus action-aware
// causal attention); history keys/values are INT8 with fp32 scales and the
// arithmetic is BF16 (same page, "单卡 4090 怎么做到的", first technique).
//
// Work decomposition
//   block  = one (head, 128-row query tile); 4 waves x 32 query rows.
//   tile   = 64 keys of one span of the tile plan, staged in LDS as bf16:
//            K as [key][d] (row pitch 136 elements) and V transposed as
//            [d][key] (row pitch 72 elements, 16-byte groups XOR-swizzled by d/8).
//            INT8 tiles are read from HBM as int8 (half the bytes), converted
//            to bf16 in registers on their way into LDS (int8 -> bf16 is exact),
//            and their fp32 scales are applied after the MFMA: the key scale to
//            the score column, the value scale to the probability.
//   math   = S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (each lane then holds
//            16 keys of one query, so the row max/sum are in-lane plus one
//            exchange with lane^32); online softmax in the log2 domain; the
//            probabilities are packed to bf16 in registers and used directly
//            as the B operand of O^T = V^T P^T, whose accumulator keeps each
//            query's 128 outputs in its own lane pair.
//   order  = the plan's span order, 64 keys at a time, double-buffered: global
//            loads of tile n+1 are in flight while tile n is computed.
//   grid   = XCD-aware: block b runs on XCD b % 8, and each XCD gets a
//            contiguous range of (head, tile) tasks, so one head's keys and
//            values stay in one XCD's L2.
#include <climits>

#include "hn_internal.h"

namespace hn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 4;                 // waves per block
constexpr int QT = 32 * NW;           // query rows per block
constexpr int KT = 64;                // keys per tile
constexpr int KP = D + 8;             // LDS pitch of a K row (bf16 elements)
constexpr int VP = KT + 8;            // LDS pitch of a V^T row (bf16 elements)
static_assert(QT == HN_TILE, "block rows must equal the plan tile");

struct Smem {
  __bf16 k[2][KT * KP];
  __bf16 vt[2][D * VP];
  float ks[2][KT];
  float vs[2][KT];
};

struct TileDesc {
  int src, kb, nk, r0, r1;
};

// Position of key `key` (0..63) in a V^T row: bits 2 and 3 swapped, so the 8
// keys one lane group feeds to a PV MFMA are contiguous.
__device__ inline int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}
// XOR swizzle of 8-key groups by d/8 against LDS bank conflicts.
__device__ inline int vt_index(int d, int pos) { return d * VP + (pos ^ (((d >> 3) & 7) << 3)); }

__device__ inline uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(b, a, sel);
}
// Low halves of a and b -> (a.lo | b.lo << 16); high halves -> (a.hi | b.hi << 16).
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// int8 -> bf16 (exact for |q| <= 127): two signed bytes -> packed bf16 pair.
__device__ inline uint32_t i8pair_to_bf16(uint32_t w, int byte0) {
  const float f0 = (float)(int8_t)((w >> (8 * byte0)) & 0xFF);
  const float f1 = (float)(int8_t)((w >> (8 * byte0 + 8)) & 0xFF);
  return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
}

struct Prefetch {
  uint4 k[4];
  uint4 v[4];
  float sc;
};

__device__ inline const int8_t* i8_base(const AttnParams& p, int src, bool is_v, int h) {
  if (src == SRC_HEADS) return (is_v ? p.heads_v : p.heads_k) + (int64_t)h * p.head_cap * D;
  return (is_v ? p.ring_v : p.ring_k) + (int64_t)h * p.ring_cap * D;
}
__device__ inline const float* sc_base(const AttnParams& p, int src, bool is_v, int h) {
  if (src == SRC_HEADS) return (is_v ? p.heads_vs : p.heads_ks) + (int64_t)h * p.head_cap;
  return (is_v ? p.ring_vs : p.ring_ks) + (int64_t)h * p.ring_cap;
}

// Global -> registers for one tile.  Rows at or past nk read as zero.
__device__ inline void load_tile(const AttnParams& p, const TileDesc& t, int h, Prefetch& pf) {
  const int tid = threadIdx.x;
  const uint4 z = make_uint4(0, 0, 0, 0);
  if (t.src >= SRC_TXT) {
    const __bf16* kbase = (t.src == SRC_TXT) ? p.k_txt : p.k_vid;
    const __bf16* vbase = (t.src == SRC_TXT) ? p.v_txt : p.v_vid;
    const int64_t rs = (int64_t)p.H * D;  // token stride
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = c * 256 + tid;
      const int key = id >> 4, dch = id & 15;
      pf.k[c] = key < t.nk
                    ? *reinterpret_cast<const uint4*>(kbase + (int64_t)(t.kb + key) * rs + h * D + dch * 8)
                    : z;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int kq = (lane & 3) + 4 * wave, dc = lane >> 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 4 * kq + r;
      pf.v[r] = key < t.nk
                    ? *reinterpret_cast<const uint4*>(vbase + (int64_t)(t.kb + key) * rs + h * D + dc * 8)
                    : z;
    }
    pf.sc = 1.0f;
  } else {
    const int8_t* kbase = i8_base(p, t.src, false, h) + (int64_t)t.kb * D;
    const int8_t* vbase = i8_base(p, t.src, true, h) + (int64_t)t.kb * D;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = c * 256 + tid;
      const int key = id >> 3, dch = id & 7;
      pf.k[c] = key < t.nk ? *reinterpret_cast<const uint4*>(kbase + key * D + dch * 16) : z;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int kq = (lane & 3) + 4 * wave, dc = lane >> 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 4 * kq + r;
      uint2 w = make_uint2(0, 0);
      if (key < t.nk) w = *reinterpret_cast<const uint2*>(vbase + key * D + dc * 8);
      pf.v[r] = make_uint4(w.x, w.y, 0, 0);
    }
    float sc = 0.0f;
    if (tid < 2 * KT) {
      const int key = tid & (KT - 1);
      const float* sb = sc_base(p, t.src, tid >= KT, h);
      sc = key < t.nk ? sb[t.kb + key] : 0.0f;
    }
    pf.sc = sc;
  }
}

// Registers -> LDS buffer `b` (bf16 K rows, bf16 V^T rows, scales).
__device__ inline void store_tile(Smem& sm, int b, const TileDesc& t, const Prefetch& pf) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kq = (lane & 3) + 4 * wave, dc = lane >> 2;
  uint32_t rows[4][4];  // V rows as 4 x (8 bf16) packed words
  if (t.src >= SRC_TXT) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int id = c * 256 + tid;
      const int key = id >> 4, dch = id & 15;
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 8]) = pf.k[c];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rows[r][0] = pf.v[r].x; rows[r][1] = pf.v[r].y; rows[r][2] = pf.v[r].z; rows[r][3] = pf.v[r].w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int id = c * 256 + tid;
      const int key = id >> 3, dch = id & 7;
      const uint4 w = pf.k[c];
      uint4 lo, hi;
      lo.x = i8pair_to_bf16(w.x, 0); lo.y = i8pair_to_bf16(w.x, 2);
      lo.z = i8pair_to_bf16(w.y, 0); lo.w = i8pair_to_bf16(w.y, 2);
      hi.x = i8pair_to_bf16(w.z, 0); hi.y = i8pair_to_bf16(w.z, 2);
      hi.z = i8pair_to_bf16(w.w, 0); hi.w = i8pair_to_bf16(w.w, 2);
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 16]) = lo;
      *reinterpret_cast<uint4*>(&sm.k[b][key * KP + dch * 16 + 8]) = hi;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rows[r][0] = i8pair_to_bf16(pf.v[r].x, 0); rows[r][1] = i8pair_to_bf16(pf.v[r].x, 2);
      rows[r][2] = i8pair_to_bf16(pf.v[r].y, 0); rows[r][3] = i8pair_to_bf16(pf.v[r].y, 2);
    }
    if (tid < KT) sm.ks[b][tid] = pf.sc;
    else if (tid < 2 * KT) sm.vs[b][tid - KT] = pf.sc;
  }
  // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
  const int pos = vt_pos(4 * kq);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int d0 = dc * 8 + 2 * w;
    uint2 e, o;
    e.x = pack_lo(rows[0][w], rows[1][w]);
    e.y = pack_lo(rows[2][w], rows[3][w]);
    o.x = pack_hi(rows[0][w], rows[1][w]);
    o.y = pack_hi(rows[2][w], rows[3][w]);
    *reinterpret_cast<uint2*>(&sm.vt[b][vt_index(d0, pos)]) = e;
    *reinterpret_cast<uint2*>(&sm.vt[b][vt_index(d0 + 1, pos)]) = o;
  }
}

__device__ inline bf16x8 lds8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ inline bf16x8 pack_p(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

__global__ __launch_bounds__(256, 2) void seg_attn_fwd_kernel(AttnParams p) {
  __shared__ Smem sm;
  const int task = (blockIdx.x & 7) * p.tasks_per_xcd + (blockIdx.x >> 3);
  if (task >= p.n_tasks) return;  // whole block leaves before any barrier
  const int h = task / p.n_qtiles;
  const int qt = task - h * p.n_qtiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int wrow0 = qt * QT + wave * 32;
  const int row = wrow0 + l32;
  const bool row_valid = row < p.lq;

  // Q^T as the B operand: lane (q, g) holds Q[q][16t + 8g .. +8] for t = 0..7
  bf16x8 qreg[8];
  {
    const __bf16* qrow = p.q + ((int64_t)(row_valid ? row : 0) * p.H + h) * D;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8 v = lds8(qrow + 16 * t + 8 * g);
      if (!row_valid) v = bf16x8{};
      qreg[t] = v;
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  const int n_spans = p.counts[qt];
  const Span* spans = p.spans + (int64_t)qt * p.max_spans;

  // tile iterator over the spans
  int e = 0;
  int kpos = n_spans > 0 ? spans[0].k0 : 0;
  auto next_tile = [&](TileDesc& t) -> bool {
    if (e >= n_spans) return false;
    const Span s = spans[e];
    t.src = s.src;
    t.kb = kpos;
    t.nk = min(KT, s.k1 - kpos);
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
  Prefetch pf;
  if (have) {
    load_tile(p, cur, h, pf);
    store_tile(sm, 0, cur, pf);
  }
  __syncthreads();
  int buf = 0;
  while (have) {
    const bool have_next = next_tile(nxt);
    if (have_next) load_tile(p, nxt, h, pf);

    // skip the math if no row of this wave can see the tile
    const bool wave_live = (cur.r0 < wrow0 + 32) && (cur.r1 > wrow0);
    if (wave_live) {
      const bool row_ok = row >= cur.r0 && row < cur.r1;
      const bool is_i8 = cur.src < SRC_TXT;
      const __bf16* kl = sm.k[buf];
      const __bf16* vl = sm.vt[buf];

      // S^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 a = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 kk = lds8(kl + (kb * 32 + l32) * KP + 16 * t + 8 * g);
          a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[t], a, 0, 0, 0);
        }
        s[kb] = a;
      }

      // scale, mask, running max (log2 domain)
      float x[2][16];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kbase = kb * 32 + 8 * r + 4 * g;
          float4 ksc = make_float4(1.f, 1.f, 1.f, 1.f);
          if (is_i8) ksc = *reinterpret_cast<const float4*>(&sm.ks[buf][kbase]);
          const float kscl[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + i;
            float v = s[kb][4 * r + i] * (p.scale_log2 * kscl[i]);
            if (key >= cur.nk || !row_ok) v = -INFINITY;
            x[kb][4 * r + i] = v;
            mx = fmaxf(mx, v);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      float psum = 0.0f;
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float4 vsc = make_float4(1.f, 1.f, 1.f, 1.f);
          if (is_i8) vsc = *reinterpret_cast<const float4*>(&sm.vs[buf][kb * 32 + 8 * r + 4 * g]);
          const float vscl[4] = {vsc.x, vsc.y, vsc.z, vsc.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e2 = __builtin_amdgcn_exp2f(x[kb][4 * r + i] - m_use);
            psum += e2;
            pv[4 * r + i] = e2 * vscl[i];
          }
        }
        pb[2 * kb] = pack_p(pv);
        pb[2 * kb + 1] = pack_p(pv + 8);
      }
      l_run = l_run * alpha + psum;

#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d = 32 * c + l32;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int pos = 16 * t + 8 * g;
          const bf16x8 vv = lds8(vl + vt_index(d, pos));
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[t], acc[c], 0, 0, 0);
        }
      }
    }

    if (have_next) store_tile(sm, buf ^ 1, nxt, pf);
    __syncthreads();
    cur = nxt;
    have = have_next;
    buf ^= 1;
  }

  // epilogue: O = acc / l, lse = (m + log2 l) * ln 2
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_valid) {
    __bf16* orow = p.o + ((int64_t)row * p.H + h) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * c + 8 * r + 4 * g;
        uint2 w;
        const __bf16 b0 = (__bf16)(acc[c][4 * r + 0] * inv), b1 = (__bf16)(acc[c][4 * r + 1] * inv);
        const __bf16 b2 = (__bf16)(acc[c][4 * r + 2] * inv), b3 = (__bf16)(acc[c][4 * r + 3] * inv);
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    }
    if (p.lse != nullptr && g == 0) {
      p.lse[(int64_t)h * p.lq + row] =
          l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  if (p.n_tasks == 0) return hipSuccess;
  const int blocks = 8 * p.tasks_per_xcd;
  hipLaunchKernelGGL(seg_attn_fwd_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hn
