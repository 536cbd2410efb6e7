// Camera cross-attention of a segment's video tokens (gfx950).
//
// Each latent frame carries one camera token (four frame poses folded into a
// 64-dimensional vector and projected), and in every block the video tokens
// read the time-aligned camera tokens of their own segment by cross-attention
// ("Hy-Nomas 拆解" teardown, section "架构", camera paragraph).  The video
// token at latent frame f sees the camera tokens of frames f' with
// |f' - f| <= radius; radius 0 is the time alignment the pages state (one
// key, weight exactly 1, so O is that frame's camera value).
//
// HBM-bound: per (token, head) it reads the 256-byte query and writes the
// 256-byte output (+ 4 bytes of lse); the camera keys and values (F x H x 256
// bytes each) stay in cache.  16 lanes own one row (8 values each, one
// 16-byte load and store; measured 8% faster than 8 lanes x 32 bytes, and
// 4 lanes x 64 bytes slower still); the score is a 16-lane butterfly; online
// softmax over the visible camera tokens in fp32, CH camera tokens at a time:
// the chunk's key and value rows are loaded together and its scores reduced
// side by side, so the cached rows cost one load round trip per chunk instead
// of two dependent ones per camera token (radius 1: +4-6%, radius 3: +10%;
// at radius 0 a 4-token chunk would waste three tokens' shuffles, so CH
// follows the radius).  Row indexing divides by host-computed multipliers.
#include "hn_internal.h"

namespace hn {
namespace {

constexpr int LANES = 16;            // lanes per (token, head) row
constexpr int ROWS = 256 / LANES;   // rows per block

constexpr int E = 8;   // values per lane

__device__ inline void unpack_row(const uint4 a, float (&x)[E]) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// n / d for n < 2^31 with the host's multiplier and shift (div_magic).
__device__ inline uint32_t udiv31(uint32_t n, uint32_t m, int k) {
  return (uint32_t)(((uint64_t)n * m) >> k);
}

// CH camera tokens per chunk: 1 for radius 0, 3 for radius 1 (the whole
// window of an inner frame), 4 beyond.
template <int CH>
__global__ __launch_bounds__(256) void camera_attn_kernel(CameraParams p) {
  const int lane = threadIdx.x & (LANES - 1);
  // a block takes ROWS consecutive tokens of one head, so that its lane
  // groups read the same camera rows (one fetch from L2, the rest from the
  // CU's cache); consecutive blocks take the heads of the same tokens
  const uint32_t tb = udiv31(blockIdx.x, p.mag_h, p.sh_h);
  const int h = (int)(blockIdx.x - tb * (uint32_t)p.H);
  const uint32_t t = tb * ROWS + (threadIdx.x / LANES);
  // whole lane groups leave together, so the butterflies stay inside active lanes
  if (t >= (uint32_t)p.rows) return;
  const int f = (int)udiv31(t, p.mag_p, p.sh_p);
  const int lo = max(0, f - p.radius);
  const int hi = min(p.F, f + p.radius + 1);

  const int64_t row = (int64_t)(t * (uint32_t)p.H + (uint32_t)h) * D + lane * E;
  float q[E];
  unpack_row(*reinterpret_cast<const uint4*>(p.q + row), q);
  float m = -INFINITY, l = 0.0f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  for (int g0 = lo; g0 < hi; g0 += CH) {
    uint4 kw[CH], vw[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      kw[c] = vw[c] = make_uint4(0u, 0u, 0u, 0u);
      if (g0 + c < hi) {
        const int64_t kv = (int64_t)((uint32_t)(g0 + c) * (uint32_t)p.H + (uint32_t)h) * D + lane * E;
        kw[c] = *reinterpret_cast<const uint4*>(p.k + kv);
        vw[c] = *reinterpret_cast<const uint4*>(p.v + kv);
      }
    }
    float s[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float k[E];
      unpack_row(kw[c], k);
      s[c] = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) s[c] = __builtin_fmaf(q[i], k[i], s[c]);
    }
#pragma unroll
    for (int x = 1; x < LANES; x <<= 1)
#pragma unroll
      for (int c = 0; c < CH; ++c) s[c] += __shfl_xor(s[c], x);
    float mc = -INFINITY;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      s[c] = g0 + c < hi ? s[c] * p.scale_log2 : -INFINITY;
      mc = fmaxf(mc, s[c]);
    }
    // the chunk holds at least one visible token, so m_new is its score max
    const float m_new = fmaxf(m, mc);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= alpha;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float w = __builtin_amdgcn_exp2f(s[c] - m_new);  // 0 past the visible range
      float v[E];
      unpack_row(vw[c], v);
      l += w;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] = __builtin_fmaf(w, v[i], acc[i]);
    }
    m = m_new;
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint32_t o[E / 2];
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const bf16x2_t pr = {(__bf16)(acc[2 * i] * inv), (__bf16)(acc[2 * i + 1] * inv)};
    o[i] = __builtin_bit_cast(uint32_t, pr);
  }
  *reinterpret_cast<uint4*>(p.o + row) = make_uint4(o[0], o[1], o[2], o[3]);
  if (p.lse != nullptr && lane == 0)
    p.lse[(int64_t)h * p.rows + t] = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_camera_attn(const CameraParams& p, hipStream_t s) {
  if (p.rows == 0 || p.H == 0) return hipSuccess;
  const int64_t blocks = (p.rows + ROWS - 1) / ROWS * p.H;
  if (p.radius == 0)
    hipLaunchKernelGGL(camera_attn_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (p.radius == 1)
    hipLaunchKernelGGL(camera_attn_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(camera_attn_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hn
