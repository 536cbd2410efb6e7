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
// softmax over the visible camera tokens in fp32.
#include "hn_internal.h"

namespace hn {
namespace {

constexpr int LANES = 16;            // lanes per (token, head) row
constexpr int ROWS = 256 / LANES;   // rows per block

constexpr int E = 8;
// E consecutive bf16 values -> float
__device__ inline void load_row(const __bf16* p, float (&x)[E]) {
#pragma unroll
  for (int c = 0; c < E / 8; ++c) {
    const uint4 a = *reinterpret_cast<const uint4*>(p + 8 * c);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
      x[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

__device__ inline float sum_lanes(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

__global__ __launch_bounds__(256) void camera_attn_kernel(CameraParams p) {
  const int lane = threadIdx.x & (LANES - 1);
  // a block takes ROWS consecutive tokens of one head, so that its lane
  // groups read the same camera rows (one fetch from L2, the rest from the
  // CU's cache); consecutive blocks take the heads of the same tokens
  const int64_t tb = blockIdx.x / p.H;
  const int h = (int)(blockIdx.x - tb * p.H);
  const int64_t t = tb * ROWS + (threadIdx.x / LANES);
  // whole lane groups leave together, so the butterflies stay inside active lanes
  if (t >= p.rows) return;
  const int f = (int)(t / p.P);
  const int lo = max(0, f - p.radius);
  const int hi = min(p.F, f + p.radius + 1);

  float q[E];
  load_row(p.q + (t * p.H + h) * D + lane * E, q);
  float m = -INFINITY, l = 0.0f;
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0f;
  for (int g = lo; g < hi; ++g) {
    const int64_t kv = ((int64_t)g * p.H + h) * D + lane * E;
    float k[E];
    load_row(p.k + kv, k);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) s = __builtin_fmaf(q[i], k[i], s);
    s = sum_lanes(s) * p.scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float w = __builtin_amdgcn_exp2f(s - m_new);
    float v[E];
    load_row(p.v + kv, v);
    l = l * alpha + w;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = acc[i] * alpha + w * v[i];
    m = m_new;
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint32_t o[E / 2];
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const bf16x2_t pr = {(__bf16)(acc[2 * i] * inv), (__bf16)(acc[2 * i + 1] * inv)};
    o[i] = __builtin_bit_cast(uint32_t, pr);
  }
  __bf16* dst = p.o + (t * p.H + h) * D + lane * E;
#pragma unroll
  for (int c = 0; c < E / 8; ++c)
    *reinterpret_cast<uint4*>(dst + 8 * c) = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
  if (p.lse != nullptr && lane == 0)
    p.lse[(int64_t)h * p.rows + t] = l > 0.0f ? (m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_camera_attn(const CameraParams& p, hipStream_t s) {
  if (p.rows == 0 || p.H == 0) return hipSuccess;
  const int64_t blocks = (p.rows + ROWS - 1) / ROWS * p.H;
  hipLaunchKernelGGL(camera_attn_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hn
