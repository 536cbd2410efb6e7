// INT8 quantize + ring append of one segment's keys and values (gfx950).
//
// Keys and values are stored INT8 with a float scale and computed in 16-bit
// floating point ("Hy-Nomas 拆解" teardown, section "单卡 4090 怎么做到的", first
// technique); history video is a window of W latent frames, oldest evicted
// first (same section, second technique).  Per (token, head) row of 128
// values:
//   scale = amax / 127 (IEEE fp32, correctly rounded),
//   q     = round_half_even(x / scale) (correctly rounded fp32 quotient),
//           clamped to [-127, 127]; a zero row stores scale 0 and q 0.
//
// The kernel streams rows: 8 lanes own one row (16 bf16 = 32 bytes
// of K and 32 of V per lane), the row max is an 8-lane butterfly, and each
// lane writes 16 int8 codes (one 16-byte store) per tensor.  Consecutive
// 8-lane groups take the heads of one token, so each wave reads 8 x 256
// contiguous bytes per tensor and writes 8 rows of codes 8 heads apart (the
// cache is head-major, so that an attention tile of 64 keys of one head is
// one contiguous 8 KB block).  A token-major cache, whose writes are as
// contiguous as the reads, made this kernel 2-10% faster but the INT8
// attention tiles (64 rows 2 KB apart) 5-7% slower on 1280x704 segments with
// history, which costs far more.  Gathering 128 rows (128 / H tokens x all
// heads) per block in LDS and writing them head by head in runs of
// contiguous bytes was slower still (3.55 against 4.73 TB/s at 337 MB).
// (16-byte stores measured 9-13% faster than
// 8-byte ones; non-temporal loads/stores, two rows per lane group, and blocks
// of 32 consecutive tokens of one head, which write their codes and scales
// contiguously but read rows 4 KB apart, were slower: the last by 10%; so was
// a grid-stride loop over 4-16 blocks per CU with the next row prefetched,
// by 4-20%.  Of 128-, 512- and 1024-thread blocks none beat 256 on all of
// the 155-337 MB appends.)
// The quotient is taken as x * rcp(scale) and rounded; only where that
// product lies within 2^-13 of a half-integer (where it could round apart
// from the correctly rounded quotient), and for zero, tiny, huge or
// non-finite scales, does a group of 8 values take the compiler's correctly
// rounded fp32 divide (no fast-math).  This cut the VALU work about 3x: +10%
// on a 1280x704 segment's append with an 18-frame window (206 MB), +4% with
// no window (337 MB), no change on the 480x832 segment (155 MB), whose short
// launch is latency-bound.  fp32 denormals are preserved so subnormal scales
// quantize exactly.
// Row indexing takes no integer division in the kernel: the host passes
// multipliers for the divisions by H and P and the ring slot of the first
// surviving frame (the 64-bit remainder it replaces cost ~200 instructions
// before a wave's first load), and blocks are spread over the XCDs in
// contiguous ranges, so that the scale stores of the blocks one XCD runs
// together fill whole lines in its L2 (the bytes written now equal the
// algorithmic ones; with consecutive blocks on different XCDs they were 9.5%
// more).  Together: +3% on the 480x832 and +4% on the 337 MB appends, within
// 1% on the 206 MB one.
#include "hn_internal.h"

namespace hn {
namespace {

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Codes of the 8 values this lane holds, by the correctly rounded quotient
// x / scale; zero marks an all-zero row (codes 0).
__device__ inline uint2 quant8(const float (&x)[8], float scale, bool zero) {
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y = zero ? 0.0f : rintf(x[i] / scale);
    y = fminf(fmaxf(y, -127.0f), 127.0f);
    b[i] = (uint32_t)((int32_t)y) & 0xFFu;
  }
  uint2 r;
  r.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  r.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  return r;
}

// Fast path for 8 values of a row with a normal scale: y = x * rcp(scale)
// is within 3.1e-5 of the correctly rounded quotient fl(x / scale) when
// |y| <= 127.0001 (reciprocal within 1 ulp, product rounded, quotient rounded),
// so rint(y) == rint(fl(x / scale)) unless y lies within 2^-13 of a
// half-integer.  Returns false if some value is that close; the caller then
// takes the exact quotient for the 8 values.  Codes are packed as q + 128
// (an exact integer in [1, 255]) and turned into two's complement bytes by
// flipping bit 7.
__device__ inline bool quant8_fast(const float (&x)[8], float r, uint2& out) {
  float far = 0.0f;  // largest |y - rint(y)|
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = x[i] * r;
    const float q = __builtin_rintf(y);
    far = fmaxf(far, fabsf(y - q));
    w[i / 4] = __builtin_amdgcn_cvt_pk_u8_f32(q + 128.0f, i % 4, w[i / 4]);
  }
  out.x = w[0] ^ 0x80808080u;
  out.y = w[1] ^ 0x80808080u;
  return far <= 0.5f - 0x1p-13f;
}

// Codes of 8 values with the given scale; fast is false for a zero,
// subnormal-range or non-finite scale, which always take the exact quotient.
__device__ inline uint2 quant8_any(const float (&x)[8], float scale, float r, bool fast, bool zero) {
  uint2 q;
  if (fast && quant8_fast(x, r, q)) return q;
  return quant8(x, scale, zero);
}

__device__ inline void unpack8(uint4 w, float (&x)[8], float& amax) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  amax = m;
}

__device__ inline float row_amax8(float m) {
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  m = fmaxf(m, __shfl_xor(m, 4));
  return m;
}

// n / d for n < 2^31 with the host's multiplier and shift (div_magic).
__device__ inline uint32_t udiv31(uint32_t n, uint32_t m, int k) {
  return (uint32_t)(((uint64_t)n * m) >> k);
}

__global__ __launch_bounds__(256) void quant_append_kernel(AppendParams p) {
  const int lane8 = threadIdx.x & 7;
  // Block b runs on XCD b % 8; each XCD takes a contiguous range of the
  // 32-row units, so the blocks one XCD runs together cover consecutive
  // tokens and their 4-byte scale stores meet in that XCD's L2 as whole lines.
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  const uint32_t per = nb / 8, rem = nb % 8, x = b % 8, i = b / 8;
  const uint32_t blk = x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int64_t unit = (int64_t)blk * 32 + (threadIdx.x >> 3);
  const int64_t rows = (int64_t)p.head_len + p.n_vid;
  // Whole 8-lane groups leave together, so the butterflies below stay inside
  // active lanes.
  if (unit >= rows * p.H) return;
  // units stay below 2^31 (the host checks), so the 31-bit divisions hold
  const uint32_t u32 = (uint32_t)unit;
  const int t = (int)udiv31(u32, p.mag_h, p.sh_h);
  const int h = (int)(u32 - (uint32_t)t * (uint32_t)p.H);

  const __bf16 *ks, *vs;
  int8_t *kd, *vd;
  float *kds, *vds;
  int64_t src_row, dst_row;
  if (t < p.head_len) {
    src_row = t;
    dst_row = (int64_t)h * p.head_cap + p.head_pos + t;
    ks = p.k_txt; vs = p.v_txt;
    kd = p.heads_k; vd = p.heads_v; kds = p.heads_ks; vds = p.heads_vs;
  } else {
    // surviving video row rv: frame fl < W of the surviving ones, row pp in it
    const uint32_t rv = (uint32_t)(t - p.head_len);
    const uint32_t fl = udiv31(rv, p.mag_p, p.sh_p);
    const uint32_t pp = rv - fl * (uint32_t)p.P;
    uint32_t slot = (uint32_t)p.slot0 + fl;  // < 2W
    if (slot >= (uint32_t)p.W) slot -= (uint32_t)p.W;
    src_row = (int64_t)p.vid_first + rv;
    dst_row = (int64_t)h * p.ring_cap + (int64_t)(slot * (uint32_t)p.P + pp);
    ks = p.k_vid; vs = p.v_vid;
    kd = p.ring_k; vd = p.ring_v; kds = p.ring_ks; vds = p.ring_vs;
  }
  const int64_t src = (src_row * p.H + h) * D + lane8 * 16;
  const uint4 kw0 = *reinterpret_cast<const uint4*>(ks + src);
  const uint4 kw1 = *reinterpret_cast<const uint4*>(ks + src + 8);
  const uint4 vw0 = *reinterpret_cast<const uint4*>(vs + src);
  const uint4 vw1 = *reinterpret_cast<const uint4*>(vs + src + 8);

  float kx0[8], kx1[8], vx0[8], vx1[8], ka0, ka1, va0, va1;
  unpack8(kw0, kx0, ka0);
  unpack8(kw1, kx1, ka1);
  unpack8(vw0, vx0, va0);
  unpack8(vw1, vx1, va1);
  const float ka = row_amax8(fmaxf(ka0, ka1));
  const float va = row_amax8(fmaxf(va0, va1));
  const float ksc = ka / 127.0f;
  const float vsc = va / 127.0f;
  // a reciprocal within 1 ulp needs a normal, finite scale well inside range
  const bool kfast = ksc >= 0x1p-100f && ksc <= 0x1p100f;
  const bool vfast = vsc >= 0x1p-100f && vsc <= 0x1p100f;
  const float kr = __builtin_amdgcn_rcpf(kfast ? ksc : 1.0f);
  const float vr = __builtin_amdgcn_rcpf(vfast ? vsc : 1.0f);
  const uint2 kq0 = quant8_any(kx0, ksc, kr, kfast, ka == 0.0f);
  const uint2 kq1 = quant8_any(kx1, ksc, kr, kfast, ka == 0.0f);
  const uint2 vq0 = quant8_any(vx0, vsc, vr, vfast, va == 0.0f);
  const uint2 vq1 = quant8_any(vx1, vsc, vr, vfast, va == 0.0f);

  *reinterpret_cast<uint4*>(kd + dst_row * D + lane8 * 16) = make_uint4(kq0.x, kq0.y, kq1.x, kq1.y);
  *reinterpret_cast<uint4*>(vd + dst_row * D + lane8 * 16) = make_uint4(vq0.x, vq0.y, vq1.x, vq1.y);
  if (lane8 == 0) {
    kds[dst_row] = ka == 0.0f ? 0.0f : ksc;
    vds[dst_row] = va == 0.0f ? 0.0f : vsc;
  }
}

}  // namespace

hipError_t launch_quant_append(const AppendParams& p, hipStream_t s) {
  const int64_t units = ((int64_t)p.head_len + p.n_vid) * p.H;
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 31) / 32;
  hipLaunchKernelGGL(quant_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hn
