// Device-side helpers shared by the Beam attention kernels (gfx950 / CDNA4).
//
// Types for the bf16 MFMA operands, bf16 packing, the visibility predicate,
// the RMSNorm + RoPE/SSMax prologue math and the workspace indexing scheme.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

constexpr int D = 128;  // head dimension (the only one supported)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round two floats to bf16 (nearest-even) and pack (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

// ---- FP8 E4M3 (OCP E4M3FN) cache codes ----
// Code of the E4M3FN value nearest to x: ties to the even code, |x| >= 448
// saturates to +-448, NaN -> 0x7F. Normal range: round the fp32 exponent and
// top 3 mantissa bits to nearest even in one integer step (a carry moves into
// the exponent), then rebias 127 -> 7. Below 2^-6 the grid is k * 2^-9.
__device__ __forceinline__ uint32_t fp8_e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);  // 0..8; 8 is the smallest normal, 2^-6
  } else {
    const uint32_t ua = __float_as_uint(a);
    code = ((ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}
// Four codes (bytes of w, low first) -> four bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
// Four floats -> four codes of x / scale, packed low byte first.
__device__ __forceinline__ uint32_t fp8x4_encode(const float (&x)[4], float scale) {
  return fp8_e4m3_encode(x[0] / scale) | (fp8_e4m3_encode(x[1] / scale) << 8) | (fp8_e4m3_encode(x[2] / scale) << 16) |
         (fp8_e4m3_encode(x[3] / scale) << 24);
}
// Four codes -> four floats (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float (&f)[4]) {
  const u32x2 b = fp8x4_to_bf16x4(w);
  f[0] = bf16lo(b[0]);
  f[1] = bf16hi(b[0]);
  f[2] = bf16lo(b[1]);
  f[3] = bf16hi(b[1]);
}

// Visibility of key position s to query position t: causal, plus the window on
// local layers (window counts the current token, so window-1 earlier ones).
__device__ __forceinline__ bool visible(int kind, int window, int t, int s) {
  int dlt = t - s;
  return dlt >= 0 && (kind == 1 || dlt <= window - 1);
}

// SSMax query scale a(p) = (1 + p/base)^exponent at one-based p = t + 1, as
// 2^(exponent * log2(1 + p/base)) in float32 (relative error ~2e-7, far below
// the bf16 rounding of the scaled query).
__device__ __forceinline__ float ssmax_scale(int t, float base, float expo) {
  return exp2f(expo * log2f(1.0f + (float)(t + 1) / base));
}

// RoPE inverse frequency theta^(-2i/128) of pair i (float64).
// RoPE frequency of pair i in revolutions per position: theta^(-2i/d) / (2 pi).
__device__ __forceinline__ double rope_rev_per_pos(int i, float theta) {
  return pow((double)theta, -2.0 * (double)i / (double)D) * 0.15915494309189533577;
}
// cos/sin of the angle of position t: formed in revolutions in float64 and
// reduced to [-1/2, 1/2], then v_cos_f32 / v_sin_f32 (which take revolutions)
// in float32. Their error (~1e-6) is far below the bf16 rounding of the
// rotated vectors; a float32 product t * r would carry up to 0.01 revolutions
// of error at t = 10^6.
__device__ __forceinline__ void rope_cs_rev(int t, double r, float* c, float* s) {
  const double rev = (double)t * r;
  const float fr = (float)(rev - rint(rev));
  *c = __builtin_amdgcn_cosf(fr);
  *s = __builtin_amdgcn_sinf(fr);
}
__device__ __forceinline__ void rope_cs(int t, int i, float theta, float* c, float* s) {
  rope_cs_rev(t, rope_rev_per_pos(i, theta), c, s);
}

// Sum over the 16 lanes of an aligned 16-lane group.
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// One head vector (128 bf16) is handled by a 16-lane group: lane j holds the
// coordinates lo = [4j, 4j+4) and hi = [64+4j, 64+4j+4), so every rotate-half
// RoPE pair (i, i+64) sits in one lane. Computes
//   y = w * x / sqrt(mean(x^2) + eps)       (fp32)
//   optional RoPE at position t with per-lane cos/sin of pairs 4j..4j+3
//   y *= post_scale
// and returns the bf16-packed results (2 words for lo, 2 for hi).
struct HeadFrag {
  uint32_t lo[2];
  uint32_t hi[2];
};

// The fp32 values before the final scale and rounding: a = lo coordinates,
// b = hi coordinates.
__device__ __forceinline__ void norm_rope_f32(u32x2 xlo, u32x2 xhi, u32x2 wlo, u32x2 whi, float eps, bool do_rope,
                                              const float* cs, const float* sn, float (&a)[4], float (&b)[4]) {
  a[0] = bf16lo(xlo[0]);
  a[1] = bf16hi(xlo[0]);
  a[2] = bf16lo(xlo[1]);
  a[3] = bf16hi(xlo[1]);
  b[0] = bf16lo(xhi[0]);
  b[1] = bf16hi(xhi[0]);
  b[2] = bf16lo(xhi[1]);
  b[3] = bf16hi(xhi[1]);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + b[e] * b[e];
  ss = sum16(ss);
  float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  float wa[4] = {bf16lo(wlo[0]), bf16hi(wlo[0]), bf16lo(wlo[1]), bf16hi(wlo[1])};
  float wb[4] = {bf16lo(whi[0]), bf16hi(whi[0]), bf16lo(whi[1]), bf16hi(whi[1])};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = wa[e] * (a[e] * r);
    b[e] = wb[e] * (b[e] * r);
  }
  if (do_rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x1 = a[e], x2 = b[e];
      a[e] = x1 * cs[e] - x2 * sn[e];
      b[e] = x2 * cs[e] + x1 * sn[e];
    }
  }
}

__device__ __forceinline__ HeadFrag norm_rope_head(u32x2 xlo, u32x2 xhi, u32x2 wlo, u32x2 whi,
                                                   float eps, bool do_rope, const float* cs,
                                                   const float* sn, float post_scale) {
  float a[4], b[4];
  norm_rope_f32(xlo, xhi, wlo, whi, eps, do_rope, cs, sn, a, b);
  HeadFrag f;
  f.lo[0] = pack_bf16x2(a[0] * post_scale, a[1] * post_scale);
  f.lo[1] = pack_bf16x2(a[2] * post_scale, a[3] * post_scale);
  f.hi[0] = pack_bf16x2(b[0] * post_scale, b[1] * post_scale);
  f.hi[1] = pack_bf16x2(b[2] * post_scale, b[3] * post_scale);
  return f;
}

// Prefill workspace indexing. K_hat and V^T of the chunk tokens live in
// position-aligned per-sequence regions so that key tiles of 64 absolute
// positions never straddle a region boundary and 8-key groups stay 16-byte
// aligned: sequence i's region starts at 64*(cu[i]/64 + 2*i) and absolute
// position s maps to region_base + s - (start & ~63).
__device__ __forceinline__ int ws_region_base(int cu_i, int i) { return 64 * (cu_i / 64 + 2 * i); }
__host__ __device__ inline int64_t ws_positions(int n_tok, int n_seqs) {
  return 64 * ((int64_t)n_tok / 64 + 2 * (int64_t)n_seqs + 2);
}

// Index of the sequence whose token range [cu[i], cu[i+1]) holds token `tok`.
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int tok) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace beam
