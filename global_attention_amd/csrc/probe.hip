// Measurement instruments declared in include/beam_probe.h: the bf16 MFMA
// rate on random operands and the HBM streaming-read rate of one GPU.
#include <hip/hip_runtime.h>

#include "beam_attn.h"
#include "beam_device.h"
#include "beam_kernels.h"
#include "beam_probe.h"

namespace beam {

__global__ void __launch_bounds__(256) probe_mfma_kernel(const uint32_t* operands, int iters, int distinct,
                                                         float* out) {
  const size_t th = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(operands + th * 64);
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[i % distinct];
    b[i] = src[8 + i % distinct];
  }
  f32x16 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i & 7]), as_bf16x8(b[(3 * i + (i >> 3)) & 7]),
                                                           acc[i & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[r][i];
  out[th] = s;
}

// The same work with v_mfma_f32_16x16x32_bf16: 32 MFMAs of half the flops per
// iteration over 8 accumulators (each MFMA still reads a fresh A and B).
__global__ void __launch_bounds__(256) probe_mfma16_kernel(const uint32_t* operands, int iters, int distinct,
                                                           float* out) {
  const size_t th = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(operands + th * 64);
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[i % distinct];
    b[i] = src[8 + i % distinct];
  }
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
      acc[i & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i & 7]), as_bf16x8(b[(3 * i + (i >> 3)) & 7]),
                                                           acc[i & 7], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[r][i];
  out[th] = s;
}

__global__ void __launch_bounds__(256) probe_read_kernel(const u32x4* buf, size_t n16, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace beam

namespace {
beam_status probe_launch(hipError_t e, const char* what) {
  return e == hipSuccess ? BEAM_OK : beam::set_error(BEAM_E_HIP, what, e);
}
}  // namespace

extern "C" {

beam_status beam_probe_mfma_bf16(const uint32_t* operands, int32_t n_blocks, int32_t iters, int32_t distinct,
                                 float* out, void* stream) {
  beam::clear_stale_error();
  if (!operands || !out) return beam::set_error(BEAM_E_NULL, "operands or out is NULL", hipSuccess);
  if (n_blocks <= 0 || iters <= 0 || distinct < 1 || distinct > 8)
    return beam::set_error(BEAM_E_RANGE, "n_blocks, iters > 0 and 1 <= distinct <= 8 required", hipSuccess);
  if (reinterpret_cast<uintptr_t>(operands) % 16 != 0)
    return beam::set_error(BEAM_E_RANGE, "operands must be 16-byte aligned", hipSuccess);
  hipLaunchKernelGGL(beam::probe_mfma_kernel, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream, operands,
                     iters, distinct, out);
  return probe_launch(hipGetLastError(), "probe_mfma launch");
}

beam_status beam_probe_mfma16_bf16(const uint32_t* operands, int32_t n_blocks, int32_t iters, int32_t distinct,
                                   float* out, void* stream) {
  beam::clear_stale_error();
  if (!operands || !out) return beam::set_error(BEAM_E_NULL, "operands or out is NULL", hipSuccess);
  if (n_blocks <= 0 || iters <= 0 || distinct < 1 || distinct > 8)
    return beam::set_error(BEAM_E_RANGE, "n_blocks, iters > 0 and 1 <= distinct <= 8 required", hipSuccess);
  if (reinterpret_cast<uintptr_t>(operands) % 16 != 0)
    return beam::set_error(BEAM_E_RANGE, "operands must be 16-byte aligned", hipSuccess);
  hipLaunchKernelGGL(beam::probe_mfma16_kernel, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream,
                     operands, iters, distinct, out);
  return probe_launch(hipGetLastError(), "probe_mfma16 launch");
}

beam_status beam_probe_stream_read(const void* buf, size_t bytes, int32_t n_blocks, uint32_t* out, void* stream) {
  beam::clear_stale_error();
  if (!buf || !out) return beam::set_error(BEAM_E_NULL, "buf or out is NULL", hipSuccess);
  if (n_blocks <= 0 || bytes == 0 || bytes % 16 != 0)
    return beam::set_error(BEAM_E_RANGE, "n_blocks > 0 and bytes a positive multiple of 16 required", hipSuccess);
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return beam::set_error(BEAM_E_RANGE, "buf must be 16-byte aligned", hipSuccess);
  hipLaunchKernelGGL(beam::probe_read_kernel, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const beam::u32x4*>(buf), bytes / 16, out);
  return probe_launch(hipGetLastError(), "probe_read launch");
}

}  // extern "C"
