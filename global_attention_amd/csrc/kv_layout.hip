// V of a KV cache between the token-major layout and the layout the attention
// kernels read (gfx950).
//
// The cache holds one layer's values V per position and KV head ("KV memory:
// nine growing caches, not 52": K and V of every position on the nine global
// layers, a window of them on the 43 local layers). The attention kernels read
// V as the A operand of O^T += V^T P^T, so the library stores each page (or
// local ring) of one KV head coordinate-major, [128][rows]; a caller whose
// cache is token-major, [rows][128] as K is, converts V with one batched
// transpose. The values are moved, never converted.
//
// A workgroup moves a tile of 16 rows x 128 coordinates of one block through
// LDS: 8 consecutive elements per thread on both sides, so global reads and
// writes are 16-byte (bf16) or 8-byte (FP8) vectors and a page's 16 x 128 tile
// goes out as one contiguous 4 KiB (bf16) run.
#include <stdint.h>

#include "beam_device.h"
#include "kv_layout.h"

namespace beam {
namespace {

template <typename T>
struct Vec8;  // 8 elements in one vector access
template <>
struct Vec8<uint16_t> {
  using type = uint4;
};
template <>
struct Vec8<uint8_t> {
  using type = uint2;
};

template <typename T, bool TO_CACHE>
__global__ void __launch_bounds__(256) kv_v_transpose_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                             int rows) {
  using V8 = typename Vec8<T>::type;
  // [row][coordinate]; 8 elements of padding spread a column's rows over
  // the banks
  __shared__ __attribute__((aligned(16))) T tile[kVTransposeRows][D + 8];
  const int tiles = rows / kVTransposeRows;
  const size_t blk = blockIdx.x / tiles;
  const int r0 = (int)(blockIdx.x % tiles) * kVTransposeRows;
  const size_t base = blk * (size_t)rows * D;
  const int t = threadIdx.x;
  // token-major side: row r0 + tr, coordinates tc .. tc+7
  const int tr = t >> 4, tc = 8 * (t & 15);
  // coordinate-major side: coordinate cc, rows r0 + cr .. r0 + cr + 7
  const int cc = t >> 1, cr = 8 * (t & 1);
  union U {
    V8 v;
    T e[8];
  };
  if constexpr (TO_CACHE) {
    U u;
    u.v = *reinterpret_cast<const V8*>(src + base + (size_t)(r0 + tr) * D + tc);
    *reinterpret_cast<V8*>(&tile[tr][tc]) = u.v;
    __syncthreads();
    U w;
#pragma unroll
    for (int k = 0; k < 8; ++k) w.e[k] = tile[cr + k][cc];
    *reinterpret_cast<V8*>(dst + base + (size_t)cc * rows + r0 + cr) = w.v;
  } else {
    U u;
    u.v = *reinterpret_cast<const V8*>(src + base + (size_t)cc * rows + r0 + cr);
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[cr + k][cc] = u.e[k];
    __syncthreads();
    *reinterpret_cast<V8*>(dst + base + (size_t)(r0 + tr) * D + tc) = *reinterpret_cast<const V8*>(&tile[tr][tc]);
  }
}

}  // namespace

hipError_t launch_kv_v_transpose(const void* src, void* dst, long long n_blocks, int rows, int elem_bytes,
                                 int to_cache, hipStream_t s) {
  (void)hipGetLastError();  // a stale error must not be reported as this launch's
  if (rows <= 0 || rows % kVTransposeRows != 0 || n_blocks <= 0) return hipErrorInvalidValue;
  const long long wgs = n_blocks * (rows / kVTransposeRows);
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(256);
  if (elem_bytes == 2 && to_cache)
    hipLaunchKernelGGL((kv_v_transpose_kernel<uint16_t, true>), grid, block, 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL((kv_v_transpose_kernel<uint16_t, false>), grid, block, 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows);
  else if (elem_bytes == 1 && to_cache)
    hipLaunchKernelGGL((kv_v_transpose_kernel<uint8_t, true>), grid, block, 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows);
  else if (elem_bytes == 1)
    hipLaunchKernelGGL((kv_v_transpose_kernel<uint8_t, false>), grid, block, 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace beam
