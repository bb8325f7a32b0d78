// Launcher of the cache V layout conversion (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

namespace beam {

// Rows of one workgroup's tile of the V layout conversion; the rows of a
// block (page_size, or window) must be a multiple.
constexpr int kVTransposeRows = 16;

// n_blocks blocks of `rows` x 128 elements of elem_bytes (2: bf16, 1: FP8
// code). to_cache != 0: src is token-major [block][rows][128] and dst gets
// [block][128][rows]; else the reverse. src and dst must not overlap.
hipError_t launch_kv_v_transpose(const void* src, void* dst, long long n_blocks, int rows, int elem_bytes,
                                 int to_cache, hipStream_t s);

}  // namespace beam
