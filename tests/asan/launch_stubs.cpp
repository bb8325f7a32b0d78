// Launch stubs for the AddressSanitizer build of the library's host side: the
// C ABI (beam_attn.hip compiled for the host only) runs its argument checks
// and workspace carving and then calls these instead of the HIP launchers.
// Each records the parameter block it was given, so that the driver can
// check what the host side would have launched, and returns hipSuccess.
#include "launch_stubs.h"

namespace stub {
Record last;
}

namespace beam {

hipError_t launch_prefill_prologue(const PrologueParams& p, int n_seqs, int n_tiles, hipStream_t) {
  ++stub::last.calls;
  stub::last.prologue = p;
  stub::last.grid_a = n_seqs;
  stub::last.grid_b = n_tiles;
  return hipSuccess;
}
hipError_t launch_kv_append(const AppendParams& p, hipStream_t) {
  ++stub::last.calls;
  stub::last.append = p;
  return hipSuccess;
}
hipError_t launch_decode_q_prologue(const DecodeQParams& p, hipStream_t) {
  ++stub::last.calls;
  stub::last.decode_q = p;
  return hipSuccess;
}
hipError_t launch_visibility(int, int, int, int, int, int, uint8_t*, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_validate_cache(const int32_t*, int, int, int, int, const int32_t*, int32_t*, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_kv_v_transpose(const void*, void*, long long n_blocks, int rows, int, int, hipStream_t) {
  ++stub::last.calls;
  stub::last.grid_a = (int)n_blocks;
  stub::last.grid_b = rows;
  return hipSuccess;
}
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t) {
  ++stub::last.calls;
  stub::last.prefill = p;
  return hipSuccess;
}
hipError_t launch_decode_split(const DecodeParams& p, int n_seqs, hipStream_t) {
  ++stub::last.calls;
  stub::last.decode = p;
  stub::last.grid_a = n_seqs;
  return hipSuccess;
}
hipError_t launch_decode_combine(const CombineParams& p, int, hipStream_t) {
  ++stub::last.calls;
  stub::last.combine = p;
  return hipSuccess;
}
hipError_t launch_verify_attn(const PrefillParams& p, int max_rows, hipStream_t) {
  ++stub::last.calls;
  stub::last.prefill = p;
  stub::last.grid_b = max_rows;
  return hipSuccess;
}
hipError_t launch_verify_combine(const VerifyCombineParams&, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_gemm(const GemmParams&, int, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_router_logits(const RouterParams&, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_router_select(const RouterParams&, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}
hipError_t launch_router_fused(const RouterParams&, hipStream_t) {
  ++stub::last.calls;
  return hipSuccess;
}

}  // namespace beam
