// Kernel parameter blocks and kernel declarations (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "beam_attn.h"

namespace beam {

// Largest supported number of KV heads (the append keeps one head's K/V per
// register slot).
constexpr int kMaxKvHeads = 8;

struct PrologueParams {
  const uint16_t* q_raw;
  const uint16_t* k_raw;
  const uint16_t* v_raw;
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  const int32_t* cu;
  const int32_t* start_pos;
  uint16_t* qp;  // Q' [n_tok][H][D]
  uint16_t* kw;  // K_hat [G][P][D]
  uint16_t* vw;  // V^T [G][P/64][D][64] (64-position tiles)
  // Cache of the layer: the cached keys of a chunk's first 64-key tile (from
  // start & ~63 up to start) are copied into the workspace.
  uint16_t* ck;
  uint16_t* cv;
  const int32_t* bt;
  const int32_t* seq_idx;
  int max_pages, n_cache_seqs, window;
  // Global layers: also write the chunk's K_hat and V into their cache slots
  // (the append stage, fused; new positions never share a slot with the
  // cached prefix that attention reads).
  int append;
  // 0: K/V parts only (Q' is already in the workspace)
  int with_q;
  int kind, H, G, P;
  float rope_theta, rms_eps, ssmax_base, ssmax_exp;
  // FP8 E4M3 cache: ck/cv hold one-byte codes at the same element offsets.
  int kv_fp8;
  float k_scale, v_scale;
};

struct AppendParams {
  const uint16_t* k_raw;
  const uint16_t* v_raw;
  const uint16_t* k_norm_w;
  const int32_t* seq_idx;  // per token (public append) or per sequence (prefill)
  const int32_t* pos;      // per token (public append), else null
  const int32_t* cu;       // prefill chunk description, else null
  const int32_t* start_pos;
  int n_seqs;
  uint16_t* ck;
  uint16_t* cv;
  const int32_t* bt;
  int max_pages;
  int n_cache_seqs;  // rows of the block table (global) or rings (local)
  int kind, G, window, n_tok;
  float rope_theta, rms_eps;
  // FP8 E4M3 cache: ck/cv hold one-byte codes at the same element offsets.
  int kv_fp8;
  float k_scale, v_scale;
};

struct DecodeQParams {
  const uint16_t* q_raw;
  const uint16_t* q_norm_w;
  const int32_t* pos;
  uint16_t* qp;  // Q' [n_seqs][H][D]
  int kind, H, n_seqs;
  float rope_theta, rms_eps, ssmax_base, ssmax_exp;
  float k_scale;  // FP8 cache: K scale folded into Q' (1 for bf16)
};

// Prefill attention tiling: 48 queries per wavefront and 8 wavefronts per
// block on global layers (384 queries of one head, one block per CU); 32
// queries per wavefront and 4 wavefronts per block on local layers (two
// blocks per CU: a window-limited tile range favours smaller, independent
// blocks). A local block takes two query heads of one KV group (when the
// group's head count is even) and 64 queries: its four waves then need the
// same key tiles (nine per 64 aligned queries), so none idles at a barrier
// while the others compute.
constexpr int kPrefillWavesGlobal = 8;
constexpr int kPrefillWavesLocal = 4;
constexpr int prefill_wave_queries(int kind) { return kind == 0 ? 32 : 48; }
constexpr int prefill_heads_per_block(int kind, int heads_per_group) {
  return kind == 0 && heads_per_group % 2 == 0 ? 2 : 1;
}
constexpr int prefill_block_queries(int kind, int heads_per_group) {
  return prefill_wave_queries(kind) * (kind == 0 ? kPrefillWavesLocal : kPrefillWavesGlobal) /
         prefill_heads_per_block(kind, heads_per_group);
}

struct PrefillParams {
  const uint16_t* qp;  // Q' [n_tok][H][D]
  const uint16_t* kw;  // K_hat workspace [G][P][D]
  const uint16_t* vw;  // V^T workspace [G][P/64][D][64]
  const uint16_t* gate;
  const float* gate_bias;
  uint16_t* out;
  const int32_t* cu;
  const int32_t* seq_idx;
  const int32_t* start_pos;
  const uint16_t* ck;
  const uint16_t* cv;
  const int32_t* bt;
  int max_pages;
  int n_cache_seqs;
  int kind, window, H, G, n_seqs, n_qtiles, P;
  // FP8 E4M3 cache: a cached prefix is read as codes and dequantised to bf16.
  int kv_fp8;
  float k_scale, v_scale;
  // Verify (short chunks; key range split over blocks): partials per (token,
  // query head, split), and the split size in 64-key tiles.
  float* part_ml;   // [n_tok][H][n_splits][2] (reference max, sum) in base-2 logits
  float* part_acc;  // [n_tok][H][n_splits][D]
  int split_tiles, n_splits;
  // Verify with a single split: the split kernel writes the gated output
  // itself; a sequence whose chunk ends past max_pos gets NaN rows.
  int max_pos;
};

// Verify attention: a block takes one (sequence, KV head, key split) and packs
// the (token, query head) rows of the chunk, 32 per wavefront.
constexpr int kVerifyWaves = 4;
constexpr int kVerifyMaxRows = 32 * kVerifyWaves;
constexpr int kVerifyMaxSplitTiles = 128;  // 64-key tiles per verify split (their page ids are staged in LDS)

struct VerifyCombineParams {
  const float* part_ml;
  const float* part_acc;
  const int32_t* cu;
  const int32_t* start_pos;
  const int32_t* seq_idx;
  const uint16_t* gate;
  const float* gate_bias;
  uint16_t* out;
  const int32_t* bt;
  int max_pages, n_cache_seqs;
  int kind, window, H, n_seqs, n_tok, n_splits, split_tiles;
  int max_pos;  // a sequence whose chunk ends past max_pos gets NaN rows (its keys lie beyond the split grid)
  float v_scale;  // FP8 cache: V scale applied to O (1 for bf16)
};

struct DecodeParams {
  const uint16_t* qp;  // Q' [n_seqs][H][D]
  const uint16_t* ck;
  const uint16_t* cv;
  const int32_t* bt;
  int max_pages;
  const int32_t* seq_idx;
  const int32_t* pos;
  float* part_ml;   // [n_seqs][H][S][2] (max, sum) in base-2 logits
  float* part_acc;  // [n_seqs][H][S][D]
  int n_cache_seqs;
  int max_pos;
  int kind, window, H, G, n_splits, kpw;
  int kv_fp8;  // the cache holds FP8 E4M3 codes (one byte per element)
};

struct CombineParams {
  const float* part_ml;
  const float* part_acc;
  const int32_t* pos;
  const int32_t* seq_idx;  // a row outside [0, n_cache_seqs) gets NaN (the split kernel read nothing for it)
  int n_cache_seqs;
  const uint16_t* gate;
  const float* gate_bias;
  uint16_t* out;
  int max_pos;
  int kind, window, H, n_splits, split_keys;
  float v_scale;  // FP8 cache: V scale applied to O (1 for bf16)
};

// Every launcher clears an error an earlier runtime call left unread on this
// thread before it launches, so that the status it returns (hipGetLastError
// after the launch) is about its own launch only.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Records a failed call's message for beam_last_error() (host, thread-local)
// and returns the status; for the sources other than beam_attn.hip.
beam_status set_error(beam_status s, const char* what, hipError_t e);

// Host-side launchers (each defined next to its kernel). They return the
// launch status of the HIP runtime.
hipError_t launch_prefill_prologue(const PrologueParams& p, int n_seqs, int n_tiles, hipStream_t s);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);
hipError_t launch_decode_q_prologue(const DecodeQParams& p, hipStream_t s);
hipError_t launch_visibility(int kind, int window, int t0, int n_q, int s0, int n_k, uint8_t* mask,
                             hipStream_t s);
hipError_t launch_validate_cache(const int32_t* bt, int max_pages, int n_pages, int page_size, int n_seqs,
                                 const int32_t* n_tokens, int32_t* n_bad, hipStream_t s);
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s);
hipError_t launch_decode_split(const DecodeParams& p, int n_seqs, hipStream_t s);
hipError_t launch_decode_combine(const CombineParams& p, int n_seqs, hipStream_t s);
hipError_t launch_verify_attn(const PrefillParams& p, int max_rows, hipStream_t s);
hipError_t launch_verify_combine(const VerifyCombineParams& p, hipStream_t s);

// ---- projection GEMMs: out[t][f] = sum_k x[t][k] w[f][k] (bf16, fp32 accumulate) ----
constexpr int kGemmTile = 256;  // n_feat must be a multiple; K a multiple of 128
constexpr int kEpiPlain = 0;    // out[t][ld_out], columns f
constexpr int kEpiQkvg = 1;     // Q' (fused norm + position op) / K / V / gate heads

struct GemmParams {
  const uint16_t* x;  // [n_tok][K]
  const uint16_t* w;  // [n_feat][K]
  int n_tok, n_feat, K;
  // plain epilogue
  uint16_t* out;
  int ld_out;
  // QKV/gate epilogue: rows of w are the H query heads, G key heads, G value
  // heads and H gate heads (128 rows each)
  uint16_t* q_out;  // Q' [n_tok][H][D] (base-2 softmax scale folded in)
  uint16_t* k_out;  // raw K [n_tok][G][D]
  uint16_t* v_out;  // raw V [n_tok][G][D]
  uint16_t* g_out;  // raw gate logits [n_tok][H][D]
  const uint16_t* q_norm_w;
  const int32_t* cu;
  const int32_t* start_pos;
  int n_seqs, kind, H, G;
  float rope_theta, rms_eps, ssmax_base, ssmax_exp;
};
hipError_t launch_gemm(const GemmParams& p, int epi, hipStream_t s);

// ---- group-limited sigmoid router (MoE expert selection) ----
constexpr int kRouterExperts = 256;
constexpr int kRouterGroups = 8;
constexpr int kRouterBlockTokens = 128;  // tokens per block of the logits GEMM
constexpr int kRouterKChunk = 32;        // hidden must be a multiple
constexpr int kRouterTopKMax = 8;        // largest supported top_k

struct RouterParams {
  const uint16_t* x;       // bf16 [n_tok][hidden]
  const float* w;          // [256][hidden]
  const float* bias;       // [256] or nullptr (zero)
  const float* logits_in;  // select: [n_tok][256]
  float* logits_out;       // logits: [n_tok][256]
  int32_t* idx;            // [n_tok][top_k]
  float* wts;              // [n_tok][top_k]
  int n_tok, hidden, topk_groups, top_k;
  float scale;
};
hipError_t launch_router_logits(const RouterParams& p, hipStream_t s);
hipError_t launch_router_select(const RouterParams& p, hipStream_t s);
hipError_t launch_router_fused(const RouterParams& p, hipStream_t s);

}  // namespace beam
