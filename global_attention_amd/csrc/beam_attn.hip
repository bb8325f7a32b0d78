// Host side of the C ABI declared in include/beam_attn.h: argument checks,
// workspace carving and kernel launches. Nothing here allocates, frees or
// synchronises; every call only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <initializer_list>
#include <algorithm>
#include <mutex>
#include <string>

#include "beam_attn.h"
#include "beam_proj.h"
#include "beam_router.h"
#include "beam_device.h"
#include "beam_kernels.h"
#include "kv_layout.h"

namespace {

thread_local std::string g_last_error;

beam_status fail(beam_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

beam_status ok() {
  g_last_error.clear();
  return BEAM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The kernels move tensor rows with 8- and 16-byte vector accesses (and the
// caches with 16-byte LDS DMA): every bf16 tensor must be 16-byte aligned
// (NULL, for an optional argument, passes).
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (!aligned16(q)) return false;
  return true;
}

beam_status check_cfg(const beam_attn_config* c) {
  if (!c) return fail(BEAM_E_NULL, "cfg is NULL");
  if (c->head_dim != beam::D) return fail(BEAM_E_UNSUPPORTED, "head_dim must be 128");
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0) return fail(BEAM_E_SHAPE, "head counts must be positive");
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(BEAM_E_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > 16)
    return fail(BEAM_E_UNSUPPORTED, "at most 16 query heads per KV head");
  if (c->n_kv_heads > beam::kMaxKvHeads) return fail(BEAM_E_UNSUPPORTED, "at most 8 KV heads");
  if (c->window <= 0 || c->window % 64 != 0)
    return fail(BEAM_E_UNSUPPORTED, "window must be a positive multiple of 64");
  if (!(c->rms_eps >= 0.f) || !(c->ssmax_base > 0.f) || !(c->rope_theta > 0.f))
    return fail(BEAM_E_RANGE, "rms_eps >= 0, ssmax_base > 0 and rope_theta > 0 required");
  return BEAM_OK;
}

beam_status check_cache(const beam_kv_cache* kv) {
  if (!kv) return fail(BEAM_E_NULL, "cache is NULL");
  if (kv->kind != BEAM_LOCAL && kv->kind != BEAM_GLOBAL) return fail(BEAM_E_RANGE, "cache kind must be 0 or 1");
  if (kv->dtype != BEAM_KV_BF16 && kv->dtype != BEAM_KV_FP8_E4M3)
    return fail(BEAM_E_UNSUPPORTED, "cache dtype must be BEAM_KV_BF16 or BEAM_KV_FP8_E4M3");
  if (kv->dtype == BEAM_KV_FP8_E4M3 &&
      !(kv->k_scale > 0.f && kv->v_scale > 0.f && kv->k_scale < 3.0e38f && kv->v_scale < 3.0e38f))
    return fail(BEAM_E_RANGE, "FP8 cache scales must be finite and positive");
  if (!kv->k || !kv->v) return fail(BEAM_E_NULL, "cache k/v is NULL");
  if (!all_aligned16({kv->k, kv->v})) return fail(BEAM_E_RANGE, "cache k/v must be 16-byte aligned");
  if (kv->n_seqs <= 0) return fail(BEAM_E_RANGE, "cache n_seqs must be positive");
  if (kv->kind == BEAM_GLOBAL) {
    if (kv->page_size != 16) return fail(BEAM_E_UNSUPPORTED, "page_size must be 16");
    if (!kv->block_table) return fail(BEAM_E_NULL, "block_table is NULL");
    if (kv->max_pages_per_seq <= 0 || kv->n_pages <= 0)
      return fail(BEAM_E_RANGE, "max_pages_per_seq and n_pages must be positive");
  }
  return BEAM_OK;
}

// Default decode split: 2048 keys on global layers; 128 on local layers, whose
// window holds at most 512 keys (four splits per sequence and KV head keep
// more blocks in flight: a 64-sequence local decode 49 -> 44 us per call).
int decode_keys_max(const beam_attn_config* c, int kind, int max_pos) {
  return kind == BEAM_LOCAL ? (max_pos + 1 < c->window ? max_pos + 1 : c->window) : max_pos + 1;
}

// Default decode split: 128 keys on local layers; on global layers 4096 keys
// when that still gives at least 1024 blocks (sequences x KV heads x splits),
// else 2048. Measured on one MI355X (split kernel): 64 sequences at
// 64K-128K 4.27 ms at 2048, 4.17 at 4096, 4.22 at 8192 keys (FP8 cache 2.29,
// 2.25, 2.29); one sequence at 2^20 0.700, 0.680, 0.671 ms.
int default_split_keys(const beam_attn_config* c, int kind, int n_seqs, int max_pos) {
  if (kind == BEAM_LOCAL) return 128;
  const long long nk = decode_keys_max(c, kind, max_pos);
  const long long blocks = (long long)n_seqs * c->n_kv_heads * ((nk + 4095) / 4096);
  return blocks >= 1024 ? 4096 : 2048;
}

struct DecodeWs {
  size_t qp, ml, acc, total;
  int n_splits, split_keys;
};

bool decode_ws_layout(const beam_attn_config* c, int kind, int n_seqs, int max_pos, int split_keys,
                      DecodeWs* ws) {
  if (n_seqs <= 0 || max_pos < 0) return false;
  if (split_keys == 0) split_keys = default_split_keys(c, kind, n_seqs, max_pos);
  if (split_keys < 128 || split_keys % 128 != 0 || split_keys > 65536) return false;
  const int nk = decode_keys_max(c, kind, max_pos);
  ws->split_keys = split_keys;
  ws->n_splits = (nk + split_keys - 1) / split_keys;
  const size_t rows = (size_t)n_seqs * c->n_q_heads * ws->n_splits;
  ws->qp = 0;
  ws->ml = align256((size_t)n_seqs * c->n_q_heads * beam::D * 2);
  ws->acc = ws->ml + align256(rows * 2 * sizeof(float));
  ws->total = ws->acc + align256(rows * beam::D * sizeof(float));
  return true;
}

struct PrefillWs {
  size_t qp, kw, vw, total;
  int64_t P;
};

PrefillWs prefill_ws_layout(const beam_attn_config* c, int n_tok, int n_seqs) {
  PrefillWs ws;
  ws.P = beam::ws_positions(n_tok, n_seqs);
  ws.qp = 0;
  ws.kw = align256((size_t)n_tok * c->n_q_heads * beam::D * 2);
  ws.vw = ws.kw + align256((size_t)c->n_kv_heads * ws.P * beam::D * 2);
  ws.total = ws.vw + align256((size_t)c->n_kv_heads * beam::D * ws.P * 2);
  return ws;
}

// 64-key tiles a local-layer chunk of max_chunk_len tokens can touch: the
// window before its first token and the chunk itself, one more for alignment.
int local_span_tiles(const beam_attn_config* c, int max_chunk_len) {
  return ((c->window - 1 + (max_chunk_len > 0 ? max_chunk_len - 1 : 0)) >> 6) + 2;
}

// Default keys per verify split. Local layers: one split over the whole span
// when the (sequence, KV head) pairs alone give 256 blocks or more, so no
// merge pass runs and the split kernel writes the gated output (64 sequences:
// 62 instead of 95 us per call); else 256 keys, for parallelism. Global
// layers: the longest of 8192, 4096 keys that still gives at least 1024 blocks
// (two per CU slot at two blocks per CU), else 2048. Longer splits mean fewer
// partials to merge and less per-block work.
int default_verify_split_keys(const beam_attn_config* c, int kind, int n_seqs, int max_pos, int max_chunk_len) {
  if (kind == BEAM_LOCAL) {
    if ((long long)n_seqs * c->n_kv_heads < 256) return 256;
    return 64 * std::min(local_span_tiles(c, max_chunk_len), beam::kVerifyMaxSplitTiles);
  }
  for (int keys = 8192; keys >= 4096; keys /= 2) {
    const long long blocks = (long long)n_seqs * c->n_kv_heads * (max_pos / keys + 1);
    if (blocks >= 1024) return keys;
  }
  return 2048;
}

// Verify (short-chunk) calls: the prefill workspace, then the split partials
// (reference max and sum, and the unnormalised accumulator) per (token, head,
// split). A sequence's keys span at most n_tiles 64-key tiles.
struct VerifyWs {
  PrefillWs pre;
  size_t ml, acc, total;
  int n_splits, split_tiles;
};

bool verify_ws_layout(const beam_attn_config* c, int kind, int n_tok, int n_seqs, int max_chunk_len, int max_pos,
                      int split_keys, VerifyWs* ws) {
  if (split_keys == 0) split_keys = default_verify_split_keys(c, kind, n_seqs, max_pos, max_chunk_len);
  if (split_keys < 64 || split_keys % 64 != 0 || split_keys > 64 * beam::kVerifyMaxSplitTiles) return false;
  if (n_seqs <= 0 || n_tok < 0 || max_chunk_len < 0 || max_pos < 0) return false;
  int n_tiles = (max_pos >> 6) + 1;
  if (kind == BEAM_LOCAL) n_tiles = std::min(n_tiles, local_span_tiles(c, max_chunk_len));
  ws->split_tiles = split_keys / 64;
  ws->n_splits = (n_tiles + ws->split_tiles - 1) / ws->split_tiles;
  ws->pre = prefill_ws_layout(c, n_tok, n_seqs);
  const size_t rows = (size_t)n_tok * c->n_q_heads * ws->n_splits;
  ws->ml = ws->pre.total;
  ws->acc = ws->ml + align256(rows * 2 * sizeof(float));
  ws->total = ws->acc + align256(rows * beam::D * sizeof(float));
  return true;
}

beam_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BEAM_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return BEAM_OK;
}

}  // namespace

namespace beam {
beam_status set_error(beam_status s, const char* what, hipError_t e) {
  return fail(s, std::string(what) + (e != hipSuccess ? std::string(": ") + hipGetErrorString(e) : std::string()));
}
}  // namespace beam

extern "C" {

const char* beam_status_str(beam_status s) {
  switch (s) {
    case BEAM_OK: return "ok";
    case BEAM_E_NULL: return "null pointer";
    case BEAM_E_SHAPE: return "inconsistent shape";
    case BEAM_E_RANGE: return "value out of range";
    case BEAM_E_UNSUPPORTED: return "unsupported configuration";
    case BEAM_E_WORKSPACE: return "workspace too small";
    case BEAM_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* beam_last_error(void) { return g_last_error.c_str(); }

beam_status beam_kv_bytes(int64_t n_tokens, int32_t bytes_per_scalar, int32_t n_global, int32_t n_local,
                          int32_t n_kv, int32_t d, int32_t window, int32_t page_size, uint64_t* logical,
                          uint64_t* paged) {
  if (!logical || !paged) return fail(BEAM_E_NULL, "output pointer is NULL");
  if (n_tokens < 0 || bytes_per_scalar <= 0 || n_global < 0 || n_local < 0 || n_kv <= 0 || d <= 0 ||
      window <= 0 || page_size <= 0)
    return fail(BEAM_E_RANGE, "sizes must be positive (n_tokens, n_global, n_local >= 0)");
  const uint64_t per_tok = 2ull * (uint64_t)bytes_per_scalar * (uint64_t)n_kv * (uint64_t)d;
  const uint64_t n = (uint64_t)n_tokens;
  const uint64_t slots = n < (uint64_t)window ? n : (uint64_t)window;
  const uint64_t pages = (n + (uint64_t)page_size - 1) / (uint64_t)page_size;
  *logical = per_tok * ((uint64_t)n_global * n + (uint64_t)n_local * slots);
  *paged = per_tok * ((uint64_t)n_global * pages * (uint64_t)page_size + (uint64_t)n_local * slots);
  return ok();
}

beam_status beam_kv_page_slot(const int32_t* block_table_host, int32_t max_pages_per_seq, int32_t page_size,
                              int32_t seq, int32_t t, int64_t* phys_page, int32_t* slot) {
  if (!block_table_host || !phys_page || !slot) return fail(BEAM_E_NULL, "NULL argument");
  if (page_size <= 0 || max_pages_per_seq <= 0 || seq < 0 || t < 0)
    return fail(BEAM_E_RANGE, "negative or zero size/index");
  if (t / page_size >= max_pages_per_seq) return fail(BEAM_E_RANGE, "position beyond block-table row");
  *phys_page = block_table_host[(int64_t)seq * max_pages_per_seq + t / page_size];
  *slot = t % page_size;
  return ok();
}

size_t beam_prefill_workspace_bytes(const beam_attn_config* cfg, int32_t n_tok, int32_t n_seqs) {
  if (check_cfg(cfg) != BEAM_OK || n_tok < 0 || n_seqs <= 0) return 0;
  return prefill_ws_layout(cfg, n_tok, n_seqs).total;
}

size_t beam_verify_workspace_bytes(const beam_attn_config* cfg, int32_t kind, int32_t n_tok, int32_t n_seqs,
                                   int32_t max_chunk_len, int32_t max_pos, int32_t split_keys) {
  if (check_cfg(cfg) != BEAM_OK || (kind != BEAM_LOCAL && kind != BEAM_GLOBAL)) return 0;
  VerifyWs ws;
  if (!verify_ws_layout(cfg, kind, n_tok, n_seqs, max_chunk_len, max_pos, split_keys, &ws)) return 0;
  return ws.total;
}

size_t beam_decode_workspace_bytes(const beam_attn_config* cfg, int32_t kind, int32_t n_seqs, int32_t max_pos,
                                   int32_t split_keys) {
  if (check_cfg(cfg) != BEAM_OK || (kind != BEAM_LOCAL && kind != BEAM_GLOBAL)) return 0;
  DecodeWs ws;
  if (!decode_ws_layout(cfg, kind, n_seqs, max_pos, split_keys, &ws)) return 0;
  return ws.total;
}

beam_status beam_kv_append(const beam_attn_config* cfg, const beam_kv_cache* cache, const beam_bf16* k_raw,
                           const beam_bf16* v_raw, const beam_bf16* k_norm_w, const int32_t* seq_idx,
                           const int32_t* pos, int32_t n_tok, void* stream) {
  beam_status st;
  if ((st = check_cfg(cfg)) != BEAM_OK) return st;
  if ((st = check_cache(cache)) != BEAM_OK) return st;
  if (n_tok < 0) return fail(BEAM_E_RANGE, "n_tok must be >= 0");
  if (n_tok == 0) return ok();
  if (!k_raw || !v_raw || !k_norm_w || !seq_idx || !pos) return fail(BEAM_E_NULL, "NULL input pointer");
  if (!all_aligned16({k_raw, v_raw, k_norm_w})) return fail(BEAM_E_RANGE, "k_raw, v_raw and k_norm_w must be 16-byte aligned");
  beam::AppendParams p{};
  p.k_raw = k_raw;
  p.v_raw = v_raw;
  p.k_norm_w = k_norm_w;
  p.seq_idx = seq_idx;
  p.pos = pos;
  p.cu = nullptr;
  p.start_pos = nullptr;
  p.n_seqs = 0;
  p.ck = static_cast<uint16_t*>(cache->k);
  p.cv = static_cast<uint16_t*>(cache->v);
  p.bt = cache->block_table;
  p.max_pages = cache->max_pages_per_seq;
  p.n_cache_seqs = cache->n_seqs;
  p.kind = cache->kind;
  p.G = cfg->n_kv_heads;
  p.window = cfg->window;
  p.n_tok = n_tok;
  p.rope_theta = cfg->rope_theta;
  p.rms_eps = cfg->rms_eps;
  p.kv_fp8 = cache->dtype == BEAM_KV_FP8_E4M3;
  p.k_scale = cache->k_scale;
  p.v_scale = cache->v_scale;
  if ((st = hip_status(beam::launch_kv_append(p, (hipStream_t)stream), "kv_append launch")) != BEAM_OK) return st;
  return ok();
}

}  // extern "C"

namespace {

// Prefill and verify share the prologue, the workspace layout and the append;
// verify (verify == true) runs the split-key attention and its combine instead
// of the prefill attention kernel.
beam_status chunk_call(bool verify, uint32_t stages, const beam_attn_config* cfg, const beam_kv_cache* cache,
                       const beam_bf16* q_raw, const beam_bf16* k_raw, const beam_bf16* v_raw,
                       const beam_bf16* q_norm_w, const beam_bf16* k_norm_w, const beam_bf16* gate_logits,
                       const float* gate_bias, const int32_t* cu_seqlens, const int32_t* seq_idx,
                       const int32_t* start_pos, int32_t n_seqs, int32_t n_tok, int32_t max_chunk_len,
                       int32_t max_pos, int32_t split_keys, beam_bf16* out, void* workspace, size_t ws_bytes,
                       void* stream) {
  beam_status st;
  if (stages & ~(verify ? 15u | BEAM_STAGE_PROLOGUE_KV : 7u | BEAM_STAGE_PROLOGUE_KV))
    return fail(BEAM_E_RANGE, "unknown stage bits");
  if ((stages & BEAM_STAGE_PROLOGUE) && (stages & BEAM_STAGE_PROLOGUE_KV))
    return fail(BEAM_E_RANGE, "BEAM_STAGE_PROLOGUE and BEAM_STAGE_PROLOGUE_KV are exclusive");
  if ((st = check_cfg(cfg)) != BEAM_OK) return st;
  if ((st = check_cache(cache)) != BEAM_OK) return st;
  if (n_seqs <= 0) return fail(BEAM_E_RANGE, "n_seqs must be positive");
  if (n_tok < 0 || max_chunk_len < 0) return fail(BEAM_E_RANGE, "n_tok and max_chunk_len must be >= 0");
  if (n_tok == 0) return ok();
  if (max_chunk_len == 0 || max_chunk_len > n_tok)
    return fail(BEAM_E_RANGE, "max_chunk_len must be in [1, n_tok]");
  if ((!q_raw && (stages & BEAM_STAGE_PROLOGUE)) || !k_raw || !v_raw || !q_norm_w || !k_norm_w || !gate_logits ||
      !cu_seqlens || !seq_idx || !start_pos || !out)
    return fail(BEAM_E_NULL, "NULL input/output pointer");
  if (!all_aligned16({q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate_logits, out}))
    return fail(BEAM_E_RANGE, "bf16 tensors (q_raw, k_raw, v_raw, norm weights, gate_logits, out) must be 16-byte aligned");
  if (!workspace) return fail(BEAM_E_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(BEAM_E_RANGE, "workspace must be 256-byte aligned");
  VerifyWs vws{};
  if (verify) {
    const int hpg = cfg->n_q_heads / cfg->n_kv_heads;
    if ((int64_t)max_chunk_len * hpg > beam::kVerifyMaxRows)
      return fail(BEAM_E_RANGE, "verify chunk too long: max_chunk_len x (n_q_heads / n_kv_heads) must be <= " +
                                    std::to_string(beam::kVerifyMaxRows));
    if (max_pos < max_chunk_len - 1) return fail(BEAM_E_RANGE, "max_pos must be >= max_chunk_len - 1");
    if (!verify_ws_layout(cfg, cache->kind, n_tok, n_seqs, max_chunk_len, max_pos, split_keys, &vws))
      return fail(BEAM_E_RANGE, "split_keys must be 0 or a multiple of 64 in [64, 8192]");
    if (ws_bytes < vws.total)
      return fail(BEAM_E_WORKSPACE, "verify workspace needs " + std::to_string(vws.total) + " bytes");
    if ((int64_t)cfg->n_kv_heads * vws.n_splits * n_seqs > 0x7fffffffLL || (int64_t)n_tok * cfg->n_q_heads > 0x7fffffffLL)
      return fail(BEAM_E_RANGE, "verify grid too large");
  }
  const PrefillWs ws = prefill_ws_layout(cfg, n_tok, n_seqs);
  if (!verify && ws_bytes < ws.total)
    return fail(BEAM_E_WORKSPACE, "prefill workspace needs " + std::to_string(ws.total) + " bytes");
  if (ws.P * beam::D > 0x7fffffff) return fail(BEAM_E_RANGE, "too many tokens in one call (workspace positions x 128 must stay below 2^31)");
  if (!verify) {
    const int hpg = cfg->n_q_heads / cfg->n_kv_heads;
    const int bq = beam::prefill_block_queries(cache->kind, hpg);
    const int64_t blocks = (int64_t)(cfg->n_q_heads / beam::prefill_heads_per_block(cache->kind, hpg)) * n_seqs *
                           ((max_chunk_len + bq - 1) / bq);
    if (blocks > 0x7fffffffLL) return fail(BEAM_E_RANGE, "prefill grid too large (n_seqs x max_chunk_len)");
  }
  hipStream_t s = (hipStream_t)stream;
  char* wsb = static_cast<char*>(workspace);
  uint16_t* qp = reinterpret_cast<uint16_t*>(wsb + ws.qp);
  uint16_t* kw = reinterpret_cast<uint16_t*>(wsb + ws.kw);
  uint16_t* vw = reinterpret_cast<uint16_t*>(wsb + ws.vw);

  beam::PrologueParams pp{};
  pp.q_raw = q_raw;
  pp.k_raw = k_raw;
  pp.v_raw = v_raw;
  pp.q_norm_w = q_norm_w;
  pp.k_norm_w = k_norm_w;
  pp.cu = cu_seqlens;
  pp.start_pos = start_pos;
  pp.qp = qp;
  pp.kw = kw;
  pp.vw = vw;
  pp.ck = static_cast<uint16_t*>(cache->k);
  pp.cv = static_cast<uint16_t*>(cache->v);
  // Global layers: the append rides along with the prologue when both run.
  const bool prologue = stages & (BEAM_STAGE_PROLOGUE | BEAM_STAGE_PROLOGUE_KV);
  pp.append = cache->kind == BEAM_GLOBAL && prologue && (stages & BEAM_STAGE_APPEND);
  pp.with_q = (stages & BEAM_STAGE_PROLOGUE) != 0;
  pp.kv_fp8 = cache->dtype == BEAM_KV_FP8_E4M3;
  pp.k_scale = cache->k_scale;
  pp.v_scale = cache->v_scale;
  pp.bt = cache->block_table;
  pp.seq_idx = seq_idx;
  pp.max_pages = cache->max_pages_per_seq;
  pp.n_cache_seqs = cache->n_seqs;
  pp.window = cfg->window;
  pp.kind = cache->kind;
  pp.H = cfg->n_q_heads;
  pp.G = cfg->n_kv_heads;
  pp.P = (int)ws.P;
  pp.rope_theta = cfg->rope_theta;
  pp.rms_eps = cfg->rms_eps;
  pp.ssmax_base = cfg->ssmax_base;
  pp.ssmax_exp = cfg->ssmax_exp;
  const int n_tiles = (max_chunk_len + 63) / 64 + 1;
  if (prologue &&
      (st = hip_status(beam::launch_prefill_prologue(pp, n_seqs, n_tiles, s), "prologue launch")) != BEAM_OK)
    return st;

  beam::PrefillParams ap{};
  ap.qp = qp;
  ap.kw = kw;
  ap.vw = vw;
  ap.gate = gate_logits;
  ap.gate_bias = gate_bias;
  ap.out = out;
  ap.cu = cu_seqlens;
  ap.seq_idx = seq_idx;
  ap.start_pos = start_pos;
  ap.ck = static_cast<const uint16_t*>(cache->k);
  ap.cv = static_cast<const uint16_t*>(cache->v);
  ap.bt = cache->block_table;
  ap.max_pages = cache->max_pages_per_seq;
  ap.n_cache_seqs = cache->n_seqs;
  ap.kind = cache->kind;
  ap.window = cfg->window;
  ap.H = cfg->n_q_heads;
  ap.G = cfg->n_kv_heads;
  ap.n_seqs = n_seqs;
  {
    const int bq = beam::prefill_block_queries(cache->kind, cfg->n_q_heads / cfg->n_kv_heads);
    ap.n_qtiles = (max_chunk_len + bq - 1) / bq;
  }
  ap.P = (int)ws.P;
  ap.kv_fp8 = cache->dtype == BEAM_KV_FP8_E4M3;
  ap.k_scale = cache->k_scale;
  ap.v_scale = cache->v_scale;
  if (!verify) {
    if ((stages & BEAM_STAGE_ATTENTION) &&
        (st = hip_status(beam::launch_prefill_attn(ap, s), "prefill attention launch")) != BEAM_OK)
      return st;
  } else {
    ap.part_ml = reinterpret_cast<float*>(wsb + vws.ml);
    ap.part_acc = reinterpret_cast<float*>(wsb + vws.acc);
    ap.split_tiles = vws.split_tiles;
    ap.n_splits = vws.n_splits;
    ap.max_pos = max_pos;
    if ((stages & BEAM_STAGE_ATTENTION) &&
        (st = hip_status(beam::launch_verify_attn(ap, max_chunk_len * (cfg->n_q_heads / cfg->n_kv_heads), s),
                         "verify attention launch")) != BEAM_OK)
      return st;
    beam::VerifyCombineParams cp{};
    cp.part_ml = ap.part_ml;
    cp.part_acc = ap.part_acc;
    cp.cu = cu_seqlens;
    cp.start_pos = start_pos;
    cp.seq_idx = seq_idx;
    cp.gate = gate_logits;
    cp.gate_bias = gate_bias;
    cp.out = out;
    cp.bt = cache->block_table;
    cp.max_pages = cache->max_pages_per_seq;
    cp.n_cache_seqs = cache->n_seqs;
    cp.kind = cache->kind;
    cp.window = cfg->window;
    cp.H = cfg->n_q_heads;
    cp.n_seqs = n_seqs;
    cp.n_tok = n_tok;
    cp.n_splits = vws.n_splits;
    cp.split_tiles = vws.split_tiles;
    cp.max_pos = max_pos;
    cp.v_scale = cache->dtype == BEAM_KV_FP8_E4M3 ? cache->v_scale : 1.f;
    // one split: the attention stage has already written the gated output
    if ((stages & BEAM_STAGE_VERIFY_COMBINE) && vws.n_splits > 1 &&
        (st = hip_status(beam::launch_verify_combine(cp, s), "verify combine launch")) != BEAM_OK)
      return st;
  }

  beam::AppendParams xp{};
  xp.k_raw = k_raw;
  xp.v_raw = v_raw;
  xp.k_norm_w = k_norm_w;
  xp.seq_idx = seq_idx;
  xp.pos = nullptr;
  xp.cu = cu_seqlens;
  xp.start_pos = start_pos;
  xp.n_seqs = n_seqs;
  xp.ck = static_cast<uint16_t*>(cache->k);
  xp.cv = static_cast<uint16_t*>(cache->v);
  xp.bt = cache->block_table;
  xp.max_pages = cache->max_pages_per_seq;
  xp.n_cache_seqs = cache->n_seqs;
  xp.kind = cache->kind;
  xp.G = cfg->n_kv_heads;
  xp.window = cfg->window;
  xp.n_tok = n_tok;
  xp.rope_theta = cfg->rope_theta;
  xp.rms_eps = cfg->rms_eps;
  xp.kv_fp8 = cache->dtype == BEAM_KV_FP8_E4M3;
  xp.k_scale = cache->k_scale;
  xp.v_scale = cache->v_scale;
  if ((stages & BEAM_STAGE_APPEND) && !pp.append &&
      (st = hip_status(beam::launch_kv_append(xp, s), "prefill append launch")) != BEAM_OK)
    return st;
  return ok();
}

}  // namespace

extern "C" {

beam_status beam_attn_prefill_stages(uint32_t stages, const beam_attn_config* cfg, const beam_kv_cache* cache,
                                     const beam_bf16* q_raw, const beam_bf16* k_raw, const beam_bf16* v_raw,
                                     const beam_bf16* q_norm_w, const beam_bf16* k_norm_w,
                                     const beam_bf16* gate_logits, const float* gate_bias, const int32_t* cu_seqlens,
                                     const int32_t* seq_idx, const int32_t* start_pos, int32_t n_seqs, int32_t n_tok,
                                     int32_t max_chunk_len, beam_bf16* out, void* workspace, size_t ws_bytes,
                                     void* stream) {
  return chunk_call(false, stages, cfg, cache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate_logits, gate_bias,
                    cu_seqlens, seq_idx, start_pos, n_seqs, n_tok, max_chunk_len, 0, 0, out, workspace, ws_bytes,
                    stream);
}

beam_status beam_attn_verify_stages(uint32_t stages, const beam_attn_config* cfg, const beam_kv_cache* cache,
                                    const beam_bf16* q_raw, const beam_bf16* k_raw, const beam_bf16* v_raw,
                                    const beam_bf16* q_norm_w, const beam_bf16* k_norm_w,
                                    const beam_bf16* gate_logits, const float* gate_bias, const int32_t* cu_seqlens,
                                    const int32_t* seq_idx, const int32_t* start_pos, int32_t n_seqs, int32_t n_tok,
                                    int32_t max_chunk_len, int32_t max_pos, int32_t split_keys, beam_bf16* out,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return chunk_call(true, stages, cfg, cache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate_logits, gate_bias,
                    cu_seqlens, seq_idx, start_pos, n_seqs, n_tok, max_chunk_len, max_pos, split_keys, out,
                    workspace, ws_bytes, stream);
}

beam_status beam_attn_verify(const beam_attn_config* cfg, const beam_kv_cache* cache, const beam_bf16* q_raw,
                             const beam_bf16* k_raw, const beam_bf16* v_raw, const beam_bf16* q_norm_w,
                             const beam_bf16* k_norm_w, const beam_bf16* gate_logits, const float* gate_bias,
                             const int32_t* cu_seqlens, const int32_t* seq_idx, const int32_t* start_pos,
                             int32_t n_seqs, int32_t n_tok, int32_t max_chunk_len, int32_t max_pos, int32_t split_keys,
                             beam_bf16* out, void* workspace, size_t ws_bytes, void* stream) {
  return beam_attn_verify_stages(BEAM_STAGE_VERIFY_ALL, cfg, cache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w,
                                 gate_logits, gate_bias, cu_seqlens, seq_idx, start_pos, n_seqs, n_tok, max_chunk_len,
                                 max_pos, split_keys, out, workspace, ws_bytes, stream);
}

beam_status beam_attn_prefill(const beam_attn_config* cfg, const beam_kv_cache* cache, const beam_bf16* q_raw,
                              const beam_bf16* k_raw, const beam_bf16* v_raw, const beam_bf16* q_norm_w,
                              const beam_bf16* k_norm_w, const beam_bf16* gate_logits, const float* gate_bias,
                              const int32_t* cu_seqlens, const int32_t* seq_idx, const int32_t* start_pos,
                              int32_t n_seqs, int32_t n_tok, int32_t max_chunk_len, beam_bf16* out,
                              void* workspace, size_t ws_bytes, void* stream) {
  return beam_attn_prefill_stages(BEAM_STAGE_ALL, cfg, cache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate_logits,
                                  gate_bias, cu_seqlens, seq_idx, start_pos, n_seqs, n_tok, max_chunk_len, out,
                                  workspace, ws_bytes, stream);
}

beam_status beam_attn_decode_stages(uint32_t stages, const beam_attn_config* cfg, const beam_kv_cache* cache,
                                    const beam_bf16* q_raw, const beam_bf16* q_norm_w, const beam_bf16* gate_logits,
                                    const float* gate_bias, const int32_t* seq_idx, const int32_t* pos,
                                    int32_t n_seqs, int32_t max_pos, int32_t split_keys, beam_bf16* out,
                                    void* workspace, size_t ws_bytes, void* stream) {
  beam_status st;
  if (stages & ~7u) return fail(BEAM_E_RANGE, "unknown stage bits");
  if ((st = check_cfg(cfg)) != BEAM_OK) return st;
  if ((st = check_cache(cache)) != BEAM_OK) return st;
  if (n_seqs < 0) return fail(BEAM_E_RANGE, "n_seqs must be >= 0");
  if (n_seqs == 0) return ok();
  if (max_pos < 0) return fail(BEAM_E_RANGE, "max_pos must be >= 0");
  if (cache->kind == BEAM_GLOBAL && (int64_t)max_pos + 1 > (int64_t)cache->max_pages_per_seq * cache->page_size)
    return fail(BEAM_E_RANGE, "max_pos beyond block-table capacity");
  if (!q_raw || !q_norm_w || !gate_logits || !seq_idx || !pos || !out)
    return fail(BEAM_E_NULL, "NULL input/output pointer");
  if (!all_aligned16({q_raw, q_norm_w, gate_logits, out}))
    return fail(BEAM_E_RANGE, "bf16 tensors (q_raw, q_norm_w, gate_logits, out) must be 16-byte aligned");
  if (!workspace) return fail(BEAM_E_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(BEAM_E_RANGE, "workspace must be 256-byte aligned");
  DecodeWs ws;
  if (!decode_ws_layout(cfg, cache->kind, n_seqs, max_pos, split_keys, &ws))
    return fail(BEAM_E_RANGE, "split_keys must be 0 or a multiple of 128 in [128, 65536]");
  if (ws_bytes < ws.total)
    return fail(BEAM_E_WORKSPACE, "decode workspace needs " + std::to_string(ws.total) + " bytes");
  if ((int64_t)n_seqs * cfg->n_kv_heads * ws.n_splits > 0x7fffffffLL) return fail(BEAM_E_RANGE, "grid too large");
  hipStream_t s = (hipStream_t)stream;
  char* wsb = static_cast<char*>(workspace);
  uint16_t* qp = reinterpret_cast<uint16_t*>(wsb + ws.qp);
  float* ml = reinterpret_cast<float*>(wsb + ws.ml);
  float* acc = reinterpret_cast<float*>(wsb + ws.acc);

  beam::DecodeQParams qp_{};
  qp_.q_raw = q_raw;
  qp_.q_norm_w = q_norm_w;
  qp_.pos = pos;
  qp_.qp = qp;
  qp_.kind = cache->kind;
  qp_.H = cfg->n_q_heads;
  qp_.n_seqs = n_seqs;
  qp_.rope_theta = cfg->rope_theta;
  qp_.rms_eps = cfg->rms_eps;
  qp_.ssmax_base = cfg->ssmax_base;
  qp_.ssmax_exp = cfg->ssmax_exp;
  qp_.k_scale = cache->dtype == BEAM_KV_FP8_E4M3 ? cache->k_scale : 1.f;
  if ((stages & BEAM_STAGE_PROLOGUE) &&
      (st = hip_status(beam::launch_decode_q_prologue(qp_, s), "decode prologue launch")) != BEAM_OK)
    return st;

  beam::DecodeParams dp{};
  dp.qp = qp;
  dp.ck = static_cast<const uint16_t*>(cache->k);
  dp.cv = static_cast<const uint16_t*>(cache->v);
  dp.bt = cache->block_table;
  dp.max_pages = cache->max_pages_per_seq;
  dp.seq_idx = seq_idx;
  dp.pos = pos;
  dp.part_ml = ml;
  dp.part_acc = acc;
  dp.n_cache_seqs = cache->n_seqs;
  dp.max_pos = max_pos;
  dp.kind = cache->kind;
  dp.window = cfg->window;
  dp.H = cfg->n_q_heads;
  dp.G = cfg->n_kv_heads;
  dp.n_splits = ws.n_splits;
  dp.kpw = ws.split_keys / 4;
  dp.kv_fp8 = cache->dtype == BEAM_KV_FP8_E4M3;
  if ((stages & BEAM_STAGE_ATTENTION) &&
      (st = hip_status(beam::launch_decode_split(dp, n_seqs, s), "decode split launch")) != BEAM_OK)
    return st;

  beam::CombineParams cp{};
  cp.part_ml = ml;
  cp.part_acc = acc;
  cp.pos = pos;
  cp.seq_idx = seq_idx;
  cp.n_cache_seqs = cache->n_seqs;
  cp.gate = gate_logits;
  cp.gate_bias = gate_bias;
  cp.out = out;
  cp.max_pos = max_pos;
  cp.kind = cache->kind;
  cp.window = cfg->window;
  cp.H = cfg->n_q_heads;
  cp.n_splits = ws.n_splits;
  cp.split_keys = ws.split_keys;
  cp.v_scale = cache->dtype == BEAM_KV_FP8_E4M3 ? cache->v_scale : 1.f;
  if ((stages & BEAM_STAGE_COMBINE) &&
      (st = hip_status(beam::launch_decode_combine(cp, n_seqs, s), "decode combine launch")) != BEAM_OK)
    return st;
  return ok();
}

}  // extern "C"

namespace {

// Library-owned decode scratch for beam_attn_decode_noalloc: the split
// partials and Q' of one call. A file-scope device array, so each GPU the
// library runs on holds its own copy until the process ends. Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the device address is looked up once per device with hipGetSymbolAddress
// and kept here.
__device__ __attribute__((aligned(256))) unsigned char scratch[BEAM_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).
beam_status scratch_address(void** ptr) {
  int dev = -1;
  beam_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != BEAM_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(BEAM_E_UNSUPPORTED, "device index beyond the scratch table (64)");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != BEAM_OK) return st;
    if (!p) return fail(BEAM_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BEAM_OK;
}

}  // namespace

extern "C" {

beam_status beam_attn_decode_noalloc(const beam_attn_config* cfg, const beam_kv_cache* cache, const beam_bf16* q_raw,
                                     const beam_bf16* q_norm_w, const beam_bf16* gate_logits, const float* gate_bias,
                                     const int32_t* seq_idx, const int32_t* pos, int32_t n_seqs, int32_t max_pos,
                                     int32_t split_keys, beam_bf16* out, void* stream) {
  beam_status st;
  if ((st = check_cfg(cfg)) != BEAM_OK) return st;
  if ((st = check_cache(cache)) != BEAM_OK) return st;
  if (n_seqs < 0) return fail(BEAM_E_RANGE, "n_seqs must be >= 0");
  if (n_seqs == 0) return ok();
  if (max_pos < 0) return fail(BEAM_E_RANGE, "max_pos must be >= 0");
  DecodeWs ws;
  if (!decode_ws_layout(cfg, cache->kind, n_seqs, max_pos, split_keys, &ws))
    return fail(BEAM_E_RANGE, "split_keys must be 0 or a multiple of 128 in [128, 65536]");
  if (ws.total > (size_t)BEAM_DECODE_SCRATCH_BYTES)
    return fail(BEAM_E_WORKSPACE, "decode needs " + std::to_string(ws.total) +
                                      " bytes of scratch; the library's array holds " +
                                      std::to_string((size_t)BEAM_DECODE_SCRATCH_BYTES) +
                                      " (pass fewer sequences or a larger split_keys)");
  void* ptr = nullptr;
  if ((st = scratch_address(&ptr)) != BEAM_OK) return st;
  return beam_attn_decode_stages(BEAM_STAGE_ALL, cfg, cache, q_raw, q_norm_w, gate_logits, gate_bias, seq_idx, pos,
                                 n_seqs, max_pos, split_keys, out, ptr, (size_t)BEAM_DECODE_SCRATCH_BYTES, stream);
}

beam_status beam_attn_decode(const beam_attn_config* cfg, const beam_kv_cache* cache, const beam_bf16* q_raw,
                             const beam_bf16* q_norm_w, const beam_bf16* gate_logits, const float* gate_bias,
                             const int32_t* seq_idx, const int32_t* pos, int32_t n_seqs, int32_t max_pos,
                             int32_t split_keys, beam_bf16* out, void* workspace, size_t ws_bytes,
                             void* stream) {
  return beam_attn_decode_stages(BEAM_STAGE_ALL, cfg, cache, q_raw, q_norm_w, gate_logits, gate_bias, seq_idx, pos,
                                 n_seqs, max_pos, split_keys, out, workspace, ws_bytes, stream);
}

beam_status beam_debug_visibility(int32_t kind, int32_t window, int32_t t0, int32_t n_q, int32_t s0, int32_t n_k,
                                  uint8_t* mask, void* stream) {
  if (kind != BEAM_LOCAL && kind != BEAM_GLOBAL) return fail(BEAM_E_RANGE, "kind must be 0 or 1");
  if (!mask) return fail(BEAM_E_NULL, "mask is NULL");
  if (window <= 0 || n_q < 0 || n_k < 0) return fail(BEAM_E_RANGE, "window > 0, n_q >= 0, n_k >= 0 required");
  if ((int64_t)n_q * n_k == 0) return ok();
  beam_status st = hip_status(beam::launch_visibility(kind, window, t0, n_q, s0, n_k, mask, (hipStream_t)stream),
                              "visibility launch");
  if (st != BEAM_OK) return st;
  return ok();
}

beam_status beam_debug_validate_cache(const beam_kv_cache* cache, const int32_t* n_tokens, int32_t* n_bad,
                                      void* stream) {
  if (!cache) return fail(BEAM_E_NULL, "cache is NULL");
  if (cache->kind != BEAM_GLOBAL) return fail(BEAM_E_RANGE, "only a paged (GLOBAL) cache has a block table");
  if (!cache->block_table || !n_bad) return fail(BEAM_E_NULL, "block_table or n_bad is NULL");
  if (cache->n_seqs <= 0 || cache->max_pages_per_seq <= 0 || cache->n_pages <= 0 || cache->page_size <= 0)
    return fail(BEAM_E_RANGE, "n_seqs, max_pages_per_seq, n_pages and page_size must be positive");
  beam_status st = hip_status(beam::launch_validate_cache(cache->block_table, cache->max_pages_per_seq,
                                                          cache->n_pages, cache->page_size, cache->n_seqs,
                                                          n_tokens, n_bad, (hipStream_t)stream),
                              "validate_cache launch");
  if (st != BEAM_OK) return st;
  return ok();
}

beam_status beam_kv_convert_v(const beam_attn_config* cfg, const beam_kv_cache* cache, void* v_token_major,
                              int32_t to_cache, void* stream) {
  if (beam_status st = check_cfg(cfg); st != BEAM_OK) return st;
  if (beam_status st = check_cache(cache); st != BEAM_OK) return st;
  if (!v_token_major) return fail(BEAM_E_NULL, "v_token_major is NULL");
  if (!aligned16(v_token_major)) return fail(BEAM_E_RANGE, "v_token_major must be 16-byte aligned");
  const bool global = cache->kind == BEAM_GLOBAL;
  if (global && cache->n_pages <= 0) return fail(BEAM_E_RANGE, "n_pages must be positive");
  const long long n_blocks = (long long)(global ? cache->n_pages : cache->n_seqs) * cfg->n_kv_heads;
  const int rows = global ? cache->page_size : cfg->window;
  const int esz = cache->dtype == BEAM_KV_FP8_E4M3 ? 1 : 2;
  const unsigned long long bytes = (unsigned long long)n_blocks * rows * beam::D * esz;
  if (n_blocks * (rows / beam::kVTransposeRows) > 0x7fffffffLL)
    return fail(BEAM_E_RANGE, "cache too large for one conversion call");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(v_token_major), b0 = reinterpret_cast<uintptr_t>(cache->v);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(BEAM_E_RANGE, "v_token_major overlaps cache->v");
  const void* src = to_cache ? v_token_major : cache->v;
  void* dst = to_cache ? cache->v : v_token_major;
  beam_status st = hip_status(beam::launch_kv_v_transpose(src, dst, n_blocks, rows, esz, to_cache ? 1 : 0,
                                                          (hipStream_t)stream),
                              "kv_convert_v launch");
  if (st != BEAM_OK) return st;
  return ok();
}

// ---------------------------------------------------------------- router

}  // extern "C"

namespace {

beam_status check_router(const beam_router_config* c, int32_t n_tok) {
  if (!c) return fail(BEAM_E_NULL, "router config is NULL");
  if (c->hidden <= 0 || c->hidden % beam::kRouterKChunk != 0)
    return fail(BEAM_E_UNSUPPORTED, "router hidden width must be a positive multiple of 32");
  if (c->n_experts != beam::kRouterExperts || c->n_groups != beam::kRouterGroups)
    return fail(BEAM_E_UNSUPPORTED, "router supports 256 experts in 8 groups");
  if (c->topk_groups < 1 || c->topk_groups > beam::kRouterGroups || c->top_k < 1 || c->top_k > 8)
    return fail(BEAM_E_UNSUPPORTED, "router needs 1 <= topk_groups <= 8 and 1 <= top_k <= 8");
  if (!std::isfinite(c->scale)) return fail(BEAM_E_RANGE, "router scale must be finite");
  if (n_tok < 0) return fail(BEAM_E_RANGE, "n_tok must be >= 0");
  return BEAM_OK;
}

beam::RouterParams router_params(const beam_router_config* c, int32_t n_tok) {
  beam::RouterParams p{};
  p.n_tok = n_tok;
  p.hidden = c->hidden;
  p.topk_groups = c->topk_groups;
  p.top_k = c->top_k;
  p.scale = c->scale;
  return p;
}

}  // namespace

extern "C" {

beam_status beam_router(const beam_router_config* cfg, const beam_bf16* x, const float* w, const float* bias,
                        int32_t n_tok, int32_t* topk_idx, float* topk_w, void* stream) {
  beam_status st;
  if ((st = check_router(cfg, n_tok)) != BEAM_OK) return st;
  if (n_tok == 0) return ok();
  if (!x || !w || !topk_idx || !topk_w) return fail(BEAM_E_NULL, "NULL input/output pointer");
  beam::RouterParams p = router_params(cfg, n_tok);
  p.x = x;
  p.w = w;
  p.bias = bias;
  p.idx = topk_idx;
  p.wts = topk_w;
  return hip_status(beam::launch_router_fused(p, (hipStream_t)stream), "router launch");
}

beam_status beam_router_logits(const beam_router_config* cfg, const beam_bf16* x, const float* w, int32_t n_tok,
                               float* logits, void* stream) {
  beam_status st;
  if ((st = check_router(cfg, n_tok)) != BEAM_OK) return st;
  if (n_tok == 0) return ok();
  if (!x || !w || !logits) return fail(BEAM_E_NULL, "NULL input/output pointer");
  beam::RouterParams p = router_params(cfg, n_tok);
  p.x = x;
  p.w = w;
  p.logits_out = logits;
  return hip_status(beam::launch_router_logits(p, (hipStream_t)stream), "router logits launch");
}

beam_status beam_router_select(const beam_router_config* cfg, const float* logits, const float* bias, int32_t n_tok,
                               int32_t* topk_idx, float* topk_w, void* stream) {
  beam_status st;
  if ((st = check_router(cfg, n_tok)) != BEAM_OK) return st;
  if (n_tok == 0) return ok();
  if (!logits || !topk_idx || !topk_w) return fail(BEAM_E_NULL, "NULL input/output pointer");
  beam::RouterParams p = router_params(cfg, n_tok);
  p.logits_in = logits;
  p.bias = bias;
  p.idx = topk_idx;
  p.wts = topk_w;
  return hip_status(beam::launch_router_select(p, (hipStream_t)stream), "router select launch");
}

}  // extern "C"

// ---------------------------------------------------------------- projections

namespace {

beam_status check_gemm_sizes(int32_t n_tok, int32_t k, int64_t n_feat, const char* what) {
  if (n_tok < 0) return fail(BEAM_E_RANGE, "n_tok must be >= 0");
  if (k <= 0 || k % 128 != 0 || k > 65536)
    return fail(BEAM_E_UNSUPPORTED, std::string(what) + ": the contraction width must be a multiple of 128 in [128, 65536]");
  if (n_feat <= 0 || n_feat % beam::kGemmTile != 0)
    return fail(BEAM_E_UNSUPPORTED, std::string(what) + ": the output width must be a positive multiple of 256");
  const int64_t blocks = (n_feat / beam::kGemmTile) * (((int64_t)n_tok + beam::kGemmTile - 1) / beam::kGemmTile);
  if (blocks > 0x7fffffffLL) return fail(BEAM_E_RANGE, std::string(what) + ": grid too large");
  return BEAM_OK;
}

}  // namespace

extern "C" {

beam_status beam_attn_project(const beam_attn_config* cfg, int32_t kind, const beam_bf16* x, int32_t hidden,
                              const beam_bf16* w_qkvg, const beam_bf16* q_norm_w, const int32_t* cu_seqlens,
                              const int32_t* start_pos, int32_t n_seqs, int32_t n_tok, beam_bf16* k_raw,
                              beam_bf16* v_raw, beam_bf16* gate_logits, void* workspace, size_t ws_bytes,
                              void* stream) {
  beam_status st;
  if ((st = check_cfg(cfg)) != BEAM_OK) return st;
  if (kind != BEAM_LOCAL && kind != BEAM_GLOBAL) return fail(BEAM_E_RANGE, "kind must be 0 or 1");
  if (n_seqs <= 0) return fail(BEAM_E_RANGE, "n_seqs must be positive");
  const int64_t n_feat = (int64_t)(2 * cfg->n_q_heads + 2 * cfg->n_kv_heads) * beam::D;
  if ((st = check_gemm_sizes(n_tok, hidden, n_feat, "projection")) != BEAM_OK) return st;
  if (n_tok == 0) return ok();
  if (!x || !w_qkvg || !q_norm_w || !cu_seqlens || !start_pos || !k_raw || !v_raw || !gate_logits)
    return fail(BEAM_E_NULL, "NULL input/output pointer");
  if (!aligned16(x) || !aligned16(w_qkvg) || !aligned16(k_raw) || !aligned16(v_raw) || !aligned16(gate_logits))
    return fail(BEAM_E_RANGE, "x, w_qkvg, k_raw, v_raw and gate_logits must be 16-byte aligned");
  if (!workspace) return fail(BEAM_E_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(BEAM_E_RANGE, "workspace must be 256-byte aligned");
  const PrefillWs ws = prefill_ws_layout(cfg, n_tok, n_seqs);
  if (ws_bytes < ws.total) return fail(BEAM_E_WORKSPACE, "prefill workspace needs " + std::to_string(ws.total) + " bytes");
  beam::GemmParams p{};
  p.x = x;
  p.w = w_qkvg;
  p.n_tok = n_tok;
  p.n_feat = (int)n_feat;
  p.K = hidden;
  p.q_out = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + ws.qp);
  p.k_out = k_raw;
  p.v_out = v_raw;
  p.g_out = gate_logits;
  p.q_norm_w = q_norm_w;
  p.cu = cu_seqlens;
  p.start_pos = start_pos;
  p.n_seqs = n_seqs;
  p.kind = kind;
  p.H = cfg->n_q_heads;
  p.G = cfg->n_kv_heads;
  p.rope_theta = cfg->rope_theta;
  p.rms_eps = cfg->rms_eps;
  p.ssmax_base = cfg->ssmax_base;
  p.ssmax_exp = cfg->ssmax_exp;
  return hip_status(beam::launch_gemm(p, beam::kEpiQkvg, (hipStream_t)stream), "projection launch");
}

beam_status beam_out_project(const beam_bf16* y, const beam_bf16* w_o, int32_t n_tok, int32_t in_features,
                             int32_t out_features, beam_bf16* out, void* stream) {
  beam_status st;
  if ((st = check_gemm_sizes(n_tok, in_features, out_features, "output projection")) != BEAM_OK) return st;
  if (n_tok == 0) return ok();
  if (!y || !w_o || !out) return fail(BEAM_E_NULL, "NULL input/output pointer");
  if (!aligned16(y) || !aligned16(w_o) || !aligned16(out)) return fail(BEAM_E_RANGE, "y, w_o and out must be 16-byte aligned");
  beam::GemmParams p{};
  p.x = y;
  p.w = w_o;
  p.n_tok = n_tok;
  p.n_feat = out_features;
  p.K = in_features;
  p.out = out;
  p.ld_out = out_features;
  return hip_status(beam::launch_gemm(p, beam::kEpiPlain, (hipStream_t)stream), "output projection launch");
}

}  // extern "C"
