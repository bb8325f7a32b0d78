/*
 * beam_attn.h — C ABI of the Beam 1.0 hybrid GQA attention library (gfx950 only).
 *
 * The operation is the attention sublayer of Beam 1.0 as described on
 *   "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax" (flozi.net, English),
 *   sections "Two attention paths in one decoder", "Follow the tensors, not the
 *   parameter label" and "KV memory: nine growing caches, not 52", with the SSMax
 *   formula as given on techfi24.com ("Architecture et mécanismes d'inférence"):
 *
 *   Q_hat = RMSNorm(Q) * w_q, K_hat = RMSNorm(K) * w_k   (per head, 128 coords, eps)
 *   local  layer: q' = RoPE(Q_hat, t), k' = RoPE(K_hat, s), visible iff 0 <= t-s <= window-1
 *   global layer: q' = a(t+1) * Q_hat, k' = K_hat,          visible iff s <= t
 *                 a(p) = (1 + p/ssmax_base)^ssmax_exp, p one-based absolute position
 *   S = q'.k'/sqrt(d), P = softmax over visible keys, O = P V (V not normalised)
 *   Y = O * sigmoid(gate_logits + gate_bias[h])           (per coordinate)
 *   Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless marked "host". The caller owns
 *     all memory; the library never allocates, frees or synchronises.
 *   - bf16 values are raw bfloat16 bit patterns (uint16_t).
 *   - `stream` is a hipStream_t (NULL = the null stream). All work of a call is
 *     enqueued on it in order; faults surface at the caller's next sync.
 *   - Arguments are checked on the host before anything is enqueued. On error a
 *     call returns a non-zero beam_status, launches nothing, and sets a
 *     thread-local message readable with beam_last_error(). BEAM_E_HIP reports
 *     a launch of the call itself: an error that an earlier runtime call left
 *     unread on the thread is cleared before the call launches.
 *   - Device-resident indices (block-table entries, seq_idx, positions,
 *     cu_seqlens) are not read by the host; out-of-range values in them are
 *     undefined behaviour.
 *   - Only head_dim == 128 is supported (BEAM_E_UNSUPPORTED). Inputs and
 *     outputs are bf16; the KV cache is bf16 or FP8 E4M3 (below).
 *   - Every bf16 tensor and the cache's k/v buffers must be 16-byte aligned
 *     (BEAM_E_RANGE otherwise); the workspaces 256-byte aligned.
 *   - Calls hold no global mutable state and may be made from several threads.
 *
 * KV cache layouts (beam_kv_cache.k / .v)
 *   GLOBAL (paged, page_size 16):
 *     k: bf16 [n_pages][n_kv_heads][page_size][head_dim]   token-major rows
 *     v: bf16 [n_pages][n_kv_heads][head_dim][page_size]   transposed within the page
 *     position t of cache sequence c lives in page block_table[c][t / page_size],
 *     slot t % page_size.
 *   LOCAL (window-sized ring, one per cache sequence):
 *     k: bf16 [n_seqs][n_kv_heads][window][head_dim]
 *     v: bf16 [n_seqs][n_kv_heads][head_dim][window]
 *     position t lives in slot t % window.
 *   The cache stores K_hat (normalised; rotated on local layers) and raw V.
 *   V kept token-major like K (another engine's layout) converts to and from
 *   this layout with beam_kv_convert_v.
 *
 * FP8 KV cache (dtype BEAM_KV_FP8_E4M3; one byte per element, same layouts)
 *   The pages' serving recipes keep the cache in FP8 E4M3 (18 KiB per token
 *   across the nine global layers, "KV memory: nine growing caches, not 52";
 *   the German serving article: FP8 E4M3 cache by default). They state no
 *   scale convention; here each layer's cache has one scale for K and one for
 *   V. A value x is stored as the OCP E4M3FN code nearest to x / scale (ties
 *   to the even code, |x / scale| >= 448 saturates to +-448) and read back as
 *   decode(code) * scale. Decode reads codes exactly (k_scale is folded into
 *   the query, v_scale into the output); prefill dequantises a cached prefix
 *   to bf16. The chunk being prefilled attends to its own keys unquantised.
 */
#ifndef BEAM_ATTN_H
#define BEAM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t beam_bf16; /* raw bfloat16 bits */

typedef enum { BEAM_LOCAL = 0, BEAM_GLOBAL = 1 } beam_layer_kind;

typedef enum { BEAM_KV_BF16 = 0, BEAM_KV_FP8_E4M3 = 1 } beam_kv_dtype;

typedef enum {
  BEAM_OK = 0,
  BEAM_E_NULL = 1,        /* a required pointer is NULL */
  BEAM_E_SHAPE = 2,       /* inconsistent sizes (e.g. n_q_heads % n_kv_heads != 0) */
  BEAM_E_RANGE = 3,       /* a size or position is out of its valid range */
  BEAM_E_UNSUPPORTED = 4, /* head_dim != 128, page_size != 16, ... */
  BEAM_E_WORKSPACE = 5,   /* workspace too small */
  BEAM_E_HIP = 6          /* the HIP runtime refused a launch */
} beam_status;

/* Layer geometry. Defaults for Beam 1.0: 48, 8, 128, 512, 1e4, 1e-6, 2048, 0.1. */
typedef struct {
  int32_t n_q_heads;  /* 48 */
  int32_t n_kv_heads; /* 8; at most 8, must divide n_q_heads, n_q_heads/n_kv_heads <= 16 */
  int32_t head_dim;   /* 128 (only value supported) */
  int32_t window;     /* local window incl. the current token; 512 */
  float rope_theta;   /* 10000 */
  float rms_eps;      /* 1e-6 */
  float ssmax_base;   /* 2048 */
  float ssmax_exp;    /* 0.1 */
} beam_attn_config;

/* One layer's KV cache (layouts above). */
typedef struct {
  int32_t kind;               /* beam_layer_kind */
  void *k;                    /* device, bf16 or FP8 codes (dtype) */
  void *v;                    /* device, bf16 or FP8 codes (dtype) */
  int32_t page_size;          /* GLOBAL: 16. LOCAL: ignored */
  int32_t n_pages;            /* GLOBAL: physical pages. LOCAL: ignored */
  const int32_t *block_table; /* GLOBAL: device [n_seqs][max_pages_per_seq]. LOCAL: ignored */
  int32_t max_pages_per_seq;  /* GLOBAL: row length of block_table */
  int32_t n_seqs;             /* GLOBAL: rows of block_table. LOCAL: rings allocated */
  int32_t dtype;              /* beam_kv_dtype (0 = bf16) */
  float k_scale;              /* FP8: K_hat = decode(code) * k_scale; finite, > 0. bf16: ignored */
  float v_scale;              /* FP8: V = decode(code) * v_scale; finite, > 0. bf16: ignored */
} beam_kv_cache;

/* Append new tokens to a layer's cache.
 * k_raw, v_raw: bf16 [n_tok][n_kv_heads][head_dim] raw projections.
 * k_norm_w:     bf16 [head_dim] RMSNorm weight of K for this layer.
 * seq_idx:      int32 [n_tok] cache sequence (block-table row / ring) of each token.
 * pos:          int32 [n_tok] zero-based absolute position t of each token.
 * Writes K_hat (RMSNorm, then RoPE at t on LOCAL) and raw V at the token's slot.
 * Two tokens of one call that map to the same slot race (the ring keeps one). */
beam_status beam_kv_append(const beam_attn_config *cfg, const beam_kv_cache *cache,
                           const beam_bf16 *k_raw, const beam_bf16 *v_raw,
                           const beam_bf16 *k_norm_w, const int32_t *seq_idx,
                           const int32_t *pos, int32_t n_tok, void *stream);

/* Causal (chunked, varlen) prefill of one layer.
 * The chunk of sequence i is tokens [cu_seqlens[i], cu_seqlens[i+1]) of the packed
 * inputs, at absolute positions start_pos[i] + 0, 1, ...; positions < start_pos[i]
 * must already be in the cache (cache sequence seq_idx[i]).
 * q_raw, gate_logits, out: bf16 [n_tok][n_q_heads][head_dim].
 * k_raw, v_raw:            bf16 [n_tok][n_kv_heads][head_dim].
 * q_norm_w, k_norm_w:      bf16 [head_dim].  gate_bias: float [n_q_heads] or NULL.
 * cu_seqlens: int32 [n_seqs+1] (cu_seqlens[0] == 0, cu_seqlens[n_seqs] == n_tok),
 * seq_idx, start_pos: int32 [n_seqs]. max_chunk_len >= every chunk length.
 * In stream order: prologue (norm, RoPE/SSMax) into the workspace, attention over
 * cached prefix + chunk with the gate applied, then the chunk's K_hat/V are appended
 * to the cache (last, so a local ring is never overwritten while it is read). On a
 * global (paged) cache the append is done by the prologue itself: the chunk's
 * positions never share a slot with the prefix that attention reads.
 * workspace: device, >= beam_prefill_workspace_bytes(cfg, n_tok, n_seqs) bytes,
 * 256-byte aligned. */
beam_status beam_attn_prefill(const beam_attn_config *cfg, const beam_kv_cache *cache,
                              const beam_bf16 *q_raw, const beam_bf16 *k_raw,
                              const beam_bf16 *v_raw, const beam_bf16 *q_norm_w,
                              const beam_bf16 *k_norm_w, const beam_bf16 *gate_logits,
                              const float *gate_bias, const int32_t *cu_seqlens,
                              const int32_t *seq_idx, const int32_t *start_pos,
                              int32_t n_seqs, int32_t n_tok, int32_t max_chunk_len,
                              beam_bf16 *out, void *workspace, size_t ws_bytes,
                              void *stream);

/* One-token decode of one layer for n_seqs sequences (split-K over the cache).
 * The new token (position pos[i], cache sequence seq_idx[i]) must already have
 * been appended with beam_kv_append.
 * q_raw, gate_logits, out: bf16 [n_seqs][n_q_heads][head_dim].
 * max_pos >= every pos[i] (sizes the split grid). A sequence whose pos[i] lies
 * outside [0, max_pos], or whose seq_idx[i] names no cache sequence, is not read
 * and its output rows are NaN.
 * split_keys: keys per split (multiple of 128, <= 65536), or 0 for the default
 * (128 on LOCAL layers; on GLOBAL layers 4096 when n_seqs * n_kv_heads *
 * ((max_pos + 1 + 4095) / 4096) >= 1024, else 2048).
 * workspace: >= beam_decode_workspace_bytes(cfg, kind, n_seqs, max_pos, split_keys). */
beam_status beam_attn_decode(const beam_attn_config *cfg, const beam_kv_cache *cache,
                             const beam_bf16 *q_raw, const beam_bf16 *q_norm_w,
                             const beam_bf16 *gate_logits, const float *gate_bias,
                             const int32_t *seq_idx, const int32_t *pos, int32_t n_seqs,
                             int32_t max_pos, int32_t split_keys, beam_bf16 *out,
                             void *workspace, size_t ws_bytes, void *stream);

/* beam_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, stages (all three) and
 * results as beam_attn_decode. The split partials and the normalised queries
 * live instead in a library-owned device array of BEAM_DECODE_SCRATCH_BYTES,
 * one per GPU the library runs on, held until the process ends; its address is
 * looked up on the first call on a device (that device current). The call
 * allocates and frees nothing. Nothing in the array needs to start at zero:
 * every value a call reads was written earlier in the same call.
 * Errors: BEAM_E_WORKSPACE if beam_decode_workspace_bytes(cfg, kind, n_seqs,
 * max_pos, split_keys) exceeds BEAM_DECODE_SCRATCH_BYTES (a larger split_keys
 * or fewer sequences per call shrink it), plus those of beam_attn_decode.
 * Calls that overlap on one GPU (several streams or threads) share the array
 * and race: the caller serialises them. */
#define BEAM_DECODE_SCRATCH_BYTES (32u << 20)
beam_status beam_attn_decode_noalloc(const beam_attn_config *cfg, const beam_kv_cache *cache,
                                     const beam_bf16 *q_raw, const beam_bf16 *q_norm_w,
                                     const beam_bf16 *gate_logits, const float *gate_bias,
                                     const int32_t *seq_idx, const int32_t *pos, int32_t n_seqs,
                                     int32_t max_pos, int32_t split_keys, beam_bf16 *out, void *stream);

/* Verify step of speculative decoding: causal attention of a few new tokens per
 * sequence (the draft tokens plus the last accepted one) over the cached history,
 * in one call for n_seqs sequences. The drafter proposes blocks of 8 tokens
 * ("Beam 1.0 auf vier B300s", orcarouter.ai, the serving recipe) or up to 15
 * that Beam checks in one pass (news.hamidun.com, the paragraph on reasoning
 * levels and acceleration); the step is a prefill chunk of that length. Same inputs,
 * outputs, semantics and append as beam_attn_prefill, computed the way decode
 * is: the (token, query head) rows of one KV head share every K/V tile, and the
 * keys are split across blocks with a log-sum-exp merge.
 * Limits: max_chunk_len * (n_q_heads / n_kv_heads) <= 128 (21 tokens at 48/8).
 * max_pos >= start_pos[i] + chunk length - 1 for every i (sizes the split grid).
 * A sequence that breaks this (or has start_pos[i] < 0) gets NaN output rows:
 * the split grid does not cover its keys. split_keys: keys per split (multiple of 64, <= 8192), or 0 for the
 * default: local one split over the keys a chunk can see (64 * ((window - 1 +
 * max_chunk_len - 1) / 64 + 2) keys) when n_seqs * n_kv_heads >= 256, else 256;
 * global the longest of 8192 and 4096 keys for which
 * n_seqs * n_kv_heads * (max_pos / keys + 1) >= 1024, else 2048.
 * Rejected draft tokens: on a GLOBAL cache the next call simply starts at the
 * first rejected position (its slots are overwritten). A LOCAL ring keeps only
 * the last `window` positions, so appending a rejected token would evict a key
 * the next chunk needs: on local layers run beam_attn_verify_stages without
 * BEAM_STAGE_APPEND and append the accepted tokens with beam_kv_append.
 * workspace: >= beam_verify_workspace_bytes(cfg, cache->kind, n_tok, n_seqs,
 * max_chunk_len, max_pos, split_keys) bytes, 256-byte aligned. */
beam_status beam_attn_verify(const beam_attn_config *cfg, const beam_kv_cache *cache,
                             const beam_bf16 *q_raw, const beam_bf16 *k_raw,
                             const beam_bf16 *v_raw, const beam_bf16 *q_norm_w,
                             const beam_bf16 *k_norm_w, const beam_bf16 *gate_logits,
                             const float *gate_bias, const int32_t *cu_seqlens,
                             const int32_t *seq_idx, const int32_t *start_pos,
                             int32_t n_seqs, int32_t n_tok, int32_t max_chunk_len,
                             int32_t max_pos, int32_t split_keys, beam_bf16 *out,
                             void *workspace, size_t ws_bytes, void *stream);

/* Stage selection for the *_stages variants. Running the stages of one call
 * separately, in this order, on one stream, with the same arguments and
 * workspace, is identical to the single call (the workspace carries the state
 * between stages). Lets a caller bracket one stage with events, or overlap the
 * cache append with other work.
 *   prefill: PROLOGUE = norm + RoPE/SSMax into the workspace, ATTENTION =
 *            attention + gate into `out`, APPEND = chunk K_hat/V into the cache.
 *            On a global cache, PROLOGUE | APPEND in one call fuses the append
 *            into the prologue; ATTENTION may follow it (the order of the two
 *            does not matter there). On a local cache APPEND must come after
 *            ATTENTION when the chunk has a cached prefix.
 *   decode:  PROLOGUE = query norm + RoPE/SSMax, ATTENTION = split-K partials,
 *            COMBINE = merge of the splits + gate into `out`.
 *   verify:  PROLOGUE, APPEND as prefill; ATTENTION = split-key partials,
 *            VERIFY_COMBINE = merge of the splits + gate into `out` (order:
 *            PROLOGUE, ATTENTION, VERIFY_COMBINE, APPEND; ALL = VERIFY_ALL).
 *            With a single key split (beam_verify_workspace_bytes' grid; the
 *            default on LOCAL layers) ATTENTION writes the gated `out` itself
 *            and VERIFY_COMBINE does nothing. */
#define BEAM_STAGE_PROLOGUE 1u
#define BEAM_STAGE_ATTENTION 2u
#define BEAM_STAGE_APPEND 4u
#define BEAM_STAGE_COMBINE 4u
#define BEAM_STAGE_ALL 7u
#define BEAM_STAGE_VERIFY_COMBINE 8u
#define BEAM_STAGE_VERIFY_ALL 15u
/* The prologue without the queries: K_hat and V^T into the workspace (and the
 * fused append on a global cache), with Q' already in the workspace's query
 * region, written by beam_attn_project (beam_proj.h). q_raw may then be NULL.
 * Takes the place of BEAM_STAGE_PROLOGUE (prefill and verify). */
#define BEAM_STAGE_PROLOGUE_KV 16u

beam_status beam_attn_prefill_stages(uint32_t stages, const beam_attn_config *cfg,
                                     const beam_kv_cache *cache, const beam_bf16 *q_raw,
                                     const beam_bf16 *k_raw, const beam_bf16 *v_raw,
                                     const beam_bf16 *q_norm_w, const beam_bf16 *k_norm_w,
                                     const beam_bf16 *gate_logits, const float *gate_bias,
                                     const int32_t *cu_seqlens, const int32_t *seq_idx,
                                     const int32_t *start_pos, int32_t n_seqs, int32_t n_tok,
                                     int32_t max_chunk_len, beam_bf16 *out, void *workspace,
                                     size_t ws_bytes, void *stream);
beam_status beam_attn_verify_stages(uint32_t stages, const beam_attn_config *cfg,
                                    const beam_kv_cache *cache, const beam_bf16 *q_raw,
                                    const beam_bf16 *k_raw, const beam_bf16 *v_raw,
                                    const beam_bf16 *q_norm_w, const beam_bf16 *k_norm_w,
                                    const beam_bf16 *gate_logits, const float *gate_bias,
                                    const int32_t *cu_seqlens, const int32_t *seq_idx,
                                    const int32_t *start_pos, int32_t n_seqs, int32_t n_tok,
                                    int32_t max_chunk_len, int32_t max_pos, int32_t split_keys,
                                    beam_bf16 *out, void *workspace, size_t ws_bytes,
                                    void *stream);
beam_status beam_attn_decode_stages(uint32_t stages, const beam_attn_config *cfg,
                                    const beam_kv_cache *cache, const beam_bf16 *q_raw,
                                    const beam_bf16 *q_norm_w, const beam_bf16 *gate_logits,
                                    const float *gate_bias, const int32_t *seq_idx,
                                    const int32_t *pos, int32_t n_seqs, int32_t max_pos,
                                    int32_t split_keys, beam_bf16 *out, void *workspace,
                                    size_t ws_bytes, void *stream);

/* Workspace sizes in bytes (host-only, no GPU needed). 0 on invalid arguments. */
size_t beam_prefill_workspace_bytes(const beam_attn_config *cfg, int32_t n_tok, int32_t n_seqs);
size_t beam_decode_workspace_bytes(const beam_attn_config *cfg, int32_t kind, int32_t n_seqs,
                                   int32_t max_pos, int32_t split_keys);
size_t beam_verify_workspace_bytes(const beam_attn_config *cfg, int32_t kind, int32_t n_tok,
                                   int32_t n_seqs, int32_t max_chunk_len, int32_t max_pos,
                                   int32_t split_keys);

/* KV payload of n_global growing caches plus n_local window-sized caches, per
 * sequence ("KV memory: nine growing caches, not 52"): logical =
 * 2*b*n_kv*d*(n_global*N + n_local*min(N, window)); paged rounds N up to pages
 * in the global term. Host-only; logical/paged are host pointers. */
beam_status beam_kv_bytes(int64_t n_tokens, int32_t bytes_per_scalar, int32_t n_global,
                          int32_t n_local, int32_t n_kv, int32_t d, int32_t window,
                          int32_t page_size, uint64_t *logical, uint64_t *paged);

/* Physical page and slot of position t of sequence seq. Host-only; block_table_host
 * is a host copy [.. ][max_pages_per_seq]. */
beam_status beam_kv_page_slot(const int32_t *block_table_host, int32_t max_pages_per_seq,
                              int32_t page_size, int32_t seq, int32_t t, int64_t *phys_page,
                              int32_t *slot);

/* mask[i][j] = 1 iff key position s0+j is visible to query position t0+i for the
 * layer kind, computed on the GPU by the predicate the decode and verify kernels
 * use (the prefill kernel applies the same rule per tile as two bounds on the
 * key's offset in the tile).
 * mask: device uint8 [n_q][n_k]. */
beam_status beam_debug_visibility(int32_t kind, int32_t window, int32_t t0, int32_t n_q,
                                  int32_t s0, int32_t n_k, uint8_t *mask, void *stream);

/* Opt-in check of a paged (GLOBAL) cache's block table. Block-table entries are
 * device data that the attention calls take on trust; a serving stack fills
 * them from its page allocator (the pages' serving recipes run a paged FP8 E4M3
 * cache with 64-token pages: "Beam 1.0 auf vier B300s", orcarouter.ai, section
 * "Was vier B300s hinsichtlich des Speichers tatsächlich bringen").
 * For every cache sequence c (0 <= c < cache->n_seqs):
 *   n_bad[c] = number of entries block_table[c][i], 0 <= i < ceil(n_tokens[c] / page_size),
 *              that are < 0 or >= cache->n_pages;
 *            = -1 if n_tokens[c] < 0 or needs more pages than the row holds.
 * n_tokens: device int32 [cache->n_seqs], positions held per sequence, or NULL
 * to check whole rows. n_bad: device int32 [cache->n_seqs], written by the call.
 * Only ids are compared: no page of k/v is read, so a bad entry is safe here.
 * Enqueued on `stream`; read n_bad after a sync. A LOCAL cache has no block
 * table (BEAM_E_RANGE). */
beam_status beam_debug_validate_cache(const beam_kv_cache *cache, const int32_t *n_tokens, int32_t *n_bad,
                                      void *stream);

/* V of a layer's cache between the token-major layout, in which K is stored
 * too, and the layout the attention calls read (coordinate-major within each
 * page or ring, "KV cache layouts" above). The cache holds V of every position
 * of the nine global layers and a window of positions on the local layers
 * ("Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax", section "KV
 * memory: nine growing caches, not 52"); a caller that filled V token-major
 * (page_size x head_dim rows per page and KV head, as another engine's paged
 * cache keeps it) converts it here before any attention call, or reads the
 * cache back that way.
 *   token-major V: GLOBAL [n_pages][n_kv_heads][page_size][head_dim],
 *                  LOCAL  [n_seqs][n_kv_heads][window][head_dim]
 *                  (page_size 16; the element type of cache->dtype, bf16 or FP8 E4M3 codes)
 * to_cache != 0: reads v_token_major, writes all of cache->v (every page, or
 *                every ring of cache->n_seqs).
 * to_cache == 0: reads cache->v, writes v_token_major.
 * The bytes are moved unchanged (no scaling or rounding). v_token_major:
 * device, caller-owned, the size of cache->v, 16-byte aligned
 * (BEAM_E_RANGE), not overlapping cache->v (BEAM_E_RANGE: there is no
 * in-place form). Enqueued on `stream`; nothing is allocated. K needs no
 * conversion. */
beam_status beam_kv_convert_v(const beam_attn_config *cfg, const beam_kv_cache *cache, void *v_token_major,
                              int32_t to_cache, void *stream);

const char *beam_status_str(beam_status s);
/* Message of the last failed call on this thread ("" if none). */
const char *beam_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_ATTN_H */
