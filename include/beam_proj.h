/*
 * beam_proj.h — C ABI of the projections around Beam 1.0's attention
 * sublayer, in the same library as beam_attn.h (gfx950).
 *
 * The operation ("Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax",
 * flozi.net, section "Follow the tensors, not the parameter label"): the
 * normalised sublayer input X [n_tok][hidden] (hidden 5,120) is projected by
 * weights in the output-by-input convention to
 *   Q = X Wq^T [n_tok][n_q_heads * 128]     (6,144: the attention width)
 *   K = X Wk^T, V = X Wv^T [n_tok][n_kv_heads * 128]   (1,024 each)
 *   G = X Wg^T [n_tok][n_q_heads * 128]     (the 6,144 gate logits)
 * and after attention the gated result Y [n_tok][n_q_heads * 128] is mixed
 * back by Wo [hidden][n_q_heads * 128]: out = Y Wo^T.
 *
 * Both run as bf16 MFMA GEMMs with fp32 accumulation and one bf16 rounding of
 * each output. The QKV/gate projection finishes the query heads in its
 * epilogue (RMSNorm with q_norm_w, then RoPE at t on local layers or the
 * SSMax factor a(t+1) on global layers, exactly the query part of the
 * prefill prologue, see beam_attn.h) and writes them as Q' into the query
 * region of the prefill workspace; the raw queries are never stored. A
 * prefill of the same chunk then runs with BEAM_STAGE_PROLOGUE_KV instead of
 * BEAM_STAGE_PROLOGUE and q_raw = NULL.
 *
 * All pointers are device pointers; the library never allocates, frees or
 * synchronises; errors as in beam_attn.h.
 */
#ifndef BEAM_PROJ_H
#define BEAM_PROJ_H

#include "beam_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* QKV/gate projection of one layer's prefill chunk with the query prologue fused.
 * kind:        beam_layer_kind of the layer (selects RoPE or SSMax for Q).
 * x:           bf16 [n_tok][hidden], the chunk tokens packed as for beam_attn_prefill.
 * w_qkvg:      bf16 [(2 n_q_heads + 2 n_kv_heads) * 128][hidden]: the rows of Wq, Wk,
 *              Wv and Wg stacked in this order.
 * q_norm_w:    bf16 [128].
 * cu_seqlens, start_pos, n_seqs, n_tok: as for beam_attn_prefill (token i of sequence
 *              s is at absolute position start_pos[s] + i - cu_seqlens[s]).
 * k_raw, v_raw: out, bf16 [n_tok][n_kv_heads][128]; gate_logits: out, bf16
 *              [n_tok][n_q_heads][128] (the inputs of the prefill call).
 * workspace:   the prefill workspace of the chunk (>= beam_prefill_workspace_bytes,
 *              256-byte aligned); Q' is written into its query region.
 * Supported: hidden a positive multiple of 128, at most 65,536. */
beam_status beam_attn_project(const beam_attn_config *cfg, int32_t kind, const beam_bf16 *x,
                              int32_t hidden, const beam_bf16 *w_qkvg, const beam_bf16 *q_norm_w,
                              const int32_t *cu_seqlens, const int32_t *start_pos, int32_t n_seqs,
                              int32_t n_tok, beam_bf16 *k_raw, beam_bf16 *v_raw,
                              beam_bf16 *gate_logits, void *workspace, size_t ws_bytes,
                              void *stream);

/* Output projection: out[t][f] = sum_k y[t][k] w_o[f][k] (bf16 in and out).
 * y: bf16 [n_tok][in_features]; w_o: bf16 [out_features][in_features];
 * out: bf16 [n_tok][out_features].
 * Supported: in_features a positive multiple of 128 (at most 65,536), out_features a
 * positive multiple of 256. */
beam_status beam_out_project(const beam_bf16 *y, const beam_bf16 *w_o, int32_t n_tok,
                             int32_t in_features, int32_t out_features, beam_bf16 *out,
                             void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_PROJ_H */
