/*
 * beam_router.h — C ABI of the group-limited sigmoid router of Beam 1.0's MoE
 * layers (expert selection), in the same library as beam_attn.h (gfx950).
 *
 * The operation ("Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax",
 * flozi.net, section "The surrounding model and serving boundary";
 * techfi24.com, "Architecture et mécanismes d'inférence"; news.hamidun.com,
 * the MoE paragraph), per token:
 *   z_e = x . W_e, computed in fp32 (e = 0..255);
 *   s_e = sigmoid(z_e) as the nearest float32;  c_e = s_e + bias_e (float32);
 *   group g (experts 32g .. 32g+31) scores the sum of its two largest c;
 *   the topk_groups best groups are kept (ties: lower group);
 *   the top_k experts by c inside the kept groups are chosen, best first
 *   (ties: lower expert index);
 *   weight_k = s_k / (sum of the chosen s) * scale.
 * The bias only chooses; the weights use the uncorrected scores.
 *
 * All pointers are device pointers unless stated; the library never
 * allocates, frees or synchronises; errors as in beam_attn.h.
 */
#ifndef BEAM_ROUTER_H
#define BEAM_ROUTER_H

#include "beam_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Router geometry. Defaults for Beam 1.0: 5120, 256, 8, 4, 8, 2.5. Supported:
 * hidden a positive multiple of 32, n_experts 256, n_groups 8,
 * 1 <= topk_groups <= 8, 1 <= top_k <= 8, finite scale. */
typedef struct beam_router_config {
  int32_t hidden;
  int32_t n_experts;
  int32_t n_groups;
  int32_t topk_groups;
  int32_t top_k;
  float scale;
} beam_router_config;

/* The whole router in one kernel (logits stay on chip).
 * x: bf16 [n_tok][hidden] (the normalised hidden states).
 * w: float [n_experts][hidden]. bias: float [n_experts], or NULL for zero.
 * topk_idx: int32 [n_tok][top_k], topk_w: float [n_tok][top_k], best first. */
beam_status beam_router(const beam_router_config *cfg, const beam_bf16 *x, const float *w,
                        const float *bias, int32_t n_tok, int32_t *topk_idx, float *topk_w,
                        void *stream);

/* The logits alone: logits float [n_tok][n_experts] = x W^T in fp32. */
beam_status beam_router_logits(const beam_router_config *cfg, const beam_bf16 *x, const float *w,
                               int32_t n_tok, float *logits, void *stream);

/* The selection alone, from float32 logits [n_tok][n_experts]; outputs as
 * beam_router. Identical decisions to beam_router for the same logits. */
beam_status beam_router_select(const beam_router_config *cfg, const float *logits,
                               const float *bias, int32_t n_tok, int32_t *topk_idx,
                               float *topk_w, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_ROUTER_H */
