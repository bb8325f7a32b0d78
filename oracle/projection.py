"""CPU oracle for the projections around Beam 1.0's attention sublayer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU baseline
leg of the benchmark may import this module. The product path never calls it
and shares no code with it.

Source: [BEAM-EN] "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax"
(flozi.net, English guide), section "Follow the tensors, not the parameter
label": the normalised sublayer input X has width 5,120; the projections use
the PyTorch output-by-input weight convention; the attention width is 6,144
(48 query heads of 128), K and V have 8 heads of 128, the gate projection has
6,144 outputs; after the coordinate-wise gate, W_o mixes the heads.

Readings where the pages are silent (each is listed in the design notes):
  * No projection carries a bias (the pages name only the gate's per-head
    additive bias, which the attention oracle already takes).
  * Head h of a projection is its output columns 128h .. 128h+127.
  * The library stacks the weights as one matrix with the rows of Wq, Wk,
    Wv and Wg in this order; this is a layout of the library, not a fact of
    the pages, and the oracle only splits it back.

Everything is evaluated in float64 from the bf16 inputs; nothing is rounded.
Pinned by tests/test_oracle_projection.py: a brute-force sum for the weight
convention, selection weights that reduce the composed layer to the pinned
attention oracle on known bf16 inputs (head split and stacking order), and
the head order that W_o sees.
"""
from __future__ import annotations

import numpy as np

from .beam_attention import (Config, attend, bf16_to_f64, output_gate, position_op, rms_norm)


def linear(x_bits, w_bits) -> np.ndarray:
    """out[t, f] = sum_k x[t, k] * W[f, k] in float64 (W output-by-input)."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T


def split_qkvg(proj: np.ndarray, n_q: int = 48, n_kv: int = 8, d: int = 128):
    """Split stacked projection outputs [n, (2 n_q + 2 n_kv) d] into Q, K, V and
    gate logits, each [n, heads, d]."""
    n = proj.shape[0]
    b = np.cumsum([0, n_q * d, n_kv * d, n_kv * d, n_q * d])
    q, k, v, g = (proj[:, b[i]:b[i + 1]] for i in range(4))
    return (q.reshape(n, n_q, d), k.reshape(n, n_kv, d), v.reshape(n, n_kv, d), g.reshape(n, n_q, d))


def project_qkvg(x_bits, w_qkvg_bits, n_q: int = 48, n_kv: int = 8, d: int = 128):
    """Q, K, V and gate logits of the tokens x [n, hidden] (float64)."""
    return split_qkvg(linear(x_bits, w_qkvg_bits), n_q, n_kv, d)


def queries_prime(kind: int, q: np.ndarray, q_norm_w_bits, q_pos, cfg: Config = Config()) -> np.ndarray:
    """Normalised, position-op'd queries (RMSNorm, then RoPE on local layers or
    a(t+1) on global layers) of raw queries q [n, H, d] at positions q_pos."""
    qn = rms_norm(q, bf16_to_f64(q_norm_w_bits), cfg.rms_eps)
    qp, _ = position_op(kind, qn, qn[:, :1], np.asarray(q_pos), np.asarray(q_pos), cfg)
    return qp


def attention_from_projections(kind: int, q, k, v, g, q_norm_w_bits, k_norm_w_bits, q_pos, k_pos,
                               cfg: Config = Config(), gate_bias=None) -> np.ndarray:
    """The attention sublayer on float64 projections: q [nq, H, d] at q_pos;
    k, v [nk, G, d] at k_pos (the sequence's history including the queries'
    own tokens); g [nq, H, d]. Returns Y [nq, H, d]."""
    qn = rms_norm(q, bf16_to_f64(q_norm_w_bits), cfg.rms_eps)
    kn = rms_norm(k, bf16_to_f64(k_norm_w_bits), cfg.rms_eps)
    qp, kp = position_op(kind, qn, kn, np.asarray(q_pos), np.asarray(k_pos), cfg)
    o = attend(kind, qp, kp, v, q_pos, k_pos, cfg)
    return output_gate(o, g, gate_bias)


def output_projection(y: np.ndarray, w_o_bits) -> np.ndarray:
    """out[t, f] = sum over (h, i) of Y[t, h, i] * W_o[f, 128 h + i] (float64);
    y is [n, H, d] (heads in order) or already [n, H d]."""
    y2 = np.asarray(y, dtype=np.float64).reshape(y.shape[0], -1)
    return y2 @ bf16_to_f64(w_o_bits).T
