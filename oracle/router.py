"""CPU oracle for Beam 1.0's group-limited sigmoid router (expert selection of
the 49 MoE layers).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU baseline
leg of the benchmark may import this module. The product path never calls it
and shares no code with it.

Sources:
  [BEAM-EN] "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax"
            (flozi.net, English guide), section "The surrounding model and
            serving boundary": router logits in FP32 become sigmoid scores;
            each of eight groups is scored by the sum of its two largest
            bias-corrected scores; four groups are kept; eight experts are
            chosen from them; the mixture weights are the uncorrected scores
            of the chosen experts, normalised, times 2.5.
  [BEAM-FR] techfi24.com, "Architecture et mécanismes d'inférence": 256
            experts in 8 groups of 32, the 4 best groups, the top 8 inside.
  [BEAM-AR] news.hamidun.com, the MoE paragraph: the same grouping and the
            factor 2.5.

Readings where the pages are silent (each is listed in the design notes):
  * The logits are x . W_e over the hidden width with x the (bf16) normalised
    hidden state and W a float32 weight [n_experts][hidden]; "FP32 logits"
    fixes the precision the path computes in. The oracle evaluates the dot
    products exactly (float64) for the value comparison.
  * A score is the float32 value nearest to sigmoid(z) (evaluated in float64,
    then rounded), so that every integer decision below is taken on float32
    numbers as the pages state.
  * Selection arithmetic is float32: corrected = s + b, group score =
    largest + second largest corrected score of the group.
  * Ties (equal group scores, equal corrected scores) go to the lower index.
    The chosen experts are reported in selection order: corrected score
    descending, lower index first on ties.
  * Weights are evaluated in float64 from the float32 scores.

Parity: pinned by CPU tests against hand-built cases in which each plausible
mistake (max instead of top-2 sum, corrected scores as weights, uncorrected
scores for selection, no normalisation or no 2.5, softmax instead of sigmoid,
wrong number of groups kept, the tie rule) changes the result, against the
reduction to a plain top-k when every group is kept and the bias is zero, and
against invariants.
"""
from __future__ import annotations

import numpy as np

N_EXPERTS = 256
N_GROUPS = 8
TOPK_GROUPS = 4
TOP_K = 8
SCALE = 2.5


def router_logits(x_bits, w) -> np.ndarray:
    """z[t, e] = sum_k x[t, k] * W[e, k], exactly (float64): x are bf16 bit
    patterns [n_tok][hidden], W float32 [n_experts][hidden]."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x @ np.asarray(w, dtype=np.float64).T


def sigmoid_f32(z) -> np.ndarray:
    """The float32 value nearest to 1 / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _order(values, n_pick: int) -> np.ndarray:
    """Indices of the n_pick largest values, largest first, lower index first
    among equal values (a stable sort of the negated values)."""
    return np.argsort(-np.asarray(values, dtype=np.float64), kind="stable")[:n_pick]


def select(scores, bias, n_groups: int = N_GROUPS, topk_groups: int = TOPK_GROUPS, top_k: int = TOP_K,
           scale: float = SCALE):
    """Group-limited top-k of one layer for every token.

    scores: float32 sigmoid scores [n_tok][n_experts]; bias: float32 [n_experts].
    Returns (idx int32 [n_tok][top_k] in selection order, weights float64
    [n_tok][top_k], kept groups int32 [n_tok][topk_groups] in order).
    """
    s = np.asarray(scores, dtype=np.float32)
    b = np.asarray(bias, dtype=np.float32)
    n_tok, n_exp = s.shape
    per = n_exp // n_groups
    idx = np.zeros((n_tok, top_k), dtype=np.int32)
    wts = np.zeros((n_tok, top_k), dtype=np.float64)
    kept = np.zeros((n_tok, topk_groups), dtype=np.int32)
    for t in range(n_tok):
        # 1. bias-corrected scores, used only to choose
        corr = s[t] + b                                        # float32 adds
        # 2. group score: the two largest corrected scores of the group
        gsc = np.empty(n_groups, dtype=np.float32)
        for g in range(n_groups):
            top2 = np.sort(corr[g * per:(g + 1) * per])[::-1][:2]
            gsc[g] = top2[0] + top2[1]                         # float32 add
        # 3. keep the best groups
        kg = _order(gsc, topk_groups)
        kept[t] = kg
        # 4. the best experts inside the kept groups
        cand = np.full(n_exp, -np.inf, dtype=np.float64)
        for g in kg:
            cand[g * per:(g + 1) * per] = corr[g * per:(g + 1) * per]
        chosen = _order(cand, top_k)
        idx[t] = chosen
        # 5. weights from the uncorrected scores, normalised, times the scale
        sel = s[t, chosen].astype(np.float64)
        wts[t] = sel / sel.sum() * scale
    return idx, wts, kept


def route(x_bits, w, bias, **kw):
    """The whole router: logits, float32 scores, selection. Also returns the
    float64 logits."""
    z = router_logits(x_bits, w)
    idx, wts, kept = select(sigmoid_f32(z), bias, **kw)
    return idx, wts, kept, z
