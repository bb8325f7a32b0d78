"""CPU oracle for Beam 1.0 hybrid GQA attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU baseline
leg of the benchmark may import this module. The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

It evaluates the plain definition of the attention sublayer in float64 with
NumPy: no tiling, no online softmax, no splitting. Every input arrives as
bf16 bit patterns and is widened exactly; nothing is rounded afterwards.

Sources (the pages the method is described on):
  [BEAM-EN] "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax"
            (flozi.net, English guide), sections "Two attention paths in one
            decoder", "Follow the tensors, not the parameter label", "What
            scalable softmax changes mathematically", "KV memory: nine growing
            caches, not 52".
  [BEAM-FR] "Beam propose un LLM MoE de 501 milliards de paramètres..."
            (techfi24.com), section "Architecture et mécanismes d'inférence".
  [BEAM-AR] "Reflection launches Beam: an open 501B MoE" (news.hamidun.com,
            Arabic), section on hybrid attention and unusual residuals.

Readings where the pages are silent (each is listed in the design notes):
  * 1/sqrt(d) score scale on both layer kinds; a(p) multiplies on top.
  * RMSNorm is y = w * x / sqrt(mean(x^2) + eps), with one learned 128-vector
    per layer for Q and one for K, shared by all heads.
  * RoPE is the rotate-half form over all 128 coordinates, theta = 10000,
    zero-based position t.
  * GQA maps query head h to KV head floor(h / (n_q / n_kv)).
  * Gate: Y = O * sigmoid(G + b_h); b is absent (zero) unless given.

Parity status: every function below is pinned by a CPU test against printed
numbers, closed forms, invariants or brute force, except the RoPE rotation
convention and the 1/sqrt(d) factor on global layers, which no printed number
distinguishes ("parity unpinned" for those two readings).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

LOCAL = 0
GLOBAL = 1


@dataclass(frozen=True)
class Config:
    """Attention geometry of one Beam layer ([BEAM-EN] "Follow the tensors";
    window from "Two attention paths in one decoder"; SSMax base/exponent from
    [BEAM-FR]/[BEAM-AR]; eps from [BEAM-EN] "Follow the tensors")."""
    n_q_heads: int = 48
    n_kv_heads: int = 8
    head_dim: int = 128
    window: int = 512
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    ssmax_base: float = 2048.0
    ssmax_exp: float = 0.1


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-vector RMSNorm along the last (head) axis, then the learned weight.

    [BEAM-EN] "Follow the tensors": Q and K are RMS-normalised over their 128
    head coordinates with eps 1e-6 before the position operation; V is not.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return w * (x / np.sqrt(ms + eps))


def rope_frequencies(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i = 0 .. d/2-1 (rotate-half RoPE)."""
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def rope(x: np.ndarray, t: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE at zero-based positions t.

    x: [n, heads, d]; t: [n]. Pair (i, i+d/2) is rotated by angle t*omega_i.
    [BEAM-EN] "Follow the tensors": on local layers RoPE rotates the
    normalised Q and K. Angles are formed in float64.
    """
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(t, dtype=np.float64)[:, None] * rope_frequencies(d, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ssmax_scale(t, base: float = 2048.0, exponent: float = 0.1) -> np.ndarray:
    """Scalable-softmax query scale a(p) = (1 + p/base)^exponent with p = t + 1.

    [BEAM-EN] "Follow the tensors": p is the one-based absolute position of the
    query, not the number of new tokens in a cached call. Formula from
    [BEAM-FR] "Architecture et mécanismes d'inférence" and [BEAM-AR].
    """
    p = np.asarray(t, dtype=np.float64) + 1.0
    return (1.0 + p / base) ** exponent


def visible(kind: int, t, s, window: int) -> np.ndarray:
    """Key at position s is visible to the query at position t.

    Global: causal, s <= t. Local: causal and t - s <= window - 1, i.e. the
    window counts the current token plus window-1 earlier positions
    ([BEAM-EN] "Two attention paths in one decoder").
    """
    t = np.asarray(t)[..., :, None]
    s = np.asarray(s)[..., None, :]
    diff = t - s
    vis = diff >= 0
    if kind == LOCAL:
        vis &= diff <= window - 1
    return vis


def kv_head_of(h: int, n_q: int, n_kv: int) -> int:
    """GQA: six consecutive query heads share one KV head ([BEAM-EN]
    "Follow the tensors"); generally n_q/n_kv of them."""
    return h // (n_q // n_kv)


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax over the masked logits; -inf entries get probability 0."""
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def position_op(kind: int, qn: np.ndarray, kn: np.ndarray, tq, tk, cfg: Config):
    """Apply the path-specific position operation to normalised Q and K.

    Local: RoPE on both. Global: K unchanged, Q times a(t+1)
    ([BEAM-EN] "Follow the tensors"; [BEAM-FR]; [BEAM-AR]).
    """
    if kind == LOCAL:
        return rope(qn, tq, cfg.rope_theta), rope(kn, tk, cfg.rope_theta)
    a = ssmax_scale(tq, cfg.ssmax_base, cfg.ssmax_exp)
    return qn * a[:, None, None], kn


def attend(kind: int, qp: np.ndarray, kp: np.ndarray, v: np.ndarray, tq, tk,
           cfg: Config, q_block: int = 256) -> np.ndarray:
    """Exact softmax attention with the layer's visibility rule.

    qp: position-op'd queries [nq, H, d]; kp: keys [nk, G, d]; v: [nk, G, d].
    S = qp.kp / sqrt(d) over visible keys, P = softmax(S), O = P V.
    Query rows are processed in blocks only to bound memory.
    """
    nq, H, d = qp.shape
    G = kp.shape[1]
    tq = np.asarray(tq)
    tk = np.asarray(tk)
    out = np.zeros((nq, H, d), dtype=np.float64)
    inv = 1.0 / math.sqrt(d)
    for h in range(H):
        g = kv_head_of(h, H, G)
        kg = kp[:, g, :]
        vg = v[:, g, :]
        for r0 in range(0, nq, q_block):
            r1 = min(nq, r0 + q_block)
            z = (qp[r0:r1, h, :] @ kg.T) * inv
            vis = visible(kind, tq[r0:r1], tk, cfg.window)
            z = np.where(vis, z, -np.inf)
            out[r0:r1, h, :] = softmax(z) @ vg
    return out


def output_gate(o: np.ndarray, gate_logits: np.ndarray, gate_bias=None) -> np.ndarray:
    """Per-coordinate sigmoid gate Y = O * sigmoid(G + b_h).

    [BEAM-EN] "Follow the tensors": the gate has 6,144 outputs per token and
    only its additive bias is one value per head.
    """
    z = gate_logits
    if gate_bias is not None:
        z = z + np.asarray(gate_bias, dtype=np.float64)[None, :, None]
    return o * (1.0 / (1.0 + np.exp(-z)))


def attention_layer(kind: int, q_bits, k_bits, v_bits, q_norm_w_bits, k_norm_w_bits,
                    gate_bits, q_pos, k_pos, cfg: Config = Config(), gate_bias=None,
                    return_pre_gate: bool = False, fp8_cache=None):
    """One attention sublayer for the queries of one sequence.

    q_bits [nq, H, d]: raw query projections at positions q_pos.
    k_bits, v_bits [nk, G, d]: raw K/V projections of the sequence's history
    (the oracle's own cache model) at positions k_pos, including the queries'
    own tokens. Returns Y [nq, H, d] in float64 (and O if asked).
    fp8_cache: None, or (k_scale, v_scale, cached_end): keys at positions below
    cached_end come from an FP8 cache, so their K_hat (after the position op,
    which is what the cache holds) and V pass through fp8_roundtrip.
    """
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    qn = rms_norm(q, bf16_to_f64(q_norm_w_bits), cfg.rms_eps)
    kn = rms_norm(k, bf16_to_f64(k_norm_w_bits), cfg.rms_eps)
    qp, kp = position_op(kind, qn, kn, np.asarray(q_pos), np.asarray(k_pos), cfg)
    if fp8_cache is not None:
        k_scale, v_scale, cached_end = fp8_cache
        m = np.asarray(k_pos) < cached_end
        kp = kp.copy()
        v = v.copy()
        kp[m] = fp8_roundtrip(kp[m], k_scale)
        v[m] = fp8_roundtrip(v[m], v_scale)
    o = attend(kind, qp, kp, v, q_pos, k_pos, cfg)
    y = output_gate(o, bf16_to_f64(gate_bits), gate_bias)
    return (y, o) if return_pre_gate else y


# ---------------------------------------------------------------- FP8 KV cache
# The pages' serving recipes keep the KV cache in FP8 E4M3 ([BEAM-EN] "KV
# memory: nine growing caches, not 52": 18 KiB per token across the nine
# global layers in FP8; the German serving article: FP8 E4M3 cache by default).
# They state no scale convention. Reading used here: one scale per tensor (K
# and V of a layer), code = nearest E4M3FN value of x / scale with ties to the
# even code and saturation at +-448, value = decode(code) * scale.

def _e4m3_finite_values() -> np.ndarray:
    """Values of the non-negative finite E4M3FN codes 0x00..0x7E, in code order
    (OCP 8-bit float E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals at exponent 0, no infinities, 0x7F is NaN)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def e4m3_decode(codes) -> np.ndarray:
    """Float value of E4M3FN codes (uint8); 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    vals = np.append(_e4m3_finite_values(), np.nan)[mag]
    return np.where(c & 0x80, -vals, vals)


def e4m3_encode(x) -> np.ndarray:
    """Code of the E4M3FN value nearest to x (ties to the even code, |x| >= 448
    saturates to +-448, NaN -> 0x7F), found by searching the table of
    representable values."""
    x = np.asarray(x, dtype=np.float64)
    table = _e4m3_finite_values()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)  # first value >= a
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= table[-1], 0x7E, code)
    code = np.where(np.isnan(x), 0x7F, code).astype(np.uint8)
    return np.where(np.signbit(x) & ~np.isnan(x), code | 0x80, code).astype(np.uint8)


def fp8_roundtrip(x, scale: float) -> np.ndarray:
    """What an FP8 cache returns for values x stored with `scale`."""
    return e4m3_decode(e4m3_encode(np.asarray(x, dtype=np.float64) / scale)) * scale


def cached_key(kind: int, k_bits, k_norm_w_bits, pos, cfg: Config = Config()) -> np.ndarray:
    """What the cache holds for K: normalised K, rotated on local layers
    (the norm/position op is fused with cache insertion on the pages' BF16
    path; SSMax touches only Q) — [BEAM-EN] "The surrounding model and
    serving boundary" and "Follow the tensors"."""
    kn = rms_norm(bf16_to_f64(k_bits), bf16_to_f64(k_norm_w_bits), cfg.rms_eps)
    if kind == LOCAL:
        kn = rope(kn, np.asarray(pos), cfg.rope_theta)
    return kn


# ---------------------------------------------------------------- KV budget

def kv_bytes(n_tokens: int, bytes_per_scalar: int, n_global: int = 9, n_local: int = 43,
             n_kv: int = 8, d: int = 128, window: int = 512, page_size: int = 16,
             batch: int = 1):
    """Logical and page-rounded KV payload in bytes (exact integers).

    [BEAM-EN] "KV memory: nine growing caches, not 52": K and V (factor 2) for
    every global layer over all N tokens, plus a window-sized cache for each
    local layer. The paged figure rounds the global term up to whole pages.
    """
    per_tok = 2 * bytes_per_scalar * n_kv * d
    local_slots = min(n_tokens, window)
    logical = batch * per_tok * (n_global * n_tokens + n_local * local_slots)
    pages = -(-n_tokens // page_size)
    paged = batch * per_tok * (n_global * pages * page_size + n_local * local_slots)
    return logical, paged


def page_slot(block_table, page_size: int, seq: int, t: int):
    """Physical page and in-page slot of position t of sequence seq."""
    return int(block_table[seq][t // page_size]), t % page_size


def ring_slot(t: int, window: int = 512) -> int:
    """Slot of position t in a local layer's window-sized ring cache."""
    return t % window


def layer_kinds(n_layers: int = 52, period: int = 6):
    """Global at every sixth layer (1-based) and at the last layer; local
    otherwise ([BEAM-EN] "Two attention paths in one decoder"; [BEAM-AR])."""
    return [GLOBAL if (i % period == 0 or i == n_layers) else LOCAL
            for i in range(1, n_layers + 1)]


# ------------------------------------------------- scalable-softmax analysis

def softmax_entropy(z: np.ndarray, a: float) -> float:
    """H(a) = log Z(a) - a E_pi[z] for pi = softmax(a z), in nats
    ([BEAM-EN] "What scalable softmax changes mathematically")."""
    az = a * np.asarray(z, dtype=np.float64)
    m = az.max()
    e = np.exp(az - m)
    Z = e.sum()
    pi = e / Z
    return float(np.log(Z) + m - a * np.dot(pi, z))


def toy_needle_probability(delta: float, a: float, n: int) -> float:
    """One key beats n-1 equal distractors by delta; its softmax probability
    at scale a ([BEAM-EN] "What scalable softmax changes mathematically")."""
    e = math.exp(a * delta)
    return e / (e + n - 1)


def toy_required_scale(r: float, delta: float, n: int) -> float:
    """Scale a that gives the needle probability r in the toy model."""
    return math.log(r * (n - 1) / (1.0 - r)) / delta
