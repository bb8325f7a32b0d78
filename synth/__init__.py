"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds no arithmetic of the attention method: it only draws
numbers and converts them to the storage format (bf16 bit patterns), so that
the oracle and the GPU consume the very same input bits.

Recipe (every tensor): the tensor is cut into blocks of 1024 rows along its
first (token) axis; block b is drawn by ``numpy.random.Generator(PCG64(
SeedSequence([cfg, tensor_id, layer, b])))`` as float32 N(0,1) values (blocks
are drawn in parallel threads), which are rounded to bfloat16 with
round-to-nearest-even and kept as ``uint16`` bit patterns.
RMSNorm weights are 1 + 0.1*N(0,1), gate logits N(0,1), gate bias absent in
the workload configurations; where a test exercises the per-head gate bias it
is float32 0.5*N(0,1) per query head (``gate_bias``).
Router inputs (the MoE layers' expert selection): hidden states bf16 N(0,1),
a float32 weight 0.02*N(0,1) and a float32 selection bias 0.05*N(0,1).
Projection inputs (the GEMMs around attention): the normalised sublayer input
x bf16 N(0,1) [n_tok][hidden]; the stacked Wq/Wk/Wv/Wg rows and W_o bf16
N(0,1)/sqrt(fan_in), so that projected values are about N(0,1) like the
attention inputs above.
Position/page structure (decode contexts, random page permutation, chunked
prefill lengths) is drawn from the same kind of generator with its own id.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_ROWS = 1024
_THREADS = max(1, min(16, os.cpu_count() or 1))

# tensor ids for SeedSequence([cfg, tensor_id, layer])
T_Q, T_K, T_V, T_GATE, T_QW, T_KW, T_POS, T_PERM, T_LEN, T_MISC = range(10)
T_RX, T_RW, T_RB = 10, 11, 12  # router: hidden states, weight, selection bias
T_PX, T_PW, T_PO = 13, 14, 15  # projections: sublayer input, stacked Wq/Wk/Wv/Wg, W_o
T_GB = 16  # per-head gate bias


def rng(cfg: int, tensor_id: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor_id, layer])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs only: the sum stays below 2^32
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, cfg: int, tensor_id: int, layer: int = 0, scale: float = 1.0,
                offset: float = 0.0) -> np.ndarray:
    """bf16 bits of scale*N(0,1)+offset, drawn in seeded blocks of 1024 rows."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0] if shape else 1
    n_blocks = max(1, -(-rows // BLOCK_ROWS))

    def block(b):
        lo, hi = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor_id, layer, b])))
        x = g.standard_normal(size=(hi - lo,) + shape[1:], dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        if offset != 0.0:
            x += np.float32(offset)
        out[lo:hi] = f32_to_bf16_bits(x)

    if n_blocks == 1:
        block(0)
    else:
        with ThreadPoolExecutor(min(_THREADS, n_blocks)) as ex:
            list(ex.map(block, range(n_blocks)))
    return out


def attention_inputs(cfg: int, layer: int, n_tok: int, n_q: int = 48, n_kv: int = 8, d: int = 128):
    """Q/K/V/gate-logit bf16 bits and the two RMSNorm weight vectors of one layer."""
    return dict(
        q=normal_bf16((n_tok, n_q, d), cfg, T_Q, layer),
        k=normal_bf16((n_tok, n_kv, d), cfg, T_K, layer),
        v=normal_bf16((n_tok, n_kv, d), cfg, T_V, layer),
        gate=normal_bf16((n_tok, n_q, d), cfg, T_GATE, layer),
        q_norm_w=normal_bf16((d,), cfg, T_QW, layer, scale=0.1, offset=1.0),
        k_norm_w=normal_bf16((d,), cfg, T_KW, layer, scale=0.1, offset=1.0),
    )


def normal_f32(shape, cfg: int, tensor_id: int, layer: int = 0, scale: float = 1.0) -> np.ndarray:
    """float32 scale*N(0,1), drawn in seeded blocks of 1024 rows (kept in float32)."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0] if shape else 1
    for b in range(max(1, -(-rows // BLOCK_ROWS))):
        lo, hi = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor_id, layer, b])))
        out[lo:hi] = g.standard_normal(size=(hi - lo,) + shape[1:], dtype=np.float32) * np.float32(scale)
    return out


def router_inputs(cfg: int, layer: int, n_tok: int, hidden: int = 5120, n_experts: int = 256):
    """Router inputs of one MoE layer: bf16 bits of the normalised hidden states
    x ~ N(0,1) [n_tok][hidden], a float32 weight W ~ N(0, 0.02^2) [n_experts][hidden]
    (logits of standard deviation ~1.4) and a float32 selection bias ~ N(0, 0.05^2)."""
    return dict(
        x=normal_bf16((n_tok, hidden), cfg, T_RX, layer),
        w=normal_f32((n_experts, hidden), cfg, T_RW, layer, scale=0.02),
        bias=normal_f32((n_experts,), cfg, T_RB, layer, scale=0.05),
    )


def router_inputs_exact(cfg: int, layer: int, n_tok: int, hidden: int = 5120, n_experts: int = 256):
    """Router inputs on a coarse grid: x integers in [-8, 8] (bf16 bits), W
    integers in [-4, 4] times 2^-10 (float32), bias multiples of 2^-12 in
    [-0.125, 0.125]. Every product x*W is a multiple of 2^-10 below 2^-5 in
    magnitude, so every partial sum over up to 2^17 terms stays exact in
    float32 in any order (logits of standard deviation ~0.9)."""
    g = rng(cfg, T_RX, layer)
    x = g.integers(-8, 9, size=(n_tok, hidden)).astype(np.float32)
    w = (g.integers(-4, 5, size=(n_experts, hidden)) * 2.0 ** -10).astype(np.float32)
    bias = (g.integers(-512, 513, size=n_experts) * 2.0 ** -12).astype(np.float32)
    return dict(x=f32_to_bf16_bits(x), w=w, bias=bias)


def decode_positions(cfg: int, n_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Zero-based positions t of the new token, uniform integers in [lo, hi]."""
    return rng(cfg, T_POS).integers(lo, hi + 1, size=n_seqs).astype(np.int32)


def paged_block_table(cfg: int, ctx_lens, page_size: int = 16, extra_pages: int = 0):
    """Deal a random permutation of physical pages to sequences in order.

    Returns (block_table [n_seqs][max_pages] int32, n_pages). Unused entries are -1.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    need = (ctx_lens + page_size - 1) // page_size
    n_pages = int(need.sum()) + extra_pages
    perm = rng(cfg, T_PERM).permutation(n_pages).astype(np.int32)
    maxp = int(need.max()) if len(need) else 0
    bt = np.full((len(ctx_lens), max(maxp, 1)), -1, dtype=np.int32)
    off = 0
    for i, n in enumerate(need):
        bt[i, :n] = perm[off:off + n]
        off += n
    return bt, n_pages


def chunked_lengths(cfg: int, n_seqs: int, lo: int, hi: int) -> np.ndarray:
    return rng(cfg, T_LEN).integers(lo, hi + 1, size=n_seqs).astype(np.int64)


def projection_inputs(cfg: int, layer: int, n_tok: int, hidden: int = 5120, n_q: int = 48, n_kv: int = 8,
                      d: int = 128, with_w_o: bool = True):
    """bf16 bits of the sublayer input x [n_tok][hidden], the stacked
    projection weight [(2 n_q + 2 n_kv) d][hidden] (rows of Wq, Wk, Wv, Wg in
    this order), W_o [hidden][n_q d] and the two RMSNorm weights."""
    out = dict(
        x=normal_bf16((n_tok, hidden), cfg, T_PX, layer),
        w_qkvg=normal_bf16(((2 * n_q + 2 * n_kv) * d, hidden), cfg, T_PW, layer, scale=hidden ** -0.5),
        q_norm_w=normal_bf16((d,), cfg, T_QW, layer, scale=0.1, offset=1.0),
        k_norm_w=normal_bf16((d,), cfg, T_KW, layer, scale=0.1, offset=1.0),
    )
    if with_w_o:
        out["w_o"] = normal_bf16((hidden, n_q * d), cfg, T_PO, layer, scale=(n_q * d) ** -0.5)
    return out


def gate_bias(cfg: int, layer: int, n_q: int = 48, scale: float = 0.5) -> np.ndarray:
    """float32 per-query-head gate bias, scale*N(0,1) [n_q]."""
    return normal_f32((n_q,), cfg, T_GB, layer, scale=scale)
