"""Python binding of libbeam_attn.so (Beam 1.0 hybrid GQA attention, gfx950).

Argument marshalling only: torch tensors are passed to the C ABI as device
pointers together with torch's current HIP stream; every step of the
computation runs in the library's HIP kernels. If the library is missing this
module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbeam_attn.so")

LOCAL = 0
GLOBAL = 1
KV_BF16 = 0
KV_FP8_E4M3 = 1

STAGE_PROLOGUE = 1
STAGE_ATTENTION = 2
STAGE_APPEND = 4
STAGE_COMBINE = 4
STAGE_ALL = 7
STAGE_VERIFY_COMBINE = 8
STAGE_VERIFY_ALL = 15
STAGE_PROLOGUE_KV = 16

EXPORTED = [
    "beam_kv_append", "beam_attn_prefill", "beam_attn_decode", "beam_attn_verify",
    "beam_attn_prefill_stages", "beam_attn_decode_stages", "beam_attn_verify_stages", "beam_attn_decode_noalloc",
    "beam_prefill_workspace_bytes", "beam_decode_workspace_bytes", "beam_verify_workspace_bytes",
    "beam_kv_bytes", "beam_kv_page_slot", "beam_debug_visibility", "beam_debug_validate_cache",
    "beam_kv_convert_v", "beam_status_str", "beam_last_error",
    "beam_router", "beam_router_logits", "beam_router_select",
    "beam_attn_project", "beam_out_project",
    "beam_probe_mfma_bf16", "beam_probe_mfma16_bf16", "beam_probe_stream_read",
]


class BeamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"beam status {status}: {message}")
        self.status = status


class CConfig(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("ssmax_base", ctypes.c_float), ("ssmax_exp", ctypes.c_float)]


class CCache(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


@dataclass
class Config:
    n_q_heads: int = 48
    n_kv_heads: int = 8
    head_dim: int = 128
    window: int = 512
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    ssmax_base: float = 2048.0
    ssmax_exp: float = 0.1

    def c(self) -> CConfig:
        return CConfig(self.n_q_heads, self.n_kv_heads, self.head_dim, self.window,
                       self.rope_theta, self.rms_eps, self.ssmax_base, self.ssmax_exp)


class CRouterConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scale", ctypes.c_float)]


@dataclass
class RouterConfig:
    """Group-limited sigmoid router of one MoE layer (include/beam_router.h)."""
    hidden: int = 5120
    n_experts: int = 256
    n_groups: int = 8
    topk_groups: int = 4
    top_k: int = 8
    scale: float = 2.5

    def c(self) -> CRouterConfig:
        return CRouterConfig(self.hidden, self.n_experts, self.n_groups, self.topk_groups, self.top_k, self.scale)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbeam_attn.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m global_attention_amd.build`")
    # torch first: its HIP runtime then serves the library too. Loaded the other
    # way round, torch's libraries (which ask for the runtime by its unversioned
    # file name) would bring a second copy of the runtime into the process.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.beam_kv_append.argtypes = [P, P, P, P, P, P, P, I32, P]
    L.beam_attn_prefill.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, P, P, SZ, P]
    L.beam_attn_decode.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, P, P, SZ, P]
    U32 = ctypes.c_uint32
    L.beam_attn_prefill_stages.argtypes = [U32] + L.beam_attn_prefill.argtypes
    L.beam_attn_decode_stages.argtypes = [U32] + L.beam_attn_decode.argtypes
    L.beam_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, P, P]
    L.beam_attn_verify.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, SZ, P]
    L.beam_attn_verify_stages.argtypes = [U32] + L.beam_attn_verify.argtypes
    L.beam_verify_workspace_bytes.argtypes = [P, I32, I32, I32, I32, I32, I32]
    L.beam_verify_workspace_bytes.restype = SZ
    L.beam_prefill_workspace_bytes.argtypes = [P, I32, I32]
    L.beam_prefill_workspace_bytes.restype = SZ
    L.beam_decode_workspace_bytes.argtypes = [P, I32, I32, I32, I32]
    L.beam_decode_workspace_bytes.restype = SZ
    L.beam_kv_bytes.argtypes = [I64, I32, I32, I32, I32, I32, I32, I32, P, P]
    L.beam_kv_page_slot.argtypes = [P, I32, I32, I32, I32, P, P]
    L.beam_debug_visibility.argtypes = [I32, I32, I32, I32, I32, I32, P, P]
    L.beam_debug_validate_cache.argtypes = [P, P, P, P]
    L.beam_kv_convert_v.argtypes = [P, P, P, I32, P]
    L.beam_router.argtypes = [P, P, P, P, I32, P, P, P]
    L.beam_router_logits.argtypes = [P, P, P, I32, P, P]
    L.beam_router_select.argtypes = [P, P, P, I32, P, P, P]
    L.beam_attn_project.argtypes = [P, I32, P, I32, P, P, P, P, I32, I32, P, P, P, P, SZ, P]
    L.beam_out_project.argtypes = [P, P, I32, I32, I32, P, P]
    L.beam_probe_mfma_bf16.argtypes = [P, I32, I32, I32, P, P]
    L.beam_probe_mfma16_bf16.argtypes = [P, I32, I32, I32, P, P]
    L.beam_probe_stream_read.argtypes = [P, SZ, I32, P, P]
    L.beam_status_str.argtypes = [I32]
    L.beam_status_str.restype = ctypes.c_char_p
    L.beam_last_error.restype = ctypes.c_char_p
    for name in ("beam_kv_append", "beam_attn_prefill", "beam_attn_decode", "beam_attn_decode_noalloc",
                 "beam_attn_prefill_stages",
                 "beam_attn_decode_stages", "beam_attn_verify", "beam_attn_verify_stages", "beam_kv_bytes",
                 "beam_kv_page_slot", "beam_debug_visibility", "beam_debug_validate_cache", "beam_kv_convert_v",
                 "beam_router",
                 "beam_router_logits", "beam_router_select", "beam_attn_project", "beam_out_project",
                 "beam_probe_mfma_bf16", "beam_probe_mfma16_bf16", "beam_probe_stream_read"):
        getattr(L, name).restype = I32
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise BeamError(status, lib().beam_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape=None, name="tensor"):
    import torch
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


@dataclass
class KVCache:
    """One layer's cache as torch device tensors (layouts in include/beam_attn.h).
    dtype KV_BF16 holds bfloat16 tensors, KV_FP8_E4M3 uint8 codes with the
    per-tensor scales k_scale / v_scale."""
    kind: int
    k: object
    v: object
    block_table: object = None  # int32 [n_seqs][max_pages] (global)
    n_pages: int = 0
    page_size: int = 16
    dtype: int = KV_BF16
    k_scale: float = 1.0
    v_scale: float = 1.0
    _c: CCache = field(default=None, repr=False)

    @staticmethod
    def _alloc(shape_k, shape_v, dtype, device, fill):
        import torch
        tdt = torch.bfloat16 if dtype == KV_BF16 else torch.uint8
        k = torch.empty(shape_k, dtype=tdt, device=device)
        v = torch.empty(shape_v, dtype=tdt, device=device)
        if fill is not None:
            view = torch.int16 if dtype == KV_BF16 else torch.uint8
            k.view(view).fill_(fill)
            v.view(view).fill_(fill)
        return k, v

    @staticmethod
    def allocate_global(cfg: Config, n_pages: int, block_table, device="cuda", fill=None, dtype=KV_BF16,
                        k_scale=1.0, v_scale=1.0):
        k, v = KVCache._alloc((n_pages, cfg.n_kv_heads, 16, cfg.head_dim), (n_pages, cfg.n_kv_heads, cfg.head_dim, 16),
                              dtype, device, fill)
        import torch
        bt = block_table.to(device=device, dtype=torch.int32).contiguous()
        return KVCache(GLOBAL, k, v, bt, n_pages, 16, dtype, float(k_scale), float(v_scale))

    @staticmethod
    def allocate_local(cfg: Config, n_seqs: int, device="cuda", fill=None, dtype=KV_BF16, k_scale=1.0, v_scale=1.0):
        k, v = KVCache._alloc((n_seqs, cfg.n_kv_heads, cfg.window, cfg.head_dim),
                              (n_seqs, cfg.n_kv_heads, cfg.head_dim, cfg.window), dtype, device, fill)
        return KVCache(LOCAL, k, v, None, 0, 16, dtype, float(k_scale), float(v_scale))

    def c(self) -> CCache:
        if self.kind == GLOBAL:
            bt = self.block_table
            return CCache(GLOBAL, self.k.data_ptr(), self.v.data_ptr(), self.page_size, self.n_pages,
                          bt.data_ptr(), bt.shape[1], bt.shape[0], self.dtype, self.k_scale, self.v_scale)
        return CCache(LOCAL, self.k.data_ptr(), self.v.data_ptr(), 0, 0, None, 0, self.k.shape[0], self.dtype,
                      self.k_scale, self.v_scale)


def prefill_workspace_bytes(cfg: Config, n_tok: int, n_seqs: int) -> int:
    c = cfg.c()
    return int(lib().beam_prefill_workspace_bytes(ctypes.byref(c), n_tok, n_seqs))


def decode_workspace_bytes(cfg: Config, kind: int, n_seqs: int, max_pos: int, split_keys: int = 0) -> int:
    c = cfg.c()
    return int(lib().beam_decode_workspace_bytes(ctypes.byref(c), kind, n_seqs, max_pos, split_keys))


def verify_workspace_bytes(cfg: Config, kind: int, n_tok: int, n_seqs: int, max_chunk_len: int, max_pos: int,
                           split_keys: int = 0) -> int:
    c = cfg.c()
    return int(lib().beam_verify_workspace_bytes(ctypes.byref(c), kind, n_tok, n_seqs, max_chunk_len, max_pos,
                                                 split_keys))


def _workspace(nbytes, device, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


def kv_append(cfg: Config, cache: KVCache, k_raw, v_raw, k_norm_w, seq_idx, pos, stream=None):
    import torch
    n = k_raw.shape[0]
    for t, nm in ((k_raw, "k_raw"), (v_raw, "v_raw"), (k_norm_w, "k_norm_w")):
        _need(t, torch.bfloat16, name=nm)
    _need(seq_idx, torch.int32, (n,), "seq_idx")
    _need(pos, torch.int32, (n,), "pos")
    c, kc = cfg.c(), cache.c()
    _check(lib().beam_kv_append(ctypes.byref(c), ctypes.byref(kc), _ptr(k_raw), _ptr(v_raw), _ptr(k_norm_w),
                                _ptr(seq_idx), _ptr(pos), n, _stream(stream)))


def prefill(cfg: Config, cache: KVCache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate, cu_seqlens, seq_idx,
            start_pos, max_chunk_len: int, gate_bias=None, out=None, workspace=None, stream=None,
            stages: int = STAGE_ALL):
    """Chunked varlen prefill of one layer; returns out [n_tok][H][d] (bf16).
    `stages` selects prologue / attention / append (beam_attn_prefill_stages)."""
    n_tok, n_seqs, out = _chunk_args(cfg, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate, cu_seqlens, seq_idx,
                                     start_pos, gate_bias, out)
    nbytes = prefill_workspace_bytes(cfg, n_tok, n_seqs)
    workspace = _workspace(nbytes, k_raw.device, workspace)
    c, kc = cfg.c(), cache.c()
    _check(lib().beam_attn_prefill_stages(
        stages, ctypes.byref(c), ctypes.byref(kc), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(q_norm_w),
        _ptr(k_norm_w), _ptr(gate), _ptr(gate_bias), _ptr(cu_seqlens), _ptr(seq_idx), _ptr(start_pos),
        n_seqs, n_tok, max_chunk_len, _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def verify(cfg: Config, cache: KVCache, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate, cu_seqlens, seq_idx,
           start_pos, max_chunk_len: int, max_pos: int, gate_bias=None, split_keys: int = 0, out=None,
           workspace=None, stream=None, stages: int = STAGE_VERIFY_ALL):
    """Verify step (a short chunk per sequence over its cache); same semantics as
    prefill, returns out [n_tok][H][d] (bf16). max_pos bounds start_pos + chunk
    length - 1. `stages` selects prologue / split attention / combine / append
    (beam_attn_verify_stages)."""
    n_tok, n_seqs, out = _chunk_args(cfg, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate, cu_seqlens, seq_idx,
                                     start_pos, gate_bias, out)
    nbytes = verify_workspace_bytes(cfg, cache.kind, n_tok, n_seqs, max_chunk_len, max_pos, split_keys)
    if nbytes == 0:
        raise BeamError(3, "invalid verify sizes (max_chunk_len / max_pos / split_keys)")
    workspace = _workspace(nbytes, k_raw.device, workspace)
    c, kc = cfg.c(), cache.c()
    _check(lib().beam_attn_verify_stages(
        stages, ctypes.byref(c), ctypes.byref(kc), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(q_norm_w),
        _ptr(k_norm_w), _ptr(gate), _ptr(gate_bias), _ptr(cu_seqlens), _ptr(seq_idx), _ptr(start_pos),
        n_seqs, n_tok, max_chunk_len, max_pos, split_keys, _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


def _chunk_args(cfg, q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate, cu_seqlens, seq_idx, start_pos, gate_bias, out):
    import torch
    n_tok = k_raw.shape[0]
    n_seqs = cu_seqlens.shape[0] - 1
    H, G, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    if q_raw is not None:
        _need(q_raw, torch.bfloat16, (n_tok, H, d), "q_raw")
    _need(k_raw, torch.bfloat16, (n_tok, G, d), "k_raw")
    _need(v_raw, torch.bfloat16, (n_tok, G, d), "v_raw")
    _need(gate, torch.bfloat16, (n_tok, H, d), "gate")
    _need(q_norm_w, torch.bfloat16, (d,), "q_norm_w")
    _need(k_norm_w, torch.bfloat16, (d,), "k_norm_w")
    _need(cu_seqlens, torch.int32, (n_seqs + 1,), "cu_seqlens")
    _need(seq_idx, torch.int32, (n_seqs,), "seq_idx")
    _need(start_pos, torch.int32, (n_seqs,), "start_pos")
    if gate_bias is not None:
        _need(gate_bias, torch.float32, (H,), "gate_bias")
    if out is None:
        out = torch.empty((n_tok, H, d), dtype=torch.bfloat16, device=k_raw.device)
    _need(out, torch.bfloat16, (n_tok, H, d), "out")
    return n_tok, n_seqs, out


def decode(cfg: Config, cache: KVCache, q_raw, q_norm_w, gate, seq_idx, pos, max_pos: int, gate_bias=None,
           split_keys: int = 0, out=None, workspace=None, stream=None, stages: int = STAGE_ALL):
    """One-token decode of one layer; returns out [n_seqs][H][d] (bf16).
    `stages` selects prologue / split attention / combine (beam_attn_decode_stages)."""
    import torch
    n = q_raw.shape[0]
    H, d = cfg.n_q_heads, cfg.head_dim
    _need(q_raw, torch.bfloat16, (n, H, d), "q_raw")
    _need(gate, torch.bfloat16, (n, H, d), "gate")
    _need(q_norm_w, torch.bfloat16, (d,), "q_norm_w")
    _need(seq_idx, torch.int32, (n,), "seq_idx")
    _need(pos, torch.int32, (n,), "pos")
    if gate_bias is not None:
        _need(gate_bias, torch.float32, (H,), "gate_bias")
    if out is None:
        out = torch.empty((n, H, d), dtype=torch.bfloat16, device=q_raw.device)
    _need(out, torch.bfloat16, (n, H, d), "out")
    nbytes = decode_workspace_bytes(cfg, cache.kind, n, max_pos, split_keys)
    if nbytes == 0:
        raise BeamError(3, "invalid decode sizes (max_pos / split_keys)")
    workspace = _workspace(nbytes, q_raw.device, workspace)
    c, kc = cfg.c(), cache.c()
    _check(lib().beam_attn_decode_stages(
        stages, ctypes.byref(c), ctypes.byref(kc), _ptr(q_raw), _ptr(q_norm_w), _ptr(gate), _ptr(gate_bias),
        _ptr(seq_idx), _ptr(pos), n, max_pos, split_keys, _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


DECODE_SCRATCH_BYTES = 32 << 20  # BEAM_DECODE_SCRATCH_BYTES


def decode_noalloc(cfg: Config, cache: KVCache, q_raw, q_norm_w, gate, seq_idx, pos, max_pos: int, out,
                   gate_bias=None, split_keys: int = 0, stream=None):
    """decode() through beam_attn_decode_noalloc: no workspace; the library's
    own per-GPU scratch array holds the split partials. `out` [n_seqs][H][d]
    (bf16) is the caller's; the call allocates nothing."""
    import torch
    n = q_raw.shape[0]
    H, d = cfg.n_q_heads, cfg.head_dim
    _need(q_raw, torch.bfloat16, (n, H, d), "q_raw")
    _need(gate, torch.bfloat16, (n, H, d), "gate")
    _need(q_norm_w, torch.bfloat16, (d,), "q_norm_w")
    _need(seq_idx, torch.int32, (n,), "seq_idx")
    _need(pos, torch.int32, (n,), "pos")
    _need(out, torch.bfloat16, (n, H, d), "out")
    if gate_bias is not None:
        _need(gate_bias, torch.float32, (H,), "gate_bias")
    c, kc = cfg.c(), cache.c()
    _check(lib().beam_attn_decode_noalloc(
        ctypes.byref(c), ctypes.byref(kc), _ptr(q_raw), _ptr(q_norm_w), _ptr(gate), _ptr(gate_bias),
        _ptr(seq_idx), _ptr(pos), n, max_pos, split_keys, _ptr(out), _stream(stream)))
    return out


def kv_bytes(n_tokens: int, bytes_per_scalar: int = 2, n_global: int = 9, n_local: int = 43, n_kv: int = 8,
             d: int = 128, window: int = 512, page_size: int = 16):
    """(logical, paged) KV payload bytes; host-only, no GPU needed."""
    lg, pg = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().beam_kv_bytes(n_tokens, bytes_per_scalar, n_global, n_local, n_kv, d, window, page_size,
                               ctypes.byref(lg), ctypes.byref(pg)))
    return lg.value, pg.value


def kv_page_slot(block_table_host, page_size: int, seq: int, t: int):
    """(physical page, slot) of position t of sequence seq; host-only."""
    import numpy as np
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    pg, sl = ctypes.c_int64(), ctypes.c_int32()
    _check(lib().beam_kv_page_slot(bt.ctypes.data_as(ctypes.c_void_p), bt.shape[1], page_size, seq, t,
                                   ctypes.byref(pg), ctypes.byref(sl)))
    return pg.value, sl.value


def debug_visibility(kind: int, window: int, t0: int, n_q: int, s0: int, n_k: int, device="cuda", stream=None):
    import torch
    mask = torch.empty((n_q, n_k), dtype=torch.uint8, device=device)
    _check(lib().beam_debug_visibility(kind, window, t0, n_q, s0, n_k, _ptr(mask), _stream(stream)))
    return mask


def debug_validate_cache(cache: KVCache, n_tokens=None, stream=None):
    """Per cache sequence, the number of used block-table entries that name no
    physical page (-1: the length does not fit the row); int32 device tensor
    [n_seqs] (beam_debug_validate_cache). n_tokens: int32 device [n_seqs] or
    None for whole rows."""
    import torch
    if cache.kind != GLOBAL:
        raise ValueError("only a paged (global) cache has a block table")
    n = cache.block_table.shape[0]
    if n_tokens is not None:
        _need(n_tokens, torch.int32, (n,), "n_tokens")
    n_bad = torch.empty((n,), dtype=torch.int32, device=cache.block_table.device)
    kc = cache.c()
    _check(lib().beam_debug_validate_cache(ctypes.byref(kc), _ptr(n_tokens), _ptr(n_bad), _stream(stream)))
    return n_bad


def kv_convert_v(cfg: Config, cache: KVCache, v_token_major, to_cache: bool, stream=None):
    """V of the cache between the token-major layout ([n_pages][n_kv][16][d]
    global, [n_seqs][n_kv][window][d] local, as K) and the cache's own
    coordinate-major layout (beam_kv_convert_v). to_cache: v_token_major ->
    cache.v, else cache.v -> v_token_major. v_token_major: device tensor of the
    cache's element type (bfloat16, or uint8 FP8 codes) and that shape."""
    import torch
    rows = cache.page_size if cache.kind == GLOBAL else cfg.window
    shape = (cache.v.shape[0], cfg.n_kv_heads, rows, cfg.head_dim)
    _need(v_token_major, torch.bfloat16 if cache.dtype == KV_BF16 else torch.uint8, shape, "v_token_major")
    kc = cache.c()
    _check(lib().beam_kv_convert_v(ctypes.byref(cfg.c()), ctypes.byref(kc), _ptr(v_token_major),
                                   1 if to_cache else 0, _stream(stream)))
    return v_token_major


# ---------------------------------------------------------------- router

def _router_outputs(rc: RouterConfig, n_tok: int, device, idx, wts):
    import torch
    if idx is None:
        idx = torch.empty((n_tok, rc.top_k), dtype=torch.int32, device=device)
    if wts is None:
        wts = torch.empty((n_tok, rc.top_k), dtype=torch.float32, device=device)
    _need(idx, torch.int32, (n_tok, rc.top_k), "topk_idx")
    _need(wts, torch.float32, (n_tok, rc.top_k), "topk_w")
    return idx, wts


def router(rc: RouterConfig, x, w, bias=None, topk_idx=None, topk_w=None, stream=None):
    """Expert selection of one MoE layer: returns (topk_idx int32, topk_w float32),
    each [n_tok][top_k], best first (beam_router)."""
    import torch
    n_tok = x.shape[0]
    _need(x, torch.bfloat16, (n_tok, rc.hidden), "x")
    _need(w, torch.float32, (rc.n_experts, rc.hidden), "w")
    if bias is not None:
        _need(bias, torch.float32, (rc.n_experts,), "bias")
    topk_idx, topk_w = _router_outputs(rc, n_tok, x.device, topk_idx, topk_w)
    c = rc.c()
    _check(lib().beam_router(ctypes.byref(c), _ptr(x), _ptr(w), _ptr(bias), n_tok, _ptr(topk_idx), _ptr(topk_w),
                             _stream(stream)))
    return topk_idx, topk_w


def router_logits(rc: RouterConfig, x, w, out=None, stream=None):
    """fp32 router logits [n_tok][n_experts] = x W^T (beam_router_logits)."""
    import torch
    n_tok = x.shape[0]
    _need(x, torch.bfloat16, (n_tok, rc.hidden), "x")
    _need(w, torch.float32, (rc.n_experts, rc.hidden), "w")
    if out is None:
        out = torch.empty((n_tok, rc.n_experts), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (n_tok, rc.n_experts), "logits")
    c = rc.c()
    _check(lib().beam_router_logits(ctypes.byref(c), _ptr(x), _ptr(w), n_tok, _ptr(out), _stream(stream)))
    return out


def router_select(rc: RouterConfig, logits, bias=None, topk_idx=None, topk_w=None, stream=None):
    """Selection from fp32 logits [n_tok][n_experts] (beam_router_select)."""
    import torch
    n_tok = logits.shape[0]
    _need(logits, torch.float32, (n_tok, rc.n_experts), "logits")
    if bias is not None:
        _need(bias, torch.float32, (rc.n_experts,), "bias")
    topk_idx, topk_w = _router_outputs(rc, n_tok, logits.device, topk_idx, topk_w)
    c = rc.c()
    _check(lib().beam_router_select(ctypes.byref(c), _ptr(logits), _ptr(bias), n_tok, _ptr(topk_idx), _ptr(topk_w),
                                    _stream(stream)))
    return topk_idx, topk_w


def attn_project(cfg: Config, kind: int, x, w_qkvg, q_norm_w, cu_seqlens, start_pos, workspace=None, k_raw=None,
                 v_raw=None, gate=None, stream=None):
    """QKV/gate projection of a prefill chunk with the query prologue fused
    (beam_attn_project). x: bf16 [n_tok][hidden]; w_qkvg: bf16
    [(2H + 2G) d][hidden] (Wq, Wk, Wv, Wg rows). Writes Q' into the prefill
    workspace and returns (k_raw, v_raw, gate, workspace); run prefill(...,
    q_raw=None, workspace=workspace, stages=STAGE_PROLOGUE_KV | ...) next."""
    import torch
    n_tok, hidden = x.shape
    n_seqs = cu_seqlens.shape[0] - 1
    H, G, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    _need(x, torch.bfloat16, (n_tok, hidden), "x")
    _need(w_qkvg, torch.bfloat16, ((2 * H + 2 * G) * d, hidden), "w_qkvg")
    _need(q_norm_w, torch.bfloat16, (d,), "q_norm_w")
    _need(cu_seqlens, torch.int32, (n_seqs + 1,), "cu_seqlens")
    _need(start_pos, torch.int32, (n_seqs,), "start_pos")
    dev = x.device
    k_raw = torch.empty((n_tok, G, d), dtype=torch.bfloat16, device=dev) if k_raw is None else k_raw
    v_raw = torch.empty((n_tok, G, d), dtype=torch.bfloat16, device=dev) if v_raw is None else v_raw
    gate = torch.empty((n_tok, H, d), dtype=torch.bfloat16, device=dev) if gate is None else gate
    _need(k_raw, torch.bfloat16, (n_tok, G, d), "k_raw")
    _need(v_raw, torch.bfloat16, (n_tok, G, d), "v_raw")
    _need(gate, torch.bfloat16, (n_tok, H, d), "gate")
    workspace = _workspace(prefill_workspace_bytes(cfg, n_tok, n_seqs), dev, workspace)
    c = cfg.c()
    _check(lib().beam_attn_project(ctypes.byref(c), kind, _ptr(x), hidden, _ptr(w_qkvg), _ptr(q_norm_w),
                                   _ptr(cu_seqlens), _ptr(start_pos), n_seqs, n_tok, _ptr(k_raw), _ptr(v_raw),
                                   _ptr(gate), _ptr(workspace), workspace.numel(), _stream(stream)))
    return k_raw, v_raw, gate, workspace


def out_project(y, w_o, out=None, stream=None):
    """out [n_tok][out_features] = y W_o^T in bf16 (beam_out_project); y may be
    [n_tok][H][d] or [n_tok][in_features]."""
    import torch
    n_tok = y.shape[0]
    y2 = y.reshape(n_tok, -1)
    out_f, in_f = w_o.shape
    _need(y2, torch.bfloat16, (n_tok, in_f), "y")
    _need(w_o, torch.bfloat16, (out_f, in_f), "w_o")
    if out is None:
        out = torch.empty((n_tok, out_f), dtype=torch.bfloat16, device=y.device)
    _need(out, torch.bfloat16, (n_tok, out_f), "out")
    _check(lib().beam_out_project(_ptr(y2), _ptr(w_o), n_tok, in_f, out_f, _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- measurement instruments

def probe_mfma_bf16(operands, n_blocks: int, iters: int, distinct: int = 8, out=None, stream=None):
    """Register-only bf16 MFMA loop (beam_probe_mfma_bf16); operands: int32
    device tensor [n_blocks * 256 * 64] of bf16 pairs. Returns the flops it ran."""
    import torch
    _need(operands, torch.int32, (n_blocks * 256 * 64,), "operands")
    if out is None:
        out = torch.empty((n_blocks * 256,), dtype=torch.float32, device=operands.device)
    _check(lib().beam_probe_mfma_bf16(_ptr(operands), n_blocks, iters, distinct, _ptr(out), _stream(stream)))
    return n_blocks * 4 * iters * 16 * 32768


def probe_mfma16_bf16(operands, n_blocks: int, iters: int, distinct: int = 8, out=None, stream=None):
    """The same loop with the 16x16x32 bf16 MFMA (beam_probe_mfma16_bf16); the
    same work, returned as flops."""
    import torch
    _need(operands, torch.int32, (n_blocks * 256 * 64,), "operands")
    if out is None:
        out = torch.empty((n_blocks * 256,), dtype=torch.float32, device=operands.device)
    _check(lib().beam_probe_mfma16_bf16(_ptr(operands), n_blocks, iters, distinct, _ptr(out), _stream(stream)))
    return n_blocks * 4 * iters * 32 * 16384


def probe_stream_read(buf, n_blocks: int, out=None, stream=None):
    """Streaming read of a device tensor (beam_probe_stream_read); returns the bytes read."""
    import torch
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty((n_blocks * 256,), dtype=torch.int32, device=buf.device)
    _check(lib().beam_probe_stream_read(_ptr(buf), nbytes, n_blocks, _ptr(out), _stream(stream)))
    return nbytes
