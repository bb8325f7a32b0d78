#!/usr/bin/env python3
"""Benchmark of the Beam 1.0 hybrid-attention hot path on one MI355X.

Step (the timed unit): causal prefill of T = 32,768 tokens (B = 1) through one
local layer (RoPE, window 512) and one global layer (SSMax), 48 query / 8 KV
heads, head_dim 128: for each layer the prologue (QK RMSNorm + RoPE/SSMax),
attention with the fused sigmoid gate, and the append of the chunk into the
layer's cache. `value` is the algorithmic attention TFLOP/s of the whole step
(4*d*H flops per visible (query, key) pair, both layers).

Also measured in the same run (reported under "decode"): batched decode of 64
sequences at positions uniform in [65536, 131071] over a paged bf16 cache
(16-token pages, random page permutation), global and local layer; value in
GB/s of KV read (4,096 B per cached key per layer). And under "verify": the
verify step of speculative decoding on the same caches, a draft block of 8
tokens per sequence ending at the decode position, in GB/s of cached KV read.
And under "decode_1m": one sequence at position 1,048,575 (4 GiB of cache).
And under "projection" / "sublayer": the QKV/gate projection (query prologue
fused) and W_o around the same two layers, alone and end to end with the
attention, in TFLOP/s against the bf16 MFMA peak.
And under "router": the MoE router of one layer over the same 32,768 tokens
(fp32 logits GEMM with the group-limited top-8 selection fused), in TFLOP/s
against the fp32 MFMA peak.
And under "schedule52": the full 52-layer attention schedule (9 global, 43
local layers) as a chunked prefill of 8 sequences of 4K-64K tokens in
8192-token chunks, aggregate TFLOP/s, with the oracle timed on sampled rows.
And under "measured_ceilings": the bf16 MFMA rates this GPU sustains on
constant and random operands with the 32x32x16 and the 16x16x32 instruction,
and its streaming HBM read rate (include/beam_probe.h); every roofline object
also gives its fraction of the highest measured MFMA rate or of the read rate.

Prints ONE JSON line on stdout. Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s @32K; decode KV GB/s @128K ctx (% of MI355X peak)"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 bf16 flop/clk x 2.4 GHz (AMD: 2.5 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0       # HBM3E, 8 TB/s
PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 matrix (v_mfma_f32_*f32), AMD's figure
H, G, D, W = 48, 8, 128, 512
FLOP_PER_PAIR = 4 * D * H   # QK^T and PV over all query heads of one (query, key) pair


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_CSRC = os.path.join(ROOT, "global_attention_amd", "csrc")
_KERNEL_SOURCES = {
    "prefill_attn_kernel<1, 8, 0, 1>": "prefill.hip",
    "prefill_attn_kernel<0, 4, 0, 2>": "prefill.hip",
    "decode_split_kernel<1>": "decode.hip",
    "decode_split_kernel<1> (1M)": "decode.hip",
    "decode_split_kernel<0>": "decode.hip",
    "decode_fp8_kernel<1>": "decode.hip",
    "verify_attn_kernel<1, 0, 4>": "prefill.hip",
    "verify_attn_kernel<0, 0, 4>": "prefill.hip",
    "verify48_fp8_kernel<1, 2>": "prefill.hip",
    "router_gemm_kernel<true>": "router.hip",
    "gemm_bf16_kernel<1>": "gemm.hip",
    "gemm_bf16_kernel<0>": "gemm.hip",
    "prefill_prologue_kernel<0, 0>": "prologue.hip",
    "prefill_prologue_kernel<1, 0>": "prologue.hip",
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in (_KERNEL_SOURCES[kernel], "beam_device.h", "beam_kernels.h"):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_pmc.md")
    if not os.path.exists(path):
        return None
    digest = source_digest(kernel)
    with open(path) as fh:
        for line in fh:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) == 6 and cells[0] == kernel and cells[1] == digest:
                return int(cells[4])
    return None


def pairs_global(T: int) -> int:
    return T * (T + 1) // 2


def pairs_local(T: int, w: int = W) -> int:
    if T <= w:
        return T * (T + 1) // 2
    return w * (w + 1) // 2 + (T - w) * w


def _dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _r4(x):
    return None if x is None else round(x, 4)


def _i32(x):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


# --------------------------------------------------------------------------- prefill

def setup_prefill(T: int):
    import torch
    import global_attention_amd as ga
    import synth
    cfg = ga.Config()
    layers = []
    for kind in (ga.LOCAL, ga.GLOBAL):
        log(f"[bench] generating prefill inputs kind={kind} T={T}")
        inp = synth.attention_inputs(cfg=2, layer=kind, n_tok=T)
        d = {k: _dev(v) for k, v in inp.items()}
        if kind == ga.GLOBAL:
            bt, n_pages = synth.paged_block_table(2, [T])
            cache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt))
        else:
            cache = ga.KVCache.allocate_local(cfg, 1)
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ga.prefill_workspace_bytes(cfg, T, 1), dtype=torch.uint8, device="cuda")
        layers.append(dict(kind=kind, inp=inp, d=d, cache=cache, out=out, ws=ws))
    meta = dict(cu=_i32([0, T]), seq=_i32([0]), start=_i32([0]))
    return cfg, layers, meta


def prefill_step(cfg, layers, meta, T, events=None):
    import global_attention_amd as ga
    for i, L in enumerate(layers):
        d = L["d"]
        args = (cfg, L["cache"], d["q"], d["k"], d["v"], d["q_norm_w"], d["k_norm_w"], d["gate"], meta["cu"],
                meta["seq"], meta["start"], T)
        # Global layers: the append is fused into the prologue (paged slots of
        # new positions never alias the prefix). Local: append after attention.
        fused = L["kind"] == ga.GLOBAL
        first = ga.STAGE_PROLOGUE | (ga.STAGE_APPEND if fused else 0)
        ga.prefill(*args, out=L["out"], workspace=L["ws"], stages=first)
        if events is not None:
            events[i][0].record()
        ga.prefill(*args, out=L["out"], workspace=L["ws"], stages=ga.STAGE_ATTENTION)
        if events is not None:
            events[i][1].record()
        if not fused:
            ga.prefill(*args, out=L["out"], workspace=L["ws"], stages=ga.STAGE_APPEND)


def bench_prefill(T, steps, warmup):
    import torch
    cfg, layers, meta = setup_prefill(T)
    for _ in range(warmup):
        prefill_step(cfg, layers, meta, T)
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in layers] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        prefill_step(cfg, layers, meta, T, evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = [sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps)) / steps
               for i in range(len(layers))]
    return dict(cfg=cfg, layers=layers, ms_per_step=elapsed * 1e3 / steps, attn_ms=attn_ms)


# --------------------------------------------------------------------------- decode

def setup_decode(n_seqs=64, lo=65536, hi=131071, seed=3):
    import numpy as np
    import torch
    import global_attention_amd as ga
    import synth
    cfg = ga.Config()
    ts = synth.decode_positions(seed, n_seqs, lo, hi)
    ctx = ts.astype(np.int64) + 1
    bt, n_pages = synth.paged_block_table(seed, ctx)
    log(f"[bench] decode cache: {n_seqs} seqs, {n_pages} pages ({n_pages * 65536 / 1e9:.1f} GB K+V)")
    gcache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt))
    lcache = ga.KVCache.allocate_local(cfg, n_seqs)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    step = 8192
    for t in (gcache.k, gcache.v):
        for p0 in range(0, n_pages, step):
            t[p0:p0 + step].normal_(generator=gen)
    for t in (lcache.k, lcache.v):
        t.normal_(generator=gen)
    # The same global layer over an FP8 E4M3 cache (scales 1): N(0,1) values
    # rounded to E4M3 by torch are its (input) contents.
    fcache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt), dtype=ga.KV_FP8_E4M3)
    for t in (fcache.k, fcache.v):
        for p0 in range(0, n_pages, step):
            blk = t[p0:p0 + step]
            blk.copy_(torch.randn(blk.shape, generator=gen, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8))
    inp = synth.attention_inputs(cfg=seed, layer=7, n_tok=n_seqs)
    d = {k: _dev(v) for k, v in inp.items()}
    torch.cuda.synchronize()
    return cfg, ts, gcache, lcache, fcache, d


def graph_ms_per_call(call, out, calls=20, reps=5):
    """Device time of one whole library call without the host's launch cost:
    `calls` back-to-back calls captured in one HIP graph (torch.cuda.CUDAGraph;
    the library enqueues kernels only, no memset or copy), replayed `reps`
    times with eager work and a synchronisation between replays. Every
    replay's output must equal the eager call's bit for bit, else None."""
    import numpy as np
    import torch
    try:
        call()
        torch.cuda.synchronize()
        want = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                call()
        ts = []
        for _ in range(reps):
            out.zero_()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            if not torch.equal(out.view(torch.int16), want.view(torch.int16)):
                log("[bench] graph replay differs from the eager call; device time not reported")
                return None
            ts.append(e0.elapsed_time(e1) / calls)
        del g
        return float(np.median(ts))
    except Exception as e:  # capture unsupported here: report no figure
        log(f"[bench] graph timing unavailable: {e}")
        return None


def bench_decode(steps, warmup):
    import torch
    import global_attention_amd as ga
    setup = setup_decode()
    cfg, ts, gcache, lcache, fcache, d = setup
    n = len(ts)
    seq = _i32(list(range(n)))
    pos = _i32(ts)
    max_pos = int(ts.max())
    res = {}
    for name, cache in (("global", gcache), ("local", lcache), ("global_fp8", fcache)):
        out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ga.decode_workspace_bytes(cfg, cache.kind, n, max_pos), dtype=torch.uint8, device="cuda")
        args = (cfg, cache, d["q"], d["q_norm_w"], d["gate"], seq, pos, max_pos)

        def one(ev=None):
            ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_PROLOGUE)
            if ev is not None:
                ev[0].record()
            ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_ATTENTION)
            if ev is not None:
                ev[1].record()
            ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_COMBINE)

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            one(evs[s])
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / steps
        split_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        keys = [min(int(t) + 1, W) if name == "local" else int(t) + 1 for t in ts]
        nbytes = sum(keys) * G * D * 2 * (1 if cache.dtype == ga.KV_FP8_E4M3 else 2)
        dev_ms = graph_ms_per_call(lambda: ga.decode(*args, out=out, workspace=ws), out)
        res[name] = dict(bytes=nbytes, ms_per_call=el * 1e3, split_ms=split_ms, device_ms=dev_ms,
                         gbs_call=nbytes / el / 1e9, gbs_split=nbytes / (split_ms / 1e3) / 1e9)
        log(f"[bench] decode {name}: {nbytes / 1e9:.2f} GB, call {el * 1e3:.3f} ms, split kernel {split_ms:.3f} ms, "
            f"device time per call {dev_ms} ms")
    res["setup"] = setup
    return res


def bench_decode_1m(steps, warmup, cpu_sample=False):
    """One sequence at t = 1,048,575 on a global layer: 65,536 pages (4 GiB of
    bf16 K+V, far beyond the 256 MB MALL) dealt by a random permutation; the
    split-key decode with its prologue and combine, timed as in bench_decode."""
    import torch
    import global_attention_amd as ga
    import synth
    cfg = ga.Config()
    T = 1 << 20
    bt, n_pages = synth.paged_block_table(4, [T])
    cache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    for t in (cache.k, cache.v):
        for p0 in range(0, n_pages, 8192):
            t[p0:p0 + 8192].normal_(generator=gen)
    inp = synth.attention_inputs(cfg=4, layer=9, n_tok=1)
    d = {k: _dev(v) for k, v in inp.items()}
    seq, pos, max_pos = _i32([0]), _i32([T - 1]), T - 1
    out = torch.empty((1, H, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ga.decode_workspace_bytes(cfg, ga.GLOBAL, 1, max_pos), dtype=torch.uint8, device="cuda")
    args = (cfg, cache, d["q"], d["q_norm_w"], d["gate"], seq, pos, max_pos)

    def staged(ev):
        ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_PROLOGUE)
        ev[0].record()
        ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_ATTENTION)
        ev[1].record()
        ga.decode(*args, out=out, workspace=ws, stages=ga.STAGE_COMBINE)

    warmup, steps = max(warmup, 5), max(steps, 50)
    for _ in range(warmup):
        ga.decode(*args, out=out, workspace=ws)
    torch.cuda.synchronize()
    # whole calls, back to back (the GPU never waits for the host): GPU time per call
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ga.decode(*args, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / steps
    # the split kernel alone, bracketed by events on the library's stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for s_ in range(steps):
        staged(evs[s_])
    torch.cuda.synchronize()
    split_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    nbytes = T * G * D * 2 * 2
    log(f"[bench] decode 1M: {nbytes / 2 ** 30:.0f} GiB, call {call_ms:.3f} ms, split kernel {split_ms:.3f} ms")
    res = dict(bytes=nbytes, ms_per_call=call_ms, split_ms=split_ms, gbs_call=nbytes / (call_ms / 1e3) / 1e9,
               gbs_split=nbytes / (split_ms / 1e3) / 1e9)
    if cpu_sample:
        log("[bench] timing the CPU oracle on the 1M decode, KV head 0")
        res["cpu_sample"] = cpu_decode_sample(cache, T - 1, inp, 0, [0],
                                              "the 1M-token sequence (t = 1,048,575), KV head 0 and its 6 query heads")
    del cache
    return res


def bench_verify(steps, warmup, dres, block=8, split_keys=0):
    """Verify of `block` tokens per sequence (positions ts-block+1 .. ts) over the
    decode caches: prologue, split attention (timed with events), combine, append."""
    import numpy as np
    import torch
    import global_attention_amd as ga
    import synth
    cfg, ts, gcache, lcache, fcache, _ = dres["setup"]
    n = len(ts)
    starts = (ts - (block - 1)).astype(np.int32)
    inp = synth.attention_inputs(cfg=3, layer=9, n_tok=n * block)
    d = {k: _dev(v) for k, v in inp.items()}
    cu = _i32(np.arange(n + 1) * block)
    seq = _i32(list(range(n)))
    st = _i32(starts)
    max_pos = int(ts.max())
    res = {}
    for name, cache in (("global", gcache), ("local", lcache), ("global_fp8", fcache)):
        out = torch.empty((n * block, H, D), dtype=torch.bfloat16, device="cuda")
        nb = ga.verify_workspace_bytes(cfg, cache.kind, n * block, n, block, max_pos, split_keys)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        args = (cfg, cache, d["q"], d["k"], d["v"], d["q_norm_w"], d["k_norm_w"], d["gate"], cu, seq, st, block,
                max_pos)
        kw = dict(split_keys=split_keys, out=out, workspace=ws)
        # global caches: the prologue also appends (one launch); local: append last
        pro = ga.STAGE_PROLOGUE | (ga.STAGE_APPEND if cache.kind == ga.GLOBAL else 0)
        tail = ga.STAGE_VERIFY_COMBINE | (ga.STAGE_APPEND if cache.kind == ga.LOCAL else 0)

        def one(ev=None):
            ga.verify(*args, **kw, stages=pro)
            if ev is not None:
                ev[0].record()
            ga.verify(*args, **kw, stages=ga.STAGE_ATTENTION)
            if ev is not None:
                ev[1].record()
            ga.verify(*args, **kw, stages=tail)

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            one(evs[s])
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / steps
        split_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        # cached keys each chunk reads once (the chunk's own keys come from the workspace)
        keys = [min(int(s), W - 1) if name == "local" else int(s) for s in starts]
        nbytes = sum(keys) * G * D * 2 * (1 if cache.dtype == ga.KV_FP8_E4M3 else 2)
        dev_ms = graph_ms_per_call(lambda: ga.verify(*args, **kw), out)
        res[name] = dict(bytes=nbytes, ms_per_call=el * 1e3, split_ms=split_ms, device_ms=dev_ms,
                         gbs_call=nbytes / el / 1e9, gbs_split=nbytes / (split_ms / 1e3) / 1e9,
                         vs_decode_calls=block * dres[name]["ms_per_call"] / (el * 1e3))
        log(f"[bench] verify {name} ({block} tokens/seq): {nbytes / 1e9:.2f} GB, call {el * 1e3:.3f} ms, "
            f"split kernel {split_ms:.3f} ms, {res[name]['vs_decode_calls']:.2f}x {block} decode calls")
    return res


def bench_router(T, steps, warmup):
    """The MoE router of one layer over T tokens: fp32 logits (hidden 5120 x 256
    experts) with the group-limited top-8 selection fused, timed with events."""
    import torch
    import global_attention_amd as ga
    import synth
    rc = ga.RouterConfig()
    inp = synth.router_inputs(40, 0, T)
    x = _dev(inp["x"]).view(T, rc.hidden)
    w = torch.from_numpy(inp["w"]).cuda()
    b = torch.from_numpy(inp["bias"]).cuda()
    idx = torch.empty((T, rc.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, rc.top_k), dtype=torch.float32, device="cuda")
    # a call lasts ~0.7 ms: warm up and time at least 20 (the clock settles
    # over the first few dozen calls)
    warmup, steps = max(warmup, 20), max(steps, 20)
    for _ in range(warmup):
        ga.router(rc, x, w, b, topk_idx=idx, topk_w=wts)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        ga.router(rc, x, w, b, topk_idx=idx, topk_w=wts)
        e[1].record()
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    flops = 2.0 * T * rc.n_experts * rc.hidden
    log(f"[bench] router T={T}: {ms:.3f} ms, {flops / (ms / 1e3) / 1e12:.1f} TFLOP/s (fp32 MFMA)")
    return dict(ms=ms, flops=flops)


# --------------------------------------------------------------------------- projections

HIDDEN = 5120
N_QKVG = (2 * H + 2 * G) * D   # stacked Wq/Wk/Wv/Wg rows


def setup_projection(T):
    import torch
    import synth
    log(f"[bench] generating projection inputs T={T} hidden={HIDDEN}")
    inp = synth.projection_inputs(41, 0, T, hidden=HIDDEN)
    d = {k: _dev(v) for k, v in inp.items()}
    d["x"] = d["x"].view(T, HIDDEN)
    d["w_qkvg"] = d["w_qkvg"].view(N_QKVG, HIDDEN)
    d["w_o"] = d["w_o"].view(HIDDEN, H * D)
    d["k_raw"] = torch.empty((T, G, D), dtype=torch.bfloat16, device="cuda")
    d["v_raw"] = torch.empty((T, G, D), dtype=torch.bfloat16, device="cuda")
    d["gate"] = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    d["out"] = torch.empty((T, HIDDEN), dtype=torch.bfloat16, device="cuda")
    return d


def proj_flops(T):
    return 2.0 * T * HIDDEN * N_QKVG, 2.0 * T * (H * D) * HIDDEN


def bench_projection(T, steps, warmup, pd, ws, meta):
    """The QKV/gate projection with the fused query prologue (both layer kinds)
    and W_o, each timed alone with events, at least 20 launches."""
    import torch
    import global_attention_amd as ga
    cfg = ga.Config()
    warmup, steps = max(warmup, 5), max(steps, 20)
    calls = {
        "qkvg_global": lambda: ga.attn_project(cfg, ga.GLOBAL, pd["x"], pd["w_qkvg"], pd["q_norm_w"], meta["cu"],
                                               meta["start"], workspace=ws, k_raw=pd["k_raw"], v_raw=pd["v_raw"],
                                               gate=pd["gate"]),
        "qkvg_local": lambda: ga.attn_project(cfg, ga.LOCAL, pd["x"], pd["w_qkvg"], pd["q_norm_w"], meta["cu"],
                                              meta["start"], workspace=ws, k_raw=pd["k_raw"], v_raw=pd["v_raw"],
                                              gate=pd["gate"]),
        "w_o": lambda: ga.out_project(pd["gate"].view(T, H * D), pd["w_o"], out=pd["out"]),
    }
    res = {}
    for name, f in calls.items():
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in evs:
            e[0].record()
            f()
            e[1].record()
        torch.cuda.synchronize()
        res[name] = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    fq, fo = proj_flops(T)
    log(f"[bench] projections T={T}: QKV/gate {res['qkvg_global']:.3f} ms ({fq / res['qkvg_global'] / 1e9:.1f} "
        f"TFLOP/s), W_o {res['w_o']:.3f} ms ({fo / res['w_o'] / 1e9:.1f} TFLOP/s)")
    return res


def sublayer_step(cfg, layers, meta, pd, T):
    """Both layers end to end: x -> QKV/gate projection (query prologue fused)
    -> prefill without the query prologue -> W_o."""
    import global_attention_amd as ga
    for L in layers:
        ga.attn_project(cfg, L["kind"], pd["x"], pd["w_qkvg"], pd["q_norm_w"], meta["cu"], meta["start"],
                        workspace=L["ws"], k_raw=pd["k_raw"], v_raw=pd["v_raw"], gate=pd["gate"])
        args = (cfg, L["cache"], None, pd["k_raw"], pd["v_raw"], pd["q_norm_w"], pd["k_norm_w"], pd["gate"],
                meta["cu"], meta["seq"], meta["start"], T)
        if L["kind"] == ga.GLOBAL:
            ga.prefill(*args, out=L["out"], workspace=L["ws"],
                       stages=ga.STAGE_PROLOGUE_KV | ga.STAGE_APPEND | ga.STAGE_ATTENTION)
        else:
            ga.prefill(*args, out=L["out"], workspace=L["ws"], stages=ga.STAGE_PROLOGUE_KV | ga.STAGE_ATTENTION)
            ga.prefill(*args, out=L["out"], workspace=L["ws"], stages=ga.STAGE_APPEND)
        ga.out_project(L["out"].view(T, H * D), pd["w_o"], out=pd["out"])


def bench_sublayer(T, steps, warmup, layers, meta, pd):
    import torch
    import global_attention_amd as ga
    cfg = ga.Config()
    for _ in range(warmup):
        sublayer_step(cfg, layers, meta, pd, T)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sublayer_step(cfg, layers, meta, pd, T)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fq, fo = proj_flops(T)
    flops = 2 * (fq + fo) + FLOP_PER_PAIR * (pairs_global(T) + pairs_local(T))
    log(f"[bench] sublayer pair (projections + attention) T={T}: {ms:.3f} ms, {flops / ms / 1e9:.1f} TFLOP/s")
    return dict(ms=ms, flops=flops)


# --------------------------------------------------------------------------- CPU oracle

def cpu_baseline(layers, T, rows):
    """Time the float64 oracle on the last `rows` query rows of both layers."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    t0 = time.perf_counter()
    flops = 0
    for L in layers:
        inp = L["inp"]
        qs = np.arange(T - rows, T)
        O.attention_layer(L["kind"], inp["q"][qs], inp["k"], inp["v"], inp["q_norm_w"], inp["k_norm_w"],
                          inp["gate"][qs], qs, np.arange(T))
        vis = (qs + 1) if L["kind"] == O.GLOBAL else np.minimum(qs + 1, W)
        flops += FLOP_PER_PAIR * int(vis.sum())
    el = time.perf_counter() - t0
    facts = cpu_facts()
    return dict(value=flops / el / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                host_cpu_count=facts["cpu_count"], host_affinity=facts["affinity"], blas_threads=facts["blas_threads"],
                workers=1,
                sample=f"float64 NumPy oracle on the last {rows} query rows (all 48 heads) of the T=32768 "
                       f"local and global layers, full key history, incl. K normalisation; "
                       f"{flops / 1e9:.1f} GFLOP in {el:.1f} s")


def cpu_decode_sample(cache, t, inp, sq, heads_kv, what):
    """Time the float64 oracle for one decode row (sequence sq at position t,
    global layer) over its cached history, KV heads `heads_kv` and their
    query heads: q normalisation and SSMax scale, exact softmax over all t+1
    keys, PV, gate. The cache contents are gathered to the host first
    (untimed); the bf16-to-float64 widening of K/V is timed, as in the prefill
    sample. Rate: bytes of bf16 K+V the oracle processed per second."""
    import numpy as np
    import torch
    import oracle as O
    n_keys = t + 1
    n_pg = (n_keys + 15) // 16
    bt_row = cache.block_table[sq].cpu().numpy()
    idx = torch.from_numpy(np.ascontiguousarray(bt_row[:n_pg]).astype(np.int64)).cuda()
    hs = torch.tensor(heads_kv, device="cuda")
    k = cache.k.index_select(0, idx).index_select(1, hs).permute(0, 2, 1, 3).reshape(n_pg * 16, len(heads_kv), D)
    v = cache.v.index_select(0, idx).index_select(1, hs).permute(0, 3, 1, 2).reshape(n_pg * 16, len(heads_kv), D)
    kb = k[:n_keys].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    vb = v[:n_keys].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    del k, v
    hpg = H // G
    ocfg = O.Config()
    t0 = time.perf_counter()
    qn = O.rms_norm(O.bf16_to_f64(inp["q"][sq])[None], O.bf16_to_f64(inp["q_norm_w"]), ocfg.rms_eps)
    qp, _ = O.position_op(O.GLOBAL, qn, qn, np.array([t]), np.array([t]), ocfg)
    key_pos = np.arange(n_keys)
    for i, g in enumerate(heads_kv):
        hq = list(range(hpg * g, hpg * g + hpg))
        o = O.attend(O.GLOBAL, qp[:, hq], O.bf16_to_f64(kb[:, i:i + 1]), O.bf16_to_f64(vb[:, i:i + 1]),
                     np.array([t]), key_pos, O.Config(n_q_heads=hpg, n_kv_heads=1))
        O.output_gate(o, O.bf16_to_f64(inp["gate"][sq])[None][:, hq])
    el = time.perf_counter() - t0
    nbytes = n_keys * len(heads_kv) * D * 2 * 2
    facts = cpu_facts()
    return dict(value=round(nbytes / el / 1e9, 3), unit="GB/s", seconds=round(el, 2), kind="oracle",
                cores=facts["blas_threads"], host_cpu_count=facts["cpu_count"], host_affinity=facts["affinity"],
                blas_threads=facts["blas_threads"], workers=1,
                sample=f"float64 NumPy oracle, {what}: {n_keys} keys x {len(heads_kv)} KV head(s) "
                       f"({nbytes / 1e9:.2f} GB of bf16 K+V) in {el:.1f} s")


def cpu_facts():
    """Host cores the oracle can use, and the BLAS threads it does use."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return dict(cpu_count=os.cpu_count(), affinity=affinity, blas_threads=int(blas))


# --------------------------------------------------------------------------- ceilings

def _probe_mfma(ops, n_blocks, iters, distinct, reps, shape=32):
    """Median TFLOP/s of `reps` runs of the MFMA probe (shape 32: the 32x32x16
    loop, 16: the 16x16x32 loop), after one untimed run of the same length."""
    import statistics
    import torch
    import global_attention_amd as ga
    probe = ga.probe_mfma_bf16 if shape == 32 else ga.probe_mfma16_bf16
    out = torch.empty((n_blocks * 256,), dtype=torch.float32, device="cuda")
    probe(ops[:n_blocks * 256 * 64], n_blocks, iters, distinct, out)
    rates = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = probe(ops[:n_blocks * 256 * 64], n_blocks, iters, distinct, out)
        e1.record()
        torch.cuda.synchronize()
        rates.append(flops / (e0.elapsed_time(e1) / 1e3) / 1e12)
    return statistics.median(rates), e0.elapsed_time(e1)


def measure_ceilings(reps=3, sweep=False):
    """What this GPU sustains, measured with the library's probes
    (include/beam_probe.h): bf16 MFMA on N(0,1) operands that change on every
    MFMA, in a register-only loop run for about 5 ms (the chip boosts for a
    fraction of a millisecond, then settles at its power limit); and a
    streaming HBM read of 8 GiB (best of four grid sizes). With sweep=True
    also the boosted short run, and operands repeated or constant."""
    import torch
    import global_attention_amd as ga
    nb_max = 1024
    rnd = torch.randn((nb_max * 256 * 128,), device="cuda").to(torch.bfloat16).view(torch.int32)
    one = torch.ones((nb_max * 256 * 128,), device="cuda").to(torch.bfloat16).view(torch.int32)
    # the matrix pipe's own sustained ceiling (operands that never switch), and
    # the rate on N(0,1) operands that change on every MFMA
    mfma, ms = _probe_mfma(one, 1024, 3000, 1, reps)
    mfma_rnd, _ = _probe_mfma(rnd, 1024, 3000, 8, reps)
    # the same loop with the 16x16x32 instruction, which the chip sustains at a
    # higher rate under the same power limit
    mfma16, _ = _probe_mfma(one, 1024, 3000, 1, reps, shape=16)
    mfma16_rnd, _ = _probe_mfma(rnd, 1024, 3000, 8, reps, shape=16)
    res = dict(mfma_bf16_tflops=round(mfma, 1), mfma_bf16_random_tflops=round(mfma_rnd, 1),
               mfma_bf16_16x16_tflops=round(mfma16, 1), mfma_bf16_16x16_random_tflops=round(mfma16_rnd, 1),
               mfma_measured_peak_tflops=round(max(mfma, mfma_rnd, mfma16, mfma16_rnd), 1))
    if sweep:
        rows = []
        for shape in (32, 16):
            for name, ops in (("random N(0,1)", rnd), ("constant 1.0", one)):
                for distinct in (8, 1):
                    for nb, iters in ((512, 400), (1024, 3000)):
                        r, t = _probe_mfma(ops, nb, iters, distinct, reps, shape=shape)
                        rows.append(dict(mfma=f"{shape}x{shape}", operands=name, distinct=distinct, blocks=nb,
                                         iters=iters, ms=round(t, 3), tflops=round(r, 1)))
                        log(f"[bench] mfma probe {shape}x{shape} {name}, {distinct} distinct, {nb} x {iters}: "
                            f"{t:.3f} ms, {r:.1f} TFLOP/s")
        res["mfma_sweep"] = rows
    del rnd, one
    buf = torch.empty((8 << 30,), dtype=torch.uint8, device="cuda")
    rout = torch.empty((16384 * 256,), dtype=torch.int32, device="cuda")
    best_read, best_grid = 0.0, 0
    for nb in (1024, 2048, 4096, 8192):
        ga.probe_stream_read(buf, nb, rout[:nb * 256])
        torch.cuda.synchronize()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            nbytes = ga.probe_stream_read(buf, nb, rout[:nb * 256])
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
            if gbs > best_read:
                best_read, best_grid = gbs, nb
    del buf, rout
    torch.cuda.empty_cache()
    log(f"[bench] ceilings: bf16 MFMA sustained, 32x32x16: {mfma:.1f} TFLOP/s (constant operands), {mfma_rnd:.1f} "
        f"TFLOP/s (N(0,1) operands changing every MFMA); 16x16x32: {mfma16:.1f} / {mfma16_rnd:.1f} TFLOP/s; "
        f"{ms:.1f} ms runs; streaming read {best_read:.1f} GB/s ({best_grid} blocks)")
    res.update(hbm_read_gbs=round(best_read, 1),
               method="beam_probe_mfma_bf16: 1024 blocks x 4 waves x 3000 iterations x 16 "
                      "v_mfma_f32_32x32x16_bf16 from registers, ~5 ms per run (past the boost), median of "
                      f"{reps} runs after one untimed run; mfma_bf16_tflops: constant 1.0 operands (no operand "
                      "switching), mfma_bf16_random_tflops: N(0,1) operands changing on every MFMA; "
                      "beam_probe_mfma16_bf16: the same work as 32 v_mfma_f32_16x16x32_bf16 per iteration "
                      "(mfma_bf16_16x16_*); mfma_measured_peak_tflops: the highest of the four, the ceiling "
                      "frac_of_measured_peak divides by; beam_probe_stream_read: "
                      f"8 GiB, 16-byte non-temporal loads, best of 4 grids x {reps}")
    return res


# --------------------------------------------------------------------------- 52-layer schedule

def bench_schedule52(reps=2, oracle_rows=32):
    """The full 52-layer attention schedule (global at 6, 12, ..., 48, 52, local
    elsewhere): chunked varlen prefill of 8 sequences with lengths U[4096,
    65536] in 8192-token chunks, each layer with its own cache (paged for
    global layers, 512-slot rings for local ones). Raw projections per
    (sequence, layer kind) come from torch's seeded device RNG and are reused
    by every layer of that kind; norm weights are per layer. Every chunk's
    batch is assembled before the timed region. Returns aggregate TFLOP/s
    over all layers and steps, and the oracle timed on sampled rows."""
    import numpy as np
    import torch
    import global_attention_amd as ga
    import oracle as O
    import synth
    cfg = ga.Config()
    CH = 8192
    lens = synth.chunked_lengths(5, 8, 4096, 65536)
    n = len(lens)
    kinds = O.layer_kinds(52)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    raw = {}
    for kind in (ga.LOCAL, ga.GLOBAL):
        for i in range(n):
            L = int(lens[i])
            raw[kind, i] = {key: torch.randn((L, hh, D), generator=gen, device="cuda").to(torch.bfloat16)
                            for key, hh in (("q", H), ("k", G), ("v", G), ("gate", H))}
    qw = [_dev(synth.normal_bf16((D,), 5, synth.T_QW, l, scale=0.1, offset=1.0)) for l in range(52)]
    kw = [_dev(synth.normal_bf16((D,), 5, synth.T_KW, l, scale=0.1, offset=1.0)) for l in range(52)]

    def fresh_caches():
        cs = []
        for l, kind in enumerate(kinds):
            if kind == ga.GLOBAL:
                bt, n_pages = synth.paged_block_table(1000 + l, lens)
                cs.append(ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt)))
            else:
                cs.append(ga.KVCache.allocate_local(cfg, n))
        return cs

    n_steps = int(-(-int(lens.max()) // CH))
    steps = []
    flops = 0
    for st in range(n_steps):
        s0 = st * CH
        seqs = [i for i in range(n) if lens[i] > s0]
        clen = [min(CH, int(lens[i]) - s0) for i in seqs]
        cu = np.concatenate([[0], np.cumsum(clen)]).astype(np.int32)
        batch = {kind: {key: torch.cat([raw[kind, i][key][s0:s0 + c] for i, c in zip(seqs, clen)])
                        for key in ("q", "k", "v", "gate")} for kind in (ga.LOCAL, ga.GLOBAL)}
        steps.append(dict(s0=s0, seqs=seqs, clen=clen, cu=cu, batch=batch, cu_d=_i32(cu), seq_d=_i32(seqs),
                          start_d=_i32([s0] * len(seqs)), n_tok=int(cu[-1])))
        for c in clen:
            t = np.arange(s0, s0 + c)
            flops += FLOP_PER_PAIR * (9 * int((t + 1).sum()) + 43 * int(np.minimum(t + 1, W).sum()))
    max_tok = n * CH
    ws = torch.empty(ga.prefill_workspace_bytes(cfg, max_tok, n), dtype=torch.uint8, device="cuda")
    out = torch.empty((max_tok, H, D), dtype=torch.bfloat16, device="cuda")
    keep = {}  # (layer, step) -> out rows of the longest sequence's last chunk
    longest = int(np.argmax(lens))

    def run(caches, record=False):
        for si, stp in enumerate(steps):
            for l, kind in enumerate(kinds):
                b = stp["batch"][kind]
                ga.prefill(cfg, caches[l], b["q"], b["k"], b["v"], qw[l], kw[l], b["gate"], stp["cu_d"],
                           stp["seq_d"], stp["start_d"], max(stp["clen"]), out=out[:stp["n_tok"]], workspace=ws)
                if record and si == len(steps) - 1 and l in (kinds.index(ga.LOCAL), kinds.index(ga.GLOBAL)):
                    j = stp["seqs"].index(longest)
                    keep[l] = out[int(stp["cu"][j]):int(stp["cu"][j + 1])].clone()

    ms = []
    for r in range(reps):
        caches = fresh_caches()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run(caches, record=(r == reps - 1))
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        del caches
    best = min(ms)
    log(f"[bench] 52-layer chunked prefill: {flops / 1e12:.1f} TFLOP in {best:.1f} ms = "
        f"{flops / best / 1e9:.1f} TFLOP/s (runs {', '.join(f'{m:.1f}' for m in ms)} ms)")
    # oracle on sampled rows of the longest sequence's last chunk, first local and first global layer
    from tests.helpers import Agreement  # comparison helper only; the oracle itself is oracle/
    stp = steps[-1]
    c = stp["clen"][stp["seqs"].index(longest)]
    rows = np.unique(np.linspace(0, c - 1, oracle_rows).astype(np.int64))
    pos = stp["s0"] + rows
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ofl, oel, agree = 0, 0.0, {}
    for l in sorted(keep):
        kind = kinds[l]
        rr = raw[kind, longest]
        last = int(pos.max()) + 1
        idx = torch.from_numpy(pos).cuda()
        args = (kind, bits(rr["q"][idx]), bits(rr["k"][:last]), bits(rr["v"][:last]), bits(qw[l]), bits(kw[l]),
                bits(rr["gate"][idx]), pos, np.arange(last))
        t0 = time.perf_counter()
        ref = O.attention_layer(*args)
        oel += time.perf_counter() - t0
        vis = (pos + 1) if kind == ga.GLOBAL else np.minimum(pos + 1, W)
        ofl += FLOP_PER_PAIR * int(vis.sum())
        a = Agreement(f"52-layer schedule layer {l + 1}, {len(rows)} rows")
        a.add(bits(keep[l])[rows], ref)
        import contextlib
        with contextlib.redirect_stdout(sys.stderr):  # stdout carries only the JSON line
            mx, rl2, _ = a.check()
        agree[f"layer_{l + 1}"] = dict(max_abs=float(f"{mx:.3e}"), rel_l2=float(f"{rl2:.3e}"))
    del raw, steps, out, ws
    torch.cuda.empty_cache()
    return dict(flops=flops, ms=best, ms_runs=[round(m, 2) for m in ms], lens=[int(x) for x in lens],
                oracle=dict(value=ofl / oel / 1e12, unit="TFLOP/s", seconds=round(oel, 2), **cpu_facts(),
                            sample=f"float64 oracle on {len(rows)} rows of the last chunk of the longest sequence, "
                                   f"first local and first global layer ({ofl / 1e9:.1f} GFLOP)",
                            parity=agree))


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE counters."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes")


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seq-len", type=int, default=32768)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--verify-split-keys", type=int, default=0)
    ap.add_argument("--skip-router", action="store_true")
    ap.add_argument("--skip-decode-1m", action="store_true",
                    help="leave out the 1M-token decode (it launches decode_split_kernel<1> at another size, which "
                         "would mix into that kernel's per-kernel profile averages)")
    ap.add_argument("--decode-1m-only", action="store_true",
                    help="of the decode lines run only the 1M-token decode (for its own counter runs)")
    ap.add_argument("--skip-projection", action="store_true")
    ap.add_argument("--skip-schedule", action="store_true", help="leave out the 52-layer chunked schedule")
    ap.add_argument("--skip-ceilings", action="store_true", help="leave out the measured MFMA / HBM ceilings")
    ap.add_argument("--ceilings-sweep", action="store_true",
                    help="only the ceilings, with the MFMA probe also boosted (short) and on repeated or constant "
                         "operands")
    ap.add_argument("--schedule-reps", type=int, default=2)
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=384)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention path shards by "
              f"KV head or sequence with no exchange, and no multi-GPU run is implemented.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceilings_sweep:
        import global_attention_amd as ga
        ga.lib()
        print(json.dumps({"measured_ceilings": measure_ceilings(sweep=True)}), flush=True)
        return

    import torch
    import global_attention_amd as ga
    ga.lib()
    T = args.seq_len

    rec = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"causal prefill T={T} B=1, one local (RoPE, window 512) + one global "
                                  f"(SSMax) layer, 48 Q / 8 KV heads, d=128, bf16 N(0,1) inputs",
                      "seq_len": T, "global_batch": 1, "parallelism": "none (1 GPU)"}}
    layers = None
    ceil = None
    if not args.skip_ceilings:
        ceil = measure_ceilings()
        rec["measured_ceilings"] = ceil

    def measured(_unused, value, kind):
        if ceil is None:
            return {}
        peak = ceil["mfma_measured_peak_tflops"] if kind == "mfma" else ceil["hbm_read_gbs"]
        return {"measured_peak": peak, "frac_of_measured_peak": round(value / peak, 4)}

    if not args.skip_prefill:
        r = bench_prefill(T, args.steps, args.warmup)
        layers = r["layers"]
        flops_step = FLOP_PER_PAIR * (pairs_global(T) + pairs_local(T))
        rec["ms_per_step"] = round(r["ms_per_step"], 4)
        rec["value"] = round(flops_step / (r["ms_per_step"] / 1e3) / 1e12, 2)
        g_ms = r["attn_ms"][1]
        l_ms = r["attn_ms"][0]
        g_flops = FLOP_PER_PAIR * pairs_global(T)
        achieved = g_flops / (g_ms / 1e3) / 1e12
        rec["roofline"] = {"kernel": "prefill_attn_kernel<1, 8, 0, 1> (global layer)", "bound": "mfma",
                           "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                           "traffic": recorded_traffic("prefill_attn_kernel<1, 8, 0, 1>"),
                           "avg_launch_ms": round(g_ms, 4), "flop_per_launch": g_flops,
                           **measured(None, achieved, "mfma")}
        l_flops = FLOP_PER_PAIR * pairs_local(T)
        l_tf = l_flops / (l_ms / 1e3) / 1e12
        rec["prefill_layers"] = {
            "global_attn_ms": round(g_ms, 4), "global_attn_tflops": round(achieved, 2),
            "local_attn_ms": round(l_ms, 4), "local_attn_tflops": round(l_tf, 2),
            "local_roofline": {"kernel": "prefill_attn_kernel<0, 4, 0, 2> (local layer)", "bound": "mfma",
                               "achieved": round(l_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(l_tf / PEAK_BF16_TFLOPS, 4),
                               "traffic": recorded_traffic("prefill_attn_kernel<0, 4, 0, 2>"),
                               "avg_launch_ms": round(l_ms, 4), "flop_per_launch": l_flops,
                               **measured(None, l_tf, "mfma")}}
        log(f"[bench] prefill step {r['ms_per_step']:.3f} ms -> {rec['value']} TFLOP/s; "
            f"global attn {g_ms:.3f} ms ({achieved:.1f} TFLOP/s), local attn {l_ms:.3f} ms")
    if not args.skip_prefill and not args.skip_projection:
        pf_layers = layers  # the prefill layers' caches and workspaces
        meta = dict(cu=_i32([0, T]), seq=_i32([0]), start=_i32([0]))
        pd = setup_projection(T)
        pr = bench_projection(T, args.steps, args.warmup, pd, pf_layers[1]["ws"], meta)
        fq, fo = proj_flops(T)
        tq = fq / (pr["qkvg_global"] / 1e3) / 1e12
        to = fo / (pr["w_o"] / 1e3) / 1e12
        tot = (fq + fo) / ((pr["qkvg_global"] + pr["w_o"]) / 1e3) / 1e12
        rec["projection"] = {
            "workload": f"QKV/gate projection of {T} tokens (hidden 5120 -> 6144 + 1024 + 1024 + 6144, bf16, "
                        "query RMSNorm + position op fused, Q' into the prefill workspace) and W_o (6144 -> 5120)",
            "value": round(tot, 2), "unit": "TFLOP/s",
            "qkvg_ms": {"global": round(pr["qkvg_global"], 4), "local": round(pr["qkvg_local"], 4)},
            "w_o_ms": round(pr["w_o"], 4), "w_o_tflops": round(to, 2),
            "roofline": {"kernel": "gemm_bf16_kernel<1>", "bound": "mfma", "achieved": round(tq, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tq / PEAK_BF16_TFLOPS, 4),
                         "traffic": recorded_traffic("gemm_bf16_kernel<1>"),
                         "avg_launch_ms": round(pr["qkvg_global"], 4), "flop_per_launch": fq},
        }
        sr = bench_sublayer(T, args.steps, args.warmup, pf_layers, meta, pd)
        rec["sublayer"] = {
            "workload": f"one local + one global attention sublayer end to end at T={T}: QKV/gate projection with "
                        "the query prologue fused, K/V prologue + attention + append, W_o",
            "value": round(sr["flops"] / (sr["ms"] / 1e3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(sr["ms"], 4), "flop_per_step": sr["flops"],
        }
        del pd
        torch.cuda.empty_cache()
    if not args.skip_schedule:
        sc = bench_schedule52(args.schedule_reps)
        tf = sc["flops"] / (sc["ms"] / 1e3) / 1e12
        rec["schedule52"] = {
            "workload": "full 52-layer attention schedule (global at 6,12,...,48,52; 43 local, window 512): "
                        "chunked varlen prefill of 8 sequences, lengths U[4096,65536] "
                        f"({', '.join(str(x) for x in sc['lens'])}), 8192-token chunks, one cache per layer "
                        "(paged for global, 512-slot rings for local)",
            "value": round(tf, 2), "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            **({"frac_of_measured_peak": round(tf / ceil["mfma_measured_peak_tflops"], 4)} if ceil else {}),
            "ms_per_pass": round(sc["ms"], 2), "ms_runs": sc["ms_runs"], "flop_per_pass": sc["flops"],
            "cpu_sample": sc["oracle"],
        }
    if not args.skip_decode and not args.decode_1m_only:
        dres = bench_decode(args.decode_steps, 3)
        g = dres["global"]
        rec["decode"] = {
            "workload": "64 seqs, 1 new token each at positions U[65536,131071], global layer over a paged "
                        "bf16 cache (16-token pages, random permutation); local layer over its 512-slot ring",
            "value": round(g["gbs_call"], 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(g["gbs_call"] / PEAK_HBM_GBS, 4),
            "global_bytes": g["bytes"], "global_ms_per_call": round(g["ms_per_call"], 4),
            "roofline": {"kernel": "decode_split_kernel<1>", "bound": "hbm", "achieved": round(g["gbs_split"], 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(g["gbs_split"] / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("decode_split_kernel<1>"),
                         "avg_launch_ms": round(g["split_ms"], 4), "bytes_per_launch": g["bytes"],
                         **measured(None, g["gbs_split"], "hbm")},
            "global_device_ms_per_call": _r4(g["device_ms"]),
            "local": {"bytes": dres["local"]["bytes"], "ms_per_call": round(dres["local"]["ms_per_call"], 4),
                      "device_ms_per_call": _r4(dres["local"]["device_ms"]),
                      "gbs_call": round(dres["local"]["gbs_call"], 1),
                      "note": "134 MB of rings can stay resident in the 256 MB MALL between calls"},
            "device_ms_note": "device_ms_per_call: 20 whole calls (prologue, split kernel, combine) captured in "
                              "one HIP graph and replayed, so no host launch cost; ms_per_call: the calls "
                              "launched from Python one by one",
        }
        f = dres["global_fp8"]
        rec["decode_fp8"] = {
            "workload": "the same 64-sequence global-layer decode over an FP8 E4M3 cache (1 byte per element, "
                        "per-tensor scales 1): half the bytes per token",
            "value": round(f["gbs_call"], 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(f["gbs_call"] / PEAK_HBM_GBS, 4),
            "global_bytes": f["bytes"], "global_ms_per_call": round(f["ms_per_call"], 4),
            "speedup_vs_bf16_call": round(g["ms_per_call"] / f["ms_per_call"], 3),
            "global_device_ms_per_call": _r4(f["device_ms"]),
            "roofline": {"kernel": "decode_fp8_kernel<1>", "bound": "hbm", "achieved": round(f["gbs_split"], 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(f["gbs_split"] / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("decode_fp8_kernel<1>"),
                         "avg_launch_ms": round(f["split_ms"], 4), "bytes_per_launch": f["bytes"],
                         **measured(None, f["gbs_split"], "hbm")},
        }
        v = bench_verify(args.decode_steps, 3, dres, split_keys=args.verify_split_keys)
        vg = v["global"]
        rec["verify"] = {
            "workload": "verify step of an 8-token draft per sequence (positions t-7..t) on the decode caches: "
                        "prologue, split-key attention, combine, append; global and local layer, and the "
                        "global layer over the FP8 cache",
            "value": round(vg["gbs_call"], 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(vg["gbs_call"] / PEAK_HBM_GBS, 4),
            "global_bytes": vg["bytes"], "global_ms_per_call": round(vg["ms_per_call"], 4),
            "speedup_vs_8_decode_calls": round(vg["vs_decode_calls"], 2),
            "global_device_ms_per_call": _r4(vg["device_ms"]),
            "roofline": {"kernel": "verify_attn_kernel<1, 0, 4>", "bound": "hbm", "achieved": round(vg["gbs_split"], 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(vg["gbs_split"] / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("verify_attn_kernel<1, 0, 4>"),
                         "avg_launch_ms": round(vg["split_ms"], 4), "bytes_per_launch": vg["bytes"],
                         **measured(None, vg["gbs_split"], "hbm")},
            "local": {"ms_per_call": round(v["local"]["ms_per_call"], 4),
                      "device_ms_per_call": _r4(v["local"]["device_ms"]),
                      "speedup_vs_8_decode_calls": round(v["local"]["vs_decode_calls"], 2)},
            "global_fp8": {"ms_per_call": round(v["global_fp8"]["ms_per_call"], 4),
                           "device_ms_per_call": _r4(v["global_fp8"]["device_ms"]),
                           "gbs_split": round(v["global_fp8"]["gbs_split"], 1),
                           "speedup_vs_8_decode_calls": round(v["global_fp8"]["vs_decode_calls"], 2),
                           "roofline": {"kernel": "verify48_fp8_kernel<1, 2>", "bound": "hbm",
                                        "achieved": round(v["global_fp8"]["gbs_split"], 1), "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s",
                                        "frac": round(v["global_fp8"]["gbs_split"] / PEAK_HBM_GBS, 4),
                                        "traffic": recorded_traffic("verify48_fp8_kernel<1, 2>"),
                                        "avg_launch_ms": round(v["global_fp8"]["split_ms"], 4),
                                        "bytes_per_launch": v["global_fp8"]["bytes"],
                                        **measured(None, v["global_fp8"]["gbs_split"], "hbm")}},
        }
        if not args.no_cpu_baseline:
            import numpy as np
            import synth
            cfg_d, ts_d, gcache_d = dres["setup"][:3]
            inp_d = synth.attention_inputs(cfg=3, layer=7, n_tok=len(ts_d))
            sq = int(np.argmax(ts_d))
            log(f"[bench] timing the CPU oracle on decode sequence {sq} (t = {int(ts_d[sq])}), all KV heads")
            cs = cpu_decode_sample(gcache_d, int(ts_d[sq]), inp_d, sq, list(range(G)),
                                   f"the longest of the 64 sequences (t = {int(ts_d[sq])}), all 48 query heads")
            cs["gpu_over_oracle"] = round(g["gbs_call"] / cs["value"], 1)
            rec["decode"]["cpu_sample"] = cs
        del dres, v
        torch.cuda.empty_cache()
    if not args.skip_decode_1m and not (args.skip_decode and not args.decode_1m_only):
        m = bench_decode_1m(args.decode_steps, 5, cpu_sample=not args.no_cpu_baseline)
        rec["decode_1m"] = {
            "workload": "one sequence at position 1,048,575 on a global layer: 65,536 permuted 16-token pages, "
                        "4 GiB of bf16 K+V",
            "value": round(m["gbs_call"], 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(m["gbs_call"] / PEAK_HBM_GBS, 4),
            "ms_per_call": round(m["ms_per_call"], 4), "bytes": m["bytes"],
            "roofline": {"kernel": "decode_split_kernel<1>", "bound": "hbm", "achieved": round(m["gbs_split"], 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(m["gbs_split"] / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("decode_split_kernel<1> (1M)"),
                         "avg_launch_ms": round(m["split_ms"], 4), "bytes_per_launch": m["bytes"],
                         **measured(None, m["gbs_split"], "hbm")},
        }
        if "cpu_sample" in m:
            m["cpu_sample"]["gpu_over_oracle"] = round(m["gbs_call"] / m["cpu_sample"]["value"], 1)
            rec["decode_1m"]["cpu_sample"] = m["cpu_sample"]
    if not args.skip_router:
        rr = bench_router(T, args.steps, args.warmup)
        tf = rr["flops"] / (rr["ms"] / 1e3) / 1e12
        rec["router"] = {
            "workload": f"group-limited sigmoid router of one MoE layer: {T} tokens, hidden 5120 (bf16), 256 experts "
                        "(fp32 weight), fp32 logits, 8 groups keep 4, top-8, weights x2.5; logits fused with the "
                        "selection",
            "value": round(tf, 2), "unit": "TFLOP/s", "ms_per_call": round(rr["ms"], 4),
            "roofline": {"kernel": "router_gemm_kernel<true>", "bound": "mfma", "achieved": round(tf, 2),
                         "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                         "traffic": recorded_traffic("router_gemm_kernel<true>"),
                         "avg_launch_ms": round(rr["ms"], 4), "flop_per_launch": rr["flops"]},
        }
    if not args.no_cpu_baseline and layers is not None:
        log(f"[bench] timing the CPU oracle on {args.cpu_rows} rows per layer")
        rec["cpu_baseline"] = cpu_baseline(layers, T, args.cpu_rows)
        if rec["value"]:
            # vs_baseline stays null: the pages publish no throughput for this path
            rec["cpu_baseline"]["gpu_over_oracle"] = round(rec["value"] / rec["cpu_baseline"]["value"], 1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
