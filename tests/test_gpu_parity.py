"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances on bf16 outputs: max-abs 2e-2 and relative L2 5e-3 (whole output
and reported per head); bit-exact for visibility masks, cache addressing and
V bytes. Inputs come from the shared seeded generator (synth), or, for the
multi-GB cache configurations, from torch's seeded device RNG written straight
into the cache (those cache contents are inputs, not results of this library).
"""
import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O
import synth
from tests.helpers import compare, dev_bf16, dev_i32, host_bits, bf16_to_f64, say

pytestmark = pytest.mark.gpu

CFG = ga.Config()
OCFG = O.Config()
SENT = 0x7F7F  # sentinel bf16 pattern (finite, large) for stray-write detection


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.lib()
    yield
    torch.cuda.synchronize()


def sync():
    import torch
    torch.cuda.synchronize()


def _inputs(cfg_id, layer, n_tok):
    return synth.attention_inputs(cfg_id, layer, n_tok)


def _global_cache(cfg_id, ctx_lens, extra_pages=3):
    bt, n_pages = synth.paged_block_table(cfg_id, ctx_lens, extra_pages=extra_pages)
    import torch
    cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt), fill=SENT)
    return cache, bt


def _oracle_layer(kind, inp, qrows, krows, q_pos, k_pos):
    return O.attention_layer(kind, inp["q"][qrows], inp["k"][krows], inp["v"][krows], inp["q_norm_w"],
                             inp["k_norm_w"], inp["gate"][qrows], q_pos, k_pos)


# ----------------------------------------------------------------- masks

@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_visibility_mask_bit_exact(kind):
    for t0, s0 in ((0, 0), (1000, 400), (5000, 4400), (1048000, 1047500)):
        say(f"[case] visibility kind={kind} t0={t0} s0={s0}")
        m = ga.debug_visibility(kind, 512, t0, 200, s0, 700).cpu().numpy().astype(bool)
        ref = O.visible(kind, np.arange(t0, t0 + 200), np.arange(s0, s0 + 700), 512)
        assert np.array_equal(m, ref)


# ----------------------------------------------------------------- append

def _check_global_cache(cache, bt, kinds_tokens, inp, seqs, poss, kind=O.GLOBAL):
    """V bytes bit-exact at the oracle's addresses, K_hat within bf16 rounding,
    every other byte still the sentinel."""
    k = host_bits(cache.k)
    v = host_bits(cache.v)
    touched_k = np.zeros(k.shape[:3], dtype=bool)
    khat = O.cached_key(kind, inp["k"], inp["k_norm_w"], np.asarray(poss))
    for i, (sq, t) in enumerate(zip(seqs, poss)):
        page, slot = O.page_slot(bt, 16, sq, t)
        assert np.array_equal(v[page, :, :, slot], inp["v"][i]), (sq, t)
        got = bf16_to_f64(k[page, :, slot, :])
        assert np.max(np.abs(got - khat[i]) / (np.abs(khat[i]) + 1e-3)) < 2 ** -7
        touched_k[page, :, slot] = True
    assert np.all(k[~touched_k] == SENT)
    vt = np.transpose(v, (0, 1, 3, 2))
    assert np.all(vt[~touched_k] == SENT)


def test_kv_append_global_addressing():
    import torch
    g = np.random.default_rng(11)
    ctx = [40, 300, 17]
    cache, bt = _global_cache(101, ctx)
    seqs, poss = [], []
    for sq, n in enumerate(ctx):
        for t in sorted(g.choice(n, size=min(n, 25), replace=False)):
            seqs.append(sq)
            poss.append(int(t))
    inp = _inputs(101, 0, len(seqs))
    say(f"[case] kv_append global n_tok={len(seqs)}")
    ga.kv_append(CFG, cache, dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_bf16(inp["k_norm_w"]),
                 dev_i32(seqs), dev_i32(poss))
    sync()
    _check_global_cache(cache, bt, None, inp, seqs, poss)


def test_kv_append_local_ring():
    seqs = [0, 0, 1, 2, 2, 2]
    poss = [0, 700, 511, 512, 1023, 1048574]  # distinct ring slots per sequence
    cache = ga.KVCache.allocate_local(CFG, 3, fill=SENT)
    inp = _inputs(102, 0, len(seqs))
    say("[case] kv_append local")
    ga.kv_append(CFG, cache, dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_bf16(inp["k_norm_w"]),
                 dev_i32(seqs), dev_i32(poss))
    sync()
    k = host_bits(cache.k)
    v = host_bits(cache.v)
    khat = O.cached_key(O.LOCAL, inp["k"], inp["k_norm_w"], np.asarray(poss))
    touched = np.zeros(k.shape[:3], dtype=bool)
    for i, (sq, t) in enumerate(zip(seqs, poss)):
        slot = O.ring_slot(t)
        assert np.array_equal(v[sq, :, :, slot], inp["v"][i])
        got = bf16_to_f64(k[sq, :, slot, :])
        assert np.max(np.abs(got - khat[i]) / (np.abs(khat[i]) + 1e-3)) < 2 ** -7
        touched[sq, :, slot] = True
    assert np.all(k[~touched] == SENT)
    assert np.all(np.transpose(v, (0, 1, 3, 2))[~touched] == SENT)


# ----------------------------------------------------------------- prefill

def _run_prefill(kind, inp_list, starts, cache, seq_idx, max_chunk=None, cfg=CFG):
    """inp_list: per sequence dict of the chunk's inputs; returns out bits per seq."""
    import torch
    lens = [x["q"].shape[0] for x in inp_list]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cat = lambda key: np.concatenate([x[key] for x in inp_list])
    w = inp_list[0]
    out = ga.prefill(cfg, cache, dev_bf16(cat("q")), dev_bf16(cat("k")), dev_bf16(cat("v")),
                     dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]), dev_bf16(cat("gate")),
                     dev_i32(cu), dev_i32(seq_idx), dev_i32(starts), max_chunk or max(lens))
    sync()
    o = host_bits(out)
    return [o[cu[i]:cu[i + 1]] for i in range(len(lens))]


def _cache_for(kind, cfg_id, ctx):
    if kind == O.GLOBAL:
        return _global_cache(cfg_id, ctx)
    return ga.KVCache.allocate_local(CFG, len(ctx), fill=SENT), None


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_t640_full(kind):
    """T=640, B=1, both layer kinds: every output element, then the cache."""
    T = 640
    inp = _inputs(1, kind, T)
    cache, bt = _cache_for(kind, 1, [T])
    say(f"[case] prefill T=640 kind={kind}")
    (out,) = _run_prefill(kind, [inp], [0], cache, [0])
    pos = np.arange(T)
    ref = _oracle_layer(kind, inp, slice(None), slice(None), pos, pos)
    compare(out, ref, f"prefill T=640 kind={kind}")
    # the chunk's K_hat/V landed in the cache
    if kind == O.GLOBAL:
        _check_global_cache(cache, bt, None, inp, [0] * T, list(range(T)))
    else:
        k = host_bits(cache.k)
        v = host_bits(cache.v)
        khat = O.cached_key(O.LOCAL, inp["k"], inp["k_norm_w"], pos)
        for t in range(T - 512, T):
            assert np.array_equal(v[0, :, :, t % 512], inp["v"][t])
            got = bf16_to_f64(k[0, :, t % 512, :])
            assert np.max(np.abs(got - khat[t]) / (np.abs(khat[t]) + 1e-3)) < 2 ** -7


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_varlen_ragged(kind):
    """Several sequences of ragged lengths in one call (1 token to >1 tile)."""
    lens = [1, 77, 333, 1000, 64, 129]
    inps = [_inputs(3, 10 * kind + i, n) for i, n in enumerate(lens)]
    for x in inps[1:]:
        x["q_norm_w"], x["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    cache, _ = _cache_for(kind, 3, lens)
    say(f"[case] prefill varlen kind={kind} lens={lens}")
    outs = _run_prefill(kind, inps, [0] * len(lens), cache, list(range(len(lens))))
    for i, (x, o) in enumerate(zip(inps, outs)):
        pos = np.arange(lens[i])
        compare(o, _oracle_layer(kind, x, slice(None), slice(None), pos, pos), f"varlen seq{i} len={lens[i]}")


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_batch_with_empty_sequences(kind):
    """Zero-length sequences inside and at the end of a varlen batch: the
    others match the oracle, and the empty ones' cache stays untouched."""
    import torch
    lens = [5, 0, 200, 0]
    inps = [_inputs(11, 10 * kind + i, max(n, 1)) for i, n in enumerate(lens)]
    inps = [{k: (v[:n] if v.ndim == 3 else v) for k, v in x.items()} for x, n in zip(inps, lens)]
    for x in inps[1:]:
        x["q_norm_w"], x["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    cache, bt = _cache_for(kind, 11, lens)
    say(f"[case] prefill with empty sequences kind={kind} lens={lens}")
    outs = _run_prefill(kind, inps, [0] * len(lens), cache, list(range(len(lens))), max_chunk=max(lens))
    for i, (x, o) in enumerate(zip(inps, outs)):
        assert o.shape[0] == lens[i]
        if lens[i]:
            pos = np.arange(lens[i])
            compare(o, _oracle_layer(kind, x, slice(None), slice(None), pos, pos), f"seq{i} len={lens[i]}")
    k = host_bits(cache.k)
    if kind == O.GLOBAL:
        used = set(int(p) for row in bt for p in row if p >= 0)
        unused = [p for p in range(k.shape[0]) if p not in used]
        assert unused and np.all(k[unused] == SENT)
    else:
        assert np.all(k[1] == SENT) and np.all(k[3] == SENT)


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_chunked_prefill_with_cached_prefix(kind):
    """Unaligned chunks of two interleaved sequences; each chunk attends to the
    cached prefix written by earlier chunks."""
    total = [1500, 900]
    chunks = [[600, 37, 700, 163], [511, 1, 388]]
    inps = [_inputs(4, 10 * kind + i, n) for i, n in enumerate(total)]
    inps[1]["q_norm_w"], inps[1]["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    cache, _ = _cache_for(kind, 4, total)
    pos_done = [0, 0]
    for step in range(4):
        batch, starts, seqs = [], [], []
        for sq in (0, 1):
            if step < len(chunks[sq]):
                n = chunks[sq][step]
                s0 = pos_done[sq]
                batch.append({k: (v[s0:s0 + n] if v.ndim == 3 else v) for k, v in inps[sq].items()})
                starts.append(s0)
                seqs.append(sq)
        say(f"[case] chunked prefill kind={kind} step={step} starts={starts}")
        outs = _run_prefill(kind, batch, starts, cache, seqs)
        for sq, s0, o, b in zip(seqs, starts, outs, batch):
            n = b["q"].shape[0]
            ref = _oracle_layer(kind, inps[sq], slice(s0, s0 + n), slice(0, s0 + n), np.arange(s0, s0 + n),
                                np.arange(s0 + n))
            compare(o, ref, f"chunk seq{sq} [{s0},{s0 + n})")
            pos_done[sq] += n


@pytest.mark.parametrize("heads", [(8, 8), (24, 8), (16, 8), (32, 2)])
@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_head_layouts(kind, heads):
    """Other grouped-query layouts: one query head per KV head, an odd number
    per KV head (local blocks then take one head), two, and sixteen; two
    sequences in two chunks each, the second chunk unaligned over the cached
    prefix of the first."""
    import torch
    nq, nkv = heads
    cfg, ocfg = ga.Config(n_q_heads=nq, n_kv_heads=nkv), O.Config(n_q_heads=nq, n_kv_heads=nkv)
    total = [533, 677]
    first = [333, 77]
    inps = [synth.attention_inputs(5, 100 * kind + 10 * nq + i, n, n_q=nq, n_kv=nkv) for i, n in enumerate(total)]
    inps[1]["q_norm_w"], inps[1]["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(5, total)
        cache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt), fill=SENT)
    else:
        cache = ga.KVCache.allocate_local(cfg, 2, fill=SENT)
    for step in range(2):
        starts = [0, 0] if step == 0 else first
        ends = first if step == 0 else total
        batch = [{k: (v[s0:e] if v.ndim == 3 else v) for k, v in x.items()} for x, s0, e in zip(inps, starts, ends)]
        say(f"[case] prefill heads={nq}/{nkv} kind={kind} step={step} starts={starts}")
        outs = _run_prefill(kind, batch, starts, cache, [0, 1], cfg=cfg)
        for sq, (x, s0, e, o) in enumerate(zip(inps, starts, ends, outs)):
            ref = O.attention_layer(kind, x["q"][s0:e], x["k"][:e], x["v"][:e], x["q_norm_w"], x["k_norm_w"],
                                    x["gate"][s0:e], np.arange(s0, e), np.arange(e), ocfg)
            compare(o, ref, f"heads {nq}/{nkv} seq{sq} [{s0},{e})")


@pytest.mark.parametrize("heads", [(8, 8), (24, 8), (16, 8), (32, 2)])
@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_and_decode_head_layouts(kind, heads):
    """The same grouped-query layouts on the verify and decode paths: two
    sequences with a prefilled history (900 and 300 tokens), a 5-token verify
    chunk each, then a one-token decode (its K/V appended first)."""
    import torch
    nq, nkv = heads
    cfg, ocfg = ga.Config(n_q_heads=nq, n_kv_heads=nkv), O.Config(n_q_heads=nq, n_kv_heads=nkv)
    hist = [900, 300]
    total = [h + 6 for h in hist]
    inps = [synth.attention_inputs(7, 100 * kind + 10 * nq + i, n, n_q=nq, n_kv=nkv) for i, n in enumerate(total)]
    inps[1]["q_norm_w"], inps[1]["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    qw, kw = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(7, total)
        cache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt), fill=SENT)
    else:
        cache = ga.KVCache.allocate_local(cfg, 2, fill=SENT)
    say(f"[case] verify/decode heads={nq}/{nkv} kind={kind}")
    _run_prefill(kind, [{k: (v[:h] if v.ndim == 3 else v) for k, v in x.items()} for x, h in zip(inps, hist)],
                 [0, 0], cache, [0, 1], cfg=cfg)
    cat = lambda key, lo, hi: dev_bf16(np.concatenate([x[key][l:h] for x, l, h in zip(inps, lo, hi)]))
    lo, hi = hist, [h + 5 for h in hist]
    out = ga.verify(cfg, cache, cat("q", lo, hi), cat("k", lo, hi), cat("v", lo, hi), dev_bf16(qw), dev_bf16(kw),
                    cat("gate", lo, hi), dev_i32([0, 5, 10]), dev_i32([0, 1]), dev_i32(hist), 5, max(hi) - 1)
    sync()
    o = host_bits(out)
    for i, x in enumerate(inps):
        ref = O.attention_layer(kind, x["q"][lo[i]:hi[i]], x["k"][:hi[i]], x["v"][:hi[i]], qw, kw,
                                x["gate"][lo[i]:hi[i]], np.arange(lo[i], hi[i]), np.arange(hi[i]), ocfg)
        compare(o[5 * i:5 * i + 5], ref, f"verify heads {nq}/{nkv} seq{i}")
    ts = hi
    ga.kv_append(cfg, cache, cat("k", ts, total), cat("v", ts, total), dev_bf16(kw), dev_i32([0, 1]), dev_i32(ts))
    out = ga.decode(cfg, cache, cat("q", ts, total), dev_bf16(qw), cat("gate", ts, total), dev_i32([0, 1]),
                    dev_i32(ts), max(ts))
    sync()
    o = host_bits(out)
    for i, x in enumerate(inps):
        t = ts[i]
        ref = O.attention_layer(kind, x["q"][t:t + 1], x["k"][:t + 1], x["v"][:t + 1], qw, kw, x["gate"][t:t + 1],
                                np.array([t]), np.arange(t + 1), ocfg)
        compare(o[i:i + 1], ref, f"decode heads {nq}/{nkv} seq{i}")


@pytest.mark.parametrize("window", [64, 128, 1024])
def test_local_window_sizes(window):
    """Local layers with other windows (multiples of 64): with 64 the window
    edge falls on the tile next to the diagonal one, with 1024 a chunk spans
    17 tiles, and the ring holds that many slots. Two sequences: chunked
    prefill over the cached ring (unaligned chunks), a 5-token verify step,
    then a one-token decode (its K/V appended first)."""
    cfg, ocfg = ga.Config(window=window), O.Config(window=window)
    chunks = [[600, 37, 363], [511, 189]]
    hist = [sum(c) for c in chunks]
    total = [h + 6 for h in hist]
    inps = [synth.attention_inputs(8, 1000 + window + i, n) for i, n in enumerate(total)]
    inps[1]["q_norm_w"], inps[1]["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    qw, kw = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    cache = ga.KVCache.allocate_local(cfg, 2, fill=SENT)
    done = [0, 0]
    for step in range(3):
        batch, starts, seqs = [], [], []
        for sq in (0, 1):
            if step < len(chunks[sq]):
                n, s0 = chunks[sq][step], done[sq]
                batch.append({k: (v[s0:s0 + n] if v.ndim == 3 else v) for k, v in inps[sq].items()})
                starts.append(s0)
                seqs.append(sq)
        say(f"[case] local window={window} prefill step={step} starts={starts}")
        outs = _run_prefill(O.LOCAL, batch, starts, cache, seqs, cfg=cfg)
        for sq, s0, o, b in zip(seqs, starts, outs, batch):
            n = b["q"].shape[0]
            x = inps[sq]
            ref = O.attention_layer(O.LOCAL, x["q"][s0:s0 + n], x["k"][:s0 + n], x["v"][:s0 + n], qw, kw,
                                    x["gate"][s0:s0 + n], np.arange(s0, s0 + n), np.arange(s0 + n), ocfg)
            compare(o, ref, f"window {window} chunk seq{sq} [{s0},{s0 + n})")
            done[sq] += n
    cat = lambda key, lo, hi: dev_bf16(np.concatenate([x[key][l:h] for x, l, h in zip(inps, lo, hi)]))
    lo, hi = hist, [h + 5 for h in hist]
    say(f"[case] local window={window} verify")
    out = ga.verify(cfg, cache, cat("q", lo, hi), cat("k", lo, hi), cat("v", lo, hi), dev_bf16(qw), dev_bf16(kw),
                    cat("gate", lo, hi), dev_i32([0, 5, 10]), dev_i32([0, 1]), dev_i32(hist), 5, max(hi) - 1)
    sync()
    o = host_bits(out)
    for i, x in enumerate(inps):
        ref = O.attention_layer(O.LOCAL, x["q"][lo[i]:hi[i]], x["k"][:hi[i]], x["v"][:hi[i]], qw, kw,
                                x["gate"][lo[i]:hi[i]], np.arange(lo[i], hi[i]), np.arange(hi[i]), ocfg)
        compare(o[5 * i:5 * i + 5], ref, f"window {window} verify seq{i}")
    ts = hi
    say(f"[case] local window={window} decode")
    ga.kv_append(cfg, cache, cat("k", ts, total), cat("v", ts, total), dev_bf16(kw), dev_i32([0, 1]), dev_i32(ts))
    out = ga.decode(cfg, cache, cat("q", ts, total), dev_bf16(qw), cat("gate", ts, total), dev_i32([0, 1]),
                    dev_i32(ts), max(ts))
    sync()
    o = host_bits(out)
    for i, x in enumerate(inps):
        t = ts[i]
        ref = O.attention_layer(O.LOCAL, x["q"][t:t + 1], x["k"][:t + 1], x["v"][:t + 1], qw, kw,
                                x["gate"][t:t + 1], np.array([t]), np.arange(t + 1), ocfg)
        compare(o[i:i + 1], ref, f"window {window} decode seq{i}")


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_stage_orders_bit_identical(kind):
    """The stage splits of a prefill call (including the global layers' fused
    PROLOGUE|APPEND and the standalone append) give the same output and cache
    bytes as the single call, for a chunk with an unaligned cached prefix."""
    import torch
    inp = _inputs(6, kind, 633)
    c1 = {k: (v[:333] if v.ndim == 3 else v) for k, v in inp.items()}
    c2 = {k: (v[333:] if v.ndim == 3 else v) for k, v in inp.items()}
    orders = [[ga.STAGE_ALL], [ga.STAGE_PROLOGUE, ga.STAGE_ATTENTION, ga.STAGE_APPEND]]
    if kind == O.GLOBAL:
        orders.append([ga.STAGE_PROLOGUE | ga.STAGE_APPEND, ga.STAGE_ATTENTION])
    results = []
    for order in orders:
        say(f"[case] stage order kind={kind} order={order}")
        cache, _ = _cache_for(kind, 6, [633])
        _run_prefill(kind, [c1], [0], cache, [0])
        args = (CFG, cache, dev_bf16(c2["q"]), dev_bf16(c2["k"]), dev_bf16(c2["v"]), dev_bf16(c2["q_norm_w"]),
                dev_bf16(c2["k_norm_w"]), dev_bf16(c2["gate"]), dev_i32([0, 300]), dev_i32([0]), dev_i32([333]), 300)
        out = torch.empty((300, 48, 128), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ga.prefill_workspace_bytes(CFG, 300, 1), dtype=torch.uint8, device="cuda")
        for st in order:
            ga.prefill(*args, out=out, workspace=ws, stages=st)
        sync()
        results.append((host_bits(out), host_bits(cache.k), host_bits(cache.v)))
    for r in results[1:]:
        for a_, b_ in zip(results[0], r):
            assert np.array_equal(a_, b_)
    ref = _oracle_layer(kind, inp, slice(333, 633), slice(0, 633), np.arange(333, 633), np.arange(633))
    compare(results[0][0], ref, f"stage orders kind={kind}")


# ----------------------------------------------------------------- decode

def _decode_setup(kind, cfg_id, ts):
    """Fill a cache with the raw history of each sequence via kv_append; return
    (cache, inputs per seq)."""
    import torch
    ctx = [t + 1 for t in ts]
    cache, bt = _cache_for(kind, cfg_id, ctx)
    hist = [_inputs(cfg_id, 100 + i, t + 1) for i, t in enumerate(ts)]
    for x in hist[1:]:
        x["q_norm_w"], x["k_norm_w"] = hist[0]["q_norm_w"], hist[0]["k_norm_w"]
    for i, t in enumerate(ts):
        lo = 0 if kind == O.GLOBAL else max(0, t + 1 - 512)
        n = t + 1 - lo
        ga.kv_append(CFG, cache, dev_bf16(hist[i]["k"][lo:]), dev_bf16(hist[i]["v"][lo:]),
                     dev_bf16(hist[0]["k_norm_w"]), dev_i32(np.full(n, i)), dev_i32(np.arange(lo, t + 1)))
    sync()
    return cache, hist


def _decode_ref(kind, hist, ts):
    refs = []
    for x, t in zip(hist, ts):
        refs.append(_oracle_layer(kind, x, slice(t, t + 1), slice(0, t + 1), np.array([t]), np.arange(t + 1)))
    return np.concatenate(refs)


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_decode_small(kind):
    ts = [0, 15, 16, 31, 511, 512, 700, 2999]
    cache, hist = _decode_setup(kind, 5, ts)
    q = np.stack([x["q"][t] for x, t in zip(hist, ts)])
    gate = np.stack([x["gate"][t] for x, t in zip(hist, ts)])
    ref = _decode_ref(kind, hist, ts)
    for sk in (0, 128, 512, 2048):
        say(f"[case] decode kind={kind} split_keys={sk}")
        out = ga.decode(CFG, cache, dev_bf16(q), dev_bf16(hist[0]["q_norm_w"]), dev_bf16(gate),
                        dev_i32(np.arange(len(ts))), dev_i32(ts), max(ts), split_keys=sk)
        sync()
        compare(host_bits(out), ref, f"decode kind={kind} split={sk}")


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_decode_is_deterministic(kind):
    ts = [1234, 77]
    cache, hist = _decode_setup(kind, 6, ts)
    q = np.stack([x["q"][t] for x, t in zip(hist, ts)])
    gate = np.stack([x["gate"][t] for x, t in zip(hist, ts)])
    outs = []
    for _ in range(3):
        say(f"[case] decode determinism kind={kind}")
        out = ga.decode(CFG, cache, dev_bf16(q), dev_bf16(hist[0]["q_norm_w"]), dev_bf16(gate),
                        dev_i32([0, 1]), dev_i32(ts), max(ts))
        sync()
        outs.append(host_bits(out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_then_decode_matches_one_shot(kind):
    """Prefill T-1 tokens, append the last token, decode it: equals the last row
    of a one-shot prefill of all T tokens (and the oracle)."""
    T = 900
    inp = _inputs(7, kind, T)
    cache, _ = _cache_for(kind, 7, [T])
    say(f"[case] prefill+decode kind={kind}")
    _run_prefill(kind, [{k: (v[:T - 1] if v.ndim == 3 else v) for k, v in inp.items()}], [0], cache, [0])
    ga.kv_append(CFG, cache, dev_bf16(inp["k"][T - 1:]), dev_bf16(inp["v"][T - 1:]), dev_bf16(inp["k_norm_w"]),
                 dev_i32([0]), dev_i32([T - 1]))
    dec = ga.decode(CFG, cache, dev_bf16(inp["q"][T - 1:]), dev_bf16(inp["q_norm_w"]), dev_bf16(inp["gate"][T - 1:]),
                    dev_i32([0]), dev_i32([T - 1]), T - 1)
    sync()
    cache2, _ = _cache_for(kind, 7, [T])
    (full,) = _run_prefill(kind, [inp], [0], cache2, [0])
    ref = _oracle_layer(kind, inp, slice(T - 1, T), slice(None), np.array([T - 1]), np.arange(T))
    d = host_bits(dec)
    compare(d, ref, "decode row")
    compare(full[T - 1:], ref, "prefill last row")
    assert np.max(np.abs(bf16_to_f64(d) - bf16_to_f64(full[T - 1:]))) < 1e-2
