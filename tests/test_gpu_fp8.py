"""GPU parity for the FP8 E4M3 KV cache (through the C ABI) against the float64
oracle's own quantiser (oracle.e4m3_encode / fp8_roundtrip).

The pages keep the serving KV cache in FP8 E4M3 ("Beam 1.0: Local RoPE, Global
NoPE and Scalable Softmax", section "KV memory: nine growing caches, not 52",
and the German serving article) without a scale convention; the reading here
is one scale per tensor, nearest code with ties to even, saturation at 448.

Stored codes are compared byte for byte. V codes come from exact bf16 inputs
divided by a power-of-two scale, so both sides decide on the same value and
must agree everywhere. K_hat is a computed value (float32 on the GPU, float64
in the oracle): its code must agree except where the oracle's value lies
within a relative 1e-5 of a rounding midpoint, and there it must be one of the
two neighbouring codes. Attention outputs use the bf16 tolerances.
"""
import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O
import synth
from tests.helpers import compare, dev_bf16, dev_i32, host_bits, bf16_to_f64, say

pytestmark = pytest.mark.gpu
CFG = ga.Config()
FILL = 0x55  # sentinel code for stray-write detection


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


def codes(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def _fp8_cache(kind, cfg_id, ctx, k_scale, v_scale, fill=FILL):
    import torch
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(cfg_id, ctx, extra_pages=3)
        c = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt), fill=fill, dtype=ga.KV_FP8_E4M3,
                                       k_scale=k_scale, v_scale=v_scale)
        return c, bt
    return ga.KVCache.allocate_local(CFG, len(ctx), fill=fill, dtype=ga.KV_FP8_E4M3, k_scale=k_scale,
                                     v_scale=v_scale), None


def _check_k_codes(got, x, what):
    """got: GPU codes; x: the oracle's K_hat / k_scale (float64), same shape.
    Where the two codes differ, x must lie at the midpoint of two adjacent
    codes (within a relative 1e-5, the float32 error of K_hat), one of them
    being the GPU's."""
    ref = O.e4m3_encode(x)
    diff = got != ref
    if diff.any():
        a, b = O.e4m3_decode(got[diff]), O.e4m3_decode(ref[diff])
        near = np.abs(x[diff] - (a + b) / 2) <= 1e-5 * np.abs(x[diff])
        adjacent = np.abs(got[diff].astype(int) - ref[diff].astype(int)) == 1
        assert np.all(near & adjacent), f"{what}: {int((~(near & adjacent)).sum())} K codes off a rounding boundary"
    say(f"[fp8] {what}: {int(diff.sum())} of {diff.size} K codes at a rounding boundary")
    assert diff.mean() < 1e-3


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_fp8_append_codes(kind):
    """kv_append into an FP8 cache: every written code against the oracle's
    quantiser, untouched bytes keep the sentinel."""
    k_scale, v_scale = 0.5, 0.25
    if kind == O.GLOBAL:
        ctx = [40, 300, 17]
        g = np.random.default_rng(12)
        seqs, poss = [], []
        for sq, n in enumerate(ctx):
            for t in sorted(g.choice(n, size=min(n, 25), replace=False)):
                seqs.append(sq)
                poss.append(int(t))
    else:
        ctx = [1, 1, 1]
        seqs = [0, 0, 1, 2, 2, 2]
        poss = [0, 700, 511, 512, 1023, 1048574]
    cache, bt = _fp8_cache(kind, 103, ctx, k_scale, v_scale)
    inp = synth.attention_inputs(103, kind, len(seqs))
    say(f"[case] fp8 kv_append kind={kind} n_tok={len(seqs)}")
    ga.kv_append(CFG, cache, dev_bf16(inp["k"]), dev_bf16(inp["v"]), dev_bf16(inp["k_norm_w"]),
                 dev_i32(seqs), dev_i32(poss))
    sync()
    k, v = codes(cache.k), codes(cache.v)
    khat = O.cached_key(kind, inp["k"], inp["k_norm_w"], np.asarray(poss))
    vref = O.e4m3_encode(bf16_to_f64(inp["v"]) / v_scale)
    touched_k = np.zeros(k.shape[:3], dtype=bool)
    got_k = []
    for i, (sq, t) in enumerate(zip(seqs, poss)):
        if kind == O.GLOBAL:
            page, slot = O.page_slot(bt, 16, sq, t)
            got_k.append(k[page, :, slot, :])
            assert np.array_equal(v[page, :, :, slot], vref[i])
            touched_k[page, :, slot] = True
        else:
            slot = O.ring_slot(t)
            got_k.append(k[sq, :, slot, :])
            assert np.array_equal(v[sq, :, :, slot], vref[i])
            touched_k[sq, :, slot] = True
    _check_k_codes(np.stack(got_k), khat / k_scale, f"append kind={kind}")
    assert np.all(k[~touched_k] == FILL)
    assert np.all(np.transpose(v, (0, 1, 3, 2))[~touched_k] == FILL)


def _fp8_decode_setup(kind, cfg_id, ts, k_scale, v_scale):
    ctx = [t + 1 for t in ts]
    cache, bt = _fp8_cache(kind, cfg_id, ctx, k_scale, v_scale)
    hist = [synth.attention_inputs(cfg_id, 100 + i, t + 1) for i, t in enumerate(ts)]
    for x in hist[1:]:
        x["q_norm_w"], x["k_norm_w"] = hist[0]["q_norm_w"], hist[0]["k_norm_w"]
    for i, t in enumerate(ts):
        lo = 0 if kind == O.GLOBAL else max(0, t + 1 - 512)
        n = t + 1 - lo
        ga.kv_append(CFG, cache, dev_bf16(hist[i]["k"][lo:]), dev_bf16(hist[i]["v"][lo:]),
                     dev_bf16(hist[0]["k_norm_w"]), dev_i32(np.full(n, i)), dev_i32(np.arange(lo, t + 1)))
    sync()
    return cache, hist


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_fp8_decode_small(kind):
    """Decode over an FP8 cache (scales that are not powers of two) against the
    oracle with every cached key and value passed through the FP8 round trip."""
    ks, vs = 0.7, 1.3
    ts = [0, 15, 16, 31, 511, 512, 700, 2999]
    cache, hist = _fp8_decode_setup(kind, 15, ts, ks, vs)
    q = np.stack([x["q"][t] for x, t in zip(hist, ts)])
    gate = np.stack([x["gate"][t] for x, t in zip(hist, ts)])
    ref = np.concatenate([
        O.attention_layer(kind, x["q"][t:t + 1], x["k"][:t + 1], x["v"][:t + 1], x["q_norm_w"], x["k_norm_w"],
                          x["gate"][t:t + 1], np.array([t]), np.arange(t + 1), fp8_cache=(ks, vs, t + 1))
        for x, t in zip(hist, ts)])
    for sk in (0, 128, 2048):
        say(f"[case] fp8 decode kind={kind} split_keys={sk}")
        out = ga.decode(CFG, cache, dev_bf16(q), dev_bf16(hist[0]["q_norm_w"]), dev_bf16(gate),
                        dev_i32(np.arange(len(ts))), dev_i32(ts), max(ts), split_keys=sk)
        sync()
        compare(host_bits(out), ref, f"fp8 decode kind={kind} split={sk}")


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_fp8_chunked_prefill_with_cached_prefix(kind):
    """Unaligned chunks over an FP8 cache: each chunk attends to its own keys
    unquantised and to the FP8 prefix written by earlier chunks."""
    ks, vs = 0.6, 0.9
    total = [1500, 900]
    chunks = [[600, 37, 700, 163], [511, 1, 388]]
    inps = [synth.attention_inputs(16, 10 * kind + i, n) for i, n in enumerate(total)]
    inps[1]["q_norm_w"], inps[1]["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    cache, _ = _fp8_cache(kind, 16, total, ks, vs)
    done = [0, 0]
    for step in range(4):
        batch, starts, seqs = [], [], []
        for sq in (0, 1):
            if step < len(chunks[sq]):
                n, s0 = chunks[sq][step], done[sq]
                batch.append({k: (v[s0:s0 + n] if v.ndim == 3 else v) for k, v in inps[sq].items()})
                starts.append(s0)
                seqs.append(sq)
        lens = [b["q"].shape[0] for b in batch]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        cat = lambda key: np.concatenate([b[key] for b in batch])
        say(f"[case] fp8 chunked prefill kind={kind} step={step} starts={starts}")
        out = ga.prefill(CFG, cache, dev_bf16(cat("q")), dev_bf16(cat("k")), dev_bf16(cat("v")),
                         dev_bf16(inps[0]["q_norm_w"]), dev_bf16(inps[0]["k_norm_w"]), dev_bf16(cat("gate")),
                         dev_i32(cu), dev_i32(seqs), dev_i32(starts), max(lens))
        sync()
        o = host_bits(out)
        for i, (sq, s0, n) in enumerate(zip(seqs, starts, lens)):
            x = inps[sq]
            ref = O.attention_layer(kind, x["q"][s0:s0 + n], x["k"][:s0 + n], x["v"][:s0 + n], x["q_norm_w"],
                                    x["k_norm_w"], x["gate"][s0:s0 + n], np.arange(s0, s0 + n), np.arange(s0 + n),
                                    fp8_cache=(ks, vs, s0))
            compare(o[cu[i]:cu[i + 1]], ref, f"fp8 chunk seq{sq} [{s0},{s0 + n})")
            done[sq] += n


def test_fp8_fused_and_standalone_append_identical():
    """Global layers: the append fused into the prologue writes the same codes
    as the standalone append stage, and the outputs agree bit for bit."""
    import torch
    inp = synth.attention_inputs(17, 1, 633)
    c1 = {k: (v[:333] if v.ndim == 3 else v) for k, v in inp.items()}
    c2 = {k: (v[333:] if v.ndim == 3 else v) for k, v in inp.items()}
    results = []
    for order in ([ga.STAGE_ALL], [ga.STAGE_PROLOGUE, ga.STAGE_ATTENTION, ga.STAGE_APPEND]):
        say(f"[case] fp8 stage order {order}")
        cache, _ = _fp8_cache(O.GLOBAL, 17, [633], 0.8, 0.4)
        for c, s0, n in ((c1, 0, 333), (c2, 333, 300)):
            args = (CFG, cache, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]), dev_bf16(c["q_norm_w"]),
                    dev_bf16(c["k_norm_w"]), dev_bf16(c["gate"]), dev_i32([0, n]), dev_i32([0]), dev_i32([s0]), n)
            out = torch.empty((n, 48, 128), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(ga.prefill_workspace_bytes(CFG, n, 1), dtype=torch.uint8, device="cuda")
            for st in order:
                ga.prefill(*args, out=out, workspace=ws, stages=st)
        sync()
        results.append((host_bits(out), codes(cache.k), codes(cache.v)))
    for a_, b_ in zip(results[0], results[1]):
        assert np.array_equal(a_, b_)


def _fill_codes(t, gen, step=4096):
    """Random cache contents (inputs): N(0,1) values rounded to E4M3 by torch."""
    import torch
    for p0 in range(0, t.shape[0], step):
        blk = t[p0:p0 + step]
        blk.copy_(torch.randn(blk.shape, generator=gen, device=t.device).to(torch.float8_e4m3fn).view(torch.uint8))


def test_fp8_decode_64seq_128k_sampled():
    """The 64-sequence decode at 64K-128K context over an FP8 cache filled with
    seeded random codes (inputs); sampled sequences against the oracle, which
    decodes the codes itself."""
    import torch
    n = 64
    ks, vs = 0.75, 1.25
    ts = synth.decode_positions(3, n, 65536, 131071)
    bt, n_pages = synth.paged_block_table(3, ts.astype(np.int64) + 1)
    say(f"[case] fp8 decode 64 seqs: {n_pages} pages")
    cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt), dtype=ga.KV_FP8_E4M3, k_scale=ks,
                                       v_scale=vs)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    _fill_codes(cache.k, gen)
    _fill_codes(cache.v, gen)
    inp = synth.attention_inputs(cfg=3, layer=7, n_tok=n)
    d = {k: dev_bf16(v) for k, v in inp.items()}
    out = ga.decode(CFG, cache, d["q"], d["q_norm_w"], d["gate"], dev_i32(np.arange(n)), dev_i32(ts), int(ts.max()))
    sync()
    o = host_bits(out)
    assert np.all(np.isfinite(bf16_to_f64(o)))
    cfg = O.Config()
    for sq in (0, int(np.argmax(ts)), 37):
        t = int(ts[sq])
        n_pg = (t + 1 + 15) // 16
        idx = torch.from_numpy(np.ascontiguousarray(bt[sq][:n_pg]).astype(np.int64)).cuda()
        kc = cache.k.index_select(0, idx).permute(0, 2, 1, 3).reshape(n_pg * 16, 8, 128)[:t + 1]
        vc = cache.v.index_select(0, idx).permute(0, 3, 1, 2).reshape(n_pg * 16, 8, 128)[:t + 1]
        kh = O.e4m3_decode(codes(kc)) * ks
        vv = O.e4m3_decode(codes(vc)) * vs
        qn = O.rms_norm(bf16_to_f64(inp["q"][sq])[None], bf16_to_f64(inp["q_norm_w"]), cfg.rms_eps)
        qp, _ = O.position_op(O.GLOBAL, qn, qn, np.array([t]), np.array([t]), cfg)
        ob = O.attend(O.GLOBAL, qp, kh, vv, np.array([t]), np.arange(t + 1), cfg)
        ref = O.output_gate(ob, bf16_to_f64(inp["gate"][sq])[None])
        compare(o[sq:sq + 1], ref, f"fp8 decode seq {sq} t={t}")
