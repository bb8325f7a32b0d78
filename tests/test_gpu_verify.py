"""GPU parity of the verify step (a short chunk per sequence over its cache,
the step that checks a speculative draft) through the C ABI, against the
float64 oracle.

The drafter's block is 8 tokens in the serving recipe ("Beam 1.0 auf vier
B300s", orcarouter.ai) and up to 15 on news.hamidun.com; chunks here run from
1 to 21 tokens (the kernel's limit at 48/8 heads). The step has prefill
semantics, so the reference is the oracle's attention layer over the cached
history plus the chunk. Tolerances on bf16 outputs: max-abs 2e-2 and relative
L2 5e-3; the cache after a verify call must equal, bit for bit, the cache after
a prefill call of the same chunk.
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
SENT = 0x7F7F


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


def _cache(kind, cfg_id, ctx, fp8=None):
    import torch
    kw = {} if fp8 is None else dict(dtype=ga.KV_FP8_E4M3, k_scale=fp8[0], v_scale=fp8[1])
    fill = SENT if fp8 is None else 0x55
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(cfg_id, ctx, extra_pages=3)
        return ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt), fill=fill, **kw), bt
    return ga.KVCache.allocate_local(CFG, len(ctx), fill=fill, **kw), None


def _slice(inp, s0, n):
    return {k: (v[s0:s0 + n] if v.ndim == 3 else v) for k, v in inp.items()}


def _packed(batch):
    lens = [b["q"].shape[0] for b in batch]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cat = lambda key: dev_bf16(np.concatenate([b[key] for b in batch]))
    return lens, cu, cat


def _call(fn, cache, batch, starts, seqs, **kw):
    lens, cu, cat = _packed(batch)
    w = batch[0]
    out = fn(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]),
             cat("gate"), dev_i32(cu), dev_i32(seqs), dev_i32(starts), max(lens), **kw)
    sync()
    o = host_bits(out)
    return [o[cu[i]:cu[i + 1]] for i in range(len(lens))]


def _verify(cache, batch, starts, seqs, split_keys=0):
    max_pos = max(s + b["q"].shape[0] - 1 for s, b in zip(starts, batch))
    return _call(ga.verify, cache, batch, starts, seqs, max_pos=max_pos, split_keys=split_keys)


def _prefill(cache, batch, starts, seqs):
    return _call(ga.prefill, cache, batch, starts, seqs)


# History lengths (positions already cached) and the verify chunks of three
# steps per sequence: unaligned histories, a chunk across a 64-key tile
# boundary (63 + 8), a history of one token and one of none.
HIST = [1500, 700, 63, 1, 0]
STEPS = [[8, 1, 21, 15, 3], [15, 21, 3, 8, 1], [1, 8, 16, 2, 21]]


def _inputs(cfg_id, kind):
    total = [h + sum(s[i] for s in STEPS) for i, h in enumerate(HIST)]
    inps = [synth.attention_inputs(cfg_id, 10 * kind + i, n) for i, n in enumerate(total)]
    for x in inps[1:]:
        x["q_norm_w"], x["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    return total, inps


@pytest.mark.parametrize("fp8", [None, (0.6, 0.9)], ids=["bf16", "fp8"])
@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_chunks_over_cached_history(kind, fp8):
    total, inps = _inputs(20, kind)
    # cache rows permuted against the batch order
    rows = [3, 0, 4, 1, 2]
    cache, _ = _cache(kind, 20, [total[i] for i in np.argsort(rows)], fp8)
    hist = [i for i, h in enumerate(HIST) if h > 0]
    say(f"[case] verify kind={kind} fp8={fp8}: prefill history {HIST}")
    _prefill(cache, [_slice(inps[i], 0, HIST[i]) for i in hist], [0] * len(hist), [rows[i] for i in hist])
    done = list(HIST)
    for step, chunk in enumerate(STEPS):
        batch = [_slice(inps[i], done[i], chunk[i]) for i in range(len(HIST))]
        sk = 64 if step == 1 else 0  # one key tile per split, then the default
        say(f"[case] verify kind={kind} fp8={fp8} step={step} starts={done} lens={chunk} split={sk}")
        outs = _verify(cache, batch, list(done), rows, split_keys=sk)
        for i, o in enumerate(outs):
            s0, n, x = done[i], chunk[i], inps[i]
            ref = O.attention_layer(kind, x["q"][s0:s0 + n], x["k"][:s0 + n], x["v"][:s0 + n], x["q_norm_w"],
                                    x["k_norm_w"], x["gate"][s0:s0 + n], np.arange(s0, s0 + n),
                                    np.arange(s0 + n), fp8_cache=None if fp8 is None else (*fp8, s0))
            compare(o, ref, f"verify step{step} seq{i} [{s0},{s0 + n})")
        done = [d + c for d, c in zip(done, chunk)]


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_and_prefill_leave_identical_caches(kind):
    """The same chunks through verify (cache A) and prefill (cache B): the two
    caches match bit for bit after every step, and both outputs pass the
    oracle tolerance against each other's reference."""
    total, inps = _inputs(21, kind)
    rows = list(range(len(HIST)))
    ca, _ = _cache(kind, 21, total)
    cb, _ = _cache(kind, 21, total)
    hist = [i for i, h in enumerate(HIST) if h > 0]
    for c in (ca, cb):
        _prefill(c, [_slice(inps[i], 0, HIST[i]) for i in hist], [0] * len(hist), hist)
    done = list(HIST)
    for step, chunk in enumerate(STEPS):
        batch = [_slice(inps[i], done[i], chunk[i]) for i in range(len(HIST))]
        say(f"[case] verify vs prefill kind={kind} step={step}")
        ov = _verify(ca, batch, list(done), rows)
        op = _prefill(cb, batch, list(done), rows)
        assert np.array_equal(host_bits(ca.k), host_bits(cb.k)), f"K differs after step {step}"
        assert np.array_equal(host_bits(ca.v), host_bits(cb.v)), f"V differs after step {step}"
        for i in range(len(HIST)):
            compare(ov[i], bf16_to_f64(op[i]), f"verify vs prefill step{step} seq{i}")
        done = [d + c for d, c in zip(done, chunk)]


# ------------------------------------------------------------- 64 x 128K, draft of 8

def _fill_random(t, gen, step=8192):
    for p0 in range(0, t.shape[0], step):
        t[p0:p0 + step].normal_(generator=gen)


def _gather_global(cache, bt_row, n_keys):
    """Host float64 copy of K_hat/V of one sequence's first n_keys positions,
    all KV heads, in logical order: [n_keys, 8, 128]."""
    import torch
    n_pg = (n_keys + 15) // 16
    idx = torch.from_numpy(np.ascontiguousarray(bt_row[:n_pg]).astype(np.int64)).cuda()
    k = cache.k.index_select(0, idx).permute(0, 2, 1, 3).reshape(n_pg * 16, 8, 128)[:n_keys]
    v = cache.v.index_select(0, idx).permute(0, 3, 1, 2).reshape(n_pg * 16, 8, 128)[:n_keys]
    return bf16_to_f64(host_bits(k.contiguous())), bf16_to_f64(host_bits(v.contiguous()))


def _gather_ring(cache, sq):
    """Host float64 copy of one sequence's ring: K_hat, V as [slot, 8, 128]."""
    k = cache.k[sq].permute(1, 0, 2).contiguous()
    v = cache.v[sq].permute(2, 0, 1).contiguous()
    return bf16_to_f64(host_bits(k)), bf16_to_f64(host_bits(v))


def _chunk_oracle(kind, x, start, kh_prev, v_prev, pos_prev):
    """Oracle of one sequence's chunk given the cache contents before the call."""
    n = x["q"].shape[0]
    tq = start + np.arange(n)
    qn = O.rms_norm(bf16_to_f64(x["q"]), bf16_to_f64(x["q_norm_w"]), OCFG.rms_eps)
    qp, _ = O.position_op(kind, qn, qn, tq, tq, OCFG)
    kh = np.concatenate([kh_prev, O.cached_key(kind, x["k"], x["k_norm_w"], tq)])
    v = np.concatenate([v_prev, bf16_to_f64(x["v"])])
    pos = np.concatenate([pos_prev, tq])
    return O.output_gate(O.attend(kind, qp, kh, v, tq, pos, OCFG), bf16_to_f64(x["gate"]))


def test_verify_64seq_128k_draft8_sampled():
    import torch
    n, L = 64, 8
    starts = synth.decode_positions(3, n, 65536, 131071 - L)
    bt, n_pages = synth.paged_block_table(3, starts.astype(np.int64) + L)
    say(f"[case] verify 64 seqs x {L} tokens: {n_pages} pages")
    gcache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    lcache = ga.KVCache.allocate_local(CFG, n)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    for t in (gcache.k, gcache.v, lcache.k, lcache.v):
        _fill_random(t, gen)
    inp = synth.attention_inputs(cfg=3, layer=9, n_tok=n * L)
    batch = [_slice(inp, L * i, L) for i in range(n)]
    sample = (0, int(np.argmax(starts)), 37)
    for name, cache, kind in (("global", gcache, O.GLOBAL), ("local", lcache, O.LOCAL)):
        before = {sq: _gather_ring(cache, sq) for sq in sample} if kind == O.LOCAL else None
        say(f"[case] verify 64 seqs {name}: launching")
        outs = _verify(cache, batch, [int(s) for s in starts], list(range(n)))
        assert all(np.all(np.isfinite(bf16_to_f64(o))) for o in outs)
        for sq in sample:
            s0 = int(starts[sq])
            if kind == O.GLOBAL:
                kh, v = _gather_global(cache, bt[sq], s0)
                pos = np.arange(s0)
            else:
                kh, v = before[sq]
                slots = np.arange(512)
                pos = (s0 - 1) - ((s0 - 1 - slots) % 512)  # position each slot held before the call
            ref = _chunk_oracle(kind, batch[sq], s0, kh, v, pos)
            compare(outs[sq], ref, f"verify {name} seq {sq} start={s0}")
    del gcache, lcache


def _gather_global_codes(cache, bt_row, n_keys):
    """Host float64 K_hat/V of one sequence's first n_keys positions from an
    FP8 cache: the codes decoded by the oracle, times the scales: [n_keys, 8, 128]."""
    import torch
    n_pg = (n_keys + 15) // 16
    idx = torch.from_numpy(np.ascontiguousarray(bt_row[:n_pg]).astype(np.int64)).cuda()
    k = cache.k.index_select(0, idx).permute(0, 2, 1, 3).reshape(n_pg * 16, 8, 128)[:n_keys]
    v = cache.v.index_select(0, idx).permute(0, 3, 1, 2).reshape(n_pg * 16, 8, 128)[:n_keys]
    kc, vc = k.contiguous().cpu().numpy(), v.contiguous().cpu().numpy()
    return O.e4m3_decode(kc) * cache.k_scale, O.e4m3_decode(vc) * cache.v_scale


def test_verify_64seq_128k_draft8_fp8_sampled():
    """The full-size verify step over an FP8 cache of seeded random codes
    (inputs), 8-token drafts: the one-wave kernel that holds all 48 (token,
    head) rows of a chunk. Three sampled sequences against the oracle, which
    decodes the cached codes itself."""
    import torch
    n, L = 64, 8
    starts = synth.decode_positions(3, n, 65536, 131071 - L)
    bt, n_pages = synth.paged_block_table(3, starts.astype(np.int64) + L)
    say(f"[case] verify 64 seqs x {L} tokens over an FP8 cache: {n_pages} pages")
    cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt), dtype=ga.KV_FP8_E4M3, k_scale=0.6,
                                       v_scale=0.9)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(33)
    for t in (cache.k, cache.v):
        for p0 in range(0, t.shape[0], 8192):
            blk = t[p0:p0 + 8192]
            blk.copy_(torch.randn(blk.shape, generator=gen, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8))
    inp = synth.attention_inputs(cfg=33, layer=9, n_tok=n * L)
    batch = [_slice(inp, L * i, L) for i in range(n)]
    sample = (0, int(np.argmax(starts)), 41)
    say("[case] verify 64 seqs fp8: launching")
    outs = _verify(cache, batch, [int(s) for s in starts], list(range(n)))
    assert all(np.all(np.isfinite(bf16_to_f64(o))) for o in outs)
    for sq in sample:
        s0 = int(starts[sq])
        kh, v = _gather_global_codes(cache, bt[sq], s0)
        ref = _chunk_oracle(O.GLOBAL, batch[sq], s0, kh, v, np.arange(s0))
        compare(outs[sq], ref, f"verify fp8 seq {sq} start={s0}")
    del cache


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_fp8_short_chunks_both_block_shapes(kind):
    """Chunks of at most 10 tokens (at most 64 rows of a KV head) over an FP8
    cache run in two-wave blocks; the same call with max_chunk_len 11 runs in
    four-wave blocks. Both must equal each other bit for bit (every row does the
    same arithmetic in either shape) and match the oracle."""
    import torch
    fp8 = (0.6, 0.9)
    hist = [700, 130, 64, 1]
    steps = [[8, 1, 10, 3], [2, 10, 7, 8]]
    total = [h + sum(st[i] for st in steps) for i, h in enumerate(hist)]
    inps = [synth.attention_inputs(34, 10 * kind + i, m) for i, m in enumerate(total)]
    for x in inps[1:]:
        x["q_norm_w"], x["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    caches = [_cache(kind, 34, total, fp8)[0] for _ in range(2)]
    for c in caches:
        _prefill(c, [_slice(inps[i], 0, hist[i]) for i in range(len(hist))], [0] * len(hist), list(range(len(hist))))
    done = list(hist)
    for step, chunk in enumerate(steps):
        batch = [_slice(inps[i], done[i], chunk[i]) for i in range(len(hist))]
        max_pos = max(s + b["q"].shape[0] - 1 for s, b in zip(done, batch))
        say(f"[case] verify fp8 kind={kind} step={step} lens={chunk}: two-wave and four-wave blocks")
        o2 = _call(ga.verify, caches[0], batch, list(done), list(range(len(hist))), max_pos=max_pos)
        lens, cu, cat = _packed(batch)
        w = batch[0]
        out = ga.verify(CFG, caches[1], cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]),
                        dev_bf16(w["k_norm_w"]), cat("gate"), dev_i32(cu), dev_i32(list(range(len(hist)))),
                        dev_i32(done), 11, max_pos)
        sync()
        o4 = host_bits(out)
        for i, o in enumerate(o2):
            assert np.array_equal(o, o4[cu[i]:cu[i + 1]]), f"step {step} seq {i}: block shapes differ"
            s0, m, x = done[i], chunk[i], inps[i]
            ref = O.attention_layer(kind, x["q"][s0:s0 + m], x["k"][:s0 + m], x["v"][:s0 + m], x["q_norm_w"],
                                    x["k_norm_w"], x["gate"][s0:s0 + m], np.arange(s0, s0 + m), np.arange(s0 + m),
                                    fp8_cache=(*fp8, s0))
            compare(o, ref, f"verify fp8 kind={kind} step{step} seq{i} [{s0},{s0 + m})")
        done = [d + c for d, c in zip(done, chunk)]


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_fp8_48_row_kernel(kind):
    """Chunks of at most 8 tokens (48 rows of a KV head) over an FP8 cache run
    in the one-wave kernel (three 16-row column blocks of 16x16x32 MFMA); the
    same call with max_chunk_len 9 runs in the two-wave 32x32x16 kernel. Both
    are compared with the oracle and with each other (the MFMA shapes sum in
    different orders, so not bit for bit). Histories of 700, 130, 60 (the
    8-token chunk crosses a 64-key tile), 1 and 0 tokens; one step with
    64-key splits (one tile per split, partials and combine), one with the
    default split."""
    fp8 = (0.6, 0.9)
    hist = [700, 130, 60, 1, 0]
    steps = [[8, 1, 8, 3, 5], [2, 8, 7, 8, 1]]
    total = [h + sum(st[i] for st in steps) for i, h in enumerate(hist)]
    inps = [synth.attention_inputs(36, 10 * kind + i, m) for i, m in enumerate(total)]
    for x in inps[1:]:
        x["q_norm_w"], x["k_norm_w"] = inps[0]["q_norm_w"], inps[0]["k_norm_w"]
    caches = [_cache(kind, 36, total, fp8)[0] for _ in range(2)]
    hs = [i for i, h in enumerate(hist) if h > 0]
    for c in caches:
        _prefill(c, [_slice(inps[i], 0, hist[i]) for i in hs], [0] * len(hs), hs)
    done = list(hist)
    for step, chunk in enumerate(steps):
        batch = [_slice(inps[i], done[i], chunk[i]) for i in range(len(hist))]
        max_pos = max(s + b["q"].shape[0] - 1 for s, b in zip(done, batch))
        sk = 64 if step == 0 else 0
        say(f"[case] verify fp8 kind={kind} step={step} lens={chunk} split={sk}: 48-row and two-wave kernels")
        o1 = _call(ga.verify, caches[0], batch, list(done), list(range(len(hist))), max_pos=max_pos, split_keys=sk)
        lens, cu, cat = _packed(batch)
        w = batch[0]
        out = ga.verify(CFG, caches[1], cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]),
                        dev_bf16(w["k_norm_w"]), cat("gate"), dev_i32(cu), dev_i32(list(range(len(hist)))),
                        dev_i32(done), 9, max_pos, split_keys=sk)
        sync()
        o2 = host_bits(out)
        for i, o in enumerate(o1):
            s0, m, x = done[i], chunk[i], inps[i]
            ref = O.attention_layer(kind, x["q"][s0:s0 + m], x["k"][:s0 + m], x["v"][:s0 + m], x["q_norm_w"],
                                    x["k_norm_w"], x["gate"][s0:s0 + m], np.arange(s0, s0 + m), np.arange(s0 + m),
                                    fp8_cache=(*fp8, s0))
            compare(o, ref, f"verify fp8 48-row kind={kind} step{step} seq{i} [{s0},{s0 + m})")
            compare(o2[cu[i]:cu[i + 1]], ref, f"verify fp8 two-wave kind={kind} step{step} seq{i}")
            a, b = bf16_to_f64(o), bf16_to_f64(o2[cu[i]:cu[i + 1]])
            assert np.max(np.abs(a - b)) <= 2e-2, f"step {step} seq {i}: the two kernels differ"
        done = [d + c for d, c in zip(done, chunk)]


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_accept_and_roll_back(kind):
    """An 8-token draft of which 3 tokens are accepted, then a new draft from
    the first rejected position. Global: the call appends all 8 and the next
    chunk overwrites the rejected slots. Local: verify without the append
    stage, then the accepted tokens go in with kv_append."""
    hist, draft, acc = 900, 8, 3
    x = synth.attention_inputs(22, 10 * kind, hist + draft)          # history + first draft
    y = synth.attention_inputs(23, 10 * kind, draft)                 # second draft
    y["q_norm_w"], y["k_norm_w"] = x["q_norm_w"], x["k_norm_w"]
    cache, _ = _cache(kind, 22, [hist + acc + draft])
    _prefill(cache, [_slice(x, 0, hist)], [0], [0])
    stages = ga.STAGE_VERIFY_ALL if kind == O.GLOBAL else ga.STAGE_VERIFY_ALL & ~ga.STAGE_APPEND

    def run(chunk, s0):
        lens, cu, cat = _packed([chunk])
        out = ga.verify(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(chunk["q_norm_w"]),
                        dev_bf16(chunk["k_norm_w"]), cat("gate"), dev_i32(cu), dev_i32([0]), dev_i32([s0]), draft,
                        s0 + draft - 1, stages=stages)
        sync()
        if kind == O.LOCAL:  # append the accepted tokens only
            ga.kv_append(CFG, cache, dev_bf16(chunk["k"][:acc]), dev_bf16(chunk["v"][:acc]),
                         dev_bf16(chunk["k_norm_w"]), dev_i32([0] * acc), dev_i32(np.arange(s0, s0 + acc)))
            sync()
        return host_bits(out)

    say(f"[case] verify accept/roll back kind={kind}: first draft at {hist}")
    o1 = run(_slice(x, hist, draft), hist)
    ref1 = O.attention_layer(kind, x["q"][hist:], x["k"], x["v"], x["q_norm_w"], x["k_norm_w"], x["gate"][hist:],
                             np.arange(hist, hist + draft), np.arange(hist + draft))
    compare(o1, ref1, f"first draft kind={kind}")
    s1 = hist + acc
    say(f"[case] verify accept/roll back kind={kind}: second draft at {s1}")
    o2 = run(y, s1)
    k_all = np.concatenate([x["k"][:s1], y["k"]])
    v_all = np.concatenate([x["v"][:s1], y["v"]])
    ref2 = O.attention_layer(kind, y["q"], k_all, v_all, y["q_norm_w"], y["k_norm_w"], y["gate"],
                             np.arange(s1, s1 + draft), np.arange(s1 + draft))
    compare(o2, ref2, f"second draft kind={kind}")
