"""GPU parity of the per-head gate bias, Y = O * sigmoid(G + b_h).

"Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax" (flozi.net, English),
section "Follow the tensors, not the parameter label": the gate is one value
per coordinate of every query head, plus an additive bias with one value per
head. The workload configurations pass no bias; these tests pass a seeded
float32 bias b ~ 0.5*N(0,1) [48] to every entry point that applies the gate
(prefill, decode at two split sizes, the verify step), for both layer kinds,
and compare every output element with the float64 oracle given the same bias
(max-abs 2e-2, relative L2 5e-3). A swapped or dropped bias moves sigmoid by
up to ~0.25 per coordinate and fails the tolerance on its own.
"""
import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O
import synth
from tests.helpers import compare, dev_bf16, dev_i32, host_bits, say

pytestmark = pytest.mark.gpu
CFG = ga.Config()


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


def _bias(layer):
    import torch
    b = synth.gate_bias(60, layer)
    return b, torch.from_numpy(b).cuda()


def _cache(kind, cfg_id, ctx):
    import torch
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(cfg_id, ctx, extra_pages=2)
        return ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    return ga.KVCache.allocate_local(CFG, len(ctx))


def _ref(kind, x, q0, q1, bias):
    return O.attention_layer(kind, x["q"][q0:q1], x["k"][:q1], x["v"][:q1], x["q_norm_w"], x["k_norm_w"],
                             x["gate"][q0:q1], np.arange(q0, q1), np.arange(q1), gate_bias=bias)


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_prefill_t640_gate_bias(kind):
    T = 640
    x = synth.attention_inputs(61, kind, T)
    b, bd = _bias(kind)
    cache = _cache(kind, 61, [T])
    say(f"[case] prefill T=640 kind={kind} with gate bias")
    out = ga.prefill(CFG, cache, dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), dev_bf16(x["q_norm_w"]),
                     dev_bf16(x["k_norm_w"]), dev_bf16(x["gate"]), dev_i32([0, T]), dev_i32([0]), dev_i32([0]), T,
                     gate_bias=bd)
    sync()
    ref = _ref(kind, x, 0, T, b)
    compare(host_bits(out), ref, f"prefill T=640 kind={kind} gate bias")
    # the bias matters: without it the same output is out of tolerance
    ref0 = _ref(kind, x, 0, T, None)
    err0 = np.linalg.norm(ref - ref0) / np.linalg.norm(ref)
    assert err0 > 20 * 5e-3, err0


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_decode_gate_bias(kind):
    ts = [0, 17, 511, 512, 1300, 2999]
    hist = [synth.attention_inputs(62, 10 * kind + i, t + 1) for i, t in enumerate(ts)]
    for x in hist[1:]:
        x["q_norm_w"], x["k_norm_w"] = hist[0]["q_norm_w"], hist[0]["k_norm_w"]
    cache = _cache(kind, 62, [t + 1 for t in ts])
    for i, t in enumerate(ts):
        lo = 0 if kind == O.GLOBAL else max(0, t + 1 - 512)
        ga.kv_append(CFG, cache, dev_bf16(hist[i]["k"][lo:]), dev_bf16(hist[i]["v"][lo:]),
                     dev_bf16(hist[0]["k_norm_w"]), dev_i32(np.full(t + 1 - lo, i)), dev_i32(np.arange(lo, t + 1)))
    b, bd = _bias(10 + kind)
    q = np.stack([x["q"][t] for x, t in zip(hist, ts)])
    gate = np.stack([x["gate"][t] for x, t in zip(hist, ts)])
    ref = np.concatenate([_ref(kind, x, t, t + 1, b) for x, t in zip(hist, ts)])
    for sk in (128, 0):
        say(f"[case] decode kind={kind} split_keys={sk} with gate bias")
        out = ga.decode(CFG, cache, dev_bf16(q), dev_bf16(hist[0]["q_norm_w"]), dev_bf16(gate),
                        dev_i32(np.arange(len(ts))), dev_i32(ts), max(ts), gate_bias=bd, split_keys=sk)
        sync()
        compare(host_bits(out), ref, f"decode kind={kind} split={sk} gate bias")


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_verify_gate_bias(kind):
    hist_len, chunk = [900, 64, 0], [8, 15, 5]
    total = [h + c for h, c in zip(hist_len, chunk)]
    xs = [synth.attention_inputs(63, 10 * kind + i, n) for i, n in enumerate(total)]
    for x in xs[1:]:
        x["q_norm_w"], x["k_norm_w"] = xs[0]["q_norm_w"], xs[0]["k_norm_w"]
    cache = _cache(kind, 63, total)
    w = xs[0]
    # history by prefill (no bias involved), then one verify chunk with the bias
    hs = [i for i, h in enumerate(hist_len) if h > 0]
    lens = [hist_len[i] for i in hs]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cat = lambda key: dev_bf16(np.concatenate([xs[i][key][:hist_len[i]] for i in hs]))
    ga.prefill(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]),
               cat("gate"), dev_i32(cu), dev_i32(hs), dev_i32([0] * len(hs)), max(lens))
    b, bd = _bias(20 + kind)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    cat = lambda key: dev_bf16(np.concatenate([x[key][h:h + c] for x, h, c in zip(xs, hist_len, chunk)]))
    say(f"[case] verify kind={kind} with gate bias")
    out = ga.verify(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]),
                    cat("gate"), dev_i32(cu), dev_i32([0, 1, 2]), dev_i32(hist_len), max(chunk),
                    max(t - 1 for t in total), gate_bias=bd)
    sync()
    o = host_bits(out)
    for i, (x, h, c) in enumerate(zip(xs, hist_len, chunk)):
        compare(o[cu[i]:cu[i + 1]], _ref(kind, x, h, h + c, b), f"verify kind={kind} seq{i} gate bias")
