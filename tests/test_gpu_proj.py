"""GPU parity of the projection GEMMs (beam_attn_project, beam_out_project)
against the float64 oracle (oracle.projection), through the C ABI.

* Every output element of a plain product (W_o, and the raw K, V and gate
  heads of the QKV/gate projection) lies within the bound of one float32 sum
  of K products plus one bf16 rounding:
      |got - ref| <= 2^-8 |ref| + 2 K 2^-24 sum_k |x_k w_k|.
* Q' (the query heads finished in the projection's epilogue: RMSNorm, RoPE
  or a(t+1), the base-2 softmax scale) matches the oracle's queries element
  by element within one bf16 rounding plus 1e-3 of the head's RMS, at the
  positions of chunks that start inside a sequence.
* The whole sublayer, x -> projection -> prefill (prologue without Q) ->
  W_o, matches the oracle layer within the attention tolerance (max abs
  2e-2, relative L2 5e-3) over chunked prefill with a cached prefix.
* Full size: T = 32,768 tokens x hidden 5,120 on sampled tokens, in the
  launch configuration the benchmark times.
"""
import numpy as np
import pytest

import global_attention_amd as ga
import synth
from oracle import beam_attention as A
from oracle import projection as P
from tests.helpers import bf16_to_f64, compare, dev_bf16, dev_i32, host_bits, say

pytestmark = pytest.mark.gpu
CFG = ga.Config()
H, G, D = 48, 8, 128
QBASE = np.log2(np.e) / np.sqrt(D)


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


def _check_product(got_bits, x_bits, w_bits, what):
    """Element-wise float32-sum + bf16-rounding bound of got = x W^T."""
    xf, wf = A.bf16_to_f64(x_bits), A.bf16_to_f64(w_bits)
    ref = xf @ wf.T
    s = np.abs(xf) @ np.abs(wf).T
    k = xf.shape[1]
    got = bf16_to_f64(got_bits).reshape(ref.shape)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2 * k * 2.0 ** -24 * s + 1e-30
    say(f"[parity] {what}: max_err={err.max():.3e} max_err/bound={np.max(err / bound):.3f}")
    assert np.all(err <= bound), f"{what}: {np.sum(err > bound)} elements outside the bound"


def _queries_region(ws, n_tok):
    import torch
    return host_bits(ws[: n_tok * H * D * 2].view(torch.bfloat16)).reshape(n_tok, H, D)


def _check_qprime(got_bits, want, what):
    """want: oracle Q' [n, H, d] in float64 (softmax scale included)."""
    got = bf16_to_f64(got_bits)
    rms = np.sqrt(np.mean(want ** 2, axis=-1, keepdims=True))
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 1e-3 * rms
    say(f"[parity] {what}: max_err={err.max():.3e} max_err/bound={np.max(err / bound):.3f}")
    assert np.all(err <= bound), f"{what}: {np.sum(err > bound)} elements outside the bound"


@pytest.mark.parametrize("n_tok,k,n_out", [(300, 6144, 5120), (513, 128, 256), (1, 128, 512), (256, 384, 768)])
def test_out_project_within_fp32_bound(n_tok, k, n_out):
    y = synth.normal_bf16((n_tok, k), 50, 0)
    w = synth.normal_bf16((n_out, k), 50, 1, scale=k ** -0.5)
    say(f"[case] out_project n_tok={n_tok} k={k} n_out={n_out}")
    out = ga.out_project(dev_bf16(y), dev_bf16(w))
    sync()
    _check_product(host_bits(out), y, w, f"out_project {n_tok}x{k}->{n_out}")


def _positions(cu, starts):
    return np.concatenate([np.arange(s, s + (cu[i + 1] - cu[i])) for i, s in enumerate(starts)])


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_project_outputs(kind):
    """Two chunks (300 and 213 tokens) starting at positions 0 and 1,000;
    hidden 1,024."""
    lens, starts, hidden = [300, 213], [0, 1000], 1024
    n = sum(lens)
    inp = synth.projection_inputs(51, kind, n, hidden=hidden, with_w_o=False)
    cu = np.array([0, lens[0], n], np.int32)
    say(f"[case] attn_project kind={kind} lens={lens} starts={starts}")
    k_raw, v_raw, gate, ws = ga.attn_project(CFG, kind, dev_bf16(inp["x"]), dev_bf16(inp["w_qkvg"]),
                                             dev_bf16(inp["q_norm_w"]), dev_i32(cu), dev_i32(starts))
    sync()
    rows = np.cumsum([0, H * D, G * D, G * D, H * D])
    w = inp["w_qkvg"]
    _check_product(host_bits(k_raw), inp["x"], w[rows[1]:rows[2]], "K")
    _check_product(host_bits(v_raw), inp["x"], w[rows[2]:rows[3]], "V")
    _check_product(host_bits(gate), inp["x"], w[rows[3]:rows[4]], "gate")
    q, _, _, _ = P.project_qkvg(inp["x"], w)
    want = P.queries_prime(kind, q, inp["q_norm_w"], _positions(cu, starts)) * QBASE
    _check_qprime(_queries_region(ws, n), want, f"Q' kind={kind}")


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_sublayer_chunked_matches_oracle(kind):
    """x -> projection -> prefill without the query prologue -> W_o, in two
    chunked steps over two sequences; the second step attends to the cache."""
    import torch
    total, hidden = [450, 290], 512
    steps = [[300, 213], [150, 77]]
    inps = [synth.projection_inputs(52, 10 * kind + i, n, hidden=hidden) for i, n in enumerate(total)]
    for x in inps[1:]:
        for key in ("w_qkvg", "w_o", "q_norm_w", "k_norm_w"):
            x[key] = inps[0][key]
    w = inps[0]
    if kind == A.GLOBAL:
        bt, n_pages = synth.paged_block_table(52, total, extra_pages=2)
        cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    else:
        cache = ga.KVCache.allocate_local(CFG, 2)
    # oracle: float64 projections of every token, then the layer per chunk
    proj = [P.project_qkvg(x["x"], w["w_qkvg"]) for x in inps]
    done = [0, 0]
    for step, lens in enumerate(steps):
        starts = list(done)
        xs = np.concatenate([inps[i]["x"][starts[i]:starts[i] + n] for i, n in enumerate(lens)])
        cu = np.array([0, lens[0], sum(lens)], np.int32)
        say(f"[case] sublayer kind={kind} step={step} starts={starts} lens={lens}")
        k_raw, v_raw, gate, ws = ga.attn_project(CFG, kind, dev_bf16(xs), dev_bf16(w["w_qkvg"]),
                                                 dev_bf16(w["q_norm_w"]), dev_i32(cu), dev_i32(starts))
        y = ga.prefill(CFG, cache, None, k_raw, v_raw, dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]), gate,
                       dev_i32(cu), dev_i32([0, 1]), dev_i32(starts), max(lens), workspace=ws,
                       stages=ga.STAGE_PROLOGUE_KV | ga.STAGE_ATTENTION | ga.STAGE_APPEND)
        out = ga.out_project(y, dev_bf16(w["w_o"]))
        sync()
        yb, ob = host_bits(y), host_bits(out)
        for i, n in enumerate(lens):
            s0 = starts[i]
            q, k, v, g = proj[i]
            ref_y = P.attention_from_projections(kind, q[s0:s0 + n], k[:s0 + n], v[:s0 + n], g[s0:s0 + n],
                                                 w["q_norm_w"], w["k_norm_w"], np.arange(s0, s0 + n),
                                                 np.arange(s0 + n))
            compare(yb[cu[i]:cu[i + 1]], ref_y, f"sublayer Y kind={kind} seq{i} [{s0},{s0 + n})")
            compare(ob[cu[i]:cu[i + 1]], P.output_projection(ref_y, w["w_o"]),
                    f"sublayer out kind={kind} seq{i} [{s0},{s0 + n})")
            done[i] += n


def test_project_full_size_sampled():
    """T = 32,768, hidden 5,120 (the benchmark's launch): 48 sampled tokens of
    every output, and 48 sampled rows of W_o over the 6,144-wide gated input."""
    import torch
    T, hidden = 32768, 5120
    inp = synth.projection_inputs(53, 1, T, hidden=hidden)
    cu = np.array([0, T], np.int32)
    say("[case] attn_project full size T=32768 global")
    x = dev_bf16(inp["x"])
    k_raw, v_raw, gate, ws = ga.attn_project(CFG, A.GLOBAL, x, dev_bf16(inp["w_qkvg"]), dev_bf16(inp["q_norm_w"]),
                                             dev_i32(cu), dev_i32([0]))
    sync()
    rows = np.sort(np.random.default_rng(9).choice(T, 48, replace=False))
    rows[-1] = T - 1
    w = inp["w_qkvg"]
    b = np.cumsum([0, H * D, G * D, G * D, H * D])
    xr = inp["x"][rows]
    ri = torch.from_numpy(rows).cuda()
    _check_product(host_bits(k_raw[ri]), xr, w[b[1]:b[2]], "K full")
    _check_product(host_bits(v_raw[ri]), xr, w[b[2]:b[3]], "V full")
    _check_product(host_bits(gate[ri]), xr, w[b[3]:b[4]], "gate full")
    q, _, _, _ = P.project_qkvg(xr, w)
    want = P.queries_prime(A.GLOBAL, q, inp["q_norm_w"], rows) * QBASE
    qall = ws[: T * H * D * 2].view(torch.bfloat16).view(T, H, D)
    _check_qprime(host_bits(qall[ri]), want, "Q' full")
    say("[case] out_project full size 32768 x 6144 -> 5120")
    y = gate.view(T, H * D)  # any bf16 [T][6144] input
    out = ga.out_project(y, dev_bf16(inp["w_o"]))
    sync()
    _check_product(host_bits(out[ri]), host_bits(y[ri]), inp["w_o"], "W_o full")


def test_project_many_sequences_and_empty_chunks():
    """Six chunks, two of them empty, at scattered start positions (the
    epilogue finds each token's sequence and position); local layer, so every
    query head is rotated at its own position."""
    lens = [5, 0, 130, 1, 0, 300]
    starts = [0, 7, 4095, 70000, 12, 1]
    hidden, n = 256, sum(lens)
    inp = synth.projection_inputs(54, 0, n, hidden=hidden, with_w_o=False)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    say(f"[case] attn_project many sequences lens={lens} starts={starts}")
    k_raw, v_raw, gate, ws = ga.attn_project(CFG, A.LOCAL, dev_bf16(inp["x"]), dev_bf16(inp["w_qkvg"]),
                                             dev_bf16(inp["q_norm_w"]), dev_i32(cu), dev_i32(starts))
    sync()
    q, _, _, _ = P.project_qkvg(inp["x"], inp["w_qkvg"])
    want = P.queries_prime(A.LOCAL, q, inp["q_norm_w"], _positions(cu, starts)) * QBASE
    _check_qprime(_queries_region(ws, n), want, "Q' many sequences")
    rows = np.cumsum([0, H * D, G * D, G * D, H * D])
    _check_product(host_bits(gate), inp["x"], inp["w_qkvg"][rows[3]:rows[4]], "gate many sequences")
