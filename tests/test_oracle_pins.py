"""Pins for the CPU oracle: printed numbers, closed forms, invariants, brute force.

Every check here ties the oracle to something other than itself, so that a
plausible mistake (a dropped term, a wrong sign or index, an off-by-one
position, a transposed operand) fails at least one of them. CPU only.
"""
import math
import os

import numpy as np
import pytest

import oracle as O
from synth import f32_to_bf16_bits, bf16_bits_to_f32, attention_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


# ------------------------------------------------------------ printed numbers

def test_ssmax_printed_scales():
    """a(p) at the three printed one-based positions, to the printed decimals."""
    for p, val, dec in _rows("ssmax_scales.txt"):
        t = int(p) - 1                      # oracle takes the zero-based position
        got = float(O.ssmax_scale(t))
        assert round(got, int(dec)) == float(val), (p, got)
    # Sensitivity: if the oracle used p = t (zero-based) the first value would
    # print as 1.0717, so the one-based reading is what the page fixes.
    assert round(float(O.ssmax_scale(2047 - 1)), 4) != 1.0718


def test_ssmax_closed_forms():
    # (1 + 2048/2048)^0.1 = 2^0.1, (1 + 65536/2048)^0.1 = 33^0.1, 513^0.1
    assert float(O.ssmax_scale(2047)) == pytest.approx(2.0 ** 0.1, rel=1e-15)
    assert float(O.ssmax_scale(65535)) == pytest.approx(33.0 ** 0.1, rel=1e-15)
    assert float(O.ssmax_scale(1048575)) == pytest.approx(513.0 ** 0.1, rel=1e-15)
    # monotone increasing in position, and a(1) just above one
    a = O.ssmax_scale(np.arange(0, 100000, 997))
    assert np.all(np.diff(a) > 0) and 1.0 < a[0] < 1.0001


def test_kv_budget_printed():
    units = {"KiB": 2 ** 10, "MiB": 2 ** 20, "GiB": 2 ** 30}
    for name, n, b, ng, nl, val, unit, dec in _rows("kv_budget.txt"):
        logical, _ = O.kv_bytes(int(n), int(b), n_global=int(ng), n_local=int(nl))
        got = logical / units[unit]
        assert round(got, int(dec)) == pytest.approx(float(val)), (name, got)


def test_kv_bytes_exact_integers():
    # 36 KiB per token exactly; 1M tokens: 36 GiB + 43 local caches of 512 slots
    assert O.kv_bytes(1, 2, 9, 0)[0] == 36864
    logical, paged = O.kv_bytes(1048576, 2)
    assert logical == 36 * 2 ** 30 + 43 * 512 * 4096
    assert paged == logical                     # 1M is a whole number of 16-token pages
    # page rounding of the global term only
    logical, paged = O.kv_bytes(17, 2)
    assert logical == 4096 * (9 * 17 + 43 * 17)
    assert paged == 4096 * (9 * 32 + 43 * 17)
    # the local term saturates at the window
    assert O.kv_bytes(513, 2, 0, 43)[0] == O.kv_bytes(10 ** 6, 2, 0, 43)[0] == 43 * 512 * 4096


def test_layer_schedule_printed():
    rows = {r[0]: r[1:] for r in _rows("layer_schedule.txt")}
    kinds = O.layer_kinds(int(rows["n_layers"][0]))
    glob = [i + 1 for i, k in enumerate(kinds) if k == O.GLOBAL]
    assert glob == [int(x) for x in rows["global_layers"]]
    assert kinds.count(O.LOCAL) == int(rows["n_local"][0])
    assert O.Config().window == int(rows["window"][0])
    # window = current token + 511 earlier positions
    t = 2000
    s = np.arange(t + 5)
    vis = O.visible(O.LOCAL, np.array([t]), s, O.Config().window)[0]
    assert vis.sum() == int(rows["earlier_visible"][0]) + 1
    assert vis[t] and vis[t - 511] and not vis[t - 512] and not vis[t + 1]


def test_toy_closed_form_printed():
    (delta, a, n, p, sig), = _rows("toy_retrieval.txt")
    got = O.toy_needle_probability(float(delta), float(a), int(n))
    assert float(f"{got:.{int(sig) - 1}e}") == float(p)
    # the required-scale formula inverts the probability formula
    r = 0.5
    a_r = O.toy_required_scale(r, 1.0, int(n))
    assert O.toy_needle_probability(1.0, a_r, int(n)) == pytest.approx(r, rel=1e-12)


def _toy_inputs(n, d=8, delta=1.0, needle=123):
    """Raw Q/K/V so that, after RMSNorm and the 1/sqrt(d) scale, the needle's
    logit is delta*a and every distractor's logit is exactly 0."""
    eps = O.Config().rms_eps
    c2 = 1.0 / (1.0 + eps)                       # RMSNorm of a +-1 vector scales by 1/sqrt(1+eps)
    w0 = delta / (c2 * math.sqrt(d))
    q = np.ones((1, 1, d))
    k = np.tile(np.array([1.0, -1.0] * (d // 2)), (n, 1))[:, None, :]
    k[needle, 0, :] = 1.0
    v = np.zeros((n, 1, d))
    v[needle, 0, 0] = 1.0
    return q, k, v, w0


def test_toy_probability_through_the_attention_path():
    """The oracle's global path (RMSNorm -> SSMax at p=N -> 1/sqrt(d) -> softmax)
    reproduces the page's toy probability at N = 1,048,576."""
    (delta, a_printed, n, p_printed, sig), = _rows("toy_retrieval.txt")
    n = int(n)
    cfg = O.Config(n_q_heads=1, n_kv_heads=1, head_dim=8)
    q, k, v, w0 = _toy_inputs(n, delta=float(delta))
    t = n - 1
    qn = O.rms_norm(q, np.ones(8), cfg.rms_eps)
    kn = O.rms_norm(k, np.full(8, w0), cfg.rms_eps)
    qp, kp = O.position_op(O.GLOBAL, qn, kn, np.array([t]), np.arange(n), cfg)
    out = O.attend(O.GLOBAL, qp, kp, v, np.array([t]), np.arange(n), cfg)
    p = out[0, 0, 0]
    a = float(O.ssmax_scale(t))
    assert round(a, 4) == float(a_printed)
    assert float(f"{p:.{int(sig) - 1}e}") == float(p_printed)
    assert p == pytest.approx(O.toy_needle_probability(float(delta), a, n), rel=1e-9)
    # the rest of the mass is spread evenly over the distractors (coordinate 0 of V is 0)
    assert out[0, 0, 1:].max() == 0.0


# ----------------------------------------------------------- SSMax analysis

def test_entropy_derivative_and_order():
    """dH/da = -a Var_pi[z] (derived from H(a) = log Z - a E[z]); a sharpens a
    nonconstant logit vector and keeps its order."""
    g = np.random.default_rng(5)
    z = g.standard_normal(300)
    for a in (0.5, 1.0, 1.4186, 1.8664):
        h = 1e-5
        fd = (O.softmax_entropy(z, a + h) - O.softmax_entropy(z, a - h)) / (2 * h)
        pi = O.softmax(a * z)
        var = np.dot(pi, z * z) - np.dot(pi, z) ** 2
        assert fd == pytest.approx(-a * var, rel=1e-6)
        assert fd < 0
        assert np.array_equal(np.argsort(pi, kind="stable"), np.argsort(z, kind="stable"))
    # entropy at a = 0 is log N (uniform); a constant vector keeps entropy log N
    assert O.softmax_entropy(z, 0.0) == pytest.approx(math.log(300), rel=1e-12)
    assert O.softmax_entropy(np.full(7, 3.0), 2.0) == pytest.approx(math.log(7), rel=1e-12)


# --------------------------------------------------------- attention pieces

def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0]])
    w = np.array([1.0, 2.0])
    # mean(x^2) = 12.5
    got = O.rms_norm(x, w, 0.0)
    assert np.allclose(got, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    # eps sits inside the square root
    got = O.rms_norm(np.zeros((1, 4)), np.ones(4), 1e-6)
    assert np.all(got == 0)
    got = O.rms_norm(np.full((1, 4), 1e-3), np.ones(4), 1e-6)
    assert got[0, 0] == pytest.approx(1e-3 / math.sqrt(1e-6 + 1e-6), rel=1e-12)
    # scale invariance (eps = 0) and unit RMS of the output with w = 1
    g = np.random.default_rng(1)
    x = g.standard_normal((5, 3, 128))
    y = O.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-13)
    assert np.allclose(O.rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-13)


def test_rope_invariants():
    g = np.random.default_rng(2)
    d, theta = 128, 10000.0
    x = g.standard_normal((6, 2, d))
    # position 0 is the identity
    assert np.allclose(O.rope(x, np.zeros(6, dtype=np.int64), theta), x, rtol=0, atol=0)
    # a rotation keeps the norm
    t = np.array([1, 7, 100, 4095, 65536, 1048575])
    y = O.rope(x, t, theta)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # scores depend only on the offset t - s
    q = g.standard_normal((1, 1, d))
    k = g.standard_normal((1, 1, d))
    for ts, shift in ((5, 0), (77, 3), (1000, 123456)):
        s0 = float((O.rope(q, np.array([ts]), theta) * O.rope(k, np.array([3]), theta)).sum())
        s1 = float((O.rope(q, np.array([ts + shift]), theta) * O.rope(k, np.array([3 + shift]), theta)).sum())
        assert s0 == pytest.approx(s1, rel=1e-9, abs=1e-9)
    # pair i rotates with frequency theta^(-2i/d): the first pair turns by exactly t radians,
    # the last pair by t * theta^(-(d-2)/d); composing t1 then t2 equals t1 + t2
    e0 = np.zeros((1, 1, d)); e0[0, 0, 0] = 1.0
    r = O.rope(e0, np.array([2]), theta)[0, 0]
    assert r[0] == pytest.approx(math.cos(2.0)) and r[d // 2] == pytest.approx(math.sin(2.0))
    a1 = O.rope(O.rope(x[:1], np.array([11]), theta), np.array([30]), theta)
    assert np.allclose(a1, O.rope(x[:1], np.array([41]), theta), rtol=1e-12, atol=1e-12)
    fr = O.rope_frequencies(d, theta)
    assert fr[0] == 1.0 and fr[-1] == pytest.approx(theta ** (-(d - 2) / d), rel=1e-15)


def _plain_inputs(T, H, G, d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((T, H, d)), g.standard_normal((T, G, d)), g.standard_normal((T, G, d)))


def test_window_needles():
    """A huge score at t-511 is attended; one at t-512 must not leak (local).
    Global sees the whole causal history but never a future key."""
    cfg = O.Config(n_q_heads=1, n_kv_heads=1, head_dim=4)
    T = 1400
    t = np.array([1300])
    s = np.arange(T)
    k = np.zeros((T, 1, 4))
    v = np.zeros((T, 1, 4))
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 1.0
    for off, should_see in ((511, True), (512, False), (0, True)):
        k2 = k.copy(); v2 = v.copy()
        k2[1300 - off, 0, 0] = 200.0
        v2[1300 - off, 0, 1] = 1.0
        o = O.attend(O.LOCAL, q, k2, v2, t, s, cfg)
        assert (o[0, 0, 1] > 0.99) == should_see, off
    # global: the needle far in the past is seen, a future one is not
    k2 = k.copy(); v2 = v.copy(); k2[3, 0, 0] = 200.0; v2[3, 0, 1] = 1.0
    assert O.attend(O.GLOBAL, q, k2, v2, t, s, cfg)[0, 0, 1] > 0.99
    k2 = k.copy(); v2 = v.copy(); k2[1301, 0, 0] = 200.0; v2[1301, 0, 1] = 1.0
    assert O.attend(O.GLOBAL, q, k2, v2, t, s, cfg)[0, 0, 1] == 0.0


def test_visible_counts():
    W = 512
    t = np.arange(0, 3000, 7)
    s = np.arange(3000)
    loc = O.visible(O.LOCAL, t, s, W).sum(1)
    glo = O.visible(O.GLOBAL, t, s, W).sum(1)
    assert np.array_equal(loc, np.minimum(t + 1, W))
    assert np.array_equal(glo, t + 1)


def test_zero_query_gives_mean_of_visible_values():
    T, H, G, d = 700, 12, 2, 16
    cfg = O.Config(n_q_heads=H, n_kv_heads=G, head_dim=d)
    _, k, v = _plain_inputs(T, H, G, d, 3)
    q = np.zeros((T, H, d))
    pos = np.arange(T)
    for kind in (O.LOCAL, O.GLOBAL):
        o = O.attend(kind, q, k, v, pos, pos, cfg)
        for t in (0, 5, 511, 512, 699):
            lo = max(0, t - 511) if kind == O.LOCAL else 0
            for h in (0, 5, 6, 11):
                ref = v[lo:t + 1, h // 6, :].mean(axis=0)
                assert np.allclose(o[t, h], ref, rtol=1e-12, atol=1e-13)


def test_gqa_mapping_distinct_values():
    """Six consecutive query heads read one KV head: V_g = g+1 constant."""
    T, H, G, d = 9, 48, 8, 8
    cfg = O.Config(n_q_heads=H, n_kv_heads=G, head_dim=d)
    q, k, _ = _plain_inputs(T, H, G, d, 4)
    v = np.broadcast_to((np.arange(G) + 1.0)[None, :, None], (T, G, d)).copy()
    o = O.attend(O.GLOBAL, q, k, v, np.arange(T), np.arange(T), cfg)
    for h in range(H):
        assert np.allclose(o[:, h, :], h // 6 + 1, rtol=1e-14)
    # and the mapping is the contiguous one
    assert [O.kv_head_of(h, 48, 8) for h in (0, 5, 6, 11, 47)] == [0, 0, 1, 1, 7]


def test_single_token_returns_its_value():
    inp = attention_inputs(cfg=99, layer=0, n_tok=1)
    for kind in (O.LOCAL, O.GLOBAL):
        y, o = O.attention_layer(kind, inp["q"], inp["k"], inp["v"], inp["q_norm_w"],
                                 inp["k_norm_w"], inp["gate"], [0], [0], return_pre_gate=True)
        v = O.bf16_to_f64(inp["v"])
        for h in range(48):
            assert np.array_equal(o[0, h], v[0, h // 6])


def test_gate_closed_form():
    o = np.ones((1, 2, 3))
    g = np.array([[[0.0, 2.0, -2.0], [100.0, -100.0, 0.0]]])
    y = O.output_gate(o, g, gate_bias=np.array([0.0, 0.0]))
    assert y[0, 0, 0] == 0.5
    assert y[0, 0, 1] == pytest.approx(1 / (1 + math.exp(-2)))
    assert y[0, 1, 0] == pytest.approx(1.0) and y[0, 1, 1] == pytest.approx(0.0, abs=1e-40)
    # bias is one value per head, added to every coordinate of that head
    y = O.output_gate(o, np.zeros((1, 2, 3)), gate_bias=np.array([0.0, 2.0]))
    assert np.allclose(y[0, 1], 1 / (1 + math.exp(-2))) and np.allclose(y[0, 0], 0.5)


def test_lse_merge_of_key_splits_equals_full_softmax():
    """Splitting the keys and merging partial (max, sum, acc) triples by
    log-sum-exp reproduces the oracle's one-pass attention (flash/split-K
    reorder exact softmax)."""
    g = np.random.default_rng(6)
    n, d = 1000, 16
    z = g.standard_normal(n) * 3
    v = g.standard_normal((n, d))
    cfg = O.Config(n_q_heads=1, n_kv_heads=1, head_dim=d)
    # feed the logits through attend: q = e0 * sqrt(d), k[:,0] = z
    q = np.zeros((1, 1, d)); q[0, 0, 0] = math.sqrt(d)
    k = np.zeros((n, 1, d)); k[:, 0, 0] = z
    full = O.attend(O.GLOBAL, q, k, v[:, None, :], np.array([n - 1]), np.arange(n), cfg)[0, 0]
    parts = []
    for lo in range(0, n, 137):
        zz = z[lo:lo + 137]
        m = zz.max()
        e = np.exp(zz - m)
        parts.append((m, e.sum(), e @ v[lo:lo + 137]))
    M = max(p[0] for p in parts)
    L = sum(p[1] * math.exp(p[0] - M) for p in parts)
    A = sum(p[2] * math.exp(p[0] - M) for p in parts)
    assert np.allclose(A / L, full, rtol=1e-12, atol=1e-14)


def _brute_layer(kind, q, k, v, qw, kw, gate, pos, cfg):
    """Scalar-loop evaluation with the math module only (tiny sizes)."""
    T, H, d = len(q), cfg.n_q_heads, cfg.head_dim
    G = cfg.n_kv_heads
    half = d // 2

    def norm(x, w):
        r = math.sqrt(sum(e * e for e in x) / d + cfg.rms_eps)
        return [w[i] * x[i] / r for i in range(d)]

    def rot(x, t):
        out = [0.0] * d
        for i in range(half):
            ang = t * cfg.rope_theta ** (-2.0 * i / d)
            out[i] = x[i] * math.cos(ang) - x[i + half] * math.sin(ang)
            out[i + half] = x[i + half] * math.cos(ang) + x[i] * math.sin(ang)
        return out

    y = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    for t in range(T):
        for h in range(H):
            g = h // (H // G)
            qq = norm(q[t][h], qw)
            if kind == O.LOCAL:
                qq = rot(qq, pos[t])
            else:
                a = (1.0 + (pos[t] + 1) / cfg.ssmax_base) ** cfg.ssmax_exp
                qq = [a * e for e in qq]
            scores = []
            for s in range(T):
                dt = pos[t] - pos[s]
                if dt < 0 or (kind == O.LOCAL and dt > cfg.window - 1):
                    continue
                kk = norm(k[s][g], kw)
                if kind == O.LOCAL:
                    kk = rot(kk, pos[s])
                scores.append((sum(qq[i] * kk[i] for i in range(d)) / math.sqrt(d), s))
            mx = max(sc for sc, _ in scores)
            den = sum(math.exp(sc - mx) for sc, _ in scores)
            for i in range(d):
                o = sum(math.exp(sc - mx) * v[s][g][i] for sc, s in scores) / den
                y[t][h][i] = o / (1.0 + math.exp(-gate[t][h][i]))
    return np.array(y)


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_brute_force_tiny(kind):
    # window 4 so that the local rule cuts inside T = 11; positions start at 3000
    cfg = O.Config(n_q_heads=6, n_kv_heads=2, head_dim=8, window=4)
    T = 11
    g = np.random.default_rng(7)
    bits = lambda *s: f32_to_bf16_bits(g.standard_normal(s).astype(np.float32))
    q, k, v, gate = bits(T, 6, 8), bits(T, 2, 8), bits(T, 2, 8), bits(T, 6, 8)
    qw = f32_to_bf16_bits((1 + 0.1 * g.standard_normal(8)).astype(np.float32))
    kw = f32_to_bf16_bits((1 + 0.1 * g.standard_normal(8)).astype(np.float32))
    pos = np.arange(3000, 3000 + T)
    y = O.attention_layer(kind, q, k, v, qw, kw, gate, pos, pos, cfg)
    f = lambda b: bf16_bits_to_f32(b).astype(np.float64).tolist()
    ref = _brute_layer(kind, f(q), f(k), f(v), f(qw), f(kw), f(gate), pos.tolist(), cfg)
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_local_attention_is_shift_invariant():
    """RoPE + a relative window make a local layer independent of the absolute
    offset of the whole sequence; the global layer is not (a(p) grows)."""
    inp = attention_inputs(cfg=98, layer=0, n_tok=40)
    args = [inp[x] for x in ("q", "k", "v", "q_norm_w", "k_norm_w", "gate")]
    p0 = np.arange(40)
    y0 = O.attention_layer(O.LOCAL, *args, p0, p0)
    y1 = O.attention_layer(O.LOCAL, *args, p0 + 100003, p0 + 100003)
    assert np.allclose(y0, y1, rtol=1e-9, atol=1e-11)
    g0 = O.attention_layer(O.GLOBAL, *args, p0, p0)
    g1 = O.attention_layer(O.GLOBAL, *args, p0 + 100003, p0 + 100003)
    assert not np.allclose(g0, g1, rtol=1e-6, atol=1e-8)


def test_chunked_equals_one_shot_and_decode_equals_last_row():
    T = 700
    inp = attention_inputs(cfg=97, layer=1, n_tok=T)
    pos = np.arange(T)
    for kind in (O.LOCAL, O.GLOBAL):
        full = O.attention_layer(kind, inp["q"], inp["k"], inp["v"], inp["q_norm_w"],
                                 inp["k_norm_w"], inp["gate"], pos, pos)
        parts = []
        for lo, hi in ((0, 300), (300, 613), (613, 699)):
            parts.append(O.attention_layer(kind, inp["q"][lo:hi], inp["k"][:hi], inp["v"][:hi],
                                           inp["q_norm_w"], inp["k_norm_w"], inp["gate"][lo:hi],
                                           pos[lo:hi], pos[:hi]))
        dec = O.attention_layer(kind, inp["q"][699:], inp["k"], inp["v"], inp["q_norm_w"],
                                inp["k_norm_w"], inp["gate"][699:], pos[699:], pos)
        assert np.allclose(np.concatenate(parts + [dec]), full, rtol=1e-12, atol=1e-13)


def test_page_and_ring_addressing():
    bt = np.array([[7, 3, 9], [0, 4, -1]])
    assert O.page_slot(bt, 16, 0, 0) == (7, 0)
    assert O.page_slot(bt, 16, 0, 17) == (3, 1)
    assert O.page_slot(bt, 16, 1, 31) == (4, 15)
    assert O.page_slot(bt, 16, 0, 47) == (9, 15)
    assert [O.ring_slot(t) for t in (0, 511, 512, 1048575)] == [0, 511, 0, 511]


def test_cached_key_matches_layer_keys():
    """The cache stores normalised K, rotated on local layers only."""
    inp = attention_inputs(cfg=96, layer=0, n_tok=3)
    pos = np.array([0, 5, 513])
    kl = O.cached_key(O.LOCAL, inp["k"], inp["k_norm_w"], pos)
    kg = O.cached_key(O.GLOBAL, inp["k"], inp["k_norm_w"], pos)
    kn = O.rms_norm(O.bf16_to_f64(inp["k"]), O.bf16_to_f64(inp["k_norm_w"]), 1e-6)
    assert np.array_equal(kg, kn)
    assert np.array_equal(kl[0], kn[0]) and not np.allclose(kl[1], kn[1])


def test_synth_bf16_rounding_matches_torch():
    """The shared generator's bf16 rounding agrees with torch's conversion."""
    import torch
    g = np.random.default_rng(8)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- FP8 E4M3 cache

def test_e4m3_decode_closed_forms():
    """Code values fixed by the E4M3FN layout (bias 7, 3 mantissa bits,
    subnormals at exponent 0, no infinities, 0x7F NaN)."""
    d = O.e4m3_decode
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x38) == 1.0
    assert d(0x39) == 1.125
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = d(codes)
    assert np.all(np.diff(vals) > 0)                  # code order is value order
    assert np.array_equal(d(codes | 0x80), -vals)     # sign bit only flips the sign


def test_e4m3_encode_matches_torch_within_range():
    """Nearest-value, ties-to-even encoding, checked against torch's own
    float8_e4m3fn conversion (an independent implementation) on random values
    over the whole exponent range and on every midpoint between neighbouring
    codes (the tie cases), where torch does not overflow (|x| < 464)."""
    torch = pytest.importorskip("torch")
    # float32 inputs: torch converts wider floats through float32 first, which
    # would round a value just below a midpoint onto it.
    rng = np.random.default_rng(7)
    vals = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = (vals[1:] + vals[:-1]) / 2                 # exact in float32
    x = np.concatenate([
        (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.5, 20000)).astype(np.float32),
        mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), vals, -vals])
    x = x[np.abs(x) < 464]
    ours = O.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_saturation_and_roundtrip():
    e = O.e4m3_encode
    assert np.array_equal(e([448.0, 463.9, 464.0, 1e6, np.inf]), [0x7E] * 5)
    assert np.array_equal(e([-448.0, -1e30, -np.inf]), [0xFE] * 3)
    assert e(np.nan) == 0x7F
    codes = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    assert np.array_equal(e(O.e4m3_decode(codes)), codes)   # every finite code maps back to itself
    x = np.linspace(-500, 500, 100001)
    assert np.all(np.diff(O.e4m3_decode(e(x))) >= 0)         # monotone


def test_fp8_cache_attention_reduces_to_bf16_on_grid_values():
    """With K_hat and V on the E4M3 grid (times the scale) the FP8 cache is
    exact, so the layer equals the BF16-cache layer; with no cached position
    the argument changes nothing; off-grid values do change the result."""
    cfg = O.Config(n_q_heads=4, n_kv_heads=2, head_dim=8, window=4, rms_eps=0.0)
    rng = np.random.default_rng(3)
    n = 6
    q = f32_to_bf16_bits(rng.standard_normal((n, 4, 8)).astype(np.float32))
    # K rows of equal-magnitude entries: rms = |c|, so K_hat = w * sign(k).
    k = f32_to_bf16_bits(np.sign(rng.standard_normal((n, 2, 8))).astype(np.float32) * 3.0)
    v = f32_to_bf16_bits(rng.integers(-8, 9, (n, 2, 8)).astype(np.float32) * 0.25)
    wq = f32_to_bf16_bits(np.ones(8, np.float32))
    wk = f32_to_bf16_bits(np.array([1, 0.5, 2, 1.5, 1, 0.75, 1.25, 1], np.float32))
    g = f32_to_bf16_bits(rng.standard_normal((n, 4, 8)).astype(np.float32))
    pos = np.arange(n)
    base = O.attention_layer(O.GLOBAL, q, k, v, wq, wk, g, pos, pos, cfg)
    on_grid = O.attention_layer(O.GLOBAL, q, k, v, wq, wk, g, pos, pos, cfg, fp8_cache=(0.5, 0.25, n))
    assert np.array_equal(base, on_grid)
    none = O.attention_layer(O.GLOBAL, q, k, v, wq, wk, g, pos, pos, cfg, fp8_cache=(0.3, 0.3, 0))
    assert np.array_equal(base, none)
    off = O.attention_layer(O.GLOBAL, q, k, v, wq, wk, g, pos, pos, cfg, fp8_cache=(0.3, 0.3, n))
    assert not np.array_equal(base, off) and np.max(np.abs(off - base)) < 0.2
