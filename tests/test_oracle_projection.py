"""Pins of the projection oracle (oracle.projection) against what the pages
and plain arithmetic fix. CPU only.

* The weight convention (output-by-input, "Follow the tensors, not the
  parameter label"): brute-force sums on a tiny case, and a permuted identity
  that a transposed weight would turn into the inverse permutation.
* The head split and stacking order: with selection weights, the layer
  composed from projections equals the already pinned attention oracle on
  the same bf16 Q/K/V/gate values, for both layer kinds; a swapped block
  order moves different values into the heads.
* W_o sees the heads in order: a selection row for column 128h + i returns
  Y[:, h, i].
* Q' (what the fused query epilogue produces): a(p) at the printed value on
  a global layer, the identity rotation at t = 0 on a local layer.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import beam_attention as A
from oracle import projection as P


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_linear_brute_force_output_by_input():
    x = _bf16([[1.0, -2.0, 0.5], [3.0, 0.25, -1.0]])                 # [n=2][in=3]
    w = _bf16([[1, 0, 0], [0, 2, 0], [1, 1, 1], [-0.5, 4, 2]])        # [out=4][in=3]
    got = P.linear(x, w)
    xf, wf = A.bf16_to_f64(x), A.bf16_to_f64(w)
    want = np.zeros((2, 4))
    for t, f, k in itertools.product(range(2), range(4), range(3)):
        want[t, f] += xf[t, k] * wf[f, k]
    assert got.shape == (2, 4)
    assert np.array_equal(got, want)


def test_permuted_identity_is_not_transposed():
    n, hidden = 5, 16
    x = synth.normal_bf16((n, hidden), 7, 0)
    perm = np.random.default_rng(3).permutation(hidden)
    w = np.zeros((hidden, hidden), np.float32)
    w[np.arange(hidden), perm] = 1.0                                  # row f selects input column perm[f]
    got = P.linear(x, _bf16(w))
    assert np.array_equal(got, A.bf16_to_f64(x)[:, perm])
    assert not np.array_equal(got, A.bf16_to_f64(x)[:, np.argsort(perm)])


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_selection_weights_reduce_to_the_attention_oracle(kind):
    n_q, n_kv, d, n = 4, 2, 128, 40
    cfg = A.Config(n_q_heads=n_q, n_kv_heads=n_kv, window=512)
    inp = synth.attention_inputs(5, kind, n, n_q=n_q, n_kv=n_kv, d=d)
    blocks = [inp["q"].reshape(n, -1), inp["k"].reshape(n, -1), inp["v"].reshape(n, -1),
              inp["gate"].reshape(n, -1)]
    x = np.concatenate(blocks, axis=1)                                # hidden = (2 n_q + 2 n_kv) d
    hidden = x.shape[1]
    w = _bf16(np.eye(hidden, dtype=np.float32))
    q, k, v, g = P.project_qkvg(x, w, n_q, n_kv, d)
    pos = np.arange(n) + 100
    got = P.attention_from_projections(kind, q, k, v, g, inp["q_norm_w"], inp["k_norm_w"], pos, pos, cfg)
    want = A.attention_layer(kind, inp["q"], inp["k"], inp["v"], inp["q_norm_w"], inp["k_norm_w"], inp["gate"],
                             pos, pos, cfg)
    assert np.array_equal(got, want)
    # the stacking order matters: K and V swapped in the weight gives other values
    bad = np.concatenate([blocks[0], blocks[2], blocks[1], blocks[3]], axis=1)
    q2, k2, v2, g2 = P.project_qkvg(bad, w, n_q, n_kv, d)
    got2 = P.attention_from_projections(kind, q2, k2, v2, g2, inp["q_norm_w"], inp["k_norm_w"], pos, pos, cfg)
    assert np.max(np.abs(got2 - want)) > 1e-2


def test_output_projection_sees_heads_in_order():
    n, H, d = 3, 4, 128
    y = np.random.default_rng(1).standard_normal((n, H, d))
    picks = [(0, 0), (3, 127), (1, 5), (2, 64)]
    w = np.zeros((len(picks), H * d), np.float32)
    for f, (h, i) in enumerate(picks):
        w[f, 128 * h + i] = 1.0
    got = P.output_projection(y, _bf16(w))
    want = np.stack([y[:, h, i] for h, i in picks], axis=1)
    assert np.array_equal(got, want)


def test_queries_prime_global_scale_and_local_identity():
    cfg = A.Config()
    q = np.full((2, 3, 128), 0.75)                                    # RMSNorm of a constant vector: all ones
    w = _bf16(np.ones(128, np.float32))
    qp = P.queries_prime(A.GLOBAL, q, w, [2047, 0], cfg)
    # a(2048) = 2^0.1 = 1.0717735 (printed to 4 decimals on the pages)
    assert np.allclose(qp[0], 2 ** 0.1 / np.sqrt(1 + cfg.rms_eps / 0.5625), rtol=0, atol=1e-12)
    assert abs(2 ** 0.1 - 1.0717735) < 5e-8
    assert np.allclose(qp[1], (1 + 1 / 2048) ** 0.1 / np.sqrt(1 + cfg.rms_eps / 0.5625), rtol=0, atol=1e-12)
    qr = np.random.default_rng(2).standard_normal((1, 3, 128))
    wr = synth.normal_bf16((128,), 3, 0, scale=0.1, offset=1.0)
    assert np.array_equal(P.queries_prime(A.LOCAL, qr, wr, [0], cfg),
                          A.rms_norm(qr, A.bf16_to_f64(wr), cfg.rms_eps))
