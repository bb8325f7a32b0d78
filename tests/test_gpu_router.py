"""GPU parity of the group-limited sigmoid router (through the C ABI) against
the oracle (oracle.router).

* Selection from given float32 logits (beam_router_select): bit-exact expert
  indices and order, weights to 1e-6 relative (float32 against float64),
  including exact ties of scores and of group scores, and other group/k
  settings.
* Logits (beam_router_logits): float32 against the exact float64 dot
  products, every element within the float32 summation bound
  (K+1) 2^-24 sum|x w| and the whole within 4 sqrt(K) 2^-24 relative L2 (a
  random-walk model of the rounding errors), and exactly equal on inputs whose
  every partial sum is representable.
* The whole router (beam_router): bit-exact against the oracle on the exact
  grid inputs; on N(0,1) inputs the same experts for every token except where
  the oracle's own decision margin is below 1e-4 (a near tie that the float32
  logits may flip); identical to logits + select on the GPU.
"""
import numpy as np
import pytest

import global_attention_amd as ga
import synth
from oracle import router as R
from tests.helpers import say

pytestmark = pytest.mark.gpu
RC = ga.RouterConfig()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.lib()
    yield
    torch.cuda.synchronize()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _check_selection(idx, wts, want_idx, want_w, what):
    assert np.array_equal(idx, want_idx), f"{what}: {np.sum(np.any(idx != want_idx, axis=1))} tokens differ"
    np.testing.assert_allclose(wts, want_w, rtol=1e-6, atol=0, err_msg=what)


def _tie_logits(n):
    """Logits with exact ties: every token repeats values across experts and
    groups (equal scores, equal group scores), plus all-equal tokens."""
    g = np.random.default_rng(4)
    z = np.round(g.standard_normal((n, 256)) * 4) / 4          # 33-ish distinct values per token
    z[::7] = 0.5                                               # every expert equal
    z[3::7] = np.tile(np.repeat(g.standard_normal(8), 32), 1)  # equal within groups
    return z.astype(np.float32)


@pytest.mark.parametrize("groups,k", [(4, 8), (1, 8), (8, 8), (4, 1), (2, 5)])
def test_select_bit_exact(groups, k):
    n = 2003                                                   # not a multiple of 64 tokens per block
    z = synth.normal_f32((n, 256), 30, 0, scale=1.5)
    z[:600] = _tie_logits(600)
    bias = synth.router_inputs(30, 0, 1, hidden=32)["bias"]
    rc = ga.RouterConfig(topk_groups=groups, top_k=k)
    for b in (bias, None):
        say(f"[case] router select groups={groups} k={k} bias={b is not None}")
        idx, wts = ga.router_select(rc, _dev(z), None if b is None else _dev(b))
        want_idx, want_w, _ = R.select(R.sigmoid_f32(z), np.zeros(256, np.float32) if b is None else b,
                                       topk_groups=groups, top_k=k)
        _check_selection(_host(idx), _host(wts), want_idx, want_w, f"select groups={groups} k={k}")


@pytest.mark.parametrize("n,hidden", [(300, 5120), (1, 32), (129, 96), (128, 64)])
def test_logits_within_fp32_bound(n, hidden):
    inp = synth.router_inputs(31, 0, n, hidden=hidden)
    say(f"[case] router logits n={n} hidden={hidden}")
    got = _host(ga.router_logits(ga.RouterConfig(hidden=hidden), _dev_bf16(inp["x"]), _dev(inp["w"])))
    want = R.router_logits(inp["x"], inp["w"])
    xa = np.abs((inp["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    bound = (hidden + 1) * 2.0 ** -24 * (xa @ np.abs(inp["w"].astype(np.float64)).T)
    err = np.abs(got - want)
    assert np.all(err <= bound), f"max err {err.max()} (bound {bound[err > bound].min()})"
    # rounding errors of a running float32 sum add up like a random walk:
    # about 2^-24 sqrt(K) of the result; allow four times that
    assert np.linalg.norm(got - want) <= 4 * np.sqrt(hidden) * 2.0 ** -24 * np.linalg.norm(want)


def test_router_exact_inputs_bit_exact():
    n = 1000
    inp = synth.router_inputs_exact(32, 0, n)
    x, w, b = _dev_bf16(inp["x"]), _dev(inp["w"]), _dev(inp["bias"])
    say("[case] router exact inputs: logits")
    z = _host(ga.router_logits(RC, x, w))
    want_z = R.router_logits(inp["x"], inp["w"])
    assert np.array_equal(z.astype(np.float64), want_z)       # every partial sum exact
    say("[case] router exact inputs: fused")
    idx, wts = ga.router(RC, x, w, b)
    want_idx, want_w, _, _ = R.route(inp["x"], inp["w"], inp["bias"])
    _check_selection(_host(idx), _host(wts), want_idx, want_w, "fused router, exact inputs")


def _margin(z64, bias, groups=4, k=8):
    """The oracle's own decision margin per token: the smallest gap, in
    score units, between a kept and a dropped group score and between the
    last chosen and the best unchosen candidate."""
    s = 1 / (1 + np.exp(-z64))
    c = s + bias.astype(np.float64)
    n = z64.shape[0]
    out = np.empty(n)
    for t in range(n):
        gs = np.array([np.sort(c[t, 32 * q:32 * q + 32])[-2:].sum() for q in range(8)])
        order = np.argsort(-gs, kind="stable")
        gap_g = gs[order[groups - 1]] - gs[order[groups]] if groups < 8 else np.inf
        cand = np.concatenate([c[t, 32 * q:32 * q + 32] for q in order[:groups]])
        cs = np.sort(cand)[::-1]
        out[t] = min(gap_g, cs[k - 1] - cs[k])
    return out


def test_router_normal_inputs():
    n = 3000
    inp = synth.router_inputs(33, 0, n)
    x, w, b = _dev_bf16(inp["x"]), _dev(inp["w"]), _dev(inp["bias"])
    say("[case] router N(0,1) inputs: fused, logits + select")
    idx, wts = ga.router(RC, x, w, b)
    idx, wts = _host(idx), _host(wts)
    z = ga.router_logits(RC, x, w)
    idx2, wts2 = ga.router_select(RC, z, b)
    # the fused kernel takes the same decisions on the same float32 logits
    assert np.array_equal(idx, _host(idx2)) and np.array_equal(wts, _host(wts2))
    want_idx, want_w, _, z64 = R.route(inp["x"], inp["w"], inp["bias"])
    same = np.all(idx == want_idx, axis=1)
    diff = np.nonzero(~same)[0]
    say(f"[info] {len(diff)} of {n} tokens differ from the float64-logit oracle")
    if len(diff):
        m = _margin(z64[diff], inp["bias"])
        assert np.all(m < 1e-4), f"tokens {diff[m >= 1e-4]} differ with margins {m[m >= 1e-4]}"
    assert len(diff) <= n // 100
    np.testing.assert_allclose(wts[same], want_w[same], rtol=2e-6)
    assert np.allclose(wts.sum(axis=1), 2.5, rtol=1e-5)
