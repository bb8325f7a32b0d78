"""beam_attn_decode_noalloc (the decode entry point that takes no workspace
and allocates nothing) through the C ABI, against beam_attn_decode with a
caller workspace on the same inputs and against the float64 oracle.

Both entry points run the same kernels with the same split, so their outputs
must be bit-identical; both must also meet the oracle tolerance (max-abs
2e-2, relative L2 5e-3). Two calls in a row share the library's scratch
array, the second with fewer sequences and a shorter context, so the second
result also shows that nothing left from the first call leaks into it.
"""
import ctypes

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


def _setup(kind, cfg_id, ts):
    import torch
    hist = [synth.attention_inputs(cfg_id, 10 * kind + i, t + 1) for i, t in enumerate(ts)]
    for x in hist[1:]:
        x["q_norm_w"], x["k_norm_w"] = hist[0]["q_norm_w"], hist[0]["k_norm_w"]
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(cfg_id, [t + 1 for t in ts])
        cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    else:
        cache = ga.KVCache.allocate_local(CFG, len(ts))
    for i, t in enumerate(ts):
        lo = 0 if kind == O.GLOBAL else max(0, t + 1 - 512)
        ga.kv_append(CFG, cache, dev_bf16(hist[i]["k"][lo:]), dev_bf16(hist[i]["v"][lo:]),
                     dev_bf16(hist[0]["k_norm_w"]), dev_i32(np.full(t + 1 - lo, i)), dev_i32(np.arange(lo, t + 1)))
    return cache, hist


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_decode_noalloc_matches_decode(kind):
    import torch
    calls = [([4000, 9, 700, 3333, 1024, 130], 256), ([515, 64], 0)]  # (positions, split_keys)
    b = torch.from_numpy(synth.gate_bias(80, kind)).cuda()
    for call, (ts, sk) in enumerate(calls):
        cache, hist = _setup(kind, 81 + call, ts)
        q = dev_bf16(np.stack([x["q"][t] for x, t in zip(hist, ts)]))
        gate = dev_bf16(np.stack([x["gate"][t] for x, t in zip(hist, ts)]))
        seq, pos, qw = dev_i32(np.arange(len(ts))), dev_i32(ts), dev_bf16(hist[0]["q_norm_w"])
        out_na = torch.full((len(ts), 48, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        say(f"[case] decode_noalloc kind={kind} call={call} n_seqs={len(ts)} max_pos={max(ts)} split={sk}")
        ga.decode_noalloc(CFG, cache, q, qw, gate, seq, pos, max(ts), out_na, gate_bias=b, split_keys=sk)
        out_ws = ga.decode(CFG, cache, q, qw, gate, seq, pos, max(ts), gate_bias=b, split_keys=sk)
        torch.cuda.synchronize()
        a, w = host_bits(out_na), host_bits(out_ws)
        assert np.array_equal(a, w), f"call {call}: noalloc differs from the workspace entry point"
        ref = np.concatenate([
            O.attention_layer(kind, x["q"][t:t + 1], x["k"][:t + 1], x["v"][:t + 1], x["q_norm_w"], x["k_norm_w"],
                              x["gate"][t:t + 1], np.array([t]), np.arange(t + 1), gate_bias=b.cpu().numpy())
            for x, t in zip(hist, ts)])
        compare(a, ref, f"decode_noalloc kind={kind} call={call}")


def test_decode_noalloc_rejects_oversized_scratch():
    """A call whose partials would not fit the library's array fails with
    BEAM_E_WORKSPACE before anything is launched."""
    import torch
    ts = [131071] * 64
    need = ga.decode_workspace_bytes(CFG, ga.GLOBAL, 64, 131071, 2048)
    assert need > ga.DECODE_SCRATCH_BYTES
    bt = torch.zeros((64, 8192), dtype=torch.int32)
    cache = ga.KVCache.allocate_global(CFG, 16, bt)
    z = torch.zeros((64, 48, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ga.BeamError) as e:
        ga.decode_noalloc(CFG, cache, z, z[0, 0], z, dev_i32(np.arange(64)), dev_i32(ts), 131071, z,
                          split_keys=2048)
    assert e.value.status == 5
    # the same call with a larger split fits the array
    assert ga.decode_workspace_bytes(CFG, ga.GLOBAL, 64, 131071, 16384) <= ga.DECODE_SCRATCH_BYTES
