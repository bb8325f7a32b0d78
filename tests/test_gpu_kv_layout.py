"""GPU: beam_kv_convert_v moves V between the token-major layout (as K is
stored) and the cache's coordinate-major layout. Expected values: the
transpose itself, bit-exact, both directions, bf16 and FP8 codes, both cache
kinds; then a cache whose K and V were written token-major by the caller and
whose V was converted decodes like the oracle (the converted layout is the
one attention reads)."""
import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O
import synth
from tests.helpers import compare, dev_bf16, dev_i32, host_bits, say

pytestmark = pytest.mark.gpu

SENT = 0x7F7F


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.lib()
    yield
    torch.cuda.synchronize()


def _cache(cfg, kind, dtype, n_pages=37, n_rings=3):
    import torch
    if kind == ga.GLOBAL:
        bt = np.arange(n_pages, dtype=np.int32)[None, :]
        return ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt), dtype=dtype), n_pages, 16
    return ga.KVCache.allocate_local(cfg, n_rings, dtype=dtype), n_rings, cfg.window


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.uint8).cpu().numpy()


@pytest.mark.parametrize("dtype", [ga.KV_BF16, ga.KV_FP8_E4M3])
@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_convert_v_is_a_transpose(kind, dtype):
    import torch
    cfg = ga.Config()
    cache, nb, rows = _cache(cfg, kind, dtype)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(100 + 10 * kind + dtype)
    tdt, idt, lo, hi = ((torch.bfloat16, torch.int16, -32768, 32768) if dtype == ga.KV_BF16
                        else (torch.uint8, torch.uint8, 0, 256))
    tm = torch.randint(lo, hi, (nb, 8, rows, 128), generator=gen, device="cuda", dtype=torch.int32).to(idt)
    tm = tm.view(tdt) if tdt == torch.bfloat16 else tm
    say(f"[case] convert_v kind={kind} dtype={dtype} blocks={nb} rows={rows} -> cache")
    ga.kv_convert_v(cfg, cache, tm, to_cache=True)
    torch.cuda.synchronize()
    src = _bits(tm)
    assert np.array_equal(_bits(cache.v), np.transpose(src, (0, 1, 3, 2)))
    back = torch.empty_like(tm)
    back.view(idt).fill_(SENT if dtype == ga.KV_BF16 else 0x7F)
    say(f"[case] convert_v kind={kind} dtype={dtype} -> token-major")
    ga.kv_convert_v(cfg, cache, back, to_cache=False)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), src)


@pytest.mark.parametrize("kind", [ga.LOCAL, ga.GLOBAL])
def test_cache_written_token_major_decodes_like_the_oracle(kind):
    """A caller writes K_hat and V of 700 positions token-major into the
    cache's pages (permuted) or ring, converts V, appends one token and
    decodes it."""
    import torch
    cfg = ga.Config()
    T = 700
    inp = synth.attention_inputs(9, 50 + kind, T + 1)
    pos = np.arange(T)
    khat = torch.from_numpy(O.cached_key(kind, inp["k"][:T], inp["k_norm_w"], pos)).to(torch.bfloat16)
    v = torch.from_numpy(inp["v"][:T].view(np.int16)).view(torch.bfloat16)
    if kind == ga.GLOBAL:
        bt, n_pages = synth.paged_block_table(9, [T + 1])
        cache = ga.KVCache.allocate_global(cfg, n_pages, torch.from_numpy(bt), fill=SENT)
        page, slot = bt[0][pos // 16], pos % 16
        first = 0
    else:
        cache = ga.KVCache.allocate_local(cfg, 1, fill=SENT)
        first = T - cfg.window + 1  # positions the decode at T still sees
        page, slot = np.zeros(T, dtype=np.int64), pos % cfg.window
    vtm = torch.empty((cache.v.shape[0], 8, cache.k.shape[2], 128), dtype=torch.bfloat16)
    vtm.view(torch.int16).fill_(SENT)
    k = cache.k.cpu()
    for t in range(first, T):
        k[page[t], :, slot[t], :] = khat[t]
        vtm[page[t], :, slot[t], :] = v[t]
    cache.k.copy_(k)
    say(f"[case] token-major cache kind={kind}: convert V, append t={T}, decode")
    ga.kv_convert_v(cfg, cache, vtm.cuda(), to_cache=True)
    d = {key: dev_bf16(val) for key, val in inp.items()}
    ga.kv_append(cfg, cache, d["k"][T:], d["v"][T:], d["k_norm_w"], dev_i32([0]), dev_i32([T]))
    out = ga.decode(cfg, cache, d["q"][T:], d["q_norm_w"], d["gate"][T:], dev_i32([0]), dev_i32([T]), T)
    torch.cuda.synchronize()
    p = np.arange(T + 1)
    ref = O.attention_layer(kind, inp["q"][T:], inp["k"], inp["v"], inp["q_norm_w"], inp["k_norm_w"],
                            inp["gate"][T:], p[T:], p)
    compare(host_bits(out), ref, f"decode over a token-major cache kind={kind}")
