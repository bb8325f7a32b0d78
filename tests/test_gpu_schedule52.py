"""GPU parity for the full 52-layer schedule: chunked varlen prefill of 8
sequences (lengths uniform in [4096, 65536]) in 8192-token chunks through all
52 attention layers (global at 6, 12, ..., 48, 52; local elsewhere, window
512), each layer with its own cache, as in "Beam 1.0: Local RoPE, Global NoPE
and Scalable Softmax", section "Two attention paths in one decoder".

Inputs per (sequence, layer kind) are drawn once on the device with torch's
seeded generator and reused by every layer of that kind; RMSNorm weights are
per layer (seeded generator of synth). The oracle checks 32 deterministic rows
of every chunk for the first and last layer of each kind, on the shortest and
the longest sequence. Cache allocation is checked bit-exactly against the KV
budget formula ("KV memory: nine growing caches, not 52")."""
import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O
import synth
from tests.helpers import compare, dev_bf16, dev_i32, host_bits, say

pytestmark = pytest.mark.gpu
CFG = ga.Config()
CHUNK = 8192
ROWS_PER_CHUNK = 32


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_52_layer_chunked_prefill_sampled():
    import torch
    lens = synth.chunked_lengths(5, 8, 4096, 65536)
    n = len(lens)
    kinds = O.layer_kinds(52)
    say(f"[case] 52-layer schedule, lengths {lens.tolist()}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    # raw projections per (kind, sequence), generated on the device
    raw = {}
    for kind in (O.LOCAL, O.GLOBAL):
        for i in range(n):
            L = int(lens[i])
            raw[kind, i] = {
                "q": torch.randn((L, 48, 128), generator=gen, device="cuda").to(torch.bfloat16),
                "k": torch.randn((L, 8, 128), generator=gen, device="cuda").to(torch.bfloat16),
                "v": torch.randn((L, 8, 128), generator=gen, device="cuda").to(torch.bfloat16),
                "gate": torch.randn((L, 48, 128), generator=gen, device="cuda").to(torch.bfloat16),
            }
    qw = [synth.normal_bf16((128,), 5, synth.T_QW, l, scale=0.1, offset=1.0) for l in range(52)]
    kw = [synth.normal_bf16((128,), 5, synth.T_KW, l, scale=0.1, offset=1.0) for l in range(52)]
    # one cache per layer: paged for global layers, 512-slot rings for local ones
    caches = []
    for l, kind in enumerate(kinds):
        if kind == O.GLOBAL:
            bt, n_pages = synth.paged_block_table(1000 + l, lens)
            caches.append(ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt)))
        else:
            caches.append(ga.KVCache.allocate_local(CFG, n))
    # allocated bytes = paged KV budget of every sequence (bit-exact integers)
    alloc = sum(c.k.numel() * 2 + c.v.numel() * 2 for c in caches)
    budget = sum(ga.kv_bytes(int(L), 2, 9, 43)[1] for L in lens)
    assert alloc == budget, (alloc, budget)
    assert budget == sum(O.kv_bytes(int(L), 2)[1] for L in lens)

    check_layers = [kinds.index(O.LOCAL), kinds.index(O.GLOBAL), 50, 51]
    assert kinds[50] == O.LOCAL and kinds[51] == O.GLOBAL
    check_seqs = [int(np.argmin(lens)), int(np.argmax(lens))]
    kept = {(l, i): [] for l in check_layers for i in check_seqs}  # (rows, output bits)

    max_tok = n * CHUNK
    ws = torch.empty(ga.prefill_workspace_bytes(CFG, max_tok, n), dtype=torch.uint8, device="cuda")
    out = torch.empty((max_tok, 48, 128), dtype=torch.bfloat16, device="cuda")
    n_steps = int(-(-int(lens.max()) // CHUNK))
    gpu_ms = 0.0
    flops = 0
    for step in range(n_steps):
        s0 = step * CHUNK
        seqs = [i for i in range(n) if lens[i] > s0]
        clen = [min(CHUNK, int(lens[i]) - s0) for i in seqs]
        cu = np.concatenate([[0], np.cumsum(clen)]).astype(np.int32)
        n_tok = int(cu[-1])
        batch = {kind: {key: torch.cat([raw[kind, i][key][s0:s0 + c] for i, c in zip(seqs, clen)])
                        for key in ("q", "k", "v", "gate")} for kind in (O.LOCAL, O.GLOBAL)}
        cu_d, seq_d, start_d = dev_i32(cu), dev_i32(seqs), dev_i32([s0] * len(seqs))
        say(f"[case] 52-layer schedule step {step}: {len(seqs)} sequences, {n_tok} tokens")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for l, kind in enumerate(kinds):
            b = batch[kind]
            ga.prefill(CFG, caches[l], b["q"], b["k"], b["v"], dev_bf16(qw[l]), dev_bf16(kw[l]), b["gate"],
                       cu_d, seq_d, start_d, max(clen), out=out[:n_tok], workspace=ws)
            for i in check_seqs:
                if l in check_layers and i in seqs:
                    j = seqs.index(i)
                    c = clen[j]
                    rows = np.unique(np.linspace(0, c - 1, ROWS_PER_CHUNK).astype(np.int64))
                    sel = torch.from_numpy(int(cu[j]) + rows).cuda()
                    kept[l, i].append((s0 + rows, out.index_select(0, sel)))
        ev1.record()
        torch.cuda.synchronize()
        gpu_ms += ev0.elapsed_time(ev1)
        for c in clen:
            t = np.arange(s0, s0 + c)
            flops += 24576 * (9 * int((t + 1).sum()) + 43 * int(np.minimum(t + 1, 512).sum()))
    say(f"[perf] 52-layer chunked prefill: {flops / 1e12:.1f} TFLOP in {gpu_ms:.1f} ms "
        f"(incl. batch slicing and row sampling) = {flops / gpu_ms / 1e9:.1f} TFLOP/s")

    for (l, i), parts in kept.items():
        kind = kinds[l]
        rows = np.concatenate([p[0] for p in parts])
        got = np.concatenate([_bits(p[1]) for p in parts])
        r = raw[kind, i]
        last = int(rows.max()) + 1
        idx = torch.from_numpy(rows).cuda()
        ref = O.attention_layer(kind, _bits(r["q"][idx]), _bits(r["k"][:last]), _bits(r["v"][:last]), qw[l], kw[l],
                                _bits(r["gate"][idx]), rows, np.arange(last))
        compare(got, ref, f"52-layer schedule: layer {l + 1} ({'global' if kind else 'local'}), seq {i} "
                          f"(len {int(lens[i])}), {len(rows)} rows")
