"""GPU checks of the library's guards on device-resident indices, through the
C ABI: the opt-in block-table check and the NaN rows that decode and verify
write for a sequence they cannot serve. Every planted bad index here is one the
kernels compare and never dereference (the block-table check reads only ids;
decode skips a row whose cache sequence does not exist; verify never reads
past the split grid). Results are bit-exact: counts and NaN positions.
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


def _bad_count(bt, n_pages, n_tokens, page_size=16):
    out = []
    for c in range(bt.shape[0]):
        if n_tokens is None:
            used = bt.shape[1]
        else:
            nt = int(n_tokens[c])
            used = -(-nt // page_size) if nt >= 0 else -1
            if nt < 0 or used > bt.shape[1]:
                out.append(-1)
                continue
        row = bt[c, :used]
        out.append(int(np.count_nonzero((row < 0) | (row >= n_pages))))
    return np.array(out, dtype=np.int32)


def test_validate_cache_counts_planted_ids():
    import torch
    ctx = [1000, 37, 4096, 16, 5000, 1]
    bt, n_pages = synth.paged_block_table(70, ctx, extra_pages=5)
    n_tok = np.array(ctx, dtype=np.int32)
    # planted ids: inside the used range (counted) and past it (not counted)
    bt[0, 3] = -1
    bt[0, 62] = n_pages
    bt[2, 0] = n_pages + 7
    bt[2, 255] = -2 ** 31
    bt[2, 100] = 2 ** 31 - 1
    bt[4, 312] = -5                     # last used page of 5000 tokens (313 pages)
    bt[1, 3] = n_pages                  # 37 tokens use pages 0..2 only: not counted
    cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    say("[case] validate_cache with planted ids")
    got = ga.debug_validate_cache(cache, dev_i32(n_tok)).cpu().numpy()
    want = _bad_count(bt, n_pages, n_tok)
    assert np.array_equal(got, want), (got, want)
    assert list(want) == [2, 0, 3, 0, 1, 0]
    # whole rows: the -1 padding the table generator leaves past a sequence's pages counts too
    got_rows = ga.debug_validate_cache(cache).cpu().numpy()
    assert np.array_equal(got_rows, _bad_count(bt, n_pages, None))
    # lengths that do not fit the row (or are negative) report -1
    n_tok2 = n_tok.copy()
    n_tok2[1] = bt.shape[1] * 16 + 1
    n_tok2[3] = -4
    n_tok2[5] = bt.shape[1] * 16
    got2 = ga.debug_validate_cache(cache, dev_i32(n_tok2)).cpu().numpy()
    assert np.array_equal(got2, _bad_count(bt, n_pages, n_tok2))
    assert got2[1] == -1 and got2[3] == -1 and got2[5] >= 0


def test_validate_cache_rejects_local_cache():
    cache = ga.KVCache.allocate_local(CFG, 2)
    with pytest.raises(ValueError):
        ga.debug_validate_cache(cache)


@pytest.mark.parametrize("kind", [O.LOCAL, O.GLOBAL])
def test_decode_nan_rows_for_missing_cache_sequence(kind):
    """A decode row whose seq_idx names no cache sequence (or whose position is
    past max_pos) is NaN; the other rows still match the oracle."""
    import torch
    ts = [300, 40, 700]
    hist = [synth.attention_inputs(71, 10 * kind + i, t + 1) for i, t in enumerate(ts)]
    for x in hist[1:]:
        x["q_norm_w"], x["k_norm_w"] = hist[0]["q_norm_w"], hist[0]["k_norm_w"]
    if kind == O.GLOBAL:
        bt, n_pages = synth.paged_block_table(71, [t + 1 for t in ts])
        cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    else:
        cache = ga.KVCache.allocate_local(CFG, len(ts))
    for i, t in enumerate(ts):
        lo = 0 if kind == O.GLOBAL else max(0, t + 1 - 512)
        ga.kv_append(CFG, cache, dev_bf16(hist[i]["k"][lo:]), dev_bf16(hist[i]["v"][lo:]),
                     dev_bf16(hist[0]["k_norm_w"]), dev_i32(np.full(t + 1 - lo, i)), dev_i32(np.arange(lo, t + 1)))
    q = np.stack([x["q"][t] for x, t in zip(hist, ts)] * 2)
    gate = np.stack([x["gate"][t] for x, t in zip(hist, ts)] * 2)
    # rows 3..5 repeat rows 0..2 with a missing cache sequence, a negative one
    # and a position past max_pos
    seq = [0, 1, 2, len(ts), -1, 2]
    pos = ts + [ts[0], ts[1], 701]
    say(f"[case] decode kind={kind} NaN rows")
    out = ga.decode(CFG, cache, dev_bf16(q), dev_bf16(hist[0]["q_norm_w"]), dev_bf16(gate), dev_i32(seq),
                    dev_i32(pos), 700)
    sync()
    o = host_bits(out)
    nan = np.isnan((o.astype(np.uint32) << 16).view(np.float32))
    assert not nan[:3].any()
    assert nan[3:].all()
    for i, (x, t) in enumerate(zip(hist, ts)):
        ref = O.attention_layer(kind, x["q"][t:t + 1], x["k"][:t + 1], x["v"][:t + 1], x["q_norm_w"],
                                x["k_norm_w"], x["gate"][t:t + 1], np.array([t]), np.arange(t + 1))
        compare(o[i:i + 1], ref, f"decode kind={kind} row {i}")


@pytest.mark.parametrize("split_keys", [0, 64], ids=["one_split", "four_splits"])
def test_verify_nan_rows_past_max_pos(split_keys):
    """Verify: a sequence whose chunk ends past max_pos gets NaN rows; the
    other sequence of the call still matches the oracle. With one key split
    (the default here) the split kernel writes the rows itself; with 64-key
    splits the combine does."""
    import torch
    kind = O.GLOBAL
    hist_len, chunk = [200, 300], [6, 6]
    total = [h + c for h, c in zip(hist_len, chunk)]
    xs = [synth.attention_inputs(72, i, n) for i, n in enumerate(total)]
    xs[1]["q_norm_w"], xs[1]["k_norm_w"] = xs[0]["q_norm_w"], xs[0]["k_norm_w"]
    bt, n_pages = synth.paged_block_table(72, total)
    cache = ga.KVCache.allocate_global(CFG, n_pages, torch.from_numpy(bt))
    w = xs[0]
    cu = np.array([0, 200, 500], dtype=np.int32)
    cat = lambda key: dev_bf16(np.concatenate([x[key][:h] for x, h in zip(xs, hist_len)]))
    ga.prefill(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]),
               cat("gate"), dev_i32(cu), dev_i32([0, 1]), dev_i32([0, 0]), 300)
    cu = np.array([0, 6, 12], dtype=np.int32)
    cat = lambda key: dev_bf16(np.concatenate([x[key][h:h + c] for x, h, c in zip(xs, hist_len, chunk)]))
    max_pos = 205  # covers sequence 0 (ends at 205), not sequence 1 (ends at 305)
    say("[case] verify NaN rows past max_pos")
    out = ga.verify(CFG, cache, cat("q"), cat("k"), cat("v"), dev_bf16(w["q_norm_w"]), dev_bf16(w["k_norm_w"]),
                    cat("gate"), dev_i32(cu), dev_i32([0, 1]), dev_i32(hist_len), 6, max_pos, split_keys=split_keys,
                    stages=ga.STAGE_PROLOGUE | ga.STAGE_ATTENTION | ga.STAGE_VERIFY_COMBINE)
    sync()
    o = host_bits(out)
    f = (o.astype(np.uint32) << 16).view(np.float32)
    assert np.isnan(f[6:]).all()
    assert not np.isnan(f[:6]).any()
    x = xs[0]
    ref = O.attention_layer(kind, x["q"][200:206], x["k"][:206], x["v"][:206], x["q_norm_w"], x["k_norm_w"],
                            x["gate"][200:206], np.arange(200, 206), np.arange(206))
    compare(o[:6], ref, "verify seq0 within max_pos")
