"""CPU tests of the C-ABI library: it loads, exports every declared symbol, its
host-only functions agree with the oracle, and argument checks fail before any
launch. No GPU is touched."""
import ctypes
import os
import re

import numpy as np
import pytest

import global_attention_amd as ga
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(beam_\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = ga.lib()
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(ga.EXPORTED) == declared


def test_library_is_built_for_gfx950():
    data = open(ga.LIB_PATH, "rb").read()
    assert b"gfx950" in data


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 511, 512, 513, 131072, 1048576, 10 ** 7])
@pytest.mark.parametrize("b", [1, 2])
def test_kv_bytes_matches_oracle(n, b):
    got = ga.kv_bytes(n, b)
    assert got == O.kv_bytes(n, b)


def test_kv_bytes_printed_values():
    assert ga.kv_bytes(1, 2, 9, 0)[0] == 36 * 1024
    assert ga.kv_bytes(1, 2, 52, 0)[0] == 208 * 1024
    assert ga.kv_bytes(1048576, 2)[0] == 36 * 2 ** 30 + 86 * 2 ** 20


def test_page_slot_matches_oracle():
    g = np.random.default_rng(0)
    bt = g.permutation(4 * 9).astype(np.int32).reshape(4, 9)
    for seq in range(4):
        for t in (0, 1, 15, 16, 17, 100, 143):
            assert ga.kv_page_slot(bt, 16, seq, t) == O.page_slot(bt, 16, seq, t)
    with pytest.raises(ga.BeamError) as e:
        ga.kv_page_slot(bt, 16, 0, 144)
    assert e.value.status == 3


def test_workspace_sizes():
    cfg = ga.Config()
    a = ga.prefill_workspace_bytes(cfg, 32768, 1)
    assert a >= 32768 * 48 * 128 * 2 + 2 * 8 * 32768 * 128 * 2
    assert ga.decode_workspace_bytes(cfg, ga.GLOBAL, 64, 131071) > 0
    assert ga.decode_workspace_bytes(cfg, ga.GLOBAL, 64, 131071, split_keys=100) == 0
    assert ga.prefill_workspace_bytes(ga.Config(head_dim=64), 10, 1) == 0


def _call_prefill(cfg, cache, ws_bytes=1 << 30, n_tok=4, max_chunk=4, ws=0x1000, n_seqs=1):
    L = ga.lib()
    c = cfg.c()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: the checks fail first
    return L.beam_attn_prefill(ctypes.byref(c), ctypes.byref(cache), fake, fake, fake, fake, fake, fake,
                               None, fake, fake, fake, n_seqs, n_tok, max_chunk, fake,
                               ctypes.c_void_p(ws), ws_bytes, None)


def _cache(kind=ga.GLOBAL, page_size=16):
    return ga.CCache(kind, 0x200000, 0x300000, page_size, 10, 0x400000 if kind == ga.GLOBAL else None, 4, 2)


def test_argument_checks_fail_before_launch():
    L = ga.lib()
    assert _call_prefill(ga.Config(), _cache(), n_tok=0, max_chunk=0) == 0  # empty work, nothing launched
    assert _call_prefill(ga.Config(head_dim=64), _cache()) == 4
    assert _call_prefill(ga.Config(n_q_heads=47), _cache()) == 2
    assert _call_prefill(ga.Config(n_q_heads=48, n_kv_heads=2), _cache()) == 4   # 24 heads per KV head
    assert _call_prefill(ga.Config(n_q_heads=64, n_kv_heads=16), _cache()) == 4  # more than 8 KV heads
    # cache dtype and FP8 scales
    c = _cache()
    c.dtype = 2
    assert _call_prefill(ga.Config(), c) == 4
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        c = _cache()
        c.dtype, c.k_scale, c.v_scale = ga.KV_FP8_E4M3, ks, vs
        assert _call_prefill(ga.Config(), c) == 3
    # 2^15 sequences with 2^22-token chunks: the workspace fits 32-bit offsets but the grid would not
    assert _call_prefill(ga.Config(), _cache(), ws_bytes=1 << 40, n_tok=1 << 22, max_chunk=1 << 22, n_seqs=1 << 15) == 3
    # workspace positions x 128 beyond 2^31
    assert _call_prefill(ga.Config(), _cache(), ws_bytes=1 << 40, n_tok=1 << 24, max_chunk=64) == 3
    assert _call_prefill(ga.Config(window=500), _cache()) == 4
    assert _call_prefill(ga.Config(), _cache(page_size=64)) == 4
    assert _call_prefill(ga.Config(), _cache(), ws_bytes=10) == 5
    assert _call_prefill(ga.Config(), _cache(), max_chunk=5) == 3
    assert _call_prefill(ga.Config(), _cache(), ws=0x1001) == 3
    msg = L.beam_last_error().decode()
    assert "aligned" in msg
    # NULL config / cache
    assert L.beam_attn_prefill(None, None, *([None] * 10), 1, 4, 4, None, None, 0, None) == 1
    # decode beyond block-table capacity: 4 pages of 16 -> max_pos 63
    c = ga.Config().c()
    kc = _cache()
    fake = ctypes.c_void_p(0x100000)
    st = L.beam_attn_decode(ctypes.byref(c), ctypes.byref(kc), fake, fake, fake, None, fake, fake, 1, 64, 0,
                            fake, ctypes.c_void_p(0x1000), 1 << 30, None)
    assert st == 3 and "capacity" in L.beam_last_error().decode()
    st = L.beam_attn_decode(ctypes.byref(c), ctypes.byref(kc), fake, fake, fake, None, fake, fake, 1, 63, 100,
                            fake, ctypes.c_void_p(0x1000), 1 << 30, None)
    assert st == 3
    # empty work succeeds without launching
    assert L.beam_attn_decode(ctypes.byref(c), ctypes.byref(kc), *([None] * 6), 0, 0, 0, None, None, 0, None) == 0
    assert L.beam_kv_append(ctypes.byref(c), ctypes.byref(kc), *([None] * 5), 0, None) == 0
    assert L.beam_debug_visibility(2, 512, 0, 4, 0, 4, fake, None) == 3
    assert L.beam_status_str(5) == b"workspace too small"


def _call_verify(cfg, cache, max_chunk=4, max_pos=100, split_keys=0, ws_bytes=1 << 30, n_tok=4, n_seqs=1):
    L = ga.lib()
    c = cfg.c()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: the checks fail first
    return L.beam_attn_verify(ctypes.byref(c), ctypes.byref(cache), fake, fake, fake, fake, fake, fake, None, fake,
                              fake, fake, n_seqs, n_tok, max_chunk, max_pos, split_keys, fake,
                              ctypes.c_void_p(0x1000), ws_bytes, None)


def test_verify_workspace_and_checks():
    cfg = ga.Config()
    L = ga.lib()
    # splits: global keys 0..max_pos in 64-key tiles; the default split is the longest
    # of 8192 and 4096 keys for which 8 sequences x 8 KV heads x (max_pos // keys + 1)
    # reach 1024 blocks, else 2048
    base = ga.prefill_workspace_bytes(cfg, 64, 8)
    for max_pos, splits in ((0, 1), (2047, 1), (2048, 2), (32767, 16), (65535, 16), (65536, 17), (131071, 16)):
        rows = 64 * 48 * splits
        want = base + ((rows * 8 + 255) // 256) * 256 + ((rows * 512 + 255) // 256) * 256
        assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, max_pos) == want
    for max_pos in (0, 65535, 65536, 131071):
        explicit = next((k for k in (8192, 4096) if 64 * (max_pos // k + 1) >= 1024), 2048)
        assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, max_pos) == \
            ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, max_pos, split_keys=explicit)
    # local: the window bounds the keys (511 + 7 positions span at most 10 tiles); 8 sequences x 8 KV
    # heads (64 blocks) -> 256-key splits, 3 of them; 32 sequences (256 blocks) -> one split of 640 keys
    rows = 64 * 48 * 3
    want = base + ((rows * 8 + 255) // 256) * 256 + ((rows * 512 + 255) // 256) * 256
    assert ga.verify_workspace_bytes(cfg, ga.LOCAL, 64, 8, 8, 131071) == want
    base32 = ga.prefill_workspace_bytes(cfg, 256, 32)
    rows = 256 * 48 * 1
    want = base32 + ((rows * 8 + 255) // 256) * 256 + ((rows * 512 + 255) // 256) * 256
    assert ga.verify_workspace_bytes(cfg, ga.LOCAL, 256, 32, 8, 131071) == want
    assert want == ga.verify_workspace_bytes(cfg, ga.LOCAL, 256, 32, 8, 131071, split_keys=640)
    assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, 1000, split_keys=96) == 0
    assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, 1000, split_keys=64) > 0
    assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, 1000, split_keys=8192) > 0
    assert ga.verify_workspace_bytes(cfg, ga.GLOBAL, 64, 8, 8, 1000, split_keys=8256) == 0
    assert ga.verify_workspace_bytes(cfg, 2, 64, 8, 8, 1000) == 0
    # 21 tokens x 6 heads = 126 rows fit one 128-row block; 22 do not
    assert _call_verify(cfg, _cache(), max_chunk=22, n_tok=22) == 3
    assert "128" in L.beam_last_error().decode()
    assert _call_verify(cfg, _cache(), split_keys=100) == 3
    assert _call_verify(cfg, _cache(), max_pos=2) == 3  # below max_chunk_len - 1
    assert _call_verify(cfg, _cache(), ws_bytes=ga.prefill_workspace_bytes(cfg, 4, 1)) == 5
    # empty work succeeds without launching
    c, kc = cfg.c(), _cache()
    assert L.beam_attn_verify(ctypes.byref(c), ctypes.byref(kc), *([None] * 10), 1, 0, 0, 0, 0, None, None, 0,
                              None) == 0
    # unknown stage bits (16 and above)
    fake = ctypes.c_void_p(0x100000)
    assert L.beam_attn_verify_stages(32, ctypes.byref(c), ctypes.byref(kc), *([fake] * 6), None, fake, fake, fake,
                                     1, 4, 4, 100, 0, fake, ctypes.c_void_p(0x1000), 1 << 30, None) == 3


def test_router_argument_checks():
    L = ga.lib()
    fake = ctypes.c_void_p(0x100000)

    def call(rc, n_tok=4, x=fake):
        c = rc.c()
        return L.beam_router(ctypes.byref(c), x, fake, None, n_tok, fake, fake, None)

    assert call(ga.RouterConfig(hidden=100)) == 4
    assert call(ga.RouterConfig(hidden=0)) == 4
    assert call(ga.RouterConfig(n_experts=128)) == 4
    assert call(ga.RouterConfig(n_groups=4)) == 4
    assert call(ga.RouterConfig(topk_groups=0)) == 4
    assert call(ga.RouterConfig(topk_groups=9)) == 4
    assert call(ga.RouterConfig(top_k=9)) == 4
    assert call(ga.RouterConfig(scale=float("nan"))) == 3
    assert call(ga.RouterConfig(), n_tok=-1) == 3
    assert call(ga.RouterConfig(), x=None) == 1
    assert call(ga.RouterConfig(), n_tok=0, x=None) == 0          # empty work, nothing launched
    assert L.beam_router(None, fake, fake, None, 4, fake, fake, None) == 1
    c = ga.RouterConfig().c()
    assert L.beam_router_logits(ctypes.byref(c), fake, fake, 4, None, None) == 1
    assert L.beam_router_select(ctypes.byref(c), None, None, 4, fake, fake, None) == 1
    assert L.beam_router_select(ctypes.byref(c), None, None, 0, None, None, None) == 0


def test_projection_argument_checks():
    L = ga.lib()
    fake = ctypes.c_void_p(0x100000)
    cfg = ga.Config()
    c = cfg.c()
    ws_need = ga.prefill_workspace_bytes(cfg, 4, 1)

    def proj(kind=ga.GLOBAL, hidden=5120, n_tok=4, x=fake, ws=ctypes.c_void_p(0x1000), ws_bytes=ws_need):
        return L.beam_attn_project(ctypes.byref(c), kind, x, hidden, fake, fake, fake, fake, 1, n_tok, fake, fake,
                                   fake, ws, ws_bytes, None)

    assert proj(kind=2) == 3
    assert proj(hidden=100) == 4                       # not a multiple of 128
    assert proj(hidden=192) == 4
    assert proj(hidden=0) == 4
    assert proj(hidden=65536 + 128) == 4
    assert proj(n_tok=-1) == 3
    assert proj(x=None) == 1
    assert proj(x=ctypes.c_void_p(0x100008)) == 3      # not 16-byte aligned
    assert proj(ws=ctypes.c_void_p(0x1010)) == 3       # not 256-byte aligned
    assert proj(ws_bytes=ws_need - 1) == 5
    assert proj(n_tok=0, x=None) == 0                  # empty work, nothing launched
    assert L.beam_attn_project(None, 0, fake, 5120, fake, fake, fake, fake, 1, 4, fake, fake, fake, fake, 0,
                               None) == 1

    def outp(n_tok=4, k=6144, n_out=5120, y=fake):
        return L.beam_out_project(y, fake, n_tok, k, n_out, fake, None)

    assert outp(k=100) == 4
    assert outp(n_out=5000) == 4                       # not a multiple of 256
    assert outp(n_out=0) == 4
    assert outp(y=None) == 1
    assert outp(y=ctypes.c_void_p(0x100004)) == 3
    assert outp(n_tok=0, y=None) == 0
    assert outp(n_tok=1 << 30, n_out=1 << 30) == 3     # grid beyond 2^31 blocks


def test_prologue_kv_stage_rules():
    L = ga.lib()
    fake = ctypes.c_void_p(0x100000)
    c, kc = ga.Config().c(), _cache()

    def call(stages, q=fake):
        return L.beam_attn_prefill_stages(stages, ctypes.byref(c), ctypes.byref(kc), q, *([fake] * 5), None, fake,
                                          fake, fake, 1, 4, 4, fake, ctypes.c_void_p(0x1000), 10, None)

    # the two prologue forms exclude each other; checked before the workspace size
    assert call(ga.STAGE_PROLOGUE | ga.STAGE_PROLOGUE_KV) == 3
    # q_raw may be NULL only without the full prologue (here the small workspace is what fails next)
    assert call(ga.STAGE_PROLOGUE_KV | ga.STAGE_ATTENTION, q=None) == 5
    assert call(ga.STAGE_PROLOGUE | ga.STAGE_ATTENTION, q=None) == 1
    assert call(32) == 3


def test_tensor_alignment_checks():
    """bf16 tensors move with 8- and 16-byte vector accesses: a pointer that is
    not 16-byte aligned is rejected (BEAM_E_RANGE) before any launch."""
    L = ga.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100008)
    c = ga.Config().c()
    kc = _cache()

    def prefill(i):
        t = [fake] * 6
        t[i] = odd
        return L.beam_attn_prefill(ctypes.byref(c), ctypes.byref(kc), *t, None, fake, fake, fake, 1, 4, 4, fake,
                                   ctypes.c_void_p(0x1000), 1 << 30, None)

    for i in range(6):  # q_raw, k_raw, v_raw, q_norm_w, k_norm_w, gate_logits
        assert prefill(i) == 3 and "aligned" in L.beam_last_error().decode()
    assert L.beam_attn_prefill(ctypes.byref(c), ctypes.byref(kc), *([fake] * 6), None, fake, fake, fake, 1, 4, 4,
                               odd, ctypes.c_void_p(0x1000), 1 << 30, None) == 3  # out

    def decode(i):
        t = [fake] * 3
        t[i] = odd
        return L.beam_attn_decode(ctypes.byref(c), ctypes.byref(kc), *t, None, fake, fake, 1, 63, 0, fake,
                                  ctypes.c_void_p(0x1000), 1 << 30, None)

    for i in range(3):  # q_raw, q_norm_w, gate_logits
        assert decode(i) == 3 and "aligned" in L.beam_last_error().decode()

    def append(i):
        t = [fake] * 3
        t[i] = odd
        return L.beam_kv_append(ctypes.byref(c), ctypes.byref(kc), *t, fake, fake, 4, None)

    for i in range(3):  # k_raw, v_raw, k_norm_w
        assert append(i) == 3 and "aligned" in L.beam_last_error().decode()
    # the cache's own buffers
    bad = ga.CCache(ga.GLOBAL, 0x200008, 0x300000, 16, 10, 0x400000, 4, 2)
    assert L.beam_kv_append(ctypes.byref(c), ctypes.byref(bad), fake, fake, fake, fake, fake, 4, None) == 3


def test_validate_cache_argument_checks():
    """beam_debug_validate_cache checks its host-visible arguments before any
    launch: a local cache has no block table, NULL pointers and empty tables
    are refused."""
    L = ga.lib()
    fake = ctypes.c_void_p(0x100000)
    loc = _cache(ga.LOCAL)
    assert L.beam_debug_validate_cache(ctypes.byref(loc), None, fake, None) == 3
    assert "block table" in L.beam_last_error().decode()
    assert L.beam_debug_validate_cache(None, None, fake, None) == 1
    glb = _cache()
    assert L.beam_debug_validate_cache(ctypes.byref(glb), None, None, None) == 1
    glb.block_table = None
    assert L.beam_debug_validate_cache(ctypes.byref(glb), None, fake, None) == 1
    for field in ("n_seqs", "max_pages_per_seq", "n_pages", "page_size"):
        c = _cache()
        setattr(c, field, 0)
        assert L.beam_debug_validate_cache(ctypes.byref(c), None, fake, None) == 3, field


# ---- the host side under AddressSanitizer and UndefinedBehaviorSanitizer ----
# The C ABI (beam_attn.hip) is rebuilt with the sanitizers on its host pass only
# (its device code is not run) and linked with recording launch stubs and a
# driver (tests/asan/); the driver prints every host-only result, the status of
# argument-check failures and the workspace carving of valid calls.

def _build_asan_driver(out_dir):
    import subprocess
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "global_attention_amd", "csrc"),
           "-I" + os.path.join(ROOT, "tests", "asan")]
    import shlex
    san = shlex.split("-Xarch_host -fsanitize=address,undefined")  # host pass only
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + san + inc
    objs = []
    units = [(os.path.join(ROOT, "global_attention_amd", "csrc", "beam_attn.hip"),
              ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]),
             (os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), []),
             (os.path.join(ROOT, "tests", "asan", "host_abi_driver.cpp"), [])]
    for src, extra in units:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["hipcc"] + extra + common + ["-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    exe = os.path.join(out_dir, "host_abi_driver")
    subprocess.run(["hipcc", "--hip-link", "--offload-arch=gfx950"] + san + objs + ["-o", exe, "-lpthread"],
                   check=True, capture_output=True)
    return exe


# beam_status values (include/beam_attn.h)
E_NULL, E_RANGE, E_UNSUPPORTED, E_WORKSPACE = 1, 3, 4, 5


def test_host_side_under_address_sanitizer(tmp_path):
    import shutil
    import subprocess
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not on PATH")
    exe = _build_asan_driver(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120, cwd=str(tmp_path))
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert lines[-1] == "done"
    rows = [ln.split() for ln in lines[:-1]]
    by = {}
    for row in rows:
        by.setdefault(row[0], []).append(row[1:])

    for n, b, st, lg, pg in by["kv_bytes"]:
        assert int(st) == 0
        assert (int(lg), int(pg)) == O.kv_bytes(int(n), int(b))
    bt = (1000 - 7 * np.arange(15, dtype=np.int64)).reshape(3, 5)
    for seq, t, st, page, slot in by["page_slot"]:
        seq, t = int(seq), int(t)
        if 0 <= seq < 3 and 0 <= t < 5 * 16:
            assert int(st) == 0 and (int(page), int(slot)) == O.page_slot(bt, 16, seq, t)
        else:
            assert int(st) == E_RANGE

    cfg = ga.Config()
    for n_tok, n_seqs, got in by["ws_prefill"]:
        assert int(got) == ga.prefill_workspace_bytes(cfg, int(n_tok), int(n_seqs))
    for kind, max_pos, split, got in by["ws_decode"]:
        assert int(got) == ga.decode_workspace_bytes(cfg, int(kind), 64, int(max_pos), int(split))
    for kind, max_pos, got in by["ws_verify"]:
        assert int(got) == ga.verify_workspace_bytes(cfg, int(kind), 64, 8, 8, int(max_pos))

    # prefill of 1000 tokens in 3 chunks (longest 600) on a global cache: the
    # prologue and the attention launch (the append is fused into the
    # prologue); Q', K_hat and V^T carved without overlap inside the workspace
    st, calls, qp, kw, vw, P, n_qtiles, _ = map(int, by["prefill_call"][0])
    ws = ga.prefill_workspace_bytes(cfg, 1000, 3)
    H, G, D = 48, 8, 128
    assert st == 0 and calls == 2
    assert qp == 0 and kw >= 1000 * H * D * 2 and vw - kw >= G * P * D * 2 and vw + G * P * D * 2 <= ws
    assert kw % 256 == 0 and vw % 256 == 0 and P % 64 == 0 and P >= 1000
    assert n_qtiles == -(-600 // 384)  # 384-query blocks on global layers (8 waves x 48 queries)

    # decode of one sequence at position 2^20 - 1, default split (4096 keys:
    # 8 KV heads x 256 splits reach 1024 blocks): Q' then the (max, sum) and
    # accumulator partials of 256 splits
    st, calls, n_splits, kpw, ml, acc = map(int, by["decode_call"][0])
    assert st == 0 and calls == 3 and n_splits == 256 and kpw == 1024
    assert ml == H * D * 2 and acc == ml + -(-(H * n_splits * 2 * 4) // 256) * 256
    assert acc + H * n_splits * D * 4 <= ga.decode_workspace_bytes(cfg, ga.GLOBAL, 1, 2 ** 20 - 1)

    want = {"kv_bytes_null": E_NULL, "kv_bytes_neg": E_RANGE,
            "prefill_ws_small": E_WORKSPACE, "decode_noalloc_too_big": E_WORKSPACE,
            "append_head_dim": E_UNSUPPORTED, "append_null": E_NULL,
            "append_page": E_UNSUPPORTED, "validate_local": E_RANGE,
            "visibility_kind": E_RANGE, "router_experts": E_UNSUPPORTED,
            "out_project_k": E_UNSUPPORTED, "convert_v_null": E_NULL, "convert_v_align": E_RANGE,
            "convert_v_overlap": E_RANGE}
    got = {what: (int(st), int(msg_len)) for what, st, msg_len in by["status"]}
    assert {k: v[0] for k, v in got.items()} == want
    assert all(v[1] > 0 for v in got.values())
    # V layout conversion: one launch over every (page, KV head) block of 16
    # rows, or every (ring, KV head) block of window rows
    conv = {int(r[0]): tuple(map(int, r[1:])) for r in by["convert_v_call"]}
    assert conv[ga.GLOBAL] == (0, 1, 100 * 8, 16)
    assert conv[ga.LOCAL] == (0, 1, 3 * 8, 512)
    assert by["threads"] == [["1600"]]
