// Driver of the host side of the C ABI under AddressSanitizer (no GPU): every
// host-only function and the argument checks, workspace sizing and workspace
// carving of the entry points, with launches replaced by recording stubs.
// Prints one line per result; tests/test_abi_host.py checks them against the
// oracle and against the regular library.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "beam_attn.h"
#include "beam_proj.h"
#include "beam_router.h"
#include "launch_stubs.h"

namespace {

beam_attn_config cfg() { return beam_attn_config{48, 8, 128, 512, 1e4f, 1e-6f, 2048.f, 0.1f}; }

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }  // device address, never dereferenced here

beam_kv_cache global_cache(int n_pages, int max_pages, int n_seqs, int dtype = BEAM_KV_BF16) {
  beam_kv_cache c{};
  c.kind = BEAM_GLOBAL;
  c.k = fake(0x10000000);
  c.v = fake(0x20000000);
  c.page_size = 16;
  c.n_pages = n_pages;
  c.block_table = static_cast<const int32_t*>(fake(0x30000000));
  c.max_pages_per_seq = max_pages;
  c.n_seqs = n_seqs;
  c.dtype = dtype;
  c.k_scale = c.v_scale = 1.f;
  return c;
}

void status_line(const char* what, beam_status s) {
  // the message is copied and measured: a dangling or overrun buffer trips the sanitizer
  const std::string msg = beam_last_error();
  std::printf("status %s %d %zu\n", what, (int)s, msg.size());
}

}  // namespace

int main() {
  // kv_bytes
  const int64_t ns[] = {0, 1, 15, 16, 17, 511, 512, 513, 131072, 1048576, 1048577};
  for (int64_t n : ns)
    for (int b : {1, 2}) {
      uint64_t lg = 0, pg = 0;
      const beam_status s = beam_kv_bytes(n, b, 9, 43, 8, 128, 512, 16, &lg, &pg);
      std::printf("kv_bytes %lld %d %d %llu %llu\n", (long long)n, b, (int)s, (unsigned long long)lg,
                  (unsigned long long)pg);
    }
  uint64_t lg, pg;
  status_line("kv_bytes_null", beam_kv_bytes(4, 2, 9, 43, 8, 128, 512, 16, nullptr, &pg));
  status_line("kv_bytes_neg", beam_kv_bytes(-1, 2, 9, 43, 8, 128, 512, 16, &lg, &pg));

  // page_slot on a host block table of 3 sequences x 5 pages
  std::vector<int32_t> bt(15);
  for (int i = 0; i < 15; ++i) bt[i] = 1000 - 7 * i;
  const int pairs[][2] = {{0, 0}, {0, 15}, {0, 16}, {1, 79}, {2, 40}, {2, 80}, {-1, 3}, {0, -2}};
  for (const auto& q : pairs) {
    int64_t page = -1;
    int32_t slot = -1;
    const beam_status s = beam_kv_page_slot(bt.data(), 5, 16, q[0], q[1], &page, &slot);
    std::printf("page_slot %d %d %d %lld %d\n", q[0], q[1], (int)s, (long long)page, (int)slot);
  }

  // workspace sizes
  const beam_attn_config c = cfg();
  for (int n_tok : {0, 1, 63, 64, 640, 32768})
    for (int n_seqs : {1, 3, 8})
      std::printf("ws_prefill %d %d %zu\n", n_tok, n_seqs, beam_prefill_workspace_bytes(&c, n_tok, n_seqs));
  for (int kind : {0, 1})
    for (int max_pos : {0, 511, 512, 131071, 1048575})
      for (int split : {0, 128, 2048})
        std::printf("ws_decode %d %d %d %zu\n", kind, max_pos, split,
                    beam_decode_workspace_bytes(&c, kind, 64, max_pos, split));
  for (int kind : {0, 1})
    for (int max_pos : {7, 4095, 131071})
      std::printf("ws_verify %d %d %zu\n", kind, max_pos, beam_verify_workspace_bytes(&c, kind, 64, 8, 8, max_pos, 0));

  // a valid prefill call: the workspace as the host side carves it
  {
    beam_kv_cache kv = global_cache(3000, 64, 4);
    const int n_tok = 1000, n_seqs = 3;
    const size_t ws = beam_prefill_workspace_bytes(&c, n_tok, n_seqs);
    void* f = fake(0x40000000);
    stub::last = stub::Record();
    const beam_status s =
        beam_attn_prefill(&c, &kv, static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f),
                          static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f), nullptr,
                          static_cast<int32_t*>(f), static_cast<int32_t*>(f), static_cast<int32_t*>(f), n_seqs, n_tok,
                          600, static_cast<beam_bf16*>(f), fake(0x50000000), ws, nullptr);
    const uintptr_t base = 0x50000000;
    std::printf("prefill_call %d %d %zu %zu %zu %d %d %d\n", (int)s, stub::last.calls,
                reinterpret_cast<uintptr_t>(stub::last.prologue.qp) - base,
                reinterpret_cast<uintptr_t>(stub::last.prologue.kw) - base,
                reinterpret_cast<uintptr_t>(stub::last.prologue.vw) - base, stub::last.prologue.P,
                stub::last.prefill.n_qtiles, stub::last.grid_b);
    status_line("prefill_ws_small", beam_attn_prefill(&c, &kv, static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f),
                                                      static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f),
                                                      static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f), nullptr,
                                                      static_cast<int32_t*>(f), static_cast<int32_t*>(f),
                                                      static_cast<int32_t*>(f), n_seqs, n_tok, 600,
                                                      static_cast<beam_bf16*>(f), fake(0x50000000), ws - 1, nullptr));
  }
  // a valid decode call: split grid and partial layout
  {
    beam_kv_cache kv = global_cache(70000, 65536, 1);
    void* f = fake(0x40000000);
    const size_t ws = beam_decode_workspace_bytes(&c, BEAM_GLOBAL, 1, 1048575, 0);
    stub::last = stub::Record();
    const beam_status s = beam_attn_decode(&c, &kv, static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f),
                                           static_cast<beam_bf16*>(f), nullptr, static_cast<int32_t*>(f),
                                           static_cast<int32_t*>(f), 1, 1048575, 0, static_cast<beam_bf16*>(f),
                                           fake(0x60000000), ws, nullptr);
    std::printf("decode_call %d %d %d %d %zu %zu\n", (int)s, stub::last.calls, stub::last.decode.n_splits,
                stub::last.decode.kpw, reinterpret_cast<uintptr_t>(stub::last.decode.part_ml) - 0x60000000,
                reinterpret_cast<uintptr_t>(stub::last.decode.part_acc) - 0x60000000);
    // no-alloc decode: a size beyond the library's array is refused before any runtime call
    beam_kv_cache kv64 = global_cache(500000, 8192, 64);
    status_line("decode_noalloc_too_big",
                beam_attn_decode_noalloc(&c, &kv64, static_cast<beam_bf16*>(f), static_cast<beam_bf16*>(f),
                                         static_cast<beam_bf16*>(f), nullptr, static_cast<int32_t*>(f),
                                         static_cast<int32_t*>(f), 64, 131071, 2048, static_cast<beam_bf16*>(f),
                                         nullptr));
  }
  // argument checks of the other entry points
  {
    beam_attn_config bad = cfg();
    bad.head_dim = 64;
    beam_kv_cache kv = global_cache(100, 8, 2);
    status_line("append_head_dim", beam_kv_append(&bad, &kv, nullptr, nullptr, nullptr, nullptr, nullptr, 4, nullptr));
    status_line("append_null", beam_kv_append(&c, &kv, nullptr, nullptr, nullptr, nullptr, nullptr, 4, nullptr));
    kv.page_size = 64;
    status_line("append_page", beam_kv_append(&c, &kv, nullptr, nullptr, nullptr, nullptr, nullptr, 4, nullptr));
    beam_kv_cache loc{};
    loc.kind = BEAM_LOCAL;
    status_line("validate_local", beam_debug_validate_cache(&loc, nullptr, static_cast<int32_t*>(fake(0x100)), nullptr));
    status_line("visibility_kind", beam_debug_visibility(5, 512, 0, 4, 0, 4, static_cast<uint8_t*>(fake(0x100)), nullptr));
    beam_router_config rc{5120, 256, 8, 4, 8, 2.5f};
    rc.n_experts = 128;
    status_line("router_experts", beam_router(&rc, nullptr, nullptr, nullptr, 4, nullptr, nullptr, nullptr));
    status_line("out_project_k", beam_out_project(nullptr, nullptr, 4, 100, 256, nullptr, nullptr));
  }
  // V layout conversion: argument checks, then the blocks of a paged and a
  // local cache (bf16 and FP8)
  {
    beam_kv_cache kv = global_cache(100, 8, 2);
    status_line("convert_v_null", beam_kv_convert_v(&c, &kv, nullptr, 1, nullptr));
    status_line("convert_v_align", beam_kv_convert_v(&c, &kv, fake(0x70000008), 1, nullptr));
    status_line("convert_v_overlap", beam_kv_convert_v(&c, &kv, fake(0x20000000 + 100 * 8 * 16 * 128 * 2 - 16), 1,
                                                       nullptr));
    stub::last = stub::Record();
    beam_status s = beam_kv_convert_v(&c, &kv, fake(0x20000000 + 100 * 8 * 16 * 128 * 2), 1, nullptr);
    std::printf("convert_v_call %d %d %d %d %d\n", BEAM_GLOBAL, (int)s, stub::last.calls, stub::last.grid_a,
                stub::last.grid_b);
    beam_kv_cache loc{};
    loc.kind = BEAM_LOCAL;
    loc.k = fake(0x10000000);
    loc.v = fake(0x20000000);
    loc.n_seqs = 3;
    loc.dtype = BEAM_KV_FP8_E4M3;
    loc.k_scale = loc.v_scale = 1.f;
    stub::last = stub::Record();
    s = beam_kv_convert_v(&c, &loc, fake(0x70000000), 0, nullptr);
    std::printf("convert_v_call %d %d %d %d %d\n", BEAM_LOCAL, (int)s, stub::last.calls, stub::last.grid_a,
                stub::last.grid_b);
  }
  // the thread-local message, from several threads at once
  {
    std::vector<std::thread> th;
    std::vector<int> ok(8, 0);
    for (int i = 0; i < 8; ++i)
      th.emplace_back([&, i] {
        uint64_t a, b;
        for (int r = 0; r < 200; ++r) {
          beam_kv_bytes(-1 - i, 2, 9, 43, 8, 128, 512, 16, &a, &b);
          const std::string m = beam_last_error();
          ok[i] += m.empty() ? 0 : 1;
        }
      });
    for (auto& t : th) t.join();
    int total = 0;
    for (int v : ok) total += v;
    std::printf("threads %d\n", total);
  }
  std::printf("done\n");
  return 0;
}
