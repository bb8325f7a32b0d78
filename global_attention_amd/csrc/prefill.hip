// Flash-style causal / sliding-window prefill attention with bf16 MFMA (gfx950).
//
// Computes, per query head h and query position t of a chunk,
//   O_t = sum_s softmax_s(q'_t . k'_s) V_s over the visible keys s, then
//   Y_t = O_t * sigmoid(gate_t + b_h),
// the attention of "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax"
// (sections "Two attention paths in one decoder" and "Follow the tensors, not
// the parameter label"). The score matrix is never materialised (section "KV
// memory: nine growing caches, not 52" notes flash-style kernels avoid it).
//
// Tiling. A block is NWAVES wavefronts x QW queries of one query head. KV tiles
// of 64 keys are double-buffered in LDS. Each wave computes
// S^T = K Q'^T with v_mfma_f32_32x32x16_bf16 (keys on M, its queries on N), so
// a lane holds one query column and the row max is an in-lane max plus one
// v_permlane32_swap. The S accumulators are packed to bf16 and fed directly as
// the B operand of O^T += V^T P^T.
//
// LDS layout. Tiles that lie inside the chunk are copied from the workspace
// straight into LDS with global_load_lds_dwordx4 (no staging registers).
//   K:   two coordinate halves, each 64 rows x 128 B. LDS row m holds key
//        kappa(m) = m with bits 2 and 3 swapped; the MFMA output row order
//        then becomes natural key order, which is the order the PV operand
//        needs.
//   V^T: 128 rows (coordinates) x 128 B (64 keys, natural order).
// Both XOR-swizzle their 16-byte chunks with bits 1..3 of the row. A b128
// read is served 16 lanes per LDS cycle, and the operand reads have those
// lanes on 16 consecutive rows, two per 256-byte bank line: the swizzle puts
// their chunks on 16 different bank groups, without padding.
// Tiles of the cached prefix are also copied by DMA, each lane addressing its
// chunk in the paged cache or ring; the prologue has already copied the cached
// keys of the chunk's first tile into the workspace, so no tile mixes the two.
//
// Softmax runs in base 2 (Q' carries log2 e / sqrt d and, on global layers,
// a(t+1)). Each query keeps a reference m (its running max, moved only when
// the max grows by more than 8; exact, since the final normalisation uses the
// same reference). The S MFMA chain starts from -m instead of 0, so the scores
// arrive already shifted and feed exp2 directly; the row sum adds the bf16 P
// values that the PV product uses, two at a time (v_dot2c_f32_bf16 against
// ones). Local layers visit only the key tiles that intersect the window.
#include <type_traits>

#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

constexpr int QW = 32;                   // queries per wave (one 32-wide MFMA N-block)
constexpr int NB = QW / 32;
constexpr int BN = 64;                   // keys per tile
constexpr int K_TILE = BN * D;           // bf16 elements
constexpr int V_TILE = D * BN;
// Tiles are staged in LDS TPS at a time (one barrier per stage); two stages
// are resident, so stage s+1 streams in while stage s is computed. Global
// layers run one 8-wave block per CU and stage two tiles (128 KiB of LDS);
// local layers run two 4-wave blocks per CU and stage one (64 KiB each).
template <int KIND>
constexpr int tiles_per_stage() { return KIND == 1 ? 2 : 1; }

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
constexpr float kRescaleThreshold = 8.0f;

// Key held by LDS row m of a K tile (bits 2 and 3 swapped; an involution).
__device__ __forceinline__ int krow_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
// LDS tile layout. Every LDS row is 128 bytes (eight 16-byte chunks) and
// chunk c of row r sits at position c ^ ((r >> 1) & 7): the 16 lanes that one
// LDS cycle serves read rows r .. r+15 (two rows per 256-byte bank line), so
// their chunks land on 16 distinct bank groups. K is stored as two halves of
// 64 coordinates, [half][64 rows][64]; V^T as [128 rows][64 keys].
constexpr int K_HALF = BN * 64;  // elements of one coordinate half of a K tile
__device__ __forceinline__ int swz(int r, int c) { return (c ^ ((r >> 1) & 7)) << 3; }
// Element offsets of 16-byte chunk c (coordinates 8c .. 8c+7) of K row m, and
// of chunk c (keys 8c .. 8c+7) of V^T row d.
__device__ __forceinline__ int k_off(int m, int c) { return (c >> 3) * K_HALF + m * 64 + swz(m, c & 7); }
__device__ __forceinline__ int v_off(int d, int c) { return d * BN + swz(d, c); }

// Combine a value held by lanes l and l^32 (the two key halves of a query)
// with v_permlane32_swap, without an LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Where the keys of one (sequence, KV head) live: keys from start & ~63 on
// in the workspace, earlier ones in the cache. All pointers are wave-uniform;
// per-lane offsets from them fit in 32 bits (the host keeps P * D below
// 2^31), except the page term of the paged cache.
struct KeySource {
  const uint16_t* kw;     // workspace K rows of head g: row s + ws_off
  const uint16_t* vw;     // workspace V^T of head g: 64-key tiles [(s + ws_off) / 64][d][64]
  const uint16_t* ck;     // cache K: global page p at ck + p * page_stride; local ring rows
  const uint16_t* cv;     // cache V^T: global as ck; local ring [d][slot]
  const int32_t* bt_row;  // block-table row of the cache sequence (global)
  size_t page_stride;     // elements per page of the paged cache (all KV heads)
  int ws_off;             // workspace index = s + ws_off
  int P, kind, window;
};

// ---------------------------------------------------------------- DMA path
// One 16-byte-per-lane global -> LDS DMA (global_load_lds_dwordx4): lane l's
// 16 bytes land at dst + 16 l (dst must be wave-uniform). Kept a plain
// function: the kernel templates reach it from lambdas, and clang's host pass
// drops the stub of a second kernel instantiation when a function template on
// that path names the target builtin itself.
__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// Element offsets (relative to the tile's first key in the workspace) of the
// chunks this lane moves with each of its DMA instructions, and the LDS
// offset of each instruction's 1 KiB.
template <int NW>
struct DmaPlan {
  static constexpr int N = 16 / NW;  // 1 KiB instructions per wave per tile, for K and for V
  uint32_t k_src[N];
  uint32_t v_src[N];
  int k_lds[N];
  int v_lds[N];
  // DMA of the workspace tile whose first key is key0 (K rows kw, V^T tiles vw).
  __device__ __forceinline__ void copy(const uint16_t* kw, const uint16_t* vw, int ws_off, int key0, uint16_t* sK,
                                       uint16_t* sV) const {
    const uint16_t* kb = kw + (uint32_t)((key0 + ws_off) * D);
    const uint16_t* vb = vw + (uint32_t)((key0 + ws_off) * D);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      lds_dma16(kb + k_src[i], sK + k_lds[i]);
      lds_dma16(vb + v_src[i], sV + v_lds[i]);
    }
  }
};

template <int NW>
__device__ __forceinline__ DmaPlan<NW> make_dma_plan(int w, int lane) {
  DmaPlan<NW> pl;
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;  // K half kI / 8, rows 8(kI % 8) .. +7
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    pl.k_src[i] = (uint32_t)(krow_key(m) * D + 64 * (kI >> 3) + 8 * c);
    pl.k_lds[i] = kI * 512;
    const int vI = w * DmaPlan<NW>::N + i;  // V^T rows 8vI .. 8vI+7
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    pl.v_src[i] = (uint32_t)(d * BN + 8 * cv);
    pl.v_lds[i] = vI * 512;
  }
  return pl;
}


// Address of cached K row s and of cached V^T element (d, s) (s < start).
__device__ __forceinline__ const uint16_t* k_row_src(const KeySource& ks, int s) {
  if (ks.kind == 1) return ks.ck + ks.bt_row[s >> 4] * ks.page_stride + (uint32_t)((s & 15) * D);
  return ks.ck + (uint32_t)((s % ks.window) * D);
}
__device__ __forceinline__ const uint16_t* v_elem_src(const KeySource& ks, int d, int s) {
  if (ks.kind == 1) return ks.cv + ks.bt_row[s >> 4] * ks.page_stride + (uint32_t)(d * 16 + (s & 15));
  return ks.cv + (uint32_t)(d * ks.window + s % ks.window);
}

// DMA of a tile of the cached prefix (all keys below start & ~63): every lane
// computes the address of its 16-byte chunk from the key's page or ring slot.
// Requires a valid cache row.
template <int NW>
__device__ __forceinline__ void dma_tile_prefix(const KeySource& ks, int w, int lane, int key0, uint16_t* sK,
                                                uint16_t* sV) {
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    lds_dma16(k_row_src(ks, key0 + krow_key(m)) + 64 * (kI >> 3) + 8 * c, sK + kI * 512);

    const int vI = w * DmaPlan<NW>::N + i;
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    lds_dma16(v_elem_src(ks, d, key0 + 8 * cv), sV + vI * 512);
  }
}

// Prefix tile from an FP8 E4M3 cache: the DMA engine cannot convert, so each
// thread loads 16 codes of a K row (or of a V^T row), dequantises them to bf16
// (decode(code) * scale, one rounding) and stores the two 16-byte chunks at
// their swizzled LDS positions. k8/v8 are the byte bases of the (sequence,
// KV head) in the cache, at the element offsets the bf16 layout uses.
struct Fp8Prefix {
  const uint8_t* k8;
  const uint8_t* v8;
  const int32_t* bt_row;
  size_t page_stride;  // bytes per page of the paged cache (all KV heads)
  int kind, window;
  float k_scale, v_scale;
};

__device__ __forceinline__ u32x4 fp8x8_dequant_bf16(uint32_t w0, uint32_t w1, float scale) {
  float a[4], b[4];
  fp8x4_to_f32(w0, a);
  fp8x4_to_f32(w1, b);
  return u32x4{pack_bf16x2(a[0] * scale, a[1] * scale), pack_bf16x2(a[2] * scale, a[3] * scale),
               pack_bf16x2(b[0] * scale, b[1] * scale), pack_bf16x2(b[2] * scale, b[3] * scale)};
}

template <int NW>
__device__ __forceinline__ void fetch_prefix_fp8(const Fp8Prefix& fp, int tid, int key0, uint16_t* sK, uint16_t* sV) {
  constexpr int R = 8 / NW;  // 16-byte loads per thread, for K and for V
  u32x4 kc[R], vc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int id = tid + 64 * NW * r;  // 0..511
    {
      const int m = id >> 3, c2 = id & 7;  // LDS row m, codes 16c2 .. 16c2+15
      const int s = key0 + krow_key(m);
      const uint8_t* src = fp.kind == 1 ? fp.k8 + fp.bt_row[s >> 4] * fp.page_stride + (size_t)((s & 15) * D)
                                        : fp.k8 + (size_t)((s % fp.window) * D);
      kc[r] = *reinterpret_cast<const u32x4*>(src + 16 * c2);
    }
    {
      const int d = id >> 2, c2 = id & 3;  // V^T row d, keys 16c2 .. 16c2+15 (one page / no ring wrap)
      const int s = key0 + 16 * c2;
      const uint8_t* src = fp.kind == 1 ? fp.v8 + fp.bt_row[s >> 4] * fp.page_stride + (size_t)(d * 16)
                                        : fp.v8 + (size_t)(d * fp.window + s % fp.window);
      vc[r] = *reinterpret_cast<const u32x4*>(src);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int id = tid + 64 * NW * r;
    const int m = id >> 3, ck = id & 7;
    *reinterpret_cast<u32x4*>(sK + k_off(m, 2 * ck)) = fp8x8_dequant_bf16(kc[r][0], kc[r][1], fp.k_scale);
    *reinterpret_cast<u32x4*>(sK + k_off(m, 2 * ck + 1)) = fp8x8_dequant_bf16(kc[r][2], kc[r][3], fp.k_scale);
    const int d = id >> 2, cv = id & 3;
    *reinterpret_cast<u32x4*>(sV + v_off(d, 2 * cv)) = fp8x8_dequant_bf16(vc[r][0], vc[r][1], fp.v_scale);
    *reinterpret_cast<u32x4*>(sV + v_off(d, 2 * cv + 1)) = fp8x8_dequant_bf16(vc[r][2], vc[r][3], fp.v_scale);
  }
}

// ---------------------------------------------------------------- kernel
template <int KIND, int NWAVES, int KV_FP8>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attn_kernel(PrefillParams p) {
  constexpr int BM = NWAVES * QW;  // queries per block
  static_assert(16 % NWAVES == 0, "tile split");
  constexpr int TPS = tiles_per_stage<KIND>();
  constexpr int SLOTS = 2 * TPS;  // tile slots: two stages
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SLOTS * (K_TILE + V_TILE)];

  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;  // consecutive blocks -> consecutive XCDs -> one KV head per XCD
  b /= p.G;
  const int hh = b % hpg;
  b /= hpg;
  const int seq = b % p.n_seqs;
  const int qt = p.n_qtiles - 1 - b / p.n_seqs;  // heaviest query tiles first
  const int h = g * hpg + hh;

  const int cu0 = p.cu[seq];
  const int len = p.cu[seq + 1] - cu0;
  if (qt * BM >= len) return;
  const int start = p.start_pos[seq];
  const int cseq = p.seq_idx[seq];
  const int W = p.window;
  constexpr bool local = (KIND == 0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (DMA bases go to M0)
  const int n = lane & 31;
  const int half = lane >> 5;

  const int q0 = start + qt * BM;                   // first query position of the block
  const int qlast = min(q0 + BM, start + len) - 1;  // last valid query position
  const int wq_lo = q0 + QW * w;
  const int wq_hi = min(wq_lo + QW - 1, qlast);
  const bool wave_active = wq_lo <= qlast;

  KeySource ks;
  ks.kw = p.kw + (size_t)g * p.P * D;
  ks.vw = p.vw + (size_t)g * D * p.P;
  if (KIND == 1) {
    ks.ck = p.ck + (size_t)g * 16 * D;
    ks.cv = p.cv + (size_t)g * D * 16;
    ks.page_stride = (size_t)p.G * 16 * D;
  } else {
    const size_t ring = (size_t)cseq * p.G + g;  // (cache sequence, head) ring
    ks.ck = p.ck + ring * W * D;
    ks.cv = p.cv + ring * D * W;
    ks.page_stride = 0;
  }
  ks.bt_row = KIND == 1 ? p.bt + (size_t)cseq * p.max_pages : nullptr;
  // The cached prefix must fit the cache sequence's block-table row (global);
  // an out-of-range row leaves the prefix out (the prologue zeroed its part
  // of the first tile).
  const bool cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (KIND == 0 || ((start + 15) >> 4) <= p.max_pages);
  ks.ws_off = ws_region_base(cu0, seq) - (start & ~63);
  ks.P = p.P;
  ks.kind = KIND;
  ks.window = W;
  const DmaPlan<NWAVES> plan = make_dma_plan<NWAVES>(w, lane);
  Fp8Prefix fp8;
  if constexpr (KV_FP8) {
    const size_t head = KIND == 1 ? (size_t)g * 16 * D : ((size_t)cseq * p.G + g) * W * D;
    fp8.k8 = reinterpret_cast<const uint8_t*>(p.ck) + head;
    fp8.v8 = reinterpret_cast<const uint8_t*>(p.cv) + head;
    fp8.bt_row = ks.bt_row;
    fp8.page_stride = (size_t)p.G * 16 * D;
    fp8.kind = KIND;
    fp8.window = W;
    fp8.k_scale = p.k_scale;
    fp8.v_scale = p.v_scale;
  }

  // Q' fragments (B operand of S^T = K Q'^T): lane holds query n of N-block nb,
  // coordinates 16kk + 8*half + 0..7.
  u32x4 qf[NB][8];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = wq_lo + 32 * nb + n;
    const bool valid = t <= qlast;
    const size_t tok = (size_t)(cu0 + (t - start));
    const uint16_t* qrow = p.qp + (tok * p.H + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[nb][kk] = valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  const int j_ws = start >> 6;  // first tile in the workspace; earlier tiles are wholly cached
  const int kmin = local ? max(0, q0 - (W - 1)) : 0;
  const int j_lo = cache_ok ? kmin >> 6 : max(kmin >> 6, j_ws);
  const int j_hi = qlast >> 6;

  f32x16 o[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nb][db][i] = 0.f;
  // m_run: reference of the query (kNegInf until a key is visible); sref holds
  // -m_run (0 while m_run is kNegInf) splatted, the accumulator input of S.
  float m_run[NB], l_run[NB];
  f32x16 sref[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sref[nb][i] = 0.f;
  }
  // Loop-invariant LDS element offsets of this lane's operand chunks: K row n,
  // chunk 2q + half for q = 0..3 (chunks 8..15 are the second coordinate half,
  // K_HALF further; M-block 1 adds 32 rows); V^T row n, chunk 2kb + half (row
  // block db adds 32 rows).
  int koff[4], voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    koff[q] = k_off(n, 2 * q + half);
    voff[q] = v_off(n, 2 * q + half);
  }

  // ---- pieces of one 64-key tile of attention for this wave's queries ----
  // Tile jt uses LDS slot (jt - j_lo) % SLOTS; the loop is unrolled by SLOTS
  // so that the slot offset is a compile-time constant of every LDS read.
  auto buf = [&](auto B) -> uint16_t* { return smem + decltype(B)::value * (K_TILE + V_TILE); };
  auto active = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return wave_active && k0 <= wq_hi && !(local && k0 + BN - 1 < wq_lo - (W - 1));
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return (k0 + BN - 1 > wq_lo) || (local && k0 < wq_hi - (W - 1));
  };
  // S^T - m = K Q'^T - m: LDS rows 32mb + (lane&31) on M, queries 32nb + n on
  // N; the chain starts from sref = -m.
  auto qk = [&](auto B, f32x16 (&s)[NB][2]) {
    const uint16_t* sK = buf(B);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sK + koff[kk & 3] + K_HALF * (kk >> 2) + 32 * 64 * mb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[nb][kk]),
                                                             kk == 0 ? sref[nb] : s[nb][mb], 0, 0, 0);
      }
    }
  };
  // Element i of block mb holds key 64j + 32mb + 16(i>>3) + 8*half + (i&7).
  auto apply_mask = [&](int j, f32x16 (&s)[NB][2]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = wq_lo + 32 * nb + n;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sk = j * BN + 32 * mb + 16 * (i >> 3) + 8 * half + (i & 7);
          if (!visible(KIND, W, t, sk)) s[nb][mb][i] = kNegInf;
        }
    }
  };
  // Shift of the reference this tile needs, per query: the tile max of the
  // shifted scores when it exceeds the threshold (or is the first finite
  // score of the query), else 0.
  auto row_shift = [&](const f32x16 (&s)[NB][2], float (&delta)[NB], bool (&need)[NB]) {
    bool grow = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mt = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[nb][mb][i]);
      mt = max_halves(mt);
      need[nb] = (m_run[nb] == kNegInf) ? (mt != kNegInf) : (mt > kRescaleThreshold);
      delta[nb] = need[nb] ? mt : 0.f;
      grow = grow || need[nb];
    }
    return grow;
  };
  // Move the reference up by delta: rescale O and l by 2^-delta (nothing to
  // rescale while no key was visible) and shift this tile's scores.
  auto rescale = [&](const float (&delta)[NB], const bool (&need)[NB], f32x16 (&s)[NB][2]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool first = m_run[nb] == kNegInf;
      const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta[nb]);
      if (need[nb]) m_run[nb] = (first ? 0.f : m_run[nb]) + delta[nb];
      const float r = m_run[nb] == kNegInf ? 0.f : -m_run[nb];
#pragma unroll
      for (int i = 0; i < 16; ++i) sref[nb][i] = r;
      l_run[nb] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[nb][db][i] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][mb][i] -= delta[nb];
    }
  };
  // P^T operand of key block kb: elements 8(kb&1)..+7 of S block kb>>1, i.e.
  // keys 16kb + 8*half + 0..7 in order.
  auto softmax = [&](const f32x16 (&s)[NB][2], u32x4 (&pf)[NB][4]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float e[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) e[jj] = __builtin_amdgcn_exp2f(s[nb][kb >> 1][8 * (kb & 1) + jj]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pf[nb][kb][c] = pack_bf16x2(e[2 * c], e[2 * c + 1]);
          l_run[nb] = sum_bf16x2(pf[nb][kb][c], l_run[nb]);
        }
      }
    }
  };
  // O^T += V^T P^T: A operand = coordinates 32db + n, keys 16kb + 8*half + 0..7.
  auto pv = [&](auto B, const u32x4 (&pf)[NB][4]) {
    const uint16_t* sV = buf(B) + K_TILE;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sV + voff[kb] + 32 * BN * db);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pf[nb][kb]), o[nb][db], 0, 0, 0);
      }
    }
  };
  // Fetch tile j into its slot by DMA, from the workspace or the cache.
  auto fetch = [&](int j, auto B) __attribute__((always_inline)) {
    uint16_t* sK = buf(B);
    if (j >= j_ws)
      plan.copy(ks.kw, ks.vw, ks.ws_off, j * BN, sK, sK + K_TILE);
    else if constexpr (KV_FP8)
      fetch_prefix_fp8<NWAVES>(fp8, tid, j * BN, sK, sK + K_TILE);
    else
      dma_tile_prefix<NWAVES>(ks, w, lane, j * BN, sK, sK + K_TILE);
  };

  // One 64-key tile of attention for this wave's queries.
  auto compute_tile = [&](int j, auto B) __attribute__((always_inline)) {
    if (!active(j)) return;
    f32x16 st[NB][2];
    qk(B, st);
    if (needs_mask(j)) apply_mask(j, st);
    float delta[NB];
    bool need[NB];
    if (__any(row_shift(st, delta, need))) rescale(delta, need, st);
    u32x4 pf[NB][4];
    softmax(st, pf);
    pv(B, pf);
  };
  // Stage of tiles j0 .. j0+TPS-1 in slots S0 .. S0+TPS-1: before tile j0+u
  // is computed, tile j0+TPS+u is sent to the other stage's slot (freed by the
  // previous barrier); the barrier then publishes the next stage.
  auto stage = [&](int j0, auto S0) __attribute__((always_inline)) {
    static_for<TPS>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      constexpr int s0 = decltype(S0)::value;
      if (j0 + TPS + u <= j_hi) fetch(j0 + TPS + u, std::integral_constant<int, (s0 + TPS + u) % SLOTS>{});
      if (j0 + u <= j_hi) compute_tile(j0 + u, std::integral_constant<int, s0 + u>{});
    });
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- tile loop ----
  static_for<TPS>([&](auto U) __attribute__((always_inline)) {
    if (j_lo + decltype(U)::value <= j_hi) fetch(j_lo + decltype(U)::value, U);
  });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int jt = j_lo; jt <= j_hi; jt += SLOTS) {
    stage(jt, std::integral_constant<int, 0>{});
    if (jt + TPS > j_hi) break;
    stage(jt + TPS, std::integral_constant<int, TPS>{});
  }

  // Epilogue: normalise, gate, write bf16. Lane holds query n of each N-block
  // and coordinates d = 32db + 8a + 4*half + 0..3.
  const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = wq_lo + 32 * nb + n;
    const float l_tot = sum_halves(l_run[nb]);
    if (t > qlast) continue;
    const float inv = l_tot > 0.f ? __frcp_rn(l_tot) : 0.f;
    const size_t tok = (size_t)(cu0 + (t - start));
    const uint16_t* grow_ = p.gate + (tok * p.H + h) * D;
    uint16_t* orow = p.out + (tok * p.H + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * db + 8 * a + 4 * half;
        const u32x2 gv = *reinterpret_cast<const u32x2*>(grow_ + d0);
        const float gz[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = __frcp_rn(1.f + __expf(-(gz[e] + bias)));
          y[e] = o[nb][db][4 * a + e] * inv * sg;
        }
        *reinterpret_cast<u32x2*>(orow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
    }
  }
}

// ---------------------------------------------------------------- verify
// Attention of a short chunk (the verify step of speculative decoding: a few
// new tokens per sequence over a long cached history). The chunk's rows are
// (token, query head) pairs of one KV head, 32 per wavefront (token r / hpg,
// head r % hpg), so every K/V tile feeds all of them; a block takes one key
// split of one (sequence, KV head) and writes its partial (reference max, sum,
// accumulator) per row; verify_combine_kernel merges the splits and gates.
// Keys come from the cache below the chunk start and from the workspace
// (written by the prologue) for the chunk itself, as in prefill. Each lane's
// row has its own query position, so masks are evaluated per lane.
//
// The split's page ids are staged in LDS first, so the DMA address path of a
// cached tile reads LDS instead of waiting on a block-table load.
constexpr int kVerifyMaxPages = 4 * kVerifyMaxSplitTiles;  // 4 pages per 64-key tile

// Cached K row s / V^T element (d, s) with the page id taken from the
// LDS-staged list (pages[i] = block-table entry page0 + i) on paged caches.
__device__ __forceinline__ const uint16_t* k_row_cached(const KeySource& ks, const int* pages, int page0, int s) {
  if (ks.kind == 1) return ks.ck + pages[(s >> 4) - page0] * ks.page_stride + (uint32_t)((s & 15) * D);
  return ks.ck + (uint32_t)((s % ks.window) * D);
}
__device__ __forceinline__ const uint16_t* v_elem_cached(const KeySource& ks, const int* pages, int page0, int d,
                                                         int s) {
  if (ks.kind == 1) return ks.cv + pages[(s >> 4) - page0] * ks.page_stride + (uint32_t)(d * 16 + (s & 15));
  return ks.cv + (uint32_t)(d * ks.window + s % ks.window);
}

// DMA of a cached-prefix tile; the same chunks and LDS positions as
// dma_tile_prefix (16 / NW instructions each for K and V per wave).
template <int NW>
__device__ __forceinline__ void dma_tile_cached(const KeySource& ks, const int* pages, int page0, int w, int lane,
                                                int key0, uint16_t* sK, uint16_t* sV) {
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    lds_dma16(k_row_cached(ks, pages, page0, key0 + krow_key(m)) + 64 * (kI >> 3) + 8 * c, sK + kI * 512);
    const int vI = w * DmaPlan<NW>::N + i;
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    lds_dma16(v_elem_cached(ks, pages, page0, d, key0 + 8 * cv), sV + vI * 512);
  }
}

// FP8 prefix tile in two phases: the codes into registers, then dequantised
// into LDS (the chunks of fetch_prefix_fp8).

// s_waitcnt immediate for vmcnt <= n, lgkmcnt 0, expcnt untouched (gfx9
// fields: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
constexpr int vm_lgkm_wait(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

template <int NW>
struct Fp8Regs {
  static constexpr int R = 8 / NW;
  u32x4 k[R], v[R];
};
template <int NW>
__device__ __forceinline__ void load_prefix_fp8(const Fp8Prefix& fp, const int* pages, int page0, int tid, int key0,
                                                Fp8Regs<NW>& r) {
#pragma unroll
  for (int i = 0; i < Fp8Regs<NW>::R; ++i) {
    const int id = tid + 64 * NW * i;
    {
      const int m = id >> 3, c2 = id & 7;
      const int s = key0 + krow_key(m);
      const uint8_t* src = fp.kind == 1 ? fp.k8 + pages[(s >> 4) - page0] * fp.page_stride + (size_t)((s & 15) * D)
                                        : fp.k8 + (size_t)((s % fp.window) * D);
      r.k[i] = *reinterpret_cast<const u32x4*>(src + 16 * c2);
    }
    {
      const int d = id >> 2, c2 = id & 3;
      const int s = key0 + 16 * c2;
      const uint8_t* src = fp.kind == 1 ? fp.v8 + pages[(s >> 4) - page0] * fp.page_stride + (size_t)(d * 16)
                                        : fp.v8 + (size_t)(d * fp.window + s % fp.window);
      r.v[i] = *reinterpret_cast<const u32x4*>(src);
    }
  }
}
template <int NW>
__device__ __forceinline__ void store_prefix_fp8(const Fp8Prefix& fp, int tid, const Fp8Regs<NW>& r, uint16_t* sK,
                                                 uint16_t* sV) {
#pragma unroll
  for (int i = 0; i < Fp8Regs<NW>::R; ++i) {
    const int id = tid + 64 * NW * i;
    const int m = id >> 3, ck = id & 7;
    *reinterpret_cast<u32x4*>(sK + k_off(m, 2 * ck)) = fp8x8_dequant_bf16(r.k[i][0], r.k[i][1], fp.k_scale);
    *reinterpret_cast<u32x4*>(sK + k_off(m, 2 * ck + 1)) = fp8x8_dequant_bf16(r.k[i][2], r.k[i][3], fp.k_scale);
    const int d = id >> 2, cv = id & 3;
    *reinterpret_cast<u32x4*>(sV + v_off(d, 2 * cv)) = fp8x8_dequant_bf16(r.v[i][0], r.v[i][1], fp.v_scale);
    *reinterpret_cast<u32x4*>(sV + v_off(d, 2 * cv + 1)) = fp8x8_dequant_bf16(r.v[i][2], r.v[i][3], fp.v_scale);
  }
}

template <int KIND, int KV_FP8>
__global__ void __launch_bounds__(64 * kVerifyWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
verify_attn_kernel(PrefillParams p) {
  constexpr int NWAVES = kVerifyWaves;
  constexpr bool local = (KIND == 0);
  // One LDS object: with a second __shared__ variable the compiler tags LDS
  // accesses with alias scopes and then makes every LDS read wait for all DMA
  // into the same array (vmcnt(0) before each tile's MFMAs), which serialises
  // the fetch of tile jt + 1 with the compute of tile jt.
  constexpr int kTiles = 2 * (K_TILE + V_TILE);
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kTiles + (KIND == 1 ? 2 * kVerifyMaxPages : 0)];
  int* const s_pages = reinterpret_cast<int*>(smem + kTiles);

  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;  // consecutive blocks -> consecutive XCDs
  b /= p.G;
  const int sp = b % p.n_splits;
  const int seq = b / p.n_splits;
  const int cu0 = p.cu[seq];
  const int len = p.cu[seq + 1] - cu0;
  if (len <= 0) return;
  const int start = p.start_pos[seq];
  const int cseq = p.seq_idx[seq];
  const int W = p.window;
  const int t_last = start + len - 1;

  KeySource ks;
  ks.kw = p.kw + (size_t)g * p.P * D;
  ks.vw = p.vw + (size_t)g * D * p.P;
  if (KIND == 1) {
    ks.ck = p.ck + (size_t)g * 16 * D;
    ks.cv = p.cv + (size_t)g * D * 16;
    ks.page_stride = (size_t)p.G * 16 * D;
  } else {
    const size_t ring = (size_t)cseq * p.G + g;
    ks.ck = p.ck + ring * W * D;
    ks.cv = p.cv + ring * D * W;
    ks.page_stride = 0;
  }
  ks.bt_row = KIND == 1 ? p.bt + (size_t)cseq * p.max_pages : nullptr;
  const bool cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (KIND == 0 || ((start + 15) >> 4) <= p.max_pages);
  ks.ws_off = ws_region_base(cu0, seq) - (start & ~63);
  ks.P = p.P;
  ks.kind = KIND;
  ks.window = W;

  // Key tiles of this split.
  const int j_ws = start >> 6;
  const int kmin = local ? max(0, start - (W - 1)) : 0;
  const int j_first = cache_ok ? kmin >> 6 : max(kmin >> 6, j_ws);
  const int j_last = t_last >> 6;
  const int j_lo = j_first + sp * p.split_tiles;
  if (j_lo > j_last) return;  // past this sequence's keys; the combine skips the split
  const int j_hi = min(j_last, j_lo + p.split_tiles - 1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int half = lane >> 5;
  const DmaPlan<NWAVES> plan = make_dma_plan<NWAVES>(w, lane);
  Fp8Prefix fp8;
  if constexpr (KV_FP8) {
    const size_t head = KIND == 1 ? (size_t)g * 16 * D : ((size_t)cseq * p.G + g) * W * D;
    fp8.k8 = reinterpret_cast<const uint8_t*>(p.ck) + head;
    fp8.v8 = reinterpret_cast<const uint8_t*>(p.cv) + head;
    fp8.bt_row = ks.bt_row;
    fp8.page_stride = (size_t)p.G * 16 * D;
    fp8.kind = KIND;
    fp8.window = W;
    fp8.k_scale = p.k_scale;
    fp8.v_scale = p.v_scale;
  }

  // Page ids of the split's cached tiles (tiles j_lo .. min(j_hi, j_ws - 1);
  // pages below (start & ~63) / 16, inside the block-table row).
  const int page0 = 4 * j_lo;
  if (KIND == 1 && cache_ok) {
    const int n_pg = 4 * (min(j_hi, j_ws - 1) - j_lo + 1);
    for (int i = tid; i < n_pg; i += 64 * NWAVES) s_pages[i] = ks.bt_row[page0 + i];
  }

  // This lane's row and the wave's range of query positions.
  const int n_rows = len * hpg;
  const int r = QW * w + n;
  const bool row_valid = r < n_rows;
  const int tok_j = row_valid ? r / hpg : 0;
  const int h = g * hpg + (row_valid ? r - tok_j * hpg : 0);
  const int t_row = start + tok_j;
  const int r_lo = QW * w;
  const bool wave_active = r_lo < n_rows;
  const int wq_lo = start + r_lo / hpg;
  const int wq_hi = start + (min(r_lo + QW, n_rows) - 1) / hpg;

  u32x4 qf[8];
  {
    const uint16_t* qrow = p.qp + ((size_t)(cu0 + tok_j) * p.H + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = row_valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  f32x16 sref;
#pragma unroll
  for (int i = 0; i < 16; ++i) sref[i] = 0.f;
  int koff[4], voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    koff[q] = k_off(n, 2 * q + half);
    voff[q] = v_off(n, 2 * q + half);
  }

  auto buf = [&](auto B) -> uint16_t* { return smem + decltype(B)::value * (K_TILE + V_TILE); };
  auto active = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return wave_active && k0 <= wq_hi && !(local && k0 + BN - 1 < wq_lo - (W - 1));
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return (k0 + BN - 1 > wq_lo) || (local && k0 < wq_hi - (W - 1));
  };
  auto tile = [&](int j, auto B) __attribute__((always_inline)) {
    if (!active(j)) return;
    const uint16_t* sK = buf(B);
    f32x16 s[2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sK + koff[kk & 3] + K_HALF * (kk >> 2) + 32 * 64 * mb);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[kk]), kk == 0 ? sref : s[mb], 0,
                                                        0, 0);
      }
    if (needs_mask(j)) {  // element i of block mb holds key 64j + 32mb + 16(i>>3) + 8*half + (i&7)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sk = j * BN + 32 * mb + 16 * (i >> 3) + 8 * half + (i & 7);
          if (!visible(KIND, W, t_row, sk)) s[mb][i] = kNegInf;
        }
    }
    // Reference shift (the row max of the shifted scores when it exceeds the
    // threshold, or the first finite score of the row).
    float mt = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[mb][i]);
    mt = max_halves(mt);
    const bool need = (m_run == kNegInf) ? (mt != kNegInf) : (mt > kRescaleThreshold);
    if (__any(need)) {
      const float delta = need ? mt : 0.f;
      const bool first = m_run == kNegInf;
      const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta);
      if (need) m_run = (first ? 0.f : m_run) + delta;
      const float rr = m_run == kNegInf ? 0.f : -m_run;
#pragma unroll
      for (int i = 0; i < 16; ++i) sref[i] = rr;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[mb][i] -= delta;
    }
    u32x4 pf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float e[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) e[jj] = __builtin_amdgcn_exp2f(s[kb >> 1][8 * (kb & 1) + jj]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pf[kb][c] = pack_bf16x2(e[2 * c], e[2 * c + 1]);
        l_run = sum_bf16x2(pf[kb][c], l_run);
      }
    }
    const uint16_t* sV = buf(B) + K_TILE;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sV + voff[kb] + 32 * BN * db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pf[kb]), o[db], 0, 0, 0);
      }
  };
  // DMA of tile j (workspace or bf16 cache) into buffer B.
  auto dma = [&](int j, auto B) __attribute__((always_inline)) {
    uint16_t* sK = buf(B);
    if (j >= j_ws)
      plan.copy(ks.kw, ks.vw, ks.ws_off, j * BN, sK, sK + K_TILE);
    else
      dma_tile_cached<NWAVES>(ks, s_pages, page0, w, lane, j * BN, sK, sK + K_TILE);
  };
  __builtin_amdgcn_s_waitcnt(0);  // Q' and page ids in
  __syncthreads();
  // Two LDS buffers: tile jt + 1 arrives while tile jt is computed. DMA tiles
  // are sent one step ahead. FP8 prefix tiles go through registers two steps
  // ahead (regs[b] for the tile that will use buffer b) and are converted
  // into LDS after the MFMAs of the step before their own; such a step ends
  // waiting for its DMA and LDS stores only, leaving the newest code loads in
  // flight. The barrier is a bare s_barrier: the workgroup fence of
  // __syncthreads would wait for every load still in flight. The empty asm
  // statements keep the compiler from moving LDS accesses across it.
  [[maybe_unused]] Fp8Regs<NWAVES> regs[2];
  auto reg_tile = [&](int j) { return KV_FP8 && j <= j_hi && j < j_ws; };
  auto step_end = [&](bool codes_in_flight) __attribute__((always_inline)) {
    if (codes_in_flight)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * Fp8Regs<NWAVES>::R));
    else
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto step = [&](int jt, auto B) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    const int jn = jt + 1;
    if (jn <= j_hi && !reg_tile(jn)) dma(jn, std::integral_constant<int, 1 - b>{});
    const bool load_nn = reg_tile(jt + 2);
    if constexpr (KV_FP8) {
      asm volatile("" ::: "memory");  // the DMA is issued before the code loads below
      if (load_nn) load_prefix_fp8<NWAVES>(fp8, s_pages, page0, tid, (jt + 2) * BN, regs[b]);
    }
    tile(jt, B);
    if constexpr (KV_FP8) {
      if (reg_tile(jn))
        store_prefix_fp8<NWAVES>(fp8, tid, regs[1 - b], buf(std::integral_constant<int, 1 - b>{}),
                                 buf(std::integral_constant<int, 1 - b>{}) + K_TILE);
    }
    step_end(load_nn);
  };
  if (reg_tile(j_lo)) {
    if constexpr (KV_FP8) {
      load_prefix_fp8<NWAVES>(fp8, s_pages, page0, tid, j_lo * BN, regs[0]);
      store_prefix_fp8<NWAVES>(fp8, tid, regs[0], smem, smem + K_TILE);
    }
  } else {
    dma(j_lo, std::integral_constant<int, 0>{});
  }
  if constexpr (KV_FP8) {
    asm volatile("" ::: "memory");
    if (reg_tile(j_lo + 1)) load_prefix_fp8<NWAVES>(fp8, s_pages, page0, tid, (j_lo + 1) * BN, regs[1]);
  }
  step_end(reg_tile(j_lo + 1));
  for (int jt = j_lo; jt <= j_hi; jt += 2) {
    step(jt, std::integral_constant<int, 0>{});
    if (jt + 1 > j_hi) break;
    step(jt + 1, std::integral_constant<int, 1>{});
  }

  // Partials of this split: lane holds row n's sum half and coordinates
  // d = 32db + 8a + 4*half + 0..3.
  const float l_tot = sum_halves(l_run);
  if (!row_valid) return;
  const size_t row = ((size_t)(cu0 + tok_j) * p.H + h) * p.n_splits + sp;
  if (half == 0) {
    p.part_ml[2 * row] = m_run;
    p.part_ml[2 * row + 1] = l_tot;
  }
  float* acc = p.part_acc + row * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(acc + 32 * db + 8 * a + 4 * half) =
          f32x4{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
}

// Merge the key splits of one (token, query head) of a verify chunk by
// log-sum-exp, then apply the gate. One block of 128 threads (a coordinate each).
__global__ void __launch_bounds__(128) verify_combine_kernel(VerifyCombineParams p) {
  const int tok = blockIdx.x / p.H;
  const int h = blockIdx.x - tok * p.H;
  const int d = threadIdx.x;
  const int seq = find_seq(p.cu, p.n_seqs, tok);
  const int start = p.start_pos[seq];
  const int len = p.cu[seq + 1] - p.cu[seq];
  const int cseq = p.seq_idx[seq];
  const bool cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (p.kind == 0 || ((start + 15) >> 4) <= p.max_pages);
  const int kmin = p.kind == 0 ? max(0, start - (p.window - 1)) : 0;
  const int j_first = cache_ok ? kmin >> 6 : max(kmin >> 6, start >> 6);
  const int j_last = (start + len - 1) >> 6;
  const int ns = min(p.n_splits, (j_last - j_first + p.split_tiles) / p.split_tiles);
  const size_t row0 = ((size_t)tok * p.H + h) * p.n_splits;
  float M = kNegInf;
#pragma unroll 8
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, p.part_ml[2 * (row0 + sp)]);
  float L = 0.f, A = 0.f;
  if (M != kNegInf) {
#pragma unroll 8
    for (int sp = 0; sp < ns; ++sp) {
      const float m = p.part_ml[2 * (row0 + sp)];
      if (m == kNegInf) continue;
      const float sc = __builtin_amdgcn_exp2f(m - M);
      L += sc * p.part_ml[2 * (row0 + sp) + 1];
      A += sc * p.part_acc[(row0 + sp) * D + d];
    }
  }
  const float o = L > 0.f ? A / L : 0.f;
  const size_t idx = ((size_t)tok * p.H + h) * D + d;
  const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
  const float sg = __frcp_rn(1.f + __expf(-(bf16f(p.gate[idx]) + bias)));
  bf16x2 rr;
  rr[0] = (__bf16)(o * sg);
  p.out[idx] = __builtin_bit_cast(uint16_t, rr[0]);
}

hipError_t launch_verify_attn(const PrefillParams& p, hipStream_t s) {
  if (p.split_tiles * 4 > kVerifyMaxPages) return hipErrorInvalidValue;
  const long long blocks = (long long)p.G * p.n_splits * p.n_seqs;
  const dim3 grid((unsigned)blocks), block(64 * kVerifyWaves);
  if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL((verify_attn_kernel<0, 0>), grid, block, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL((verify_attn_kernel<0, 1>), grid, block, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL((verify_attn_kernel<1, 0>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((verify_attn_kernel<1, 1>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_combine(const VerifyCombineParams& p, hipStream_t s) {
  hipLaunchKernelGGL(verify_combine_kernel, dim3((unsigned)((long long)p.n_tok * p.H)), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  const long long blocks = (long long)p.G * (p.H / p.G) * p.n_seqs * p.n_qtiles;
  const dim3 grid((unsigned)blocks), local_block(64 * kPrefillWavesLocal), global_block(64 * kPrefillWavesGlobal);
  if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 0>), grid, local_block, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 1>), grid, local_block, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL((prefill_attn_kernel<1, kPrefillWavesGlobal, 0>), grid, global_block, 0, s, p);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<1, kPrefillWavesGlobal, 1>), grid, global_block, 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
