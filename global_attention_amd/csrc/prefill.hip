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
// Tiling. A block is NWAVES wavefronts x QW queries; on global layers 8 x 48
// queries of one query head, on local layers 4 x 32: two query heads of one
// KV group, each with 64 queries (so the four waves read the same key tiles).
// KV tiles of 64 keys are double-buffered in LDS. Each wave computes
// S^T = K Q'^T with v_mfma_f32_16x16x32_bf16 (key blocks of 16 on M, three
// or two 16-query column blocks on N, so each K or V^T operand read from LDS
// feeds three or two MFMAs): a lane holds one query of each column block,
// a query's 64 keys of a tile are spread over the four 16-lane groups, and
// the row max is an in-lane max plus two lane swaps (v_permlane16_swap, then
// v_permlane32_swap). The S accumulators are packed to bf16 and fed directly
// as the B operand of O^T += V^T P^T. Under the chip's power limit the
// 16x16x32 form holds a higher clock than 32x32x16 for the same multiply-adds
// (2-3 % faster on a 32K-token global layer). The verify kernel keeps
// 32x32x16: its rows are (token, head) pairs, 32 per wave.
//
// LDS layout. Tiles that lie inside the chunk are copied from the workspace
// straight into LDS with global_load_lds_dwordx4 (no staging registers).
//   K:   two coordinate halves, each 64 rows x 128 B. LDS row m holds key
//        kappa(m), a permutation that turns the MFMA output row order into
//        the key order the PV operand needs: in the prefill kernel row
//        16b + 4g + i holds key 32(b >> 1) + 8g + 4(b & 1) + i (krow_key16),
//        in the verify kernel m with bits 2 and 3 swapped (krow_key).
//   V^T: 128 rows (coordinates) x 128 B (64 keys, natural order).
// Both XOR-swizzle their 16-byte chunks with bits 1..3 of the row. A b128
// read is served 16 lanes per LDS cycle, and the operand reads have those
// lanes on 16 consecutive rows, two per 256-byte bank line: the swizzle puts
// their chunks on 16 different bank groups, without padding.
// Tiles of the cached prefix are also copied by DMA, each lane addressing its
// chunk in the paged cache or ring; the prologue has already copied the cached
// keys of the chunk's first tile into the workspace, so no tile mixes the two.
//
// Epilogue. The gate logits of a local block's queries are copied into the
// LDS slot its last tile leaves free while that tile is computed; every gate
// value is read before the first output store.
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

constexpr int VQW = 32;                  // (token, head) rows per verify wave (one 32x32x16 N-block)
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

// Key held by LDS row m of a K tile for the 32x32x16 operand layout (bits 2
// and 3 swapped; an involution): the verify kernel.
__device__ __forceinline__ int krow_key(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
// Key held by LDS row m of a K tile for the 16x16x32 layout of the prefill
// kernel: row 16b + 4g + i (key block b = m >> 4, lane group g) holds key
// 32(b >> 1) + 8g + 4(b & 1) + i, so lane group g's four S rows of key blocks
// 2c and 2c+1 are keys 32c + 8g + 0..7 in order, the B operand of PV. The 8
// rows of one DMA instruction (8a .. 8a+7) stay inside one 16-key page.
__device__ __forceinline__ int krow_key16(int m) { return (m & 0x23) | ((m & 0x0c) << 1) | ((m & 0x10) >> 2); }
template <bool P16>
__device__ __forceinline__ int krow(int m) { return P16 ? krow_key16(m) : krow_key(m); }
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
// max(a, b) as one v_max_f32. The scores are never NaN; fmaxf would first
// quiet each operand that came out of a lane swap (which the compiler cannot
// prove canonical), an extra v_max_f32 per operand.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Combine a value over the four lane groups l, l^16, l^32, l^48 (the 16x16
// layout spreads a query's keys over them): v_permlane16_swap, then 32.
__device__ __forceinline__ float max_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_halves(max2(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float sum_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
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
// The same with the non-temporal hint (cache policy nt): for a paged cache's
// K/V that one block reads once (verify splits), not for tiles many blocks
// share or a local layer's window-sized rings.
__device__ __forceinline__ void lds_dma16_nt(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 2);
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

template <int NW, bool P16 = false>
__device__ __forceinline__ DmaPlan<NW> make_dma_plan(int w, int lane) {
  DmaPlan<NW> pl;
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;  // K half kI / 8, rows 8(kI % 8) .. +7
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    pl.k_src[i] = (uint32_t)(krow<P16>(m) * D + 64 * (kI >> 3) + 8 * c);
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
template <int NW, bool P16 = false>
__device__ __forceinline__ void dma_tile_prefix(const KeySource& ks, int w, int lane, int key0, uint16_t* sK,
                                                uint16_t* sV) {
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    lds_dma16(k_row_src(ks, key0 + krow<P16>(m)) + 64 * (kI >> 3) + 8 * c, sK + kI * 512);

    const int vI = w * DmaPlan<NW>::N + i;
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    lds_dma16(v_elem_src(ks, d, key0 + 8 * cv), sV + vI * 512);
  }
}

// DMA of a tile of a paged cache's prefix with the tile's four page ids
// given (pg holds page id (lane & 3) of the tile in every lane). A K
// instruction moves 8 rows of one page (its page id is wave-uniform); the
// lanes of a V^T instruction span the four pages, each picks its own.
template <int NW, bool P16 = false>
__device__ __forceinline__ void dma_tile_paged(const KeySource& ks, int pg, int w, int lane, uint16_t* sK,
                                               uint16_t* sV) {
  const int p0 = __builtin_amdgcn_readlane(pg, 0), p1 = __builtin_amdgcn_readlane(pg, 1);
  const int p2 = __builtin_amdgcn_readlane(pg, 2), p3 = __builtin_amdgcn_readlane(pg, 3);
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    const int kp = krow<P16>(8 * (kI & 7)) >> 4;  // page of rows 8(kI & 7) .. +7 (one page, wave-uniform)
    const int kpage = kp == 0 ? p0 : kp == 1 ? p1 : kp == 2 ? p2 : p3;
    lds_dma16(ks.ck + kpage * ks.page_stride + (uint32_t)((krow<P16>(m) & 15) * D + 64 * (kI >> 3) + 8 * c),
              sK + kI * 512);

    const int vI = w * DmaPlan<NW>::N + i;
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    const int vp = cv >> 1;
    const int vpage = vp == 0 ? p0 : vp == 1 ? p1 : vp == 2 ? p2 : p3;
    lds_dma16(ks.cv + vpage * ks.page_stride + (uint32_t)(d * 16 + 8 * (cv & 1)), sV + vI * 512);
  }
}

// ---------------------------------------------------------------- FP8 code tiles
// A tile of the cached prefix of an FP8 cache is moved into LDS as its raw
// codes by the same LDS DMA as a bf16 tile (16 KiB instead of 32): the DMA
// copies bytes and cannot convert. The MFMA operands are read as 8 codes
// (ds_read_b64) and converted exactly to bf16 in registers (every E4M3 value
// is a bf16 value); the attention then runs in the cache's code space (Q'
// times k_scale, O times v_scale). Layout in the slot (bytes):
//   K codes  [0, 8192):    row m (key kappa(m), as the bf16 tile) of 128 B,
//                          16-byte chunk c at position c ^ ((m >> 1) & 7);
//   V^T codes [8192, 16384): row d of 64 B (keys in order), 16-byte chunk c
//                          (16 keys, one page) at position c ^ ((d >> 2) & 3).
// Each swizzle spreads the 32 lanes of one b64 read over 16 positions: two
// lanes per bank pair, the least any 128-B (64-B) row layout allows here.
constexpr int kCodeVOff = 8192;

struct CodeSource {
  const uint8_t* k8;  // K codes of (cache row or page base, KV head g): + page * page_stride
  const uint8_t* v8;
  size_t page_stride;  // bytes per page of the paged cache (all KV heads); 0 on a ring
  int kind, window;
};

__device__ __forceinline__ CodeSource make_code_source(const PrefillParams& p, int kind, int cseq, int g) {
  CodeSource c;
  const size_t head = kind == 1 ? (size_t)g * 16 * D : ((size_t)cseq * p.G + g) * p.window * D;
  c.k8 = reinterpret_cast<const uint8_t*>(p.ck) + head;
  c.v8 = reinterpret_cast<const uint8_t*>(p.cv) + head;
  c.page_stride = kind == 1 ? (size_t)p.G * 16 * D : 0;
  c.kind = kind;
  c.window = p.window;
  return c;
}

// DMA of the code tile whose first key is key0 (a multiple of 64): 8 K and 8
// V instructions of 1 KiB, 8 / NW of each per wave. page(i) is the physical
// page of logical page i (paged caches). NT: non-temporal hint.
template <int NW, bool NT = false, bool P16 = false, typename PageOf>
__device__ __forceinline__ void dma_code_tile(const CodeSource& c, PageOf page, int w, int lane, int key0,
                                              uint8_t* slot) {
  // every source address first (the page lookups together), then the DMAs
  const uint8_t* ksrc[8 / NW];
  const uint8_t* vsrc[8 / NW];
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) {
    const int ins = w * (8 / NW) + i;
    {  // K rows 8 ins .. 8 ins + 7
      const int m = 8 * ins + (lane >> 3);
      const int cc = (lane & 7) ^ ((m >> 1) & 7);
      const int s = key0 + krow<P16>(m);
      ksrc[i] = (c.kind == 1 ? c.k8 + (size_t)page(s >> 4) * c.page_stride + (uint32_t)((s & 15) * D)
                             : c.k8 + (uint32_t)((s % c.window) * D)) + 16 * cc;
    }
    {  // V^T rows 16 ins .. 16 ins + 15
      const int d = 16 * ins + (lane >> 2);
      const int cc = (lane & 3) ^ ((d >> 2) & 3);
      const int s = key0 + 16 * cc;
      vsrc[i] = c.kind == 1 ? c.v8 + (size_t)page(s >> 4) * c.page_stride + (uint32_t)(d * 16)
                            : c.v8 + (uint32_t)(d * c.window + s % c.window);
    }
  }
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) {
    const int ins = w * (8 / NW) + i;
    const uint16_t* ks = reinterpret_cast<const uint16_t*>(ksrc[i]);
    const uint16_t* vs = reinterpret_cast<const uint16_t*>(vsrc[i]);
    uint16_t* kd = reinterpret_cast<uint16_t*>(slot + 1024 * ins);
    uint16_t* vd = reinterpret_cast<uint16_t*>(slot + kCodeVOff + 1024 * ins);
    if constexpr (NT) {
      lds_dma16_nt(ks, kd);
      lds_dma16_nt(vs, vd);
    } else {
      lds_dma16(ks, kd);
      lds_dma16(vs, vd);
    }
  }
}

// Per-lane byte offsets of the code operands: K for k-step kk (8 offsets,
// + 4096 for M-block 1), V^T for key block kb (4 offsets, + 2048 per row block).
struct CodeOffsets {
  int k[8];
  int v[4];
};
__device__ __forceinline__ CodeOffsets code_offsets(int n, int half) {
  CodeOffsets co;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) co.k[kk] = n * 128 + 16 * (kk ^ ((n >> 1) & 7)) + 8 * half;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) co.v[kb] = kCodeVOff + n * 64 + 16 * (kb ^ ((n >> 2) & 3)) + 8 * half;
  return co;
}
__device__ __forceinline__ u32x4 codes_to_bf16(u32x2 c) {
  const u32x2 lo = fp8x4_to_bf16x4(c[0]), hi = fp8x4_to_bf16x4(c[1]);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// K fragment of k-step kk, M-block mb: row n + 32 mb, codes 16 kk + 8 half + 0..7.
__device__ __forceinline__ u32x4 code_kfrag(const uint8_t* slot, const CodeOffsets& co, int kk, int mb) {
  return codes_to_bf16(*reinterpret_cast<const u32x2*>(slot + co.k[kk] + 4096 * mb));
}
// V^T fragment of key block kb, row block db: row 32 db + n, keys 16 kb + 8 half + 0..7.
__device__ __forceinline__ u32x4 code_vfrag(const uint8_t* slot, const CodeOffsets& co, int kb, int db) {
  return codes_to_bf16(*reinterpret_cast<const u32x2*>(slot + co.v[kb] + 2048 * db));
}
// The same for the 16x16x32 layout of the prefill kernel: K for d-step kk
// (4 offsets, + 2048 per key block of 16 rows), V^T for key chunk c2 (2
// offsets, + 1024 per row block of 16).
struct CodeOffsets16 {
  int k[4];
  int v[2];
};
__device__ __forceinline__ CodeOffsets16 code_offsets16(int c16, int lg) {
  CodeOffsets16 co;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) co.k[kk] = c16 * 128 + 16 * ((2 * kk + (lg >> 1)) ^ ((c16 >> 1) & 7)) + 8 * (lg & 1);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
    co.v[c2] = kCodeVOff + c16 * 64 + 16 * ((2 * c2 + (lg >> 1)) ^ ((c16 >> 2) & 3)) + 8 * (lg & 1);
  return co;
}
// K fragment of d-step kk, key block kb: row 16kb + c16, codes 32kk + 8lg + 0..7.
__device__ __forceinline__ u32x4 code_kfrag16(const uint8_t* slot, const CodeOffsets16& co, int kk, int kb) {
  return codes_to_bf16(*reinterpret_cast<const u32x2*>(slot + co.k[kk] + 2048 * kb));
}
// V^T fragment of key chunk c2, row block db: row 16db + c16, keys 32c2 + 8lg + 0..7.
__device__ __forceinline__ u32x4 code_vfrag16(const uint8_t* slot, const CodeOffsets16& co, int c2, int db) {
  return codes_to_bf16(*reinterpret_cast<const u32x2*>(slot + co.v[c2] + 1024 * db));
}
// Q' fragments times k_scale (one bf16 rounding), for the code space of an FP8 cache.
template <int NF>
__device__ __forceinline__ void scale_frags(u32x4 (&qf)[NF], float k_scale) {
#pragma unroll
  for (int kk = 0; kk < NF; ++kk)
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[kk][c] = pack_bf16x2(bf16lo(qf[kk][c]) * k_scale, bf16hi(qf[kk][c]) * k_scale);
}

// ---------------------------------------------------------------- kernel
// HB query heads (of one KV group) per block; wave w takes head w / (NWAVES /
// HB) and queries QW (w % (NWAVES / HB)) .. +QW-1 of the block's query range.
template <int KIND, int NWAVES, int KV_FP8, int HB>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attn_kernel(PrefillParams p) {
  // Queries per wave: three 16-query column blocks on global layers (each K
  // and V^T operand read from LDS feeds three MFMAs), two on local layers.
  constexpr int QW = prefill_wave_queries(KIND);
  constexpr int QB = QW / 16;
  constexpr int WQ = NWAVES / HB;  // waves per head
  constexpr int BM = WQ * QW;      // queries per block
  static_assert(16 % NWAVES == 0 && NWAVES % HB == 0, "tile split");
  constexpr int TPS = tiles_per_stage<KIND>();
  constexpr int SLOTS = 2 * TPS;  // tile slots: two stages
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SLOTS * (K_TILE + V_TILE)];

  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;  // consecutive blocks -> consecutive XCDs -> one KV head per XCD
  b /= p.G;
  const int hh0 = b % (hpg / HB) * HB;
  b /= hpg / HB;
  // Sequence-major, heaviest query tiles of a sequence first: the blocks in
  // flight on one XCD then stream one sequence's K/V tiles (shared in its L2)
  // instead of one tile from each of several sequences (8 sequences of a
  // chunked prefill: 6 % faster).
  const int qt = p.n_qtiles - 1 - b % p.n_qtiles;
  const int seq = b / p.n_qtiles;

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
  const int c16 = lane & 15;  // row of the MFMA A operand, column of B and of C
  const int lg = lane >> 4;   // lane group: k-slice 8lg of A and B, C rows 4lg .. 4lg+3
  const int h = g * hpg + hh0 + w / WQ;  // this wave's query head

  const int q0 = start + qt * BM;                   // first query position of the block
  const int qlast = min(q0 + BM, start + len) - 1;  // last valid query position
  const int wq_lo = q0 + QW * (w % WQ);
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
  const DmaPlan<NWAVES> plan = make_dma_plan<NWAVES, true>(w, lane);
  CodeSource cs8;
  if constexpr (KV_FP8) cs8 = make_code_source(p, KIND, cseq, g);

  // Q' fragments (B operand of S^T = K Q'^T): lane holds query c16 of column
  // block qb, coordinates 32kk + 8lg + 0..7.
  u32x4 qf[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // a query past the chunk's end loads the last valid row: its column of
    // S, P and O only feeds its own (never written) output
    const int t = min(wq_lo + 16 * qb + c16, qlast);
    const size_t tok = (size_t)(cu0 + (t - start));
    const uint16_t* qrow = p.qp + (tok * p.H + h) * D + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk);
    if constexpr (KV_FP8) scale_frags(qf[qb], p.k_scale);  // code space: q' k_scale against the codes
  }

  const int j_ws = start >> 6;  // first tile in the workspace; earlier tiles are wholly cached
  const int kmin = local ? max(0, q0 - (W - 1)) : 0;
  const int j_lo = cache_ok ? kmin >> 6 : max(kmin >> 6, j_ws);
  const int j_hi = qlast >> 6;

  f32x4 o[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: reference of the query (kNegInf until a key is visible); sref holds
  // -m_run (0 while m_run is kNegInf) splatted, the accumulator input of S.
  float m_run[QB], l_run[QB];
  f32x4 sref[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
    sref[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Loop-invariant LDS element offsets of this lane's operand chunks: K row
  // c16, chunk 4kk + lg (chunks 8..15 are the second coordinate half; key
  // block kb adds 16 rows); V^T row c16, chunk 4c2 + lg (row block db adds 16
  // rows).
  int koff[2], voff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) koff[kk] = k_off(c16, 4 * kk + lg);  // d-steps 2, 3: + K_HALF
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) voff[c2] = v_off(c16, 4 * c2 + lg);
  [[maybe_unused]] CodeOffsets16 co;
  if constexpr (KV_FP8) co = code_offsets16(c16, lg);

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
  // S^T - m = K Q'^T - m with v_mfma_f32_16x16x32_bf16: LDS rows 16kb + c16
  // on M (key block kb), queries 16qb + c16 on N; the chain starts from
  // sref = -m. Element i of block (qb, kb) holds key 32(kb >> 1) + 8lg +
  // 4(kb & 1) + i of the tile (the K row permutation).
  // CODES: the tile holds FP8 codes (converted after the LDS read).
  auto qk = [&](auto B, auto CODES, f32x4 (&s)[QB][4]) {
    const uint16_t* sK = buf(B);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 a;
        if constexpr (decltype(CODES)::value)
          a = code_kfrag16(reinterpret_cast<const uint8_t*>(sK), co, kk, kb);
        else
          a = *reinterpret_cast<const u32x4*>(sK + koff[kk & 1] + K_HALF * (kk >> 1) + 1024 * kb);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[qb][kk]),
                                                             kk == 0 ? sref[qb] : s[qb][kb], 0, 0, 0);
      }
    }
    if constexpr (!decltype(CODES)::value) {
      // K fragment reads run two k-steps ahead of the MFMAs that use them, so
      // the LDS latency hides behind the matrix work
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      static_for<2>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      });
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * QB, 0);
    }
  };
  // Per lane and query the visible key offsets c of the tile (relative to its
  // first key k0) are [t - (W-1) - k0, t - k0]: a 64-bit mask once per lane
  // and column block (only the bounds that cut into the tile), shifted by the
  // lane group's 8lg; each element then costs a bit-field extract and a
  // bit-field insert.
  auto apply_mask = [&](int j, f32x4 (&s)[QB][4]) {
    const int k0 = j * BN;
    const bool diag = k0 + BN - 1 > wq_lo;
    const bool edge = local && k0 < wq_hi - (W - 1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int t = wq_lo + 16 * qb + c16;
      uint64_t vis = ~0ull;
      if (diag) {
        const int hi = t - k0;  // visible: c <= hi
        vis &= hi >= 63 ? ~0ull : hi < 0 ? 0ull : (2ull << hi) - 1;
      }
      if (edge) {
        const int lo = t - (W - 1) - k0;  // visible: c >= lo
        vis &= lo <= 0 ? ~0ull : lo >= 64 ? 0ull : ~((1ull << lo) - 1);
      }
      const uint64_t vs = vis >> (8 * lg);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t word = (uint32_t)(vs >> (32 * (kb >> 1)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * (kb & 1) + i;
          const uint32_t m = (uint32_t)((int32_t)(word << (31 - c)) >> 31);
          s[qb][kb][i] = __uint_as_float((__float_as_uint(s[qb][kb][i]) & m) | (0xff800000u & ~m));
        }
      }
    }
  };
  // Shift of the reference this tile needs, per query: the tile max of the
  // shifted scores when it exceeds the threshold (or is the first finite
  // score of the query), else 0. A query's 64 keys sit in its four lane
  // groups (16 each).
  auto tile_max = [&](const f32x4 (&s)[QB][4], float (&mt)[QB]) {
    bool maybe = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[qb][kb][i]);
      mt[qb] = max_groups(x);
      // a reference moves only on a query's first finite score or when the
      // tile max passes the threshold: one cheap test per lane
      maybe = maybe || mt[qb] > kRescaleThreshold || m_run[qb] == kNegInf;
    }
    return maybe;
  };
  auto row_shift = [&](const float (&mt)[QB], float (&delta)[QB], bool (&need)[QB]) {
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      need[qb] = (m_run[qb] == kNegInf) ? (mt[qb] != kNegInf) : (mt[qb] > kRescaleThreshold);
      delta[qb] = need[qb] ? mt[qb] : 0.f;
      grow = grow || need[qb];
    }
    return grow;
  };
  // Move the reference up by delta: rescale O and l by 2^-delta (nothing to
  // rescale while no key was visible) and shift this tile's scores.
  // O is still zero at a query's first visible key (alpha 1), so a block's
  // first reference move skips the O multiply.
  auto rescale = [&](const float (&delta)[QB], const bool (&need)[QB], f32x4 (&s)[QB][4]) {
    float alpha[QB];
    bool scale_o = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool first = m_run[qb] == kNegInf;
      alpha[qb] = first ? 1.f : __builtin_amdgcn_exp2f(-delta[qb]);
      scale_o = scale_o || alpha[qb] != 1.f;
      if (need[qb]) m_run[qb] = (first ? 0.f : m_run[qb]) + delta[qb];
      const float r = m_run[qb] == kNegInf ? 0.f : -m_run[qb];
      sref[qb] = f32x4{r, r, r, r};
      l_run[qb] *= alpha[qb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[qb][kb][i] -= delta[qb];
    }
    if (__any(scale_o)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[qb][db][i] *= alpha[qb];
    }
  };
  // P^T operand of key chunk c2 (keys 32c2 .. 32c2+31): lane group lg holds
  // keys 32c2 + 8lg + 0..7 in order, elements 0..3 of S blocks 2c2 and 2c2+1.
  auto softmax = [&](const f32x4 (&s)[QB][4], u32x4 (&pf)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __builtin_amdgcn_exp2f(s[qb][2 * c2][i]);
          e[4 + i] = __builtin_amdgcn_exp2f(s[qb][2 * c2 + 1][i]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pf[qb][c2][c] = pack_bf16x2(e[2 * c], e[2 * c + 1]);
          l_run[qb] = sum_bf16x2(pf[qb][c2][c], l_run[qb]);
        }
      }
    }
  };
  // O^T += V^T P^T: A operand = coordinates 16db + c16, keys 32c2 + 8lg + 0..7.
  auto pv = [&](auto B, auto CODES, const u32x4 (&pf)[QB][2]) {
    const uint16_t* sV = buf(B) + K_TILE;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x4 a;
        if constexpr (decltype(CODES)::value)
          a = code_vfrag16(reinterpret_cast<const uint8_t*>(buf(B)), co, c2, db);
        else
          a = *reinterpret_cast<const u32x4*>(sV + voff[c2] + 1024 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[qb][c2]), o[qb][db], 0, 0, 0);
      }
    }
  };
  // Page ids of tile j of a paged prefix, one per lane: lane l holds page
  // (l & 3) of the tile (global layers; loaded a stage ahead of the DMA).
  auto load_pages = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (KIND == 1) {
      if (j < j_ws && j <= j_hi) return ks.bt_row[4 * j + (lane & 3)];
    }
    return 0;
  };
  // Fetch tile j into its slot by DMA, from the workspace or the cache (pg:
  // the tile's page ids from load_pages, on a paged prefix).
  auto fetch = [&](int j, auto B, int pg) __attribute__((always_inline)) {
    uint16_t* sK = buf(B);
    if (j >= j_ws)
      plan.copy(ks.kw, ks.vw, ks.ws_off, j * BN, sK, sK + K_TILE);
    else if constexpr (KIND == 1 && !KV_FP8)
      dma_tile_paged<NWAVES, true>(ks, pg, w, lane, sK, sK + K_TILE);
    else if constexpr (KV_FP8)
      dma_code_tile<NWAVES, false, true>(cs8, [&](int pg) { return ks.bt_row[pg]; }, w, lane, j * BN,
                                         reinterpret_cast<uint8_t*>(sK));
    else
      dma_tile_prefix<NWAVES, true>(ks, w, lane, j * BN, sK, sK + K_TILE);
  };

  // One 64-key tile of attention for this wave's queries (CODES: an FP8 code tile).
  auto tile = [&](int j, auto B, auto CODES) __attribute__((always_inline)) {
    f32x4 st[QB][4];
    qk(B, CODES, st);
    if (needs_mask(j)) apply_mask(j, st);
    float mt[QB];
    if (__any(tile_max(st, mt))) {
      float delta[QB];
      bool need[QB];
      if (__any(row_shift(mt, delta, need))) rescale(delta, need, st);
    }
    u32x4 pf[QB][2];
    softmax(st, pf);
    pv(B, CODES, pf);
  };
  // The main loop sees bf16 tiles only (over an FP8 cache the code tiles of
  // the cached prefix run first, in a loop of their own).
  auto compute_tile = [&](int j, auto B) __attribute__((always_inline)) {
    if (!active(j)) return;
    tile(j, B, std::false_type{});
  };
  // Gate rows of the wave's 32 queries into LDS (local layers): 8 KiB per wave
  // in the slot the last stage leaves free, so the epilogue's gate reads do
  // not wait on memory. DMA instruction i moves rows 4i .. 4i+3, 16 bytes per
  // lane; chunk c of row r lands at chunk position c ^ (r & 15), so the
  // epilogue's reads of one chunk from 16 consecutive rows hit distinct banks.
  // Rows past the chunk's end read the last valid row (never used).
  auto fetch_gate = [&](auto B) __attribute__((always_inline)) {
    uint16_t* dst = buf(B) + w * (QW * D);
#pragma unroll
    for (int i = 0; i < QW * D / 512; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const size_t tok = (size_t)(cu0 + (min(wq_lo + r, qlast) - start));
      lds_dma16(p.gate + (tok * p.H + h) * D + 8 * c, dst + 512 * i);
    }
  };
  static_assert(!local || (QW == 32 && NWAVES * QW * D <= K_TILE + V_TILE), "gate staging fits one slot");
  // Stage of tiles j0 .. j0+TPS-1 in slots S0 .. S0+TPS-1: before tile j0+u
  // is computed, tile j0+TPS+u is sent to the other stage's slot (freed by the
  // previous barrier); the barrier then publishes the next stage. On local
  // layers the last stage sends the gate rows instead.
  int pgs[TPS];  // page ids of the tiles the next stage fetches (paged prefix)
  auto stage = [&](int j0, auto S0) __attribute__((always_inline)) {
    static_for<TPS>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      constexpr int s0 = decltype(S0)::value;
      using Next = std::integral_constant<int, (s0 + TPS + u) % SLOTS>;
      if (j0 + TPS + u <= j_hi) {
        fetch(j0 + TPS + u, Next{}, pgs[u]);
        pgs[u] = load_pages(j0 + 2 * TPS + u);
      }
      else if constexpr (local)
        fetch_gate(Next{});
      if (j0 + u <= j_hi) compute_tile(j0 + u, std::integral_constant<int, s0 + u>{});
    });
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- tile loop ----
  int j_main = j_lo;
  if constexpr (KV_FP8) {
    // FP8 code tiles of the cached prefix (below the chunk's first tile), one
    // per step in buffers 0 and 1; then the main loop starts afresh.
    const int jc = min(j_hi, j_ws - 1);
    if (j_lo <= jc) {
      const auto CODE = std::true_type{};
      const auto S0 = std::integral_constant<int, 0>{};
      const auto S1 = std::integral_constant<int, 1>{};
      fetch(j_lo, S0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (int jt = j_lo; jt <= jc; jt += 2) {
        if (jt + 1 <= jc) fetch(jt + 1, S1, 0);
        if (active(jt)) tile(jt, S0, CODE);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (jt + 1 > jc) break;
        if (jt + 2 <= jc) fetch(jt + 2, S0, 0);
        if (active(jt + 1)) tile(jt + 1, S1, CODE);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      j_main = jc + 1;
    }
  }
  // slot holding the staged gate rows: the one after the last tile's
  const int gate_slot = (j_hi - j_main + 1) % SLOTS;
  static_for<TPS>([&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    if (j_main + u <= j_hi) fetch(j_main + u, U, load_pages(j_main + u));
    pgs[u] = load_pages(j_main + TPS + u);
  });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int jt = j_main; jt <= j_hi; jt += SLOTS) {
    stage(jt, std::integral_constant<int, 0>{});
    if (jt + TPS > j_hi) break;
    stage(jt + TPS, std::integral_constant<int, TPS>{});
  }

  // Epilogue: normalise, gate, write bf16. Lane holds query c16 of each
  // column block and coordinates d = 16db + 4lg + 0..3; its l is the sum over
  // the four lane groups. Every gate value is read before the first output
  // store (gate and output are both bf16 rows, so the compiler would
  // otherwise keep each load behind the previous store).
  // Y = O v_scale / (l (1 + 2^z)), z = -(gate + bias) log2 e: the sigmoid and
  // the normalisation share one reciprocal (v_rcp_f32, 1 ulp; a correctly
  // rounded division costs ~12 instructions per element, and Y is rounded to
  // bf16 next). v_scale applies over an FP8 cache (code space). l = 0 (no
  // visible key, O = 0) gives Y = 0.
  constexpr float kLog2e = 1.4426950408889634f;
  const float zb = -(p.gate_bias ? p.gate_bias[h] : 0.f) * kLog2e;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = wq_lo + 16 * qb + c16;
    const float l_tot = sum_groups(l_run[qb]);
    if (t > qlast) continue;
    const float l_eff = l_tot > 0.f ? (KV_FP8 ? l_tot / p.v_scale : l_tot) : 1.f;
    const size_t tok = (size_t)(cu0 + (t - start));
    uint16_t* orow = p.out + (tok * p.H + h) * D + 4 * lg;
    u32x2 gvs[8];
    if constexpr (local) {
      // staged row r = 16qb + c16: chunk 2db + (lg >> 1) at position chunk ^ (r & 15)
      const int r = 16 * qb + c16;
      const uint16_t* grow_ = smem + gate_slot * (K_TILE + V_TILE) + w * (QW * D) + r * D + 4 * (lg & 1);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        gvs[db] = *reinterpret_cast<const u32x2*>(grow_ + 8 * ((2 * db + (lg >> 1)) ^ (r & 15)));
    } else {
      const uint16_t* grow_ = p.gate + (tok * p.H + h) * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < 8; ++db) gvs[db] = *reinterpret_cast<const u32x2*>(grow_ + 16 * db);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 gv = gvs[db];
      const float gz[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ex = __builtin_amdgcn_exp2f(fmaf(gz[e], -kLog2e, zb));
        y[e] = o[qb][db][e] * __builtin_amdgcn_rcpf(fmaf(ex, l_eff, l_eff));
      }
      *reinterpret_cast<u32x2*>(orow + 16 * db) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
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
// dma_tile_prefix (16 / NW instructions each for K and V per wave). NT:
// non-temporal hint (a verify split of a paged cache reads its keys once).
template <int NW, bool NT>
__device__ __forceinline__ void dma_tile_cached(const KeySource& ks, const int* pages, int page0, int w, int lane,
                                                int key0, uint16_t* sK, uint16_t* sV) {
  // every source address first (the page lookups together), then the DMAs
  const uint16_t* ksrc[DmaPlan<NW>::N];
  const uint16_t* vsrc[DmaPlan<NW>::N];
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    const int m = 8 * (kI & 7) + (lane >> 3);
    const int c = (lane & 7) ^ ((m >> 1) & 7);
    ksrc[i] = k_row_cached(ks, pages, page0, key0 + krow_key(m)) + 64 * (kI >> 3) + 8 * c;
    const int vI = w * DmaPlan<NW>::N + i;
    const int d = 8 * vI + (lane >> 3);
    const int cv = (lane & 7) ^ ((d >> 1) & 7);
    vsrc[i] = v_elem_cached(ks, pages, page0, d, key0 + 8 * cv);
  }
#pragma unroll
  for (int i = 0; i < DmaPlan<NW>::N; ++i) {
    const int kI = w * DmaPlan<NW>::N + i;
    if constexpr (NT) {
      lds_dma16_nt(ksrc[i], sK + kI * 512);
      lds_dma16_nt(vsrc[i], sV + kI * 512);
    } else {
      lds_dma16(ksrc[i], sK + kI * 512);
      lds_dma16(vsrc[i], sV + kI * 512);
    }
  }
}

// s_waitcnt immediate for vmcnt <= n, lgkmcnt 0, expcnt untouched (gfx9
// fields: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
constexpr int vm_lgkm_wait(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

// NWAVES = 4: two bf16 tile buffers (64 KiB), two blocks per CU. NWAVES = 2
// (FP8 caches, chunks of at most 64 rows): one buffer (32 KiB, two 16-KiB
// code tiles), four blocks per CU, so that every wave of the CU has rows and
// the MFMA work of a CU spreads over all four SIMDs.
template <int KIND, int KV_FP8, int NWAVES>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
verify_attn_kernel(PrefillParams p) {
  constexpr bool local = (KIND == 0);
  constexpr int NSLOT = NWAVES == 4 ? 2 : 1;  // bf16 tile buffers
  // One LDS object: with a second __shared__ variable the compiler tags LDS
  // accesses with alias scopes and then makes every LDS read wait for all DMA
  // into the same array (vmcnt(0) before each tile's MFMAs), which serialises
  // the fetch of tile jt + 1 with the compute of tile jt.
  constexpr int kTiles = NSLOT * (K_TILE + V_TILE);
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
  if (start < 0 || (p.n_splits == 1 && t_last > p.max_pos)) {
    // The sequence's keys lie outside the split grid: its rows are NaN (with
    // several splits the combine writes them).
    if (p.n_splits == 1) {
      const int hpg_ = p.H / p.G, g_ = blockIdx.x % p.G;
      for (int i = threadIdx.x; i < len * hpg_ * D; i += 64 * NWAVES) {
        const int r = i / D;
        p.out[((size_t)(cu0 + r / hpg_) * p.H + g_ * hpg_ + r % hpg_) * D + i % D] = 0x7fc0;
      }
    }
    return;
  }

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
  CodeSource cs8;
  if constexpr (KV_FP8) cs8 = make_code_source(p, KIND, cseq, g);

  // Page ids of the split's cached tiles (tiles j_lo .. min(j_hi, j_ws - 1);
  // pages below (start & ~63) / 16, inside the block-table row).
  const int page0 = 4 * j_lo;
  if (KIND == 1 && cache_ok) {
    const int n_pg = 4 * (min(j_hi, j_ws - 1) - j_lo + 1);
    for (int i = tid; i < n_pg; i += 64 * NWAVES) s_pages[i] = ks.bt_row[page0 + i];
  }

  // This lane's row and the wave's range of query positions.
  const int n_rows = len * hpg;
  const int r = VQW * w + n;
  const bool row_valid = r < n_rows;
  const int tok_j = row_valid ? r / hpg : 0;
  const int h = g * hpg + (row_valid ? r - tok_j * hpg : 0);
  const int t_row = start + tok_j;
  const int r_lo = VQW * w;
  const bool wave_active = r_lo < n_rows;
  const int wq_lo = start + r_lo / hpg;
  const int wq_hi = start + (min(r_lo + VQW, n_rows) - 1) / hpg;

  u32x4 qf[8];
  {
    const uint16_t* qrow = p.qp + ((size_t)(cu0 + tok_j) * p.H + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = row_valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (KV_FP8) scale_frags(qf, p.k_scale);  // code space: q' k_scale against the codes
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
  [[maybe_unused]] CodeOffsets co;
  if constexpr (KV_FP8) co = code_offsets(n, half);

  auto buf = [&](auto B) -> uint16_t* { return smem + decltype(B)::value * (K_TILE + V_TILE); };
  auto active = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return wave_active && k0 <= wq_hi && !(local && k0 + BN - 1 < wq_lo - (W - 1));
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return (k0 + BN - 1 > wq_lo) || (local && k0 < wq_hi - (W - 1));
  };
  // A operand fragments of one tile: bf16 tiles (workspace, bf16 cache) or
  // FP8 code tiles (converted exactly after the LDS read).
  // Code tiles sit in 16 KiB sub-buffers: `sub` of them past buffer B.
  auto kfrag = [&](auto B, auto CODES, int sub, int kk, int mb) __attribute__((always_inline)) -> u32x4 {
    if constexpr (decltype(CODES)::value)
      return code_kfrag(reinterpret_cast<const uint8_t*>(buf(B)) + 16384 * sub, co, kk, mb);
    else
      return *reinterpret_cast<const u32x4*>(buf(B) + koff[kk & 3] + K_HALF * (kk >> 2) + 32 * 64 * mb);
  };
  auto vfrag = [&](auto B, auto CODES, int sub, int kb, int db) __attribute__((always_inline)) -> u32x4 {
    if constexpr (decltype(CODES)::value)
      return code_vfrag(reinterpret_cast<const uint8_t*>(buf(B)) + 16384 * sub, co, kb, db);
    else
      return *reinterpret_cast<const u32x4*>(buf(B) + K_TILE + voff[kb] + 32 * BN * db);
  };
  auto tile = [&](int j, auto B, auto CODES, int sub = 0) __attribute__((always_inline)) {
    f32x16 s[2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kfrag(B, CODES, sub, kk, mb)), as_bf16x8(qf[kk]),
                                                        kk == 0 ? sref : s[mb], 0, 0, 0);
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
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfrag(B, CODES, sub, kb, db)), as_bf16x8(pf[kb]), o[db],
                                                        0, 0, 0);
  };
  // DMA of tile j into buffer B: the workspace, the bf16 cache, or FP8 codes.
  auto dma = [&](int j, auto B) __attribute__((always_inline)) {
    uint16_t* sK = buf(B);
    if (j >= j_ws)
      plan.copy(ks.kw, ks.vw, ks.ws_off, j * BN, sK, sK + K_TILE);
    else if constexpr (KV_FP8)
      dma_code_tile<NWAVES, KIND == 1>(cs8, [&](int pg) { return s_pages[pg - page0]; }, w, lane, j * BN,
                            reinterpret_cast<uint8_t*>(sK));
    else
      dma_tile_cached<NWAVES, KIND == 1>(ks, s_pages, page0, w, lane, j * BN, sK, sK + K_TILE);
  };
  // Each step ends with an explicit wait for its DMA and a bare s_barrier:
  // the workgroup fence of __syncthreads would also wait for loads the
  // compiler cannot see as finished. The empty asm statements keep the
  // compiler from moving LDS accesses across it.
  auto step_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // One step: tile jt + 1 is sent to the other buffer while tile jt is
  // computed from buffer B.
  // The chunk's own tiles (workspace) alone, for the second loop over an FP8
  // cache, where no cached tile follows.
  auto dma_ws = [&](int j, auto B) __attribute__((always_inline)) {
    uint16_t* sK = buf(B);
    plan.copy(ks.kw, ks.vw, ks.ws_off, j * BN, sK, sK + K_TILE);
  };
  auto step = [&](int jt, auto B, auto CODES, auto& fetch) __attribute__((always_inline)) {
    if (jt + 1 <= j_hi) fetch(jt + 1, std::integral_constant<int, 1 - decltype(B)::value>{});
    if (active(jt)) tile(jt, B, CODES);
    step_end();
  };
  const auto S0 = std::integral_constant<int, 0>{};
  const auto S1 = std::integral_constant<int, 1>{};
  __builtin_amdgcn_s_waitcnt(0);  // Q' and page ids in
  __syncthreads();
  int jt = j_lo;
  if constexpr (KV_FP8) {
    // The code tiles of an FP8 cache (the cached keys below the chunk) come
    // first, in a loop of their own: one kind of tile per loop body keeps the
    // register allocation as tight as in a single-kind kernel. A code tile
    // takes 16 KiB, so the two buffers hold four: the DMA runs three tiles
    // ahead, and each step waits only for the tile the next step computes
    // (each tile is 16 / NWAVES DMA instructions of every wave).
    constexpr int kPerTile = 16 / NWAVES;  // DMA instructions of a wave per code tile
    constexpr int NSUB = 2 * NSLOT;         // 16-KiB code tile buffers
    constexpr int AHEAD = NSUB - 1;         // tiles in flight beyond the one computed
    const int jc = min(j_hi, j_ws - 1);
    if (j_lo <= jc) {
      auto sub = [&](auto U) { return reinterpret_cast<uint8_t*>(smem) + 16384 * decltype(U)::value; };
      auto dma_c = [&](int j, auto U) __attribute__((always_inline)) {
        dma_code_tile<NWAVES, KIND == 1>(cs8, [&](int pg) { return s_pages[pg - page0]; }, w, lane, j * BN, sub(U));
      };
      // wait until tile j + 1 has landed (the tiles after it may stay in flight)
      auto wait_next = [&](int j) __attribute__((always_inline)) {
        const int ahead = min(j + AHEAD, jc) - (j + 1);
        if (AHEAD >= 3 && ahead >= 2)
          __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * kPerTile));
        else if (AHEAD >= 2 && ahead >= 1)
          __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kPerTile));
        else
          __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      };
      auto cstep = [&](int j, auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        if (j + AHEAD <= jc) dma_c(j + AHEAD, std::integral_constant<int, (u + AHEAD) % NSUB>{});
        if (active(j)) tile(j, std::integral_constant<int, 0>{}, std::true_type{}, u);
        wait_next(j);
      };
      static_for<AHEAD>([&](auto U) __attribute__((always_inline)) {
        if (j_lo + decltype(U)::value <= jc) dma_c(j_lo + decltype(U)::value, U);
      });
      wait_next(j_lo - 1);
      for (; jt <= jc; jt += NSUB) {
        bool done = false;
        static_for<NSUB>([&](auto U) __attribute__((always_inline)) {
          if (!done && jt + decltype(U)::value <= jc) cstep(jt + decltype(U)::value, U);
          else done = true;
        });
        if (done) break;
      }
      jt = jc + 1;
    }
  }
  // bf16 tiles (the workspace, or a bf16 cache) in two buffers: tile jt + 1
  // arrives while tile jt is computed.
  const auto BF = std::false_type{};
  auto& fetch2 = [&]() -> auto& {
    if constexpr (KV_FP8) return dma_ws; else return dma;
  }();
  if constexpr (NSLOT == 2) {
    if (jt <= j_hi) {
      fetch2(jt, S0);
      step_end();
    }
    for (; jt <= j_hi; jt += 2) {
      step(jt, S0, BF, fetch2);
      if (jt + 1 > j_hi) break;
      step(jt + 1, S1, BF, fetch2);
    }
  } else {
    // one buffer: fetch, compute, then free it for the next tile
    for (; jt <= j_hi; ++jt) {
      fetch2(jt, S0);
      step_end();
      if (active(jt)) tile(jt, S0, BF);
      step_end();
    }
  }

  // Partials of this split: lane holds row n's sum half and coordinates
  // d = 32db + 8a + 4*half + 0..3.
  const float l_tot = sum_halves(l_run);
  if (!row_valid) return;
  if (p.n_splits == 1) {
    // A single split needs no merge: the gated output directly, with the
    // combine's arithmetic (so either path gives the same bits).
    const size_t idx = ((size_t)(cu0 + tok_j) * p.H + h) * D + 4 * half;
    const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
    const float inv = (m_run != kNegInf && l_tot > 0.f) ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const float vs = KV_FP8 ? p.v_scale : 1.f;
    u32x2 gv[4][4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) gv[db][a] = *reinterpret_cast<const u32x2*>(p.gate + idx + 32 * db + 8 * a);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float gz[4] = {bf16lo(gv[db][a][0]), bf16hi(gv[db][a][0]), bf16lo(gv[db][a][1]), bf16hi(gv[db][a][1])};
        uint16_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ov = o[db][4 * a + e] * inv * vs;
          const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(gz[e] + bias)));
          y[e] = __builtin_bit_cast(uint16_t, (__bf16)(ov * sg));
        }
        *reinterpret_cast<u32x2*>(p.out + idx + 32 * db + 8 * a) =
            u32x2{(uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16)};
      }
    return;
  }
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
// Verify over an FP8 cache for chunks of at most 48 (token, query head) rows
// of a KV head (an 8-token draft at 6 query heads per KV head): one wave holds
// all rows as three 16-row column blocks of v_mfma_f32_16x16x32_bf16, so every
// code tile is converted to bf16 once per block (not once per wave) and no
// MFMA is spent on padding rows. Tiles, key order (krow_key16), masks and the
// softmax are those of the prefill kernel; rows are (token, head) pairs as in
// verify_attn_kernel, whose partials and single-split epilogue this kernel
// writes in the same format. NSUB 16-KiB code buffers: the DMA runs NSUB - 1
// tiles ahead; two of them hold the bf16 workspace tiles afterwards.
template <int KIND, int NSUB>
__global__ void __launch_bounds__(64) verify48_fp8_kernel(PrefillParams p) {
  constexpr bool local = (KIND == 0);
  constexpr int QB = 3;
  static_assert(NSUB >= 2, "the workspace tile needs two code buffers");
  constexpr int kCodeBytes = NSUB * 16384;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kCodeBytes / 2 + (KIND == 1 ? 2 * kVerifyMaxPages : 0)];
  int* const s_pages = reinterpret_cast<int*>(smem + kCodeBytes / 2);
  uint8_t* const codes = reinterpret_cast<uint8_t*>(smem);

  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;
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
  const int lane = threadIdx.x;
  if (start < 0 || (p.n_splits == 1 && t_last > p.max_pos)) {
    if (p.n_splits == 1)  // NaN rows (with several splits the combine writes them)
      for (int i = lane; i < len * hpg * D; i += 64) {
        const int r = i / D;
        p.out[((size_t)(cu0 + r / hpg) * p.H + g * hpg + r % hpg) * D + i % D] = 0x7fc0;
      }
    return;
  }

  KeySource ks;
  ks.kw = p.kw + (size_t)g * p.P * D;
  ks.vw = p.vw + (size_t)g * D * p.P;
  ks.ck = p.ck;
  ks.cv = p.cv;
  ks.page_stride = 0;
  ks.bt_row = KIND == 1 ? p.bt + (size_t)cseq * p.max_pages : nullptr;
  const bool cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (KIND == 0 || ((start + 15) >> 4) <= p.max_pages);
  ks.ws_off = ws_region_base(cu0, seq) - (start & ~63);
  ks.P = p.P;
  ks.kind = KIND;
  ks.window = W;
  const int j_ws = start >> 6;
  const int kmin = local ? max(0, start - (W - 1)) : 0;
  const int j_first = cache_ok ? kmin >> 6 : max(kmin >> 6, j_ws);
  const int j_last = t_last >> 6;
  const int j_lo = j_first + sp * p.split_tiles;
  if (j_lo > j_last) return;  // past this sequence's keys; the combine skips the split
  const int j_hi = min(j_last, j_lo + p.split_tiles - 1);

  const int c16 = lane & 15, lg = lane >> 4;
  const DmaPlan<1> plan = make_dma_plan<1, true>(0, lane);
  const CodeSource cs8 = make_code_source(p, KIND, cseq, g);
  const int page0 = 4 * j_lo;
  if (KIND == 1 && cache_ok) {
    const int n_pg = 4 * (min(j_hi, j_ws - 1) - j_lo + 1);
    for (int i = lane; i < n_pg; i += 64) s_pages[i] = ks.bt_row[page0 + i];
  }

  // Row 16qb + c16 of column block qb: token r / hpg, head r % hpg.
  const int n_rows = len * hpg;
  bool rv[QB];
  int rtok[QB], rh[QB], t_row[QB];
  u32x4 qf[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = 16 * qb + c16;
    rv[qb] = r < n_rows;
    rtok[qb] = rv[qb] ? r / hpg : 0;
    rh[qb] = g * hpg + (rv[qb] ? r - rtok[qb] * hpg : 0);
    t_row[qb] = start + rtok[qb];
    const uint16_t* qrow = p.qp + ((size_t)(cu0 + rtok[qb]) * p.H + rh[qb]) * D + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[qb][kk] = rv[qb] ? *reinterpret_cast<const u32x4*>(qrow + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
    scale_frags(qf[qb], p.k_scale);  // code space: q' k_scale against the codes
  }
  const int wq_lo = start, wq_hi = t_last;

  f32x4 o[QB][8];
  float m_run[QB], l_run[QB];
  f32x4 sref[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
    sref[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int koff[2], voff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) koff[kk] = k_off(c16, 4 * kk + lg);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) voff[c2] = v_off(c16, 4 * c2 + lg);
  const CodeOffsets16 co = code_offsets16(c16, lg);

  auto active = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return k0 <= wq_hi && !(local && k0 + BN - 1 < wq_lo - (W - 1));
  };
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN;
    return (k0 + BN - 1 > wq_lo) || (local && k0 < wq_hi - (W - 1));
  };
  // One 64-key tile: a code tile at `slot` (CODES) or the bf16 tile at smem.
  auto tile = [&](int j, auto CODES, const uint8_t* slot) __attribute__((always_inline)) {
    constexpr bool C = decltype(CODES)::value;
    const uint16_t* sK = smem;
    const uint16_t* sV = smem + K_TILE;
    f32x4 st[QB][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 a;
        if constexpr (C)
          a = code_kfrag16(slot, co, kk, kb);
        else
          a = *reinterpret_cast<const u32x4*>(sK + koff[kk & 1] + K_HALF * (kk >> 1) + 1024 * kb);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          st[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[qb][kk]),
                                                              kk == 0 ? sref[qb] : st[qb][kb], 0, 0, 0);
      }
    if (needs_mask(j)) {  // element i of block (qb, kb): key 32(kb >> 1) + 8lg + 4(kb & 1) + i of the tile
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sk = j * BN + 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + i;
            if (!visible(KIND, W, t_row[qb], sk)) st[qb][kb][i] = kNegInf;
          }
    }
    // Reference shift per row, as in the prefill kernel.
    bool need[QB];
    bool any_need = false;
    float mt[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, st[qb][kb][i]);
      mt[qb] = max_groups(x);
      need[qb] = (m_run[qb] == kNegInf) ? (mt[qb] != kNegInf) : (mt[qb] > kRescaleThreshold);
      any_need = any_need || need[qb];
    }
    if (__any(any_need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float delta = need[qb] ? mt[qb] : 0.f;
        const bool first = m_run[qb] == kNegInf;
        const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta);
        if (need[qb]) m_run[qb] = (first ? 0.f : m_run[qb]) + delta;
        const float rr = m_run[qb] == kNegInf ? 0.f : -m_run[qb];
        sref[qb] = f32x4{rr, rr, rr, rr};
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[qb][db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[qb][kb][i] -= delta;
      }
    }
    // P^T of key chunk c2: lane group lg holds keys 32c2 + 8lg + 0..7.
    u32x4 pf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __builtin_amdgcn_exp2f(st[qb][2 * c2][i]);
          e[4 + i] = __builtin_amdgcn_exp2f(st[qb][2 * c2 + 1][i]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pf[qb][c2][c] = pack_bf16x2(e[2 * c], e[2 * c + 1]);
          l_run[qb] = sum_bf16x2(pf[qb][c2][c], l_run[qb]);
        }
      }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x4 a;
        if constexpr (C)
          a = code_vfrag16(slot, co, c2, db);
        else
          a = *reinterpret_cast<const u32x4*>(sV + voff[c2] + 1024 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf[qb][c2]), o[qb][db], 0, 0, 0);
      }
  };
  // wait until at most VM vector memory operations are in flight, then a bare s_barrier
  auto barrier = [&](auto VM) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(decltype(VM)::value));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  __builtin_amdgcn_s_waitcnt(0);  // Q' and page ids in
  __syncthreads();

  int jt = j_lo;
  // Code tiles of the cached keys below the chunk: NSUB buffers, the DMA
  // NSUB - 1 tiles ahead; each step waits only for the tile the next step
  // computes (a code tile is 16 DMA instructions of the wave).
  constexpr int AHEAD = NSUB - 1;
  constexpr int kPerTile = 16;
  const int jc = min(j_hi, j_ws - 1);
  if (j_lo <= jc) {
    auto page_of = [&](int pg) { return s_pages[pg - page0]; };
    auto dma_c = [&](int j, int u) __attribute__((always_inline)) {
      dma_code_tile<1, KIND == 1, true>(cs8, page_of, 0, lane, j * BN, codes + 16384 * u);
    };
    auto wait_next = [&](int j) __attribute__((always_inline)) {
      const int ahead = min(j + AHEAD, jc) - (j + 1);  // tiles in flight beyond tile j + 1
      if (AHEAD >= 3 && ahead >= 2)
        barrier(std::integral_constant<int, 2 * kPerTile>{});
      else if (AHEAD >= 2 && ahead >= 1)
        barrier(std::integral_constant<int, kPerTile>{});
      else
        barrier(std::integral_constant<int, 0>{});
    };
#pragma unroll
    for (int u = 0; u < AHEAD; ++u)
      if (j_lo + u <= jc) dma_c(j_lo + u, u);
    wait_next(j_lo - 1);
    for (; jt <= jc; jt += NSUB) {
      bool done = false;
      static_for<NSUB>([&](auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        const int j = jt + u;
        if (done || j > jc) {
          done = true;
          return;
        }
        if (j + AHEAD <= jc) dma_c(j + AHEAD, (u + AHEAD) % NSUB);
        if (active(j)) tile(j, std::true_type{}, codes + 16384 * u);
        wait_next(j);
      });
      if (done) break;
    }
    jt = jc + 1;
  }
  // The chunk's own tiles (bf16, from the workspace) in the first two buffers.
  for (; jt <= j_hi; ++jt) {
    plan.copy(ks.kw, ks.vw, ks.ws_off, jt * BN, smem, smem + K_TILE);
    barrier(std::integral_constant<int, 0>{});
    if (active(jt)) tile(jt, std::false_type{}, codes);
    barrier(std::integral_constant<int, 0>{});
  }

  // Partials of this split (or, with a single split, the gated output with the
  // combine's arithmetic): lane holds row 16qb + c16, coordinates 16db + 4lg + 0..3.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_groups(l_run[qb]);
    if (!rv[qb]) continue;
    const int h = rh[qb];
    if (p.n_splits == 1) {
      const size_t idx = ((size_t)(cu0 + rtok[qb]) * p.H + h) * D + 4 * lg;
      const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
      const float inv = (m_run[qb] != kNegInf && l_tot > 0.f) ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
      u32x2 gv[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) gv[db] = *reinterpret_cast<const u32x2*>(p.gate + idx + 16 * db);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const float gz[4] = {bf16lo(gv[db][0]), bf16hi(gv[db][0]), bf16lo(gv[db][1]), bf16hi(gv[db][1])};
        uint16_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ov = o[qb][db][e] * inv * p.v_scale;
          const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(gz[e] + bias)));
          y[e] = __builtin_bit_cast(uint16_t, (__bf16)(ov * sg));
        }
        *reinterpret_cast<u32x2*>(p.out + idx + 16 * db) =
            u32x2{(uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16)};
      }
      continue;
    }
    const size_t row = ((size_t)(cu0 + rtok[qb]) * p.H + h) * p.n_splits + sp;
    if (lg == 0) {
      p.part_ml[2 * row] = m_run[qb];
      p.part_ml[2 * row + 1] = l_tot;
    }
    float* acc = p.part_acc + row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(acc + 16 * db) = o[qb][db];
  }
}

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
  const size_t idx = ((size_t)tok * p.H + h) * D + d;
  if (start < 0 || start + len - 1 > p.max_pos) {
    p.out[idx] = 0x7fc0;  // NaN: the chunk reaches past max_pos, beyond the keys the split grid covers
    return;
  }
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
  const float o = L > 0.f ? A * __builtin_amdgcn_rcpf(L) * p.v_scale : 0.f;
  const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
  const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(bf16f(p.gate[idx]) + bias)));
  bf16x2 rr;
  rr[0] = (__bf16)(o * sg);
  p.out[idx] = __builtin_bit_cast(uint16_t, rr[0]);
}

// Code buffers of verify48_fp8_kernel (16 KiB each; 2 KiB of page ids on top).
constexpr int kVerify48Bufs = 2;

hipError_t launch_verify_attn(const PrefillParams& p, int max_rows, hipStream_t s) {
  clear_stale_error();
  if (p.split_tiles * 4 > kVerifyMaxPages) return hipErrorInvalidValue;
  const long long blocks = (long long)p.G * p.n_splits * p.n_seqs;
  const dim3 grid((unsigned)blocks), block4(64 * kVerifyWaves), block2(128);
  const bool two = p.kv_fp8 && max_rows <= 64;  // FP8 cache, chunks of at most 64 rows: 2-wave blocks
  const bool one = p.kv_fp8 && max_rows <= 48;  // at most 48 rows: one wave holds them all
  const dim3 block1(64);
  if (p.kind == 0 && one)
    hipLaunchKernelGGL((verify48_fp8_kernel<0, kVerify48Bufs>), grid, block1, 0, s, p);
  else if (p.kind == 1 && one)
    hipLaunchKernelGGL((verify48_fp8_kernel<1, kVerify48Bufs>), grid, block1, 0, s, p);
  else if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL((verify_attn_kernel<0, 0, 4>), grid, block4, 0, s, p);
  else if (p.kind == 0 && two)
    hipLaunchKernelGGL((verify_attn_kernel<0, 1, 2>), grid, block2, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL((verify_attn_kernel<0, 1, 4>), grid, block4, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL((verify_attn_kernel<1, 0, 4>), grid, block4, 0, s, p);
  else if (two)
    hipLaunchKernelGGL((verify_attn_kernel<1, 1, 2>), grid, block2, 0, s, p);
  else
    hipLaunchKernelGGL((verify_attn_kernel<1, 1, 4>), grid, block4, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_combine(const VerifyCombineParams& p, hipStream_t s) {
  clear_stale_error();
  hipLaunchKernelGGL(verify_combine_kernel, dim3((unsigned)((long long)p.n_tok * p.H)), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  clear_stale_error();
  const int hpg = p.H / p.G;
  const int hb = prefill_heads_per_block(p.kind, hpg);
  const long long blocks = (long long)p.G * (hpg / hb) * p.n_seqs * p.n_qtiles;
  const dim3 grid((unsigned)blocks), local_block(64 * kPrefillWavesLocal), global_block(64 * kPrefillWavesGlobal);
  if (p.kind == 0 && hb == 2 && !p.kv_fp8)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 0, 2>), grid, local_block, 0, s, p);
  else if (p.kind == 0 && hb == 2)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 1, 2>), grid, local_block, 0, s, p);
  else if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 0, 1>), grid, local_block, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL((prefill_attn_kernel<0, kPrefillWavesLocal, 1, 1>), grid, local_block, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL((prefill_attn_kernel<1, kPrefillWavesGlobal, 0, 1>), grid, global_block, 0, s, p);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<1, kPrefillWavesGlobal, 1, 1>), grid, global_block, 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
