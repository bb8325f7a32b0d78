// Split-K paged decode attention with bf16 MFMA (gfx950).
//
// One new query token per sequence attends over its cache: all t+1 positions
// on a global layer (paged), the last min(t+1, window) on a local layer (ring);
// "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax", sections "Two
// attention paths in one decoder" and "KV memory: nine growing caches, not 52"
// (every cached token is read once per layer and query).
//
// Each block handles one (sequence, KV head, split of 4*kpw keys); its four
// wavefronts stream kpw keys each, 32 keys (two 16-token pages) per step. The
// 6 query heads that share the KV head form the N side of
// v_mfma_f32_16x16x32_bf16 (padded to 16), so every K/V byte is read from HBM
// once for all of them. K pages are token-major, V pages are stored
// transposed (d-major), so both MFMA operands are plain vector loads straight
// from HBM into registers; nothing is staged in LDS on the hot path (an FP8
// E4M3 cache has its own kernel below, with 64-key steps). The four
// waves merge their (max, sum, acc) triples through LDS; a second kernel merges
// the splits by log-sum-exp and applies the output gate.
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

constexpr float kDecRescale = 8.0f;

// Merge the four waves' (max, sum, acc) of one block through LDS and store
// the block's partials (part_ml, part_acc) for the combine kernel. Lane
// (nn, q) holds head nn's max and sum (all four lane groups agree) and o[db][i]
// = head nn, coordinate 16db + 4q + i.
__device__ __forceinline__ void store_wave_partials(const DecodeParams& p, int seq, int g, int sp, int hpg, int tid,
                                                    float m_run, float l_run, const f32x4 (&o)[8]) {
  const int lane = tid & 63, w = tid >> 6, nn = lane & 15, q = lane >> 4;
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  __shared__ float s_o[4][16][D + 4];
  if (lane < 16) {
    s_m[w][lane] = m_run;
    s_l[w][lane] = l_run;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[w][nn][16 * db + 4 * q + i] = o[db][i];
  __syncthreads();

  for (int e2 = tid; e2 < hpg * D; e2 += 256) {
    const int hn = e2 / D, d = e2 - hn * D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hn]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float sc = __builtin_amdgcn_exp2f(s_m[ww][hn] - M);
        L += sc * s_l[ww][hn];
        A += sc * s_o[ww][hn][d];
      }
    }
    const size_t row = ((size_t)seq * p.H + g * hpg + hn) * p.n_splits + sp;
    p.part_acc[row * D + d] = A;
    if (d == 0) {
      p.part_ml[2 * row] = M;
      p.part_ml[2 * row + 1] = L;
    }
  }
}


struct DecodeStep {
  u32x4 k[2][4];  // [page][d-block of 32]
  u32x2 v[2][8];  // [page][d-block of 16]
};

template <int KIND>
__global__ void __launch_bounds__(256, 2) decode_split_kernel(DecodeParams p) {
  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;
  b /= p.G;
  const int sp = b % p.n_splits;
  const int seq = b / p.n_splits;

  const int t = p.pos[seq];
  const int cseq = p.seq_idx[seq];
  // Positions beyond max_pos or bad cache rows are not read (the combine
  // kernel writes NaN for such sequences).
  if (t < 0 || t > p.max_pos || cseq < 0 || cseq >= p.n_cache_seqs) return;
  constexpr bool local = (KIND == 0);
  const int n_keys = local ? min(t + 1, p.window) : t + 1;
  const int split0 = sp * 4 * p.kpw;
  if (split0 >= n_keys) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nn = lane & 15;  // head column (valid if < hpg); also the key row of K loads
  const int q = lane >> 4;   // lane group 0..3

  const int k0 = split0 + w * p.kpw;
  const int k1 = min(k0 + p.kpw, n_keys);

  // Q' fragments (B operand of S^T = K Q'^T): head nn, coords 32kk + 8q + 0..7.
  u32x4 qf[4];
  {
    const bool hv = nn < hpg;
    const uint16_t* qrow = p.qp + ((size_t)seq * p.H + g * hpg + (hv ? nn : 0)) * D + 8 * q;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = hv ? *reinterpret_cast<const u32x4*>(qrow + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  const int32_t* bt_row = p.bt + (size_t)cseq * p.max_pages;
  const size_t ring = (size_t)cseq * p.G + g;

  // Base pointers of the 16-key group starting at logical key kg.
  auto kbase = [&](int kg) -> const uint16_t* {
    if (local) return p.ck + (ring * p.window + kg) * D;
    int page = bt_row[kg >> 4];
    return p.ck + ((size_t)page * p.G + g) * 16 * D;
  };
  auto vbase = [&](int kg, int* dstride) -> const uint16_t* {
    if (local) {
      *dstride = p.window;
      return p.cv + ring * D * p.window + kg;
    }
    *dstride = 16;
    int page = bt_row[kg >> 4];
    return p.cv + ((size_t)page * p.G + g) * D * 16;
  };
  auto load_step = [&](int kb, DecodeStep& st) {
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const int kg = kb + 16 * X;
      if (kg < k1) {
        const uint16_t* kp = kbase(kg) + nn * D + 8 * q;
        // global layers: non-temporal, every cached byte is read once per call
        // (measured 4-7 % faster on bf16 caches; in the FP8 kernel only the V
        // loads take it). A local layer's rings (window-sized) are left to the
        // caches.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          st.k[X][kk] = local ? *reinterpret_cast<const u32x4*>(kp + 32 * kk)
                              : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 32 * kk));
        int ds;
        const uint16_t* vp = vbase(kg, &ds) + 4 * q;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          st.v[X][db] = local ? *reinterpret_cast<const u32x2*>(vp + (size_t)(16 * db + nn) * ds)
                              : __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp + (size_t)(16 * db + nn) * ds));
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) st.k[X][kk] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int db = 0; db < 8; ++db) st.v[X][db] = u32x2{0u, 0u};
      }
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;

  DecodeStep cur, nxt;
  if (k0 < k1) load_step(k0, cur);
  for (int kb = k0; kb < k1; kb += 32) {
    const bool has_next = kb + 32 < k1;
    if (has_next) load_step(kb + 32, nxt);

    const bool partial = kb + 32 > k1;
    if (partial) {
      // Zero V of keys past the end (their pages may hold stale or unwritten data).
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int key0 = kb + 16 * X + 4 * q;
          u32x2 v = cur.v[X][db];
          uint32_t m0 = (key0 + 0 < k1 ? 0xffffu : 0u) | (key0 + 1 < k1 ? 0xffff0000u : 0u);
          uint32_t m1 = (key0 + 2 < k1 ? 0xffffu : 0u) | (key0 + 3 < k1 ? 0xffff0000u : 0u);
          cur.v[X][db] = u32x2{v[0] & m0, v[1] & m1};
        }
    }

    f32x4 s[2];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      s[X] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[X] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.k[X][kk]), as_bf16x8(qf[kk]), s[X], 0, 0, 0);
    }
    // lane holds head nn, keys kb + 16X + 4q + i
    if (partial) {
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * X + 4 * q + i >= k1) s[X][i] = kNegInf;
    }
    float mt = kNegInf;
#pragma unroll
    for (int X = 0; X < 2; ++X)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[X][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run + kDecRescale)) {
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= alpha;
    }
    const float mu = (m_run == kNegInf) ? 0.f : m_run;
    float e[8];
#pragma unroll
    for (int X = 0; X < 2; ++X)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[4 * X + i] = __builtin_amdgcn_exp2f(s[X][i] - mu);
        l_run += e[4 * X + i];
      }
    // P^T operand: k-slot 8q + j <-> key 16(j>>2) + 4q + (j&3)
    const u32x4 pf = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                           pack_bf16x2(e[6], e[7])};
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x4 a = u32x4{cur.v[0][db][0], cur.v[0][db][1], cur.v[1][db][0], cur.v[1][db][1]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf), o[db], 0, 0, 0);
    }
    if (has_next) cur = nxt;
  }

  // Sum of the lane partials of each head (lanes nn, nn+16, nn+32, nn+48).
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  store_wave_partials(p, seq, g, sp, hpg, tid, m_run, l_run, o);
}

// ----------------------------------------------------------------------------
// Decode over an FP8 E4M3 cache. Same split/merge structure as the bf16
// kernel, but a step covers 64 keys (four 16-token pages) and every load is
// 16 bytes, so a wave moves as many bytes per step as the bf16 kernel with
// fewer memory instructions:
//   * S MFMA b (b = 0..3) takes as row r the key (page r>>2, slot 4b + (r&3));
//     its output then gives lane group q the scores of page q, slots 4b + i.
//   * The dot product over d splits as lane group q <-> coordinates
//     [32q, 32q+32) (MFMA kk takes 32q + 8kk + 0..7), one 32-byte run of the
//     key's row; Q' is loaded with the same split.
//   * PV MFMA kh (kh = 0, 1) takes key slot 8q + j <-> (page q, slot 8kh + j),
//     which is the order of lane group q's scores and of the 16-byte V^T row
//     of page q that each lane loads.
// Codes convert exactly to bf16 in registers; k_scale rides on Q' and
// v_scale on the output.
// ----------------------------------------------------------------------------
struct Fp8Step {
  u32x4 k[4][2];  // [S block b][16-byte half]: 32 codes of one key row
  u32x4 v[8];     // [d-block]: 16 codes of one V^T row of page q
};

// Codes 8w .. 8w+7 of a 16-byte load as bf16 (exact).
__device__ __forceinline__ u32x4 fp8x8_bf16(const u32x4& c, int w) {
  const u32x2 lo = fp8x4_to_bf16x4(c[2 * w]), hi = fp8x4_to_bf16x4(c[2 * w + 1]);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

template <int KIND>
__global__ void __launch_bounds__(256, 2) decode_fp8_kernel(DecodeParams p) {
  const int hpg = p.H / p.G;
  int b = blockIdx.x;
  const int g = b % p.G;
  b /= p.G;
  const int sp = b % p.n_splits;
  const int seq = b / p.n_splits;

  const int t = p.pos[seq];
  const int cseq = p.seq_idx[seq];
  if (t < 0 || t > p.max_pos || cseq < 0 || cseq >= p.n_cache_seqs) return;
  constexpr bool local = (KIND == 0);
  const int n_keys = local ? min(t + 1, p.window) : t + 1;
  const int split0 = sp * 4 * p.kpw;
  if (split0 >= n_keys) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nn = lane & 15;  // head column of S/O; row of the K and V operands
  const int q = lane >> 4;   // lane group 0..3

  const int k0 = split0 + w * p.kpw;
  const int k1 = min(k0 + p.kpw, n_keys);

  // Q' fragments: head nn, coordinates 32q + 8kk + 0..7.
  u32x4 qf[4];
  {
    const bool hv = nn < hpg;
    const uint16_t* qrow = p.qp + ((size_t)seq * p.H + g * hpg + (hv ? nn : 0)) * D + 32 * q;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = hv ? *reinterpret_cast<const u32x4*>(qrow + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  const int32_t* bt_row = p.bt + (size_t)cseq * p.max_pages;
  const size_t ring = (size_t)cseq * p.G + g;
  const uint8_t* ck = reinterpret_cast<const uint8_t*>(p.ck);
  const uint8_t* cv = reinterpret_cast<const uint8_t*>(p.cv);
  // Byte offsets of the 16-key group starting at logical key kg.
  auto kbase = [&](int kg) -> size_t {
    if (local) return (ring * p.window + kg) * D;
    return ((size_t)bt_row[kg >> 4] * p.G + g) * 16 * D;
  };
  auto vbase = [&](int kg, int* dstride) -> size_t {
    if (local) {
      *dstride = p.window;
      return ring * D * p.window + kg;
    }
    *dstride = 16;
    return ((size_t)bt_row[kg >> 4] * p.G + g) * D * 16;
  };
  auto load_step = [&](int kb, Fp8Step& st) {
    {  // K rows: page nn >> 2, slot 4b + (nn & 3), coordinates [32q, 32q+32)
      const int kg = kb + 16 * (nn >> 2);
      if (kg < k1) {
        const uint8_t* kp = ck + kbase(kg) + (size_t)((nn & 3) * D + 32 * q);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          st.k[bb][0] = *reinterpret_cast<const u32x4*>(kp + 4 * bb * D);
          st.k[bb][1] = *reinterpret_cast<const u32x4*>(kp + 4 * bb * D + 16);
        }
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) st.k[bb][0] = st.k[bb][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    {  // V^T rows 16db + nn of page q (16 slots)
      const int kg = kb + 16 * q;
      if (kg < k1) {
        int ds;
        const uint8_t* vp = cv + vbase(kg, &ds) + (size_t)nn * ds;
#pragma unroll
        for (int db = 0; db < 8; ++db)  // non-temporal on global layers (K: each row is read as two halves; plain)
          st.v[db] = local ? *reinterpret_cast<const u32x4*>(vp + (size_t)(16 * db) * ds)
                           : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + (size_t)(16 * db) * ds));
      } else {
#pragma unroll
        for (int db = 0; db < 8; ++db) st.v[db] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;

  Fp8Step cur, nxt;
  if (k0 < k1) load_step(k0, cur);
  for (int kb = k0; kb < k1; kb += 64) {
    const bool has_next = kb + 64 < k1;
    if (has_next) load_step(kb + 64, nxt);
    const bool partial = kb + 64 > k1;

    f32x4 s[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      s[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fp8x8_bf16(cur.k[bb][kk >> 1], kk & 1)),
                                                        as_bf16x8(qf[kk]), s[bb], 0, 0, 0);
    }
    // lane holds head nn, keys kb + 16q + 4b + i
    if (partial) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * q + 4 * bb + i >= k1) s[bb][i] = kNegInf;
    }
    float mt = kNegInf;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[bb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run + kDecRescale)) {
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= alpha;
    }
    const float mu = (m_run == kNegInf) ? 0.f : m_run;
    float e[4][4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[bb][i] = __builtin_amdgcn_exp2f(s[bb][i] - mu);
        l_run += e[bb][i];
      }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // P^T operand: key slot 8q + j <-> page q, slot 8kh + j = S block 2kh + (j >> 2), element j & 3.
      const u32x4 pf = u32x4{pack_bf16x2(e[2 * kh][0], e[2 * kh][1]), pack_bf16x2(e[2 * kh][2], e[2 * kh][3]),
                             pack_bf16x2(e[2 * kh + 1][0], e[2 * kh + 1][1]),
                             pack_bf16x2(e[2 * kh + 1][2], e[2 * kh + 1][3])};
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x4 a = fp8x8_bf16(cur.v[db], kh);
        if (partial) {  // zero V of keys past the end (their slots may hold stale or unwritten codes)
          const int key0 = kb + 16 * q + 8 * kh;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t m = (key0 + 2 * c < k1 ? 0xffffu : 0u) | (key0 + 2 * c + 1 < k1 ? 0xffff0000u : 0u);
            a[c] &= m;
          }
        }
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pf), o[db], 0, 0, 0);
      }
    }
    if (has_next) cur = nxt;
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  store_wave_partials(p, seq, g, sp, hpg, tid, m_run, l_run, o);
}

// Log-sum-exp merge of the splits of one (sequence, query head), then the
// per-coordinate sigmoid gate. A block is SG groups of 128 threads (one per
// coordinate); group sg merges splits sg, sg + SG, ... and the SG partial
// merges are combined through LDS in group order (deterministic, no atomics).
// Each thread keeps eight loads in flight, so a long context (hundreds of
// splits) takes n_splits / (8 SG) memory round trips instead of n_splits / 8.
constexpr int kCombineMaxGroups = 8;

__global__ void __launch_bounds__(128 * kCombineMaxGroups) decode_combine_kernel(CombineParams p) {
  const int seq = blockIdx.x / p.H;
  const int h = blockIdx.x - seq * p.H;
  const int d = threadIdx.x & 127;
  const int sg = threadIdx.x >> 7;
  const int SG = blockDim.x >> 7;
  const int t = p.pos[seq];
  const int cseq = p.seq_idx[seq];
  const size_t idx = ((size_t)seq * p.H + h) * D + d;
  if (t < 0 || t > p.max_pos || cseq < 0 || cseq >= p.n_cache_seqs) {
    if (sg == 0) p.out[idx] = 0x7fc0;  // NaN: the position was outside the decode grid, or the cache row does not exist
    return;
  }
  const int n_keys = p.kind == 0 ? min(t + 1, p.window) : t + 1;
  const int ns = (n_keys + p.split_keys - 1) / p.split_keys;
  const size_t row0 = ((size_t)seq * p.H + h) * p.n_splits;
  float M = kNegInf;
#pragma unroll 8
  for (int s = sg; s < ns; s += SG) M = fmaxf(M, p.part_ml[2 * (row0 + s)]);
  float L = 0.f, A = 0.f;
  if (M != kNegInf) {
#pragma unroll 8
    for (int s = sg; s < ns; s += SG) {
      const float sc = __builtin_amdgcn_exp2f(p.part_ml[2 * (row0 + s)] - M);
      L += sc * p.part_ml[2 * (row0 + s) + 1];
      A += sc * p.part_acc[(row0 + s) * D + d];
    }
  }
  __shared__ float s_m[kCombineMaxGroups], s_l[kCombineMaxGroups], s_a[kCombineMaxGroups][D];
  if (SG > 1) {
    if (d == 0) {
      s_m[sg] = M;
      s_l[sg] = L;
    }
    s_a[sg][d] = A;
    __syncthreads();
    if (sg != 0) return;
    M = kNegInf;
    for (int g = 0; g < SG; ++g) M = fmaxf(M, s_m[g]);
    L = 0.f;
    A = 0.f;
    if (M != kNegInf) {
      for (int g = 0; g < SG; ++g) {
        if (s_m[g] == kNegInf) continue;
        const float sc = __builtin_amdgcn_exp2f(s_m[g] - M);
        L += sc * s_l[g];
        A += sc * s_a[g][d];
      }
    }
  }
  const float o = L > 0.f ? A * __builtin_amdgcn_rcpf(L) * p.v_scale : 0.f;
  const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
  const float gz = bf16f(p.gate[idx]) + bias;
  const float y = o * __builtin_amdgcn_rcpf(1.f + __expf(-gz));
  bf16x2 r;
  r[0] = (__bf16)y;
  p.out[idx] = __builtin_bit_cast(uint16_t, r[0]);
}

hipError_t launch_decode_split(const DecodeParams& p, int n_seqs, hipStream_t s) {
  clear_stale_error();
  const long long blocks = (long long)n_seqs * p.G * p.n_splits;
  const dim3 grid((unsigned)blocks), block(256);
  if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL(decode_split_kernel<0>, grid, block, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL(decode_fp8_kernel<0>, grid, block, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL(decode_split_kernel<1>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(decode_fp8_kernel<1>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const CombineParams& p, int n_seqs, hipStream_t s) {
  clear_stale_error();
  // groups of 128 threads per (sequence, head): about 32 splits per group
  int sg = 1;
  while (sg < kCombineMaxGroups && p.n_splits > 32 * sg) sg *= 2;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(n_seqs * p.H)), dim3(128 * sg), 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
