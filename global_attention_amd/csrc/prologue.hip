// Prologue and KV-append kernels for Beam attention (gfx950).
//
// Per-head RMSNorm of Q and K (eps inside the square root, learned 128-vector),
// then RoPE on local layers or the SSMax scale a(t+1) on global layers, as on
// "Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax", section "Follow the
// tensors, not the parameter label". Q leaves the prologue already multiplied
// by log2(e)/sqrt(d) (and a(t+1) on global layers) so the attention kernels
// work in base-2 logits; this is one bf16 rounding of Q, the same count as
// rounding the normalised Q itself.
//
// Over an FP8 cache the attention kernels work in the cache's code space: the
// chunk's own keys and values go into the workspace divided by k_scale and
// v_scale (one bf16 rounding each), cached ones as their exact codes, and the
// kernels multiply Q' by k_scale and O by v_scale.
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

// ----------------------------------------------------------------------------
// Prefill prologue. Grid (sequence, 64-position tile, part). The tile covers
// absolute positions [64*T, 64*T + 64) with T = (start >> 6) + blockIdx.y.
// Part 0 writes K_hat of the tile and parts 1..2 write V^T (KV heads
// [4(z-1), 4z)) into the position-aligned workspace: the chunk's own positions
// from the projections, the cached positions [start & ~63, start) of its first
// tile copied from the cache (zeros when the cache row is out of range), zeros
// after the chunk end. Attention then reads every tile either wholly from the
// workspace or wholly from the cache. Part z >= 3 writes Q' for query heads
// [8(z-3), 8(z-2)) of the chunk's tokens into [n_tok][H][D].
//
// A 16-lane group owns one position at a time (positions grp, grp+16, ...) and
// handles all of its heads: the position's RoPE cos/sin (local) or SSMax scale
// (global) is formed once, and the group's loads for every head are issued
// before any is used.
// ----------------------------------------------------------------------------
constexpr int kQHeadsPerBlock = 8;
constexpr int kVHeadsPerBlock = 4;
constexpr int kPrologueFixedParts = 3;  // K, V (two halves)
constexpr int kMaxHeadsPerGroup = 8;

// Element offset of the cached K_hat row of position t (paged: block-table
// page; local: ring slot). An FP8 cache uses the same offsets in bytes.
template <int KIND>
__device__ __forceinline__ size_t cache_k_off(const PrologueParams& p, int cseq, int g, int t) {
  if (KIND == 1) {
    const int page = p.bt[(size_t)cseq * p.max_pages + (t >> 4)];
    return (((size_t)page * p.G + g) * 16 + (t & 15)) * D;
  }
  return (((size_t)cseq * p.G + g) * p.window + t % p.window) * D;
}
// Element offset of cached V^T element (0, t); coordinate d is d * stride further.
template <int KIND>
__device__ __forceinline__ size_t cache_v_off(const PrologueParams& p, int cseq, int g, int t, int* stride) {
  if (KIND == 1) {
    const int page = p.bt[(size_t)cseq * p.max_pages + (t >> 4)];
    *stride = 16;
    return ((size_t)page * p.G + g) * D * 16 + (t & 15);
  }
  *stride = p.window;
  return ((size_t)cseq * p.G + g) * D * p.window + t % p.window;
}
template <int KIND, int KV_FP8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) prefill_prologue_kernel(PrologueParams p) {
  constexpr bool local = (KIND == 0);
  const int seq = blockIdx.x;
  const int part = blockIdx.z;
  const int start = p.start_pos[seq];
  const int cu0 = p.cu[seq];
  const int len = p.cu[seq + 1] - cu0;
  const int tile_pos0 = ((start >> 6) + (int)blockIdx.y) * 64;
  if (tile_pos0 >= start + len) return;
  const int region = ws_region_base(cu0, seq);
  const int ws0 = region + tile_pos0 - (start & ~63);  // workspace index of tile_pos0 (multiple of 64)

  const int tid = threadIdx.x;
  const int grp = tid >> 4;  // 16 groups of 16 lanes
  const int j = tid & 15;    // lane within group: coords [4j,4j+4) and [64+4j, 64+4j+4)

  // RoPE frequencies of this lane's pairs 4j..4j+3, in revolutions per
  // position: the block's 64 values are formed once (one float64 pow per
  // thread of the first wave) and shared through LDS.
  double rev_freq[4];
  if (local && part != 1 && part != 2) {
    __shared__ double s_rev[D / 2];
    if (tid < D / 2) s_rev[tid] = rope_rev_per_pos(tid, p.rope_theta);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) rev_freq[e] = s_rev[4 * j + e];
  }

  if (part >= kPrologueFixedParts) {
    // Q': 64 positions x up to 8 heads.
    const int h_lo = (part - kPrologueFixedParts) * kQHeadsPerBlock;
    if (h_lo >= p.H) return;
    const int nh = min(kQHeadsPerBlock, p.H - h_lo);
    const u32x2* qw = reinterpret_cast<const u32x2*>(p.q_norm_w);
    const u32x2 wq_lo = qw[j], wq_hi = qw[16 + j];
    const float qbase = kLog2e / sqrtf((float)D);
    for (int r = grp; r < 64; r += 16) {
      const int t = tile_pos0 + r;
      if (t < start || t >= start + len) continue;
      const size_t tok = (size_t)(cu0 + t - start);
      const u32x2* src = reinterpret_cast<const u32x2*>(p.q_raw + (tok * p.H + h_lo) * D);
      u32x2 xlo[kMaxHeadsPerGroup], xhi[kMaxHeadsPerGroup];
#pragma unroll
      for (int hh = 0; hh < kMaxHeadsPerGroup; ++hh)
        if (hh < nh) {
          xlo[hh] = src[hh * (D / 4) + j];
          xhi[hh] = src[hh * (D / 4) + 16 + j];
        }
      float cs[4], sn[4];
      if (local) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_cs_rev(t, rev_freq[e], &cs[e], &sn[e]);
      }
      const float scale = local ? qbase : qbase * ssmax_scale(t, p.ssmax_base, p.ssmax_exp);
      u32x2* dst = reinterpret_cast<u32x2*>(p.qp + (tok * p.H + h_lo) * D);
#pragma unroll
      for (int hh = 0; hh < kMaxHeadsPerGroup; ++hh)
        if (hh < nh) {
          HeadFrag f = norm_rope_head(xlo[hh], xhi[hh], wq_lo, wq_hi, p.rms_eps, local, cs, sn, scale);
          dst[hh * (D / 4) + j] = u32x2{f.lo[0], f.lo[1]};
          dst[hh * (D / 4) + 16 + j] = u32x2{f.hi[0], f.hi[1]};
        }
    }
    return;
  }

  // Cache row of the sequence, for the cached positions of the first tile.
  const int cseq = p.seq_idx[seq];
  const bool cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (local || ((start + 15) >> 4) <= p.max_pages);
  // Fused append (global layers): chunk positions whose page is in the row.
  const bool append = KIND == 1 && p.append && cseq >= 0 && cseq < p.n_cache_seqs;
  auto append_pos = [&](int t) { return append && t >= start && t < start + len && (t >> 4) < p.max_pages; };

  if (part == 0) {
    // K_hat: 64 positions x G heads into the workspace [G][P][D].
    if (p.G > kMaxHeadsPerGroup) return;  // rejected by the host
    const u32x2* kwgt = reinterpret_cast<const u32x2*>(p.k_norm_w);
    const u32x2 wk_lo = kwgt[j], wk_hi = kwgt[16 + j];
    for (int r = grp; r < 64; r += 16) {
      const int t = tile_pos0 + r;
      u32x2* dst0 = reinterpret_cast<u32x2*>(p.kw + ((size_t)ws0 + r) * D);
      const size_t hstride = (size_t)p.P * (D / 4);  // u32x2 units between heads
      if (t < start && cache_ok) {  // cached K_hat rows, already normalised (and rotated)
        u32x2 clo[kMaxHeadsPerGroup], chi[kMaxHeadsPerGroup];
#pragma unroll
        for (int g = 0; g < kMaxHeadsPerGroup; ++g)
          if (g < p.G) {
            const size_t off = cache_k_off<KIND>(p, cseq, g, t);
            if constexpr (KV_FP8) {  // the codes themselves (code space, exact in bf16)
              const uint8_t* src = reinterpret_cast<const uint8_t*>(p.ck) + off;
              clo[g] = fp8x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(src + 4 * j));
              chi[g] = fp8x4_to_bf16x4(*reinterpret_cast<const uint32_t*>(src + 64 + 4 * j));
            } else {
              const u32x2* src = reinterpret_cast<const u32x2*>(p.ck + off);
              clo[g] = src[j];
              chi[g] = src[16 + j];
            }
          }
#pragma unroll
        for (int g = 0; g < kMaxHeadsPerGroup; ++g)
          if (g < p.G) {
            dst0[g * hstride + j] = clo[g];
            dst0[g * hstride + 16 + j] = chi[g];
          }
        continue;
      }
      if (t < start || t >= start + len) {
        for (int g = 0; g < p.G; ++g) {
          dst0[g * hstride + j] = u32x2{0u, 0u};
          dst0[g * hstride + 16 + j] = u32x2{0u, 0u};
        }
        continue;
      }
      const size_t tok = (size_t)(cu0 + t - start);
      const u32x2* src = reinterpret_cast<const u32x2*>(p.k_raw + tok * p.G * D);
      u32x2 xlo[kMaxHeadsPerGroup], xhi[kMaxHeadsPerGroup];
#pragma unroll
      for (int g = 0; g < kMaxHeadsPerGroup; ++g)
        if (g < p.G) {
          xlo[g] = src[g * (D / 4) + j];
          xhi[g] = src[g * (D / 4) + 16 + j];
        }
      float cs[4], sn[4];
      if (local) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_cs_rev(t, rev_freq[e], &cs[e], &sn[e]);
      }
#pragma unroll
      for (int g = 0; g < kMaxHeadsPerGroup; ++g)
        if (g < p.G) {
          float a[4], bq[4];
          norm_rope_f32(xlo[g], xhi[g], wk_lo, wk_hi, p.rms_eps, local, cs, sn, a, bq);
          const float ks = KV_FP8 ? 1.f / p.k_scale : 1.f;  // code space over an FP8 cache
          const u32x2 flo = u32x2{pack_bf16x2(a[0] * ks, a[1] * ks), pack_bf16x2(a[2] * ks, a[3] * ks)};
          const u32x2 fhi = u32x2{pack_bf16x2(bq[0] * ks, bq[1] * ks), pack_bf16x2(bq[2] * ks, bq[3] * ks)};
          dst0[g * hstride + j] = flo;
          dst0[g * hstride + 16 + j] = fhi;
          if (append_pos(t)) {
            const size_t off = cache_k_off<KIND>(p, cseq, g, t);
            if constexpr (KV_FP8) {
              uint8_t* crow = reinterpret_cast<uint8_t*>(p.ck) + off;
              *reinterpret_cast<uint32_t*>(crow + 4 * j) = fp8x4_encode(a, p.k_scale);
              *reinterpret_cast<uint32_t*>(crow + 64 + 4 * j) = fp8x4_encode(bq, p.k_scale);
            } else {
              u32x2* crow = reinterpret_cast<u32x2*>(p.ck + off);
              crow[j] = flo;
              crow[16 + j] = fhi;
            }
          }
        }
    }
    return;
  }

  // V^T: transpose 64 positions x 128 coords per KV head through LDS into the
  // workspace [G][P/64][D][64] (each 64-position tile contiguous).
  __shared__ uint16_t s_v[64][D + 2];
  const int g_lo = (part - 1) * kVHeadsPerBlock;
  for (int g = g_lo; g < min(g_lo + kVHeadsPerBlock, p.G); ++g) {
    u32x4 v[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {  // 16-byte pieces: row r, coords 8c..8c+7
      const int e = tid + 256 * q4;
      const int r = e >> 4, c = e & 15;
      const int t = tile_pos0 + r;
      v[q4] = u32x4{0u, 0u, 0u, 0u};
      if (t >= start && t < start + len) {
        const size_t tok = (size_t)(cu0 + t - start);
        v[q4] = *reinterpret_cast<const u32x4*>(p.v_raw + (tok * p.G + g) * D + 8 * c);
      } else if (t < start && cache_ok) {  // cached V^T column of position t
        int stride;
        const size_t off = cache_v_off<KIND>(p, cseq, g, t, &stride);
        if constexpr (KV_FP8) {
          const uint8_t* col = reinterpret_cast<const uint8_t*>(p.cv) + off;
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // the codes themselves (code space, exact)
            float f0[4], f1[4];
            fp8x4_to_f32(col[(size_t)(8 * c + 2 * q) * stride], f0);
            fp8x4_to_f32(col[(size_t)(8 * c + 2 * q + 1) * stride], f1);
            v[q4][q] = pack_bf16x2(f0[0], f1[0]);
          }
        } else {
          const uint16_t* col = p.cv + off;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q4][q] = (uint32_t)col[(size_t)(8 * c + 2 * q) * stride] |
                       ((uint32_t)col[(size_t)(8 * c + 2 * q + 1) * stride] << 16);
        }
      }
    }
    __syncthreads();  // the previous head's transposed reads are done
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int e = tid + 256 * q4;
      const int r = e >> 4, c = e & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s_v[r][8 * c + 2 * q] = (uint16_t)(v[q4][q] & 0xffffu);
        s_v[r][8 * c + 2 * q + 1] = (uint16_t)(v[q4][q] >> 16);
      }
    }
    __syncthreads();
    uint16_t* vt = p.vw + (size_t)g * D * p.P + (size_t)(ws0 >> 6) * D * 64;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {  // row d of V^T, keys 8c..8c+7
      const int e = tid + 256 * q4;
      const int d = e >> 3, c = e & 7;
      u32x4 o;
      if constexpr (KV_FP8) {
        // code space: the chunk's own values divided by v_scale; cached ones
        // are codes already
        const float vs = 1.f / p.v_scale;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k0 = 8 * c + 2 * q;
          const float s0 = tile_pos0 + k0 >= start ? vs : 1.f, s1 = tile_pos0 + k0 + 1 >= start ? vs : 1.f;
          o[q] = pack_bf16x2(bf16f(s_v[k0][d]) * s0, bf16f(s_v[k0 + 1][d]) * s1);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = (uint32_t)s_v[8 * c + 2 * q][d] | ((uint32_t)s_v[8 * c + 2 * q + 1][d] << 16);
      }
      *reinterpret_cast<u32x4*>(vt + d * 64 + 8 * c) = o;
    }
    if (append) {
      // V^T into the cache pages of the tile, [page][g][d][16]: 16-byte pieces
      // of 8 positions; pieces at the chunk's edges go element by element.
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int e = tid + 256 * q4;  // (page q, row d, half hf)
        const int q = e >> 8, d = (e >> 1) & 127, hf = e & 1;
        const int r0 = 16 * q + 8 * hf, t0 = tile_pos0 + r0;
        int stride;
        if (append_pos(t0) && append_pos(t0 + 7)) {
          const size_t off = cache_v_off<KIND>(p, cseq, g, t0, &stride) + (size_t)d * 16;
          if constexpr (KV_FP8) {
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; ++k)
              w[k >> 2] |= fp8_e4m3_encode(bf16f(s_v[r0 + k][d]) / p.v_scale) << (8 * (k & 3));
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.cv) + off) = u32x2{w[0], w[1]};
          } else {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              o[k] = (uint32_t)s_v[r0 + 2 * k][d] | ((uint32_t)s_v[r0 + 2 * k + 1][d] << 16);
            *reinterpret_cast<u32x4*>(p.cv + off) = o;
          }
        } else {
          for (int k = 0; k < 8; ++k)
            if (append_pos(t0 + k)) {
              const size_t off = cache_v_off<KIND>(p, cseq, g, t0 + k, &stride) + (size_t)d * 16;
              if constexpr (KV_FP8)
                reinterpret_cast<uint8_t*>(p.cv)[off] = (uint8_t)fp8_e4m3_encode(bf16f(s_v[r0 + k][d]) / p.v_scale);
              else
                p.cv[off] = s_v[r0 + k][d];
            }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// KV append: one 16-lane group per token; the group loops over the KV heads.
// Token -> (cache sequence, position) comes either from explicit arrays (public
// append) or from the prefill chunk description (cu/start/seq_idx).
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) kv_append_kernel(AppendParams p) {
  const int tid = threadIdx.x;
  const int tok = blockIdx.x * 16 + (tid >> 4);
  const int j = tid & 15;
  if (tok >= p.n_tok) return;
  int cseq, t;
  if (p.cu != nullptr) {
    int s = find_seq(p.cu, p.n_seqs, tok);
    int start = p.start_pos[s];
    int len = p.cu[s + 1] - p.cu[s];
    t = start + tok - p.cu[s];
    cseq = p.seq_idx[s];
    // Local ring: only the last `window` positions of the chunk survive; the
    // earlier ones would be overwritten within this same call.
    if (p.kind == 0 && t < start + len - p.window) return;
  } else {
    cseq = p.seq_idx[tok];
    t = p.pos[tok];
  }
  // Out-of-range device indices are dropped rather than written out of bounds.
  if (t < 0 || cseq < 0 || cseq >= p.n_cache_seqs) return;
  if (p.kind == 1 && (t >> 4) >= p.max_pages) return;
  const bool local = (p.kind == 0);
  float cs[4], sn[4];
  if (local) {
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_cs(t, 4 * j + e, p.rope_theta, &cs[e], &sn[e]);
  }
  const u32x2* kwgt = reinterpret_cast<const u32x2*>(p.k_norm_w);
  const u32x2 w_lo = kwgt[j], w_hi = kwgt[16 + j];

  // Every head's K and V first, then the stores: raw K/V and the cache are all
  // bf16 rows, so the compiler would otherwise keep each head's loads behind
  // the previous head's stores (one memory round trip per head).
  u32x2 kl[kMaxKvHeads], kh[kMaxKvHeads], vl[kMaxKvHeads], vh[kMaxKvHeads];
#pragma unroll
  for (int g = 0; g < kMaxKvHeads; ++g) {
    if (g >= p.G) break;
    const u32x2* ks = reinterpret_cast<const u32x2*>(p.k_raw + ((size_t)tok * p.G + g) * D);
    const u32x2* vs = reinterpret_cast<const u32x2*>(p.v_raw + ((size_t)tok * p.G + g) * D);
    kl[g] = ks[j];
    kh[g] = ks[16 + j];
    vl[g] = vs[j];       // V coordinates 4j .. 4j+3
    vh[g] = vs[16 + j];  // 64 + 4j .. 64 + 4j+3
  }
  const int page = local ? 0 : p.bt[(size_t)cseq * p.max_pages + (t >> 4)];

#pragma unroll
  for (int g = 0; g < kMaxKvHeads; ++g) {
    if (g >= p.G) break;
    size_t krow;  // element offset of the K_hat row
    size_t vcol;  // element offset of V^T element [0][slot]; coordinate d is at vcol + d * vstride
    int vstride;
    if (local) {
      int slot = t % p.window;
      size_t base = (size_t)cseq * p.G + g;
      krow = (base * p.window + slot) * D;
      vcol = base * D * p.window + slot;
      vstride = p.window;
    } else {
      size_t base = (size_t)page * p.G + g;
      krow = (base * 16 + (t & 15)) * D;
      vcol = base * D * 16 + (t & 15);
      vstride = 16;
    }
    const uint16_t vlo[4] = {(uint16_t)vl[g][0], (uint16_t)(vl[g][0] >> 16), (uint16_t)vl[g][1],
                             (uint16_t)(vl[g][1] >> 16)};
    const uint16_t vhi[4] = {(uint16_t)vh[g][0], (uint16_t)(vh[g][0] >> 16), (uint16_t)vh[g][1],
                             (uint16_t)(vh[g][1] >> 16)};
    if (p.kv_fp8) {
      float a[4], b[4];
      norm_rope_f32(kl[g], kh[g], w_lo, w_hi, p.rms_eps, local, cs, sn, a, b);
      uint8_t* k8 = reinterpret_cast<uint8_t*>(p.ck) + krow;
      *reinterpret_cast<uint32_t*>(k8 + 4 * j) = fp8x4_encode(a, p.k_scale);
      *reinterpret_cast<uint32_t*>(k8 + 64 + 4 * j) = fp8x4_encode(b, p.k_scale);
      uint8_t* v8 = reinterpret_cast<uint8_t*>(p.cv) + vcol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v8[(size_t)(4 * j + e) * vstride] = (uint8_t)fp8_e4m3_encode(bf16f(vlo[e]) / p.v_scale);
        v8[(size_t)(64 + 4 * j + e) * vstride] = (uint8_t)fp8_e4m3_encode(bf16f(vhi[e]) / p.v_scale);
      }
      continue;
    }
    HeadFrag f = norm_rope_head(kl[g], kh[g], w_lo, w_hi, p.rms_eps, local, cs, sn, 1.0f);
    reinterpret_cast<u32x2*>(p.ck + krow)[j] = u32x2{f.lo[0], f.lo[1]};
    reinterpret_cast<u32x2*>(p.ck + krow)[16 + j] = u32x2{f.hi[0], f.hi[1]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p.cv[vcol + (size_t)(4 * j + e) * vstride] = vlo[e];
      p.cv[vcol + (size_t)(64 + 4 * j + e) * vstride] = vhi[e];
    }
  }
}

// ----------------------------------------------------------------------------
// Decode prologue: Q' for one new token per sequence, one 16-lane group per
// (sequence, head).
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_q_prologue_kernel(DecodeQParams p) {
  const int tid = threadIdx.x;
  const int pr = blockIdx.x * 16 + (tid >> 4);
  const int j = tid & 15;
  if (pr >= p.n_seqs * p.H) return;
  const int seq = pr / p.H;
  const int h = pr - seq * p.H;
  const int t = p.pos[seq];
  const bool local = (p.kind == 0);
  float cs[4], sn[4];
  if (local) {
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_cs(t, 4 * j + e, p.rope_theta, &cs[e], &sn[e]);
  }
  const u32x2* qw = reinterpret_cast<const u32x2*>(p.q_norm_w);
  const float qbase = kLog2e / sqrtf((float)D);
  float scale = (local ? qbase : qbase * ssmax_scale(t, p.ssmax_base, p.ssmax_exp)) * p.k_scale;
  const u32x2* src = reinterpret_cast<const u32x2*>(p.q_raw + ((size_t)seq * p.H + h) * D);
  HeadFrag f = norm_rope_head(src[j], src[16 + j], qw[j], qw[16 + j], p.rms_eps, local, cs, sn, scale);
  u32x2* dst = reinterpret_cast<u32x2*>(p.qp + ((size_t)seq * p.H + h) * D);
  dst[j] = u32x2{f.lo[0], f.lo[1]};
  dst[16 + j] = u32x2{f.hi[0], f.hi[1]};
}

// ----------------------------------------------------------------------------
// Visibility mask with the kernels' own predicate (debug entry point).
// ----------------------------------------------------------------------------
__global__ void visibility_kernel(int kind, int window, int t0, int n_q, int s0, int n_k,
                                  uint8_t* mask) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n_q * n_k) return;
  int r = (int)(i / n_k), c = (int)(i - (long long)r * n_k);
  mask[i] = visible(kind, window, t0 + r, s0 + c) ? 1 : 0;
}

// ----------------------------------------------------------------------------
// Block-table check of a paged cache (debug entry point): one block per cache
// sequence counts the entries of its used range that name no physical page.
// Only the ids are compared; no page is read.
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) validate_cache_kernel(const int32_t* bt, int max_pages, int n_pages,
                                                             int page_size, const int32_t* n_tokens,
                                                             int32_t* n_bad) {
  const int c = blockIdx.x;
  int used = max_pages;
  if (n_tokens) {
    const long long nt = n_tokens[c];
    const long long np = (nt + page_size - 1) / page_size;
    if (nt < 0 || np > max_pages) {
      if (threadIdx.x == 0) n_bad[c] = -1;  // the length itself does not fit the row
      return;
    }
    used = (int)np;
  }
  const int32_t* row = bt + (size_t)c * max_pages;
  int cnt = 0;
  for (int i = threadIdx.x; i < used; i += 256) {
    const int pg = row[i];
    cnt += (pg < 0 || pg >= n_pages) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  __shared__ int s_cnt[4];
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) n_bad[c] = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
}

}  // namespace beam

namespace beam {

hipError_t launch_validate_cache(const int32_t* bt, int max_pages, int n_pages, int page_size, int n_seqs,
                                 const int32_t* n_tokens, int32_t* n_bad, hipStream_t s) {
  clear_stale_error();
  hipLaunchKernelGGL(validate_cache_kernel, dim3((unsigned)n_seqs), dim3(256), 0, s, bt, max_pages, n_pages,
                     page_size, n_tokens, n_bad);
  return hipGetLastError();
}

hipError_t launch_prefill_prologue(const PrologueParams& p, int n_seqs, int n_tiles, hipStream_t s) {
  clear_stale_error();
  const int parts = kPrologueFixedParts + (p.with_q ? (p.H + kQHeadsPerBlock - 1) / kQHeadsPerBlock : 0);
  if (p.G > kMaxHeadsPerGroup || p.G > 2 * kVHeadsPerBlock) return hipErrorInvalidValue;
  const dim3 grid(n_seqs, n_tiles, parts), block(256);
  if (p.kind == 0 && !p.kv_fp8)
    hipLaunchKernelGGL((prefill_prologue_kernel<0, 0>), grid, block, 0, s, p);
  else if (p.kind == 0)
    hipLaunchKernelGGL((prefill_prologue_kernel<0, 1>), grid, block, 0, s, p);
  else if (!p.kv_fp8)
    hipLaunchKernelGGL((prefill_prologue_kernel<1, 0>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((prefill_prologue_kernel<1, 1>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
  clear_stale_error();
  hipLaunchKernelGGL(kv_append_kernel, dim3((p.n_tok + 15) / 16), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_q_prologue(const DecodeQParams& p, hipStream_t s) {
  clear_stale_error();
  hipLaunchKernelGGL(decode_q_prologue_kernel, dim3((p.n_seqs * p.H + 15) / 16), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_visibility(int kind, int window, int t0, int n_q, int s0, int n_k, uint8_t* mask,
                             hipStream_t s) {
  clear_stale_error();
  long long n = (long long)n_q * n_k;
  hipLaunchKernelGGL(visibility_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kind,
                     window, t0, n_q, s0, n_k, mask);
  return hipGetLastError();
}

}  // namespace beam
