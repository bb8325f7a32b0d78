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
// Block = 4 wavefronts = 128 queries of one query head; KV tiles of 64 keys are
// staged through LDS (double-buffered). Each wave owns 32 queries and computes
// S^T = K Q'^T with v_mfma_f32_32x32x16_bf16 (keys on M, queries on N), so each
// lane holds one query column and a row max needs a single cross-half swap.
// P^T is fed straight from the S accumulators into O^T += V^T P^T; V^T is kept
// in LDS with the key order permuted inside each 16-key group to match the
// accumulator layout. Softmax runs in base 2 (Q' carries log2 e / sqrt d and,
// on global layers, a(t+1)); the running max is only moved when it grows by
// more than 8 (exact: the final normalisation uses the same reference).
// Local layers visit only the key tiles that intersect the window.
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

constexpr int BM = 128;       // queries per block
constexpr int BN = 64;        // keys per tile
constexpr int KROW = D + 8;   // LDS row of K (bf16): 272 B, conflict-free b128 reads
constexpr int VROW = BN + 8;  // LDS row of V^T (bf16): 144 B
constexpr int K_TILE = BN * KROW;
constexpr int V_TILE = D * VROW;
constexpr float kRescaleThreshold = 8.0f;

struct KeySource {
  const uint16_t* kw;
  const uint16_t* vw;
  const uint16_t* ck;
  const uint16_t* cv;
  const int32_t* bt_row;  // block-table row of the cache sequence (global)
  int start;              // first chunk position; keys below it come from the cache
  int cache_ok;           // the cache sequence index is in range
  int ws_off;             // workspace index = s + ws_off
  int g, G, P, kind, window;
  size_t ring_base;       // (cseq*G + g) for the local ring
};

// 16 bytes of K row s, coordinates [8c, 8c+8).
__device__ __forceinline__ u32x4 load_k_piece(const KeySource& ks, int s, int c) {
  const uint16_t* src;
  if (s >= ks.start) {
    src = ks.kw + ((size_t)ks.g * ks.P + (s + ks.ws_off)) * D;
  } else if (!ks.cache_ok) {
    return u32x4{0u, 0u, 0u, 0u};
  } else if (ks.kind == 1) {
    int page = ks.bt_row[s >> 4];
    src = ks.ck + (((size_t)page * ks.G + ks.g) * 16 + (s & 15)) * D;
  } else {
    src = ks.ck + (ks.ring_base * ks.window + (s % ks.window)) * D;
  }
  return *reinterpret_cast<const u32x4*>(src + 8 * c);
}

__device__ __forceinline__ uint16_t load_v_elem(const KeySource& ks, int d, int s) {
  if (s >= ks.start) return ks.vw[((size_t)ks.g * D + d) * ks.P + (s + ks.ws_off)];
  if (!ks.cache_ok) return 0;
  if (ks.kind == 1) {
    int page = ks.bt_row[s >> 4];
    return ks.cv[(((size_t)page * ks.G + ks.g) * D + d) * 16 + (s & 15)];
  }
  return ks.cv[(ks.ring_base * D + d) * ks.window + (s % ks.window)];
}

// 8 consecutive V^T values: row d, keys [s8, s8+8) (s8 a multiple of 8).
__device__ __forceinline__ u32x4 load_v_piece(const KeySource& ks, int d, int s8) {
  if (s8 >= ks.start) {
    return *reinterpret_cast<const u32x4*>(ks.vw + ((size_t)ks.g * D + d) * ks.P + (s8 + ks.ws_off));
  }
  if (s8 + 8 <= ks.start) {
    if (!ks.cache_ok) return u32x4{0u, 0u, 0u, 0u};
    const uint16_t* src;
    if (ks.kind == 1) {
      int page = ks.bt_row[s8 >> 4];
      src = ks.cv + (((size_t)page * ks.G + ks.g) * D + d) * 16 + (s8 & 15);
    } else {
      src = ks.cv + (ks.ring_base * D + d) * ks.window + (s8 % ks.window);
    }
    return *reinterpret_cast<const u32x4*>(src);
  }
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = (uint32_t)load_v_elem(ks, d, s8 + 2 * q) | ((uint32_t)load_v_elem(ks, d, s8 + 2 * q + 1) << 16);
  return r;
}

__device__ __forceinline__ void load_tile(const KeySource& ks, int key0, int tid, u32x4 (&kr)[4],
                                          u32x4 (&vr)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int id = tid + 256 * r;
    kr[r] = load_k_piece(ks, key0 + (id >> 4), id & 15);
    vr[r] = load_v_piece(ks, id >> 3, key0 + 8 * (id & 7));
  }
}

__device__ __forceinline__ void store_tile(uint16_t* sK, uint16_t* sV, int tid, const u32x4 (&kr)[4],
                                           const u32x4 (&vr)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int id = tid + 256 * r;
    *reinterpret_cast<u32x4*>(sK + (id >> 4) * KROW + 8 * (id & 15)) = kr[r];
    // keys 8c+0..3 -> positions 16(c>>1) + 4(c&1) + 0..3, keys 8c+4..7 -> +8
    int d = id >> 3, c = id & 7;
    uint16_t* dst = sV + d * VROW + 16 * (c >> 1) + 4 * (c & 1);
    *reinterpret_cast<u32x2*>(dst) = u32x2{vr[r][0], vr[r][1]};
    *reinterpret_cast<u32x2*>(dst + 8) = u32x2{vr[r][2], vr[r][3]};
  }
}

template <int KIND>
__global__ void __launch_bounds__(256, 2) prefill_attn_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (K_TILE + V_TILE)];

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
  const int w = tid >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;

  const int q0 = start + qt * BM;                   // first query position of the block
  const int qlast = min(q0 + BM, start + len) - 1;  // last valid query position
  const int wq_lo = q0 + 32 * w;
  const int wq_hi = min(wq_lo + 31, qlast);
  const bool wave_active = wq_lo <= qlast;
  const int t = wq_lo + n;  // this lane's query position
  const bool row_valid = t <= qlast;

  KeySource ks;
  ks.kw = p.kw;
  ks.vw = p.vw;
  ks.ck = p.ck;
  ks.cv = p.cv;
  ks.bt_row = KIND == 1 ? p.bt + (size_t)cseq * p.max_pages : nullptr;
  ks.start = start;
  // The cached prefix must fit the cache sequence's block-table row (global).
  ks.cache_ok = cseq >= 0 && cseq < p.n_cache_seqs && (KIND == 0 || ((start + 15) >> 4) <= p.max_pages);
  ks.ws_off = ws_region_base(cu0, seq) - (start & ~63);
  ks.g = g;
  ks.G = p.G;
  ks.P = p.P;
  ks.kind = KIND;
  ks.window = W;
  ks.ring_base = (size_t)cseq * p.G + g;

  // Q' fragments (B operand of S^T = K Q'^T): lane holds query n, coords 16kk + 8*half + 0..7.
  u32x4 qf[8];
  {
    const size_t tok = (size_t)(cu0 + (t - start));
    const uint16_t* qrow = p.qp + (tok * p.H + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = row_valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  const int kmin = local ? max(0, q0 - (W - 1)) : 0;
  const int j_lo = kmin >> 6;
  const int j_hi = qlast >> 6;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;

  u32x4 kr[4], vr[4];
  load_tile(ks, j_lo * BN, tid, kr, vr);
  store_tile(smem, smem + 2 * K_TILE, tid, kr, vr);
  __syncthreads();

  for (int jt = j_lo; jt <= j_hi; ++jt) {
    const int buf = (jt - j_lo) & 1;
    const uint16_t* sK = smem + buf * K_TILE;
    const uint16_t* sV = smem + 2 * K_TILE + buf * V_TILE;
    const bool has_next = jt < j_hi;
    if (has_next) load_tile(ks, (jt + 1) * BN, tid, kr, vr);

    const int ks0 = jt * BN;
    const bool skip = !wave_active || ks0 > wq_hi || (local && ks0 + BN - 1 < wq_lo - (W - 1));
    if (!skip) {
      // S^T tile: keys 32mb + (lane&31) on M, queries on N.
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          u32x4 a = *reinterpret_cast<const u32x4*>(sK + (32 * mb + n) * KROW + 16 * kk + 8 * half);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qf[kk]), s[mb], 0, 0, 0);
        }
      }
      const bool need_mask = (ks0 + BN - 1 > wq_lo) || (local && ks0 < wq_hi - (W - 1));
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            int sk = ks0 + 32 * mb + 8 * (i >> 2) + 4 * half + (i & 3);
            if (!visible(KIND, W, t, sk)) s[mb][i] = kNegInf;
          }
      }
      float mt = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[mb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      if (__any(m_new > m_run + kRescaleThreshold)) {
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      const float mu = (m_run == kNegInf) ? 0.f : m_run;
      u32x4 pf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float e[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          e[jj] = __builtin_amdgcn_exp2f(s[kb >> 1][8 * (kb & 1) + jj] - mu);
          l_run += e[jj];
        }
        pf[kb] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                       pack_bf16x2(e[6], e[7])};
      }
      // O^T += V^T P^T over the 4 key blocks of 16.
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          u32x4 a = *reinterpret_cast<const u32x4*>(sV + (32 * db + n) * VROW + 16 * kb + 8 * half);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pf[kb]), o[db], 0, 0, 0);
        }
      }
    }

    if (has_next) {
      store_tile(smem + (buf ^ 1) * K_TILE, smem + 2 * K_TILE + (buf ^ 1) * V_TILE, tid, kr, vr);
    }
    __syncthreads();
  }

  // Epilogue: normalise, gate, write bf16. Lane holds query n and coordinates
  // d = 32db + 8a + 4*half + 0..3.
  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float bias = p.gate_bias ? p.gate_bias[h] : 0.f;
  const size_t tok = (size_t)(cu0 + (t - start));
  const uint16_t* grow = p.gate + (tok * p.H + h) * D;
  uint16_t* orow = p.out + (tok * p.H + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * db + 8 * a + 4 * half;
      u32x2 gv = *reinterpret_cast<const u32x2*>(grow + d0);
      float gz[4] = {bf16lo(gv[0]), bf16hi(gv[0]), bf16lo(gv[1]), bf16hi(gv[1])};
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sg = 1.f / (1.f + __expf(-(gz[e] + bias)));
        y[e] = o[db][4 * a + e] * inv * sg;
      }
      *reinterpret_cast<u32x2*>(orow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    }
  }
}

hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  const long long blocks = (long long)p.G * (p.H / p.G) * p.n_seqs * p.n_qtiles;
  if (p.kind == 0)
    hipLaunchKernelGGL(prefill_attn_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_attn_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
