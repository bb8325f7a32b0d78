// Group-limited sigmoid router of Beam 1.0's MoE layers (gfx950).
//
// Per token ("Beam 1.0: Local RoPE, Global NoPE and Scalable Softmax",
// section "The surrounding model and serving boundary"; techfi24.com,
// "Architecture et mécanismes d'inférence"; news.hamidun.com, the MoE
// paragraph):
//   z_e = x . W_e in fp32 over the hidden width, s_e = sigmoid(z_e) (the
//   float32 value nearest to it), c_e = s_e + b_e (used only to choose);
//   each of 8 groups of 32 experts scores the sum of its two largest c;
//   the best topk_groups groups are kept; the top_k experts by c inside them
//   are chosen (ties to the lower index, reported best first); their weights
//   are s / (sum of the chosen s) * scale.
//
// The logits are a dense contraction and run on fp32 MFMA
// (v_mfma_f32_32x32x2f32): a block of 8 waves computes 128 tokens x 256
// experts, a wave 64 x 64 (2 x 2 output blocks). The contraction order is
// free, so lane half h takes k = k0 + 16h + p in MFMA step p of a 32-wide
// chunk: each lane then reads 16 consecutive x values (32 bytes) and 16
// consecutive W values (64 bytes) per chunk straight from memory, no LDS on
// the GEMM path. All blocks walk k in the same order, so the W chunk every
// block needs at a time is shared through L2. The fused kernel keeps the
// logits in LDS and routes each token with a quad of four lanes (lane
// quarter q holds experts 64q .. 64q+63, i.e. groups 2q and 2q+1), so the
// 512 lanes of a block route its 128 tokens at once and every exchange is a
// DPP move inside the quad.
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

namespace {

// LDS row of the fused kernel: expert e at column e + e/64, pitch 260 floats.
// A quad's reads (token tl, quarter q, expert 64q + j) then fall on bank
// 4 tl + q + j (mod 64): the 64 lanes of a wave hit 64 different banks.
constexpr int kLogPitch = 260;

struct RtChunk {
  u32x4 a[2][2];  // [row block][16-byte piece]: 16 bf16 of x
  f32x4 b[2][4];  // [column block][16-byte piece]: 16 floats of W
};

// Exchange within a quad of lanes (DPP quad_perm, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float quad_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int quad_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int quad_bcast(int i) { return i * 0x55; }  // quad_perm [i,i,i,i]

// Route one token with the four lanes of a quad. Lane quarter q holds the
// logits z[j] of experts 64q + j (groups 2q and 2q + 1) and their bias. The
// quad swaps group scores, each lane keeps a sorted list of its best
// top_k candidates in the kept groups, and top_k rounds of a quad-wide
// argmax (score, then lower expert index) merge the four lists. Lane q == 0
// writes the chosen experts and weights, best first.
__device__ __forceinline__ void route_token_quad(const float (&z)[64], const float (&bias)[64], int q,
                                                 int topk_groups, int top_k, float scale, int32_t* idx_out,
                                                 float* w_out) {
  float s[64], c[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    s[j] = (float)(1.0 / (1.0 + exp(-(double)z[j])));  // nearest float32 of the sigmoid
    c[j] = s[j] + bias[j];
  }
  // Scores of this lane's two groups: largest + second largest corrected score.
  float gl[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float m1 = kNegInf, m2 = kNegInf;
#pragma unroll
    for (int j = 32 * half; j < 32 * half + 32; ++j) {
      m2 = fmaxf(m2, fminf(m1, c[j]));
      m1 = fmaxf(m1, c[j]);
    }
    gl[half] = m1 + m2;
  }
  float G[kRouterGroups];
  G[0] = quad_f<quad_bcast(0)>(gl[0]);
  G[1] = quad_f<quad_bcast(0)>(gl[1]);
  G[2] = quad_f<quad_bcast(1)>(gl[0]);
  G[3] = quad_f<quad_bcast(1)>(gl[1]);
  G[4] = quad_f<quad_bcast(2)>(gl[0]);
  G[5] = quad_f<quad_bcast(2)>(gl[1]);
  G[6] = quad_f<quad_bcast(3)>(gl[0]);
  G[7] = quad_f<quad_bcast(3)>(gl[1]);
  // Kept groups: rank below topk_groups (ties to the lower group).
  bool keep[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int g = 2 * q + half;
    const float gv = half ? gl[1] : gl[0];
    int rank = 0;
#pragma unroll
    for (int o = 0; o < kRouterGroups; ++o) rank += (G[o] > gv) || (G[o] == gv && o < g);
    keep[half] = rank < topk_groups;
  }

  // This lane's best candidates, sorted by score then lower index. Experts
  // arrive in index order, so a new one goes in front of the first strictly
  // smaller entry, and from there on every entry moves down one slot.
  // Entries past the lane's candidates stay at -inf, index -1.
  float tv[kRouterTopKMax], ts[kRouterTopKMax];
  int te[kRouterTopKMax];
#pragma unroll
  for (int k = 0; k < kRouterTopKMax; ++k) {
    tv[k] = kNegInf;
    ts[k] = 0.f;
    te[k] = -1;
  }
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    float v = keep[j >> 5] ? c[j] : kNegInf, sv = s[j];
    int ev = 64 * q + j;
    bool moved = false;
#pragma unroll
    for (int k = 0; k < kRouterTopKMax; ++k) {
      const bool gt = moved || v > tv[k];
      moved = gt;
      const float t0 = tv[k], t1 = ts[k];
      const int t2 = te[k];
      tv[k] = gt ? v : t0;
      ts[k] = gt ? sv : t1;
      te[k] = gt ? ev : t2;
      v = gt ? t0 : v;
      sv = gt ? t1 : sv;
      ev = gt ? t2 : ev;
    }
  }

  // Merge: the kept groups hold at least 32 >= top_k candidates, so every
  // round's winner is a real expert (index >= 0).
  int sel_e[kRouterTopKMax];
  float sel_s[kRouterTopKMax], sum = 0.f;
#pragma unroll
  for (int k = 0; k < kRouterTopKMax; ++k) {
    sel_e[k] = 0;
    sel_s[k] = 0.f;
    if (k < top_k) {
      float v = tv[0], sv = ts[0];
      int ev = te[0];
      {
        const float ov = quad_f<kQuadXor1>(v), osv = quad_f<kQuadXor1>(sv);
        const int oev = quad_i<kQuadXor1>(ev);
        const bool take = ov > v || (ov == v && oev < ev);
        v = take ? ov : v;
        sv = take ? osv : sv;
        ev = take ? oev : ev;
      }
      {
        const float ov = quad_f<kQuadXor2>(v), osv = quad_f<kQuadXor2>(sv);
        const int oev = quad_i<kQuadXor2>(ev);
        const bool take = ov > v || (ov == v && oev < ev);
        v = take ? ov : v;
        sv = take ? osv : sv;
        ev = take ? oev : ev;
      }
      const bool mine = te[0] == ev;  // the winner's lane drops its head
#pragma unroll
      for (int i = 0; i < kRouterTopKMax; ++i) {
        const float nv = i + 1 < kRouterTopKMax ? tv[i + 1] : kNegInf;
        const float ns = i + 1 < kRouterTopKMax ? ts[i + 1] : 0.f;
        const int ne = i + 1 < kRouterTopKMax ? te[i + 1] : -1;
        tv[i] = mine ? nv : tv[i];
        ts[i] = mine ? ns : ts[i];
        te[i] = mine ? ne : te[i];
      }
      sel_e[k] = ev;
      sel_s[k] = sv;
      sum += sv;
    }
  }
  if (q == 0) {
#pragma unroll
    for (int k = 0; k < kRouterTopKMax; ++k)
      if (k < top_k) {
        idx_out[k] = sel_e[k];
        w_out[k] = sel_s[k] / sum * scale;
      }
  }
}

// Bias of experts 64q .. 64q+63 (zero without a bias).
__device__ __forceinline__ void load_bias_quarter(const float* bias, int q, float (&b)[64]) {
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const f32x4 v = bias ? *reinterpret_cast<const f32x4*>(bias + 64 * q + j) : f32x4{0.f, 0.f, 0.f, 0.f};
    b[j] = v[0];
    b[j + 1] = v[1];
    b[j + 2] = v[2];
    b[j + 3] = v[3];
  }
}

}  // namespace

template <bool FUSED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) router_gemm_kernel(RouterParams p) {
  __shared__ float s_log[FUSED ? kRouterBlockTokens * kLogPitch : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = w >> 2, we = w & 3;  // token half, expert quarter
  const int r = lane & 31, h = lane >> 5;
  const int blk0 = blockIdx.x * kRouterBlockTokens;
  const int tok0 = blk0 + 64 * wt;

  const uint16_t* xa[2];
  bool va[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int t = tok0 + 32 * mb + r;
    va[mb] = t < p.n_tok;
    xa[mb] = p.x + (size_t)(va[mb] ? t : 0) * p.hidden + 16 * h;
  }
  const float* wb[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) wb[nb] = p.w + (size_t)(64 * we + 32 * nb + r) * p.hidden + 16 * h;

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  auto load = [&](int k0, RtChunk& c) __attribute__((always_inline)) {
    // Loads are unconditional (rows past n_tok read row 0 and are zeroed at
    // use): a load under a branch makes the compiler wait for every load in
    // flight at the merge, which would serialise the prefetch with the MFMAs.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 2; ++q) c.a[mb][q] = *reinterpret_cast<const u32x4*>(xa[mb] + k0 + 8 * q);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) c.b[nb][q] = *reinterpret_cast<const f32x4*>(wb[nb] + k0 + 4 * q);
  };
  // MFMA step pp: A[i][kslot h] = x[row i][k0 + 16h + pp], B[kslot h][j] = W[col j][k0 + 16h + pp].
  auto compute = [&](const RtChunk& c) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) {
      float av[2], bv[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint32_t word = c.a[mb][pp >> 3][(pp >> 1) & 3];
        av[mb] = va[mb] ? ((pp & 1) ? bf16hi(word) : bf16lo(word)) : 0.f;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bv[nb] = c.b[nb][pp >> 2][pp & 3];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  // Chunks alternate between c0 and c1, each loaded one chunk ahead; past the
  // end the offset is clamped to the last chunk (a reload nobody computes).
  const int k_last = p.hidden - kRouterKChunk;
  RtChunk c0, c1;
  load(0, c0);
  // The scheduling barriers keep each chunk's loads ahead of the previous
  // chunk's MFMAs (left alone, the scheduler sinks them next to their uses).
  for (int k0 = 0; k0 < p.hidden; k0 += 2 * kRouterKChunk) {
    load(min(k0 + kRouterKChunk, k_last), c1);
    __builtin_amdgcn_sched_barrier(0);
    compute(c0);
    __builtin_amdgcn_sched_barrier(0);
    load(min(k0 + 2 * kRouterKChunk, k_last), c0);
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + kRouterKChunk < p.hidden) compute(c1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Output element i of block (mb, nb): token 32mb + 8(i>>2) + 4h + (i&3),
  // expert 64we + 32nb + r.
  if constexpr (!FUSED) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tok0 + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
        if (t < p.n_tok) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            p.logits_out[(size_t)t * kRouterExperts + 64 * we + 32 * nb + r] = acc[mb][nb][i];
        }
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = 64 * wt + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) s_log[tl * kLogPitch + 65 * we + 32 * nb + r] = acc[mb][nb][i];
      }
    __syncthreads();
    const int tl = tid >> 2, q = tid & 3;
    const int t = blk0 + tl;
    if (t < p.n_tok) {
      float z[64], bias[64];
#pragma unroll
      for (int j = 0; j < 64; ++j) z[j] = s_log[tl * kLogPitch + 65 * q + j];
      load_bias_quarter(p.bias, q, bias);
      route_token_quad(z, bias, q, p.topk_groups, p.top_k, p.scale, p.idx + (size_t)t * p.top_k,
                       p.wts + (size_t)t * p.top_k);
    }
  }
}

// One quad of lanes per token over fp32 logits [n_tok][256]: 64 tokens per
// block of 256 lanes, each lane reading 256 contiguous bytes.
__global__ void __launch_bounds__(256) router_select_kernel(RouterParams p) {
  const int q = threadIdx.x & 3;
  const int t = blockIdx.x * 64 + (threadIdx.x >> 2);
  if (t >= p.n_tok) return;
  float z[64], bias[64];
  const float* row = p.logits_in + (size_t)t * kRouterExperts + 64 * q;
#pragma unroll
  for (int j = 0; j < 64; j += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + j);
    z[j] = v[0];
    z[j + 1] = v[1];
    z[j + 2] = v[2];
    z[j + 3] = v[3];
  }
  load_bias_quarter(p.bias, q, bias);
  route_token_quad(z, bias, q, p.topk_groups, p.top_k, p.scale, p.idx + (size_t)t * p.top_k,
                   p.wts + (size_t)t * p.top_k);
}

hipError_t launch_router_logits(const RouterParams& p, hipStream_t s) {
  clear_stale_error();
  const unsigned blocks = (unsigned)((p.n_tok + kRouterBlockTokens - 1) / kRouterBlockTokens);
  hipLaunchKernelGGL(router_gemm_kernel<false>, dim3(blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_router_fused(const RouterParams& p, hipStream_t s) {
  clear_stale_error();
  const unsigned blocks = (unsigned)((p.n_tok + kRouterBlockTokens - 1) / kRouterBlockTokens);
  hipLaunchKernelGGL(router_gemm_kernel<true>, dim3(blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_router_select(const RouterParams& p, hipStream_t s) {
  clear_stale_error();
  hipLaunchKernelGGL(router_select_kernel, dim3((unsigned)((p.n_tok + 63) / 64)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
