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
// logits in LDS and routes each token with one wavefront (lane l holds
// experts l, l+64, l+128, l+192, i.e. groups 2j + (l>>5)).
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

namespace {

constexpr int kLogStride = kRouterExperts + 1;  // LDS row pitch of the fused kernel (floats)

struct RtChunk {
  u32x4 a[2][2];  // [row block][16-byte piece]: 16 bf16 of x
  f32x4 b[2][4];  // [column block][16-byte piece]: 16 floats of W
};

// Route one token; z and bias hold this lane's experts lane + 64j. Lanes
// 0 .. top_k-1 write the chosen expert and weight of their rank.
__device__ __forceinline__ void route_token(const float (&z)[4], const float (&bias)[4], int lane, int topk_groups,
                                            int top_k, float scale, int32_t* idx_out, float* w_out) {
  const int h = lane >> 5;
  float s[4], c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s[j] = (float)(1.0 / (1.0 + exp(-(double)z[j])));  // nearest float32 of the sigmoid
    c[j] = s[j] + bias[j];
  }
  // Group scores: the two largest c among the 32 lanes of a half, per j.
  float G[kRouterGroups];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m1 = c[j], m2 = kNegInf;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float o1 = __shfl_xor(m1, off), o2 = __shfl_xor(m2, off);
      const float lo = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
      m1 = fmaxf(m1, o1);
      m2 = lo;
    }
    const float gs = m1 + m2;                // group 2j + h
    const float go = __shfl_xor(gs, 32);     // group 2j + 1 - h
    G[2 * j] = h ? go : gs;
    G[2 * j + 1] = h ? gs : go;
  }
  // Kept groups: rank below topk_groups (ties to the lower group).
  unsigned keep = 0;
#pragma unroll
  for (int g = 0; g < kRouterGroups; ++g) {
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kRouterGroups; ++q) rank += (G[q] > G[g]) || (G[q] == G[g] && q < g);
    keep |= (unsigned)(rank < topk_groups) << g;
  }
  float cand[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cand[j] = ((keep >> (2 * j + h)) & 1u) ? c[j] : kNegInf;

  // top_k rounds of a wave-wide argmax (value, then lower expert index).
  float sel_s = 0.f, sum = 0.f;
  int sel_e = 0;
  for (int k = 0; k < top_k; ++k) {
    float bv = cand[0];
    int bj = 0;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (cand[j] > bv) {
        bv = cand[j];
        bj = j;
      }
    int be = lane + 64 * bj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    const int wj = be >> 6, owner = be & 63;
    const float mine = wj == 0 ? s[0] : wj == 1 ? s[1] : wj == 2 ? s[2] : s[3];
    const float ws = __shfl(mine, owner);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j == wj && lane == owner) cand[j] = kNegInf;
    sum += ws;
    if (lane == k) {
      sel_s = ws;
      sel_e = be;
    }
  }
  if (lane < top_k) {
    idx_out[lane] = sel_e;
    w_out[lane] = sel_s / sum * scale;
  }
}

}  // namespace

template <bool FUSED>
__global__ void __launch_bounds__(512) router_gemm_kernel(RouterParams p) {
  __shared__ float s_log[FUSED ? kRouterBlockTokens * kLogStride : 1];
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
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        c.a[mb][q] = va[mb] ? *reinterpret_cast<const u32x4*>(xa[mb] + k0 + 8 * q) : u32x4{0u, 0u, 0u, 0u};
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
        av[mb] = (pp & 1) ? bf16hi(word) : bf16lo(word);
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

  RtChunk c0, c1;
  load(0, c0);
  for (int k0 = 0; k0 < p.hidden; k0 += 2 * kRouterKChunk) {
    const bool has1 = k0 + kRouterKChunk < p.hidden;
    if (has1) load(k0 + kRouterKChunk, c1);
    compute(c0);
    if (!has1) break;
    if (k0 + 2 * kRouterKChunk < p.hidden) load(k0 + 2 * kRouterKChunk, c0);
    compute(c1);
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
        for (int nb = 0; nb < 2; ++nb) s_log[tl * kLogStride + 64 * we + 32 * nb + r] = acc[mb][nb][i];
      }
    __syncthreads();
    float bias[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bias[j] = p.bias ? p.bias[lane + 64 * j] : 0.f;
    constexpr int per_wave = kRouterBlockTokens / 8;
    for (int u = 0; u < per_wave; ++u) {
      const int tl = w * per_wave + u;
      const int t = blk0 + tl;
      if (t >= p.n_tok) break;
      float z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = s_log[tl * kLogStride + lane + 64 * j];
      route_token(z, bias, lane, p.topk_groups, p.top_k, p.scale, p.idx + (size_t)t * p.top_k,
                  p.wts + (size_t)t * p.top_k);
    }
  }
}

// One wavefront per token over fp32 logits [n_tok][256].
__global__ void __launch_bounds__(256) router_select_kernel(RouterParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.n_tok) return;
  float z[4], bias[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = p.logits_in[(size_t)t * kRouterExperts + lane + 64 * j];
    bias[j] = p.bias ? p.bias[lane + 64 * j] : 0.f;
  }
  route_token(z, bias, lane, p.topk_groups, p.top_k, p.scale, p.idx + (size_t)t * p.top_k,
              p.wts + (size_t)t * p.top_k);
}

hipError_t launch_router_logits(const RouterParams& p, hipStream_t s) {
  const unsigned blocks = (unsigned)((p.n_tok + kRouterBlockTokens - 1) / kRouterBlockTokens);
  hipLaunchKernelGGL(router_gemm_kernel<false>, dim3(blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_router_fused(const RouterParams& p, hipStream_t s) {
  const unsigned blocks = (unsigned)((p.n_tok + kRouterBlockTokens - 1) / kRouterBlockTokens);
  hipLaunchKernelGGL(router_gemm_kernel<true>, dim3(blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_router_select(const RouterParams& p, hipStream_t s) {
  hipLaunchKernelGGL(router_select_kernel, dim3((unsigned)((p.n_tok + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
