// Projection GEMMs of the Beam attention sublayer with fused epilogues (gfx950).
//
// The sublayer input X [T][5120] (bf16) is projected to Q [T][6144],
// K and V [T][1024] and the gate logits [T][6144]; the gated attention result
// [T][6144] is mixed back to [T][5120] by W_o ("Beam 1.0: Local RoPE, Global
// NoPE and Scalable Softmax", section "Follow the tensors, not the parameter
// label": weights in the output-by-input convention, attention width 6,144,
// a 6,144-output gate, heads mixed by W_o after the gate).
//
// Both are out[t][f] = sum_k x[t][k] w[f][k] with x and w K-contiguous, on
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation:
//   * a block computes 256 features x 256 tokens; its four waves each own
//     128 features x 128 tokens (the A operand is w, so MFMA rows are
//     features and columns are tokens: a lane holds one token and 64 of its
//     128 features, the other 64 sit in lane l ^ 32);
//   * K advances 64 at a time through two LDS stages of 64 KiB (W and X
//     tiles, 128-byte rows with their 16-byte chunks XOR-swizzled by the low 3
//     bits of the row), filled by global_load_lds_dwordx4 while the other
//     stage is multiplied;
//   * the tile leaves through LDS (transposed to token rows) so every global
//     store is 16 bytes wide and a 256-byte head row is written by 16 lanes.
// QKV/gate epilogue: with 128-feature waves each wave holds whole heads. The
// query heads are finished in registers: RMSNorm over the head (in-lane sum
// plus one permlane32 swap), RoPE on local layers (the rotate-half partner of
// feature i is feature i + 64: same lane, two MFMA row blocks further) or the
// SSMax factor a(t+1) on global layers, and the base-2 softmax scale
// log2(e)/sqrt(d); the result Q' goes straight to the prefill workspace, so
// the raw queries never reach memory. K, V and the gate logits are stored raw.
#include "beam_device.h"
#include "beam_kernels.h"

namespace beam {

namespace {

constexpr int kTB = kGemmTile;         // features and tokens per block
constexpr int kTK = 64;                // k per LDS stage
constexpr int kOpTile = kTB * kTK;     // elements of one operand tile (32 KiB)
constexpr int kBufs = 2;               // LDS stage buffers (each a W tile and an X tile)
constexpr int kRopePairs = D / 2;      // rotate-half pairs per head
constexpr int kXcds = 8;               // XCDs of an MI355X (32 CUs each)
constexpr int kPatchF = 4, kPatchT = 8;  // tiles per patch (feature x token): 32 = one per CU of an XCD
constexpr int kGrid = kXcds * kPatchF * kPatchT;
// LDS: two stage buffers (W tile, X tile) of 64 KiB. After the k loop the
// same 128 KiB stage the output tile (4 waves x 128 x 128 bf16); the RoPE
// frequencies (revolutions per position, float64) sit behind them.
constexpr int kSmemElems = 2 * kBufs * kOpTile + 4 * (D / 2);
constexpr int kFreqOff = 2 * kBufs * kOpTile;  // element offset of the RoPE table

// Element offset of 16-byte chunk c (k = 8c .. 8c+7) of row r of an operand tile.
__device__ __forceinline__ int op_off(int r, int c) { return r * kTK + ((c ^ (r & 7)) << 3); }

// s_waitcnt: at most n vector-memory operations outstanding, LDS/scalar 0,
// export count untouched (gfx9 fields vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] at bits 15:14).
constexpr int vm_wait(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// sum of x over lanes l and l ^ 32
__device__ __forceinline__ float sum_lane_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

// Grid: kGrid = 256 persistent blocks, one per CU (one 4-wave block fills a
// CU's LDS).
template <int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmemElems];
  double* s_freq = reinterpret_cast<double*>(smem + kFreqOff);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;  // wave's feature half, token half
  const int r32 = lane & 31, h = lane >> 5;
  const int K = p.K;

  if constexpr (EPI == kEpiQkvg) {
    if (tid < kRopePairs)
      s_freq[tid] = pow((double)p.rope_theta, -2.0 * (double)tid / (double)D) * 0.15915494309189533577;
  }

  // Persistent schedule: block b = 8 j + x runs on XCD x (blocks are dealt to
  // the eight XCDs in turn) and takes tile j of patches x, x + 8, x + 16, ...
  // A patch is 4 feature tiles x 8 token tiles, so the 32 blocks of an XCD
  // share 4 W tiles and 8 X tiles and walk K together: the k-slices they read
  // are fetched into that XCD's L2 once. Consecutive patches differ in their
  // feature tiles first, so the eight XCDs work on the same token tiles.
  const int n_ft = p.n_feat / kTB, n_tt = (p.n_tok + kTB - 1) / kTB;
  const int n_pf = (n_ft + kPatchF - 1) / kPatchF, n_pt = (n_tt + kPatchT - 1) / kPatchT;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  for (int pch = xcd; pch < n_pf * n_pt; pch += kXcds) {
    const int ft = (pch % n_pf) * kPatchF + j % kPatchF;
    const int tt = (pch / n_pf) * kPatchT + j / kPatchF;
    if (ft >= n_ft || tt >= n_tt) continue;
    const int f0 = ft * kTB, n0 = tt * kTB;

    // Loads per stage and wave: 8 KiB of W rows through registers and 8 KiB
    // of X rows by LDS DMA, 1 KiB (8 rows of 128 bytes) per instruction, lane
    // l on row 8(8w + i) + (l >> 3). The W rows are read in order (chunk
    // l & 7) and written to their swizzled LDS chunk; the DMA lands lane l at
    // LDS chunk l & 7, so it reads source chunk (l & 7) ^ ((l >> 3) & 7).
    const uint16_t* wsrc = p.w + (size_t)f0 * K;
    const uint16_t* xsrc = p.x + (size_t)n0 * K;
    uint32_t w_off[8], x_off[8];
    int w_lds[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * (8 * w + i) + (lane >> 3);
      const int c = (lane & 7) ^ ((lane >> 3) & 7);
      w_off[i] = (uint32_t)(r * K + 8 * (lane & 7));
      w_lds[i] = op_off(r, lane & 7);
      const int rt = min(r, p.n_tok - 1 - n0);  // rows past the last token re-read it
      x_off[i] = (uint32_t)(rt * K + 8 * c);
    }
    u32x4 wr0[8], wr1[8];  // W rows of two stages in flight
    auto load_w = [&](int k0, u32x4(&r)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = *reinterpret_cast<const u32x4*>(wsrc + k0 + w_off[i]);
    };
    auto store_w = [&](uint16_t* st, const u32x4(&r)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(st + w_lds[i]) = r[i];
    };
    auto dma_x = [&](int k0, uint16_t* st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_dma16(xsrc + k0 + x_off[i], st + kOpTile + (8 * w + i) * 512);
    };

    // Fragment offsets: row 32b + (l & 31) of the wave's half, chunk 2kk + h.
    int frag[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) frag[kk] = op_off(r32, 2 * kk + h);
    const int a_base = 128 * wm * kTK, b_base = 128 * wn * kTK;

    f32x16 acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

    // Fragments of k-step kk + 1 are read while the 16 MFMAs of kk run (two
    // register sets; the scheduling barriers keep that order).
    struct Frags {
      u32x4 a[4], b[4];
    };
    auto read_frags = [&](const uint16_t* st, int kk, Frags& f) __attribute__((always_inline)) {
      const uint16_t* sw = st;
      const uint16_t* sx = st + kOpTile;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) f.a[mb] = *reinterpret_cast<const u32x4*>(sw + a_base + 32 * mb * kTK + frag[kk]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) f.b[nb] = *reinterpret_cast<const u32x4*>(sx + b_base + 32 * nb * kTK + frag[kk]);
    };
    auto mfmas = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(f.a[mb]), as_bf16x8(f.b[nb]), acc[mb][nb], 0, 0, 0);
    };
    // The 16 MFMAs of one k-step with the 8 fragment reads of the next
    // interleaved into the first 8 (one read per MFMA): at most 8 LDS reads
    // are in flight (the LDS counter holds 15) and each has 8 MFMAs to land.
    // In the stage's last k-step the W rows of the next stage are written to
    // LDS between the last 8 MFMAs.
    auto step = [&](const Frags& cur_f, const uint16_t* st, int kk, Frags& nxt_f) __attribute__((always_inline)) {
      read_frags(st, kk, nxt_f);
      mfmas(cur_f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // The stage's loads are spread over its first two k-steps so the memory
    // pipeline sees a steady stream instead of a burst that stalls the MFMA
    // issue behind it. The X DMAs set M0 and stay where the source puts them:
    // one after each of k-step 0's first 8 MFMAs. The W loads of k-step 1 are
    // placed by scheduling groups, one per MFMA.
    auto step_dma = [&](const Frags& cur_f, const uint16_t* st, int kk, Frags& nxt_f, int k0x, uint16_t* stx)
                        __attribute__((always_inline)) {
      read_frags(st, kk, nxt_f);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur_f.a[mb]), as_bf16x8(cur_f.b[nb]),
                                                                acc[mb][nb], 0, 0, 0);
          const int i = 4 * mb + nb;
          if (i < 8) lds_dma16(xsrc + k0x + x_off[i], stx + kOpTile + (8 * w + i) * 512);
        }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto step_loads = [&](const Frags& cur_f, const uint16_t* st, int kk, Frags& nxt_f, int k0w, u32x4(&r)[8])
                          __attribute__((always_inline)) {
      read_frags(st, kk, nxt_f);
      load_w(k0w, r);
      mfmas(cur_f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one W load
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto step_store = [&](const Frags& cur_f, const uint16_t* st, int kk, Frags& nxt_f, uint16_t* st_w,
                          const u32x4(&r)[8]) __attribute__((always_inline)) {
      read_frags(st, kk, nxt_f);
      mfmas(cur_f);
      store_w(st_w, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS write
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // Stage s lives in LDS buffer s % 2; its X rows arrive by DMA issued one
    // stage ahead, its W rows in registers loaded two stages ahead. In stage
    // s: DMA of X(s+1) into the other buffer (free: every wave passed the
    // previous barrier after its last read of it), then the loads of W(s+2)
    // (after the DMA, so the in-order counter can wait for the DMA alone);
    // k-steps 0 .. 1 with the reads of 1 .. 2; wait for W(s+1) (16 newer
    // operations may stay outstanding); k-step 2 with the reads of 3 and
    // W(s+1) written into the other buffer; wait for the DMA (W(s+2) may stay
    // outstanding) and the LDS traffic; a bare barrier (a fence would drain
    // the loads still in flight); k-step 3 with the reads of stage s + 1's
    // k-step 0. Stages go in pairs so the two W register sets have fixed
    // names; every stage is the same code (the last ones re-load the final
    // chunk and read a k-step nobody uses), so the loop has no branch and the
    // accumulators never need copies.
    const int nk = K / kTK;  // even (K is a multiple of 128)
    auto kofs = [&](int kt) { return min(kt, nk - 1) * kTK; };
    load_w(0, wr0);
    dma_x(0, smem);
    load_w(kofs(1), wr1);
    __builtin_amdgcn_s_waitcnt(vm_wait(8));
    store_w(smem, wr0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Frags fa, fb;
    read_frags(smem, 0, fa);
    // (The buffers are fixed per half of the pair: with a buffer computed from
    // kt the compiler cannot tell the DMA target from the buffer being read
    // and waits for the DMA before every read.)
    auto stage = [&](int kt, const uint16_t* cur, uint16_t* nxt, u32x4(&r_next)[8], u32x4(&r_load)[8])
                     __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      step_dma(fa, cur, 1, fb, kofs(kt + 1), nxt);
      step_loads(fb, cur, 2, fa, kofs(kt + 2), r_load);
      __builtin_amdgcn_s_waitcnt(vm_wait(16));
      __builtin_amdgcn_sched_barrier(0);
      step_store(fa, cur, 3, fb, nxt, r_next);
      __builtin_amdgcn_s_waitcnt(vm_wait(8));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      step(fb, nxt, 0, fa);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      stage(kt, smem, smem + 2 * kOpTile, wr1, wr0);
      stage(kt + 1, smem + 2 * kOpTile, smem, wr0, wr1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue ----
    // Lane l holds, for token column 32nb + (l & 31) of the wave, features
    // 32mb + 8(i >> 2) + 4h + (i & 3) of accumulator element i of block (mb, nb).
    const int head = (f0 + 128 * wm) / D;  // the wave's head among all outputs
    uint16_t* out = p.out;
    size_t ld = (size_t)p.ld_out;
    int col0 = f0 + 128 * wm;
    if constexpr (EPI == kEpiQkvg) {
      const int H = p.H, G = p.G;
      if (head < H) {
        out = p.q_out;
        ld = (size_t)H * D;
        col0 = head * D;
        // normalised Q, position op and the base-2 softmax scale, per token
        float wq[4][16];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) wq[mb][i] = bf16f(p.q_norm_w[32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)]);
        const float qbase = kLog2e / sqrtf((float)D);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int tok = min(n0 + 128 * wn + 32 * nb + r32, p.n_tok - 1);
          const int sq = find_seq(p.cu, p.n_seqs, tok);
          const int t = p.start_pos[sq] + tok - p.cu[sq];
          float ss = 0.f;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) ss += acc[mb][nb][i] * acc[mb][nb][i];
          ss = sum_lane_halves(ss);
          const float rn = 1.0f / sqrtf(ss * (1.0f / D) + p.rms_eps);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] = wq[mb][i] * (acc[mb][nb][i] * rn);
          if (p.kind == 0) {
            // RoPE: pair (i, i + 64) = rows of blocks mb and mb + 2, same element
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int pi = 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
                const double rev = (double)t * s_freq[pi];
                const float fr = (float)(rev - rint(rev));  // angle in revolutions, [-1/2, 1/2]
                const float cs = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
                const float x1 = acc[mb][nb][i], x2 = acc[mb + 2][nb][i];
                acc[mb][nb][i] = (x1 * cs - x2 * sn) * qbase;
                acc[mb + 2][nb][i] = (x2 * cs + x1 * sn) * qbase;
              }
          } else {
            const float sc = qbase * ssmax_scale(t, p.ssmax_base, p.ssmax_exp);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[mb][nb][i] *= sc;
          }
        }
      } else if (head < H + G) {
        out = p.k_out;
        ld = (size_t)G * D;
        col0 = (head - H) * D;
      } else if (head < H + 2 * G) {
        out = p.v_out;
        ld = (size_t)G * D;
        col0 = (head - H - G) * D;
      } else {
        out = p.g_out;
        ld = (size_t)H * D;
        col0 = (head - H - 2 * G) * D;
      }
    }

    // Stage the wave's 128 x 128 tile as token rows of 256 bytes (16-byte
    // chunk c at c ^ (row & 15)), then write 16 bytes per lane.
    uint16_t* so = smem + w * (128 * 128);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int row = 32 * nb + r32;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 4 * mb + q;
          const u32x2 v = u32x2{pack_bf16x2(acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1]),
                                pack_bf16x2(acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3])};
          *reinterpret_cast<u32x2*>(so + row * 128 + ((c ^ (row & 15)) << 3) + 4 * h) = v;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // own wave's rows only: no barrier needed
    const int c = lane & 15;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int row = 4 * it + (lane >> 4);
      const int tok = n0 + 128 * wn + row;
      const u32x4 v = *reinterpret_cast<const u32x4*>(so + row * 128 + ((c ^ (row & 15)) << 3));
      if (tok < p.n_tok) *reinterpret_cast<u32x4*>(out + (size_t)tok * ld + col0 + 8 * c) = v;
    }
    __syncthreads();  // the next tile's DMA overwrites the staging area
  }
}

hipError_t launch_gemm(const GemmParams& p, int epi, hipStream_t s) {
  clear_stale_error();
  if (epi == kEpiQkvg)
    hipLaunchKernelGGL(gemm_bf16_kernel<kEpiQkvg>, dim3(kGrid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<kEpiPlain>, dim3(kGrid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace beam
