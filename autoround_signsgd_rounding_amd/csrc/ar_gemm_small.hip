// Small bf16 MFMA products of the tuning step (gfx950): the forward and the
// float32-output products (weight gradient, Gram-form product and statistics)
// when each has at most SMALL_MAX_TILES tiles of 256 x 256. The operands are
// those of the 256 x 256 kernels in ar_gemm.hip (the blocked layout of
// ar_blocked.h), and so are the products they compute.
#include <hip/hip_runtime.h>

#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"
#include "ar_loss.h"

namespace {

constexpr int BK = arblk::KB;

// The 256 x 256 kernels would run such a product on one or a few workgroups,
// which is what a toy layer's step costs. Here each workgroup is one wave that owns a 64 x 64 tile (2 x 2 blocks
// of v_mfma_f32_32x32x16_bf16), or a 32 x 32 tile (one block) when the product
// has at most SM_FINE_MAX tiles of 64 x 64, so that a product's operand loads
// spread over as many CUs as it has tiles. The wave loads its fragments from the blocked
// operands straight into registers, SM_D steps ahead (the fragment layout is
// the one the LDS reads of the large kernels use); the forward's targets are
// loaded before the main loop. A product this small is bound by memory latency
// and per-CU load bandwidth, so the kernel spends registers to keep the round
// trips few. Every output element gets the same sequence of MFMAs as in the
// large kernels (per 32-wide step, substep 0 then substep 1), so G and dY come
// out the same; only the forward's sums of R² are grouped per tile.
// A float32-output product's launch has one workgroup more, which reduces the
// previous forward's loss while the others run.
constexpr int SMALL_MAX_TILES = 4;
constexpr int SM_D = 8;   // steps of fragments in flight
constexpr int SM_THR = 64;
constexpr int SM_FINE_MAX = 16;

enum { SM_FWD_F32 = 0, SM_FWD_BF16 = 1, SM_WGRAD = 2 };

struct SmallArgs {
  const uint16_t* P;   // rows rowsP (forward: X_b, gradient: dYᵀ), nkb blocks per panel
  const uint16_t* Q;   // rows rowsQ (forward: Ŵ, gradient: X_bᵀ)
  int nkb;             // reduction steps (k-blocks of Q)
  int nQ;              // tiles along Q (tile t: row t / nQ, column t % nQ)
  // P panels hold nkP blocks; step s reads P block s for s < foldP, else s - foldP
  // (nkP = foldP = nkb: P and Q side by side; the Gram product folds D)
  int nkP, foldP;
  // forward: targets and dYᵀ blocked (rows n, reduction t, nkbT blocks)
  const void* yB;
  uint16_t* dyB;
  float* partials;     // one per tile, at its tile index
  int nkbT;
  // float32 output: G [N, K] row-major, scaled; the previous forward's loss, reduced
  // by the launch's last workgroup
  float* G;
  int64_t N, K;
  float scale;
  ArLossIn loss;
};

// NB x NB blocks of 32 x 32 per wave (tile TS = 32·NB).
template <int MODE, int NB>
__global__ __launch_bounds__(SM_THR) void k_gemm_small(SmallArgs a) {
  constexpr int TS = 32 * NB;
  const int lane = threadIdx.x;
  if (MODE == SM_WGRAD && blockIdx.x == gridDim.x - 1) {   // the extra workgroup
    if (a.loss.partials) loss_reduce_wave(a.loss);
    return;
  }
  const int tP = (int)blockIdx.x / a.nQ, tQ = (int)blockIdx.x - tP * a.nQ;
  const int64_t r0 = (int64_t)tP * TS;   // the wave's rows of P
  const int64_t c0 = (int64_t)tQ * TS;   // and of Q
  const int nk = a.nkb;
  const uint16_t* pb = a.P + (r0 >> 8) * (int64_t)a.nkP * arblk::BLOCK_ELEMS;
  const uint16_t* qb = a.Q + (c0 >> 8) * (int64_t)nk * arblk::BLOCK_ELEMS;
  // fragment (b, ks): row (r0 & 255) + 32b + (lane & 31) of a block, logical chunk
  // 2 ks + (lane >> 5), stored at chunk ^ ((row >> 2) & 3) (ar_blocked.h)
  const int sw = ((lane & 31) >> 2) & 3;
  uint32_t oP[NB][2], oQ[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t ch = (uint32_t)(((2 * ks + (lane >> 5)) ^ sw) << 3);
      oP[b][ks] = (uint32_t)((r0 & 255) + 32 * b + (lane & 31)) * BK + ch;
      oQ[b][ks] = (uint32_t)((c0 & 255) + 32 * b + (lane & 31)) * BK + ch;
    }
  bf16x8_t fa[SM_D][NB][2], fb[SM_D][NB][2];
  auto load = [&](int s, int u) {
    const uint16_t* P = pb + (int64_t)(s < a.foldP ? s : s - a.foldP) * arblk::BLOCK_ELEMS;
    const uint16_t* Q = qb + (int64_t)s * arblk::BLOCK_ELEMS;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        fa[u][b][ks] = *reinterpret_cast<const bf16x8_t*>(P + oP[b][ks]);
        fb[u][b][ks] = *reinterpret_cast<const bf16x8_t*>(Q + oQ[b][ks]);
      }
  };
  f32x16_t acc[NB][NB];
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;
#pragma unroll
  for (int u = 0; u < SM_D; ++u)
    if (u < nk) load(u, u);
  // forward: the targets of the lane's accumulator elements (4 tokens each, at
  // element offset toff[bj][bi][q] of the blocked arrays), loaded up front
  uint32_t toff[NB][NB][4];
  f32x4_t yv[NB][NB][4];
  if constexpr (MODE != SM_WGRAD) {
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = c0 + bj * 32 + (lane & 31);
          const int64_t t = r0 + bi * 32 + q * 8 + (lane >> 5) * 4;
          const uint32_t off = (uint32_t)arblk::offset(n, t, a.nkbT);
          toff[bj][bi][q] = off;
          if constexpr (MODE == SM_FWD_F32) {
            yv[bj][bi][q] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.yB) + off);
          } else {
            const u32x2_t v = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(a.yB) + off);
            yv[bj][bi][q] = f32x4_t{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                                    __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
          }
        }
  }
  for (int s0 = 0; s0 < nk; s0 += SM_D) {
#pragma unroll
    for (int u = 0; u < SM_D; ++u) {
      const int s = s0 + u;
      if (s < nk) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj)
              acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[u][bi][ks], fb[u][bj][ks],
                                                                    acc[bi][bj], 0, 0, 0);
        if (s + SM_D < nk) load(s + SM_D, u);
      }
    }
  }

  // accumulator element (bi, bj, e): row r0 + bi*32 + 8*(e >> 2) + 4*(lane >> 5) + (e & 3)
  // of P, row c0 + bj*32 + (lane & 31) of Q
  if constexpr (MODE == SM_WGRAD) {
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
      const int64_t k = c0 + bj * 32 + (lane & 31);
      if (k < a.K) {
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t n = r0 + bi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (n < a.N) a.G[n * a.K + k] = acc[bi][bj][e] * a.scale;
          }
      }
    }
  } else {
    // R = Y' - Y_true, dYᵀ = bf16(R) (padding rows and columns give R = 0)
    float sq = 0.0f;
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
#pragma unroll
      for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = acc[bi][bj][q * 4 + e] - yv[bj][bi][q][e];
            sq += r[e] * r[e];
          }
          u32x2_t o;
          o[0] = bf16_bits(r[0]) | (bf16_bits(r[1]) << 16);
          o[1] = bf16_bits(r[2]) | (bf16_bits(r[3]) << 16);
          *reinterpret_cast<u32x2_t*>(a.dyB + toff[bj][bi][q]) = o;
        }
    sq = wave_sum64(sq);
    if (lane == 0) a.partials[blockIdx.x] = sq;
  }
}

int64_t tiles_of(int64_t R, int ts) { return (R + ts - 1) / ts; }
// The forward covers whole 256-row panels, padding included, as the 256 x 256
// kernels do: the gradient product reduces over every token of the padded
// panels, so every dYᵀ element there must be written (R = 0 in padding).
int64_t fwd_tiles(int64_t R, int ts) { return (arblk::ROWS / ts) * arblk::row_tiles(R); }
// Tile size of a product: 32 when it has at most SM_FINE_MAX tiles of 64 x 64.
int fwd_ts(int64_t Tb, int64_t N) {
  return fwd_tiles(Tb, 64) * fwd_tiles(N, 64) <= SM_FINE_MAX ? 32 : 64;
}
int out_ts(int64_t N, int64_t K) {
  return tiles_of(N, 64) * tiles_of(K, 64) <= SM_FINE_MAX ? 32 : 64;
}

}  // namespace

bool ar_small_product(int64_t rowsP, int64_t rowsQ) {
  return arblk::row_tiles(rowsP) * arblk::row_tiles(rowsQ) <= SMALL_MAX_TILES;
}

int ar_small_fwd_tiles(int64_t Tb, int64_t N) {
  const int ts = fwd_ts(Tb, N);
  return (int)(fwd_tiles(Tb, ts) * fwd_tiles(N, ts));
}

ar_status ar_launch_small_fwd(const uint16_t* XB, const uint16_t* WB, const void* yB, int ydt,
                              uint16_t* dyB, float* partials, int64_t Tb, int64_t N, int64_t K,
                              hipStream_t st) {
  const int ts = fwd_ts(Tb, N);
  SmallArgs s{};
  s.P = XB; s.Q = WB; s.nkb = (int)arblk::k_blocks(K); s.nQ = (int)fwd_tiles(N, ts);
  s.nkP = s.foldP = s.nkb;
  s.yB = yB; s.dyB = dyB; s.partials = partials;
  s.nkbT = (int)(arblk::row_tiles(Tb) * (arblk::ROWS / arblk::KB));
  const dim3 grid((unsigned)(fwd_tiles(Tb, ts) * fwd_tiles(N, ts)));
  if (ydt == AR_BF16) {
    if (ts == 32) hipLaunchKernelGGL((k_gemm_small<SM_FWD_BF16, 1>), grid, dim3(SM_THR), 0, st, s);
    else hipLaunchKernelGGL((k_gemm_small<SM_FWD_BF16, 2>), grid, dim3(SM_THR), 0, st, s);
  } else {
    if (ts == 32) hipLaunchKernelGGL((k_gemm_small<SM_FWD_F32, 1>), grid, dim3(SM_THR), 0, st, s);
    else hipLaunchKernelGGL((k_gemm_small<SM_FWD_F32, 2>), grid, dim3(SM_THR), 0, st, s);
  }
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

ar_status ar_launch_small_f32out(const uint16_t* P, const uint16_t* Q, float* out, int64_t N,
                                 int64_t K, int64_t nkb, float scale, const ArLossIn& loss,
                                 int64_t nkP, int64_t foldP, hipStream_t st) {
  const int ts = out_ts(N, K);
  SmallArgs s{};
  s.P = P; s.Q = Q; s.nkb = (int)nkb; s.nQ = (int)tiles_of(K, ts);
  s.nkP = (int)nkP; s.foldP = (int)foldP;
  s.G = out; s.N = N; s.K = K; s.scale = scale; s.loss = loss;
  // one workgroup per tile of out, then the loss workgroup
  const dim3 grid((unsigned)(tiles_of(N, ts) * tiles_of(K, ts) + 1));
  if (ts == 32) hipLaunchKernelGGL((k_gemm_small<SM_WGRAD, 1>), grid, dim3(SM_THR), 0, st, s);
  else hipLaunchKernelGGL((k_gemm_small<SM_WGRAD, 2>), grid, dim3(SM_THR), 0, st, s);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
