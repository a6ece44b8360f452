// bf16 MFMA contractions of the tuning step (gfx950).
//
// Both products are written as one "NT" GEMM, C[i, j] = sum_k P[i, k] * Q[j, k],
// with P and Q row-major and contiguous along the reduction index:
//   forward   Y'[t, n]  = sum_k X_b[t, k] * Ŵ[n, k]         P = X_b [Tb, K],  Q = Ŵ [N, K]
//   gradient  G[n, k]   = sum_t dYᵀ[n, t] * Xᵀ_b[k, t]      P = dYᵀ [N, Tb], Q = Xᵀ_b [K, Tb]
// (the loss and its weight gradient of the per-module loop on the llm-compressor
// AutoRound page: F.linear forward, mean-squared error, backward). The gradient
// operands are kept transposed in HBM (dYᵀ is written that way by the forward
// epilogue, Xᵀ is transposed once per Linear) so that the same LDS/MFMA main loop
// serves both products.
//
// Tile: 256 x 256 x 64 per workgroup of 4 waves (2 x 2), each wave 128 x 128 as
// 4 x 4 blocks of v_mfma_f32_32x32x16_bf16; float32 accumulators (256 per lane).
// Global -> registers -> LDS, two LDS stages (128 KiB), one barrier per k-step.
// LDS rows are 128 B (64 bf16) with the 16-byte chunk index XOR-swizzled by
// (row & 7) so that both the row-wise stores and the MFMA fragment reads are
// free of bank conflicts. Ragged tiles are zero-filled by buffer-load range checks.
#include "ar_device.h"
#include "ar_launch.h"

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int STAGE_BYTES = (BM + BN) * BK * 2;   // 64 KiB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;         // 128 KiB

struct GemmArgs {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t ld;       // row stride of P and Q in elements (== reduction length)
  int64_t rowsP, rowsQ, kred;
  int tilesI, tilesJ;
};

// Workgroup -> tile. The dispatcher places workgroup w on XCD (w mod 8); give
// each XCD one contiguous range of the tile sequence, and walk that sequence in
// groups of GI tile rows so that the ~32 tiles resident on one XCD share a few
// P and Q panels in its L2.
__device__ __forceinline__ void tile_of(int w, int nwg, int tilesI, int tilesJ, int& ti, int& tj) {
  const int xcd = w & 7, local = w >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  const int L = xcd * q + min(xcd, r) + local;
  constexpr int GI = 4;
  const int per_group = GI * tilesJ;
  const int grp = L / per_group;
  const int first = grp * GI;
  const int gsize = min(tilesI - first, GI);
  const int inner = L - grp * per_group;
  ti = first + inner % gsize;
  tj = inner / gsize;
}

template <class Epi>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_nt(GemmArgs a, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  int ti, tj;
  tile_of(blockIdx.x, gridDim.x, a.tilesI, a.tilesJ, ti, tj);
  const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
  const uint32_t rP = (uint32_t)min<int64_t>(BM, a.rowsP - i0);
  const uint32_t rQ = (uint32_t)min<int64_t>(BN, a.rowsQ - j0);
  const __amdgpu_buffer_rsrc_t bufP = make_rsrc(a.P + i0 * a.ld, rP * (uint32_t)a.ld * 2u);
  const __amdgpu_buffer_rsrc_t bufQ = make_rsrc(a.Q + j0 * a.ld, rQ * (uint32_t)a.ld * 2u);

  // Loader: thread owns chunk (tid & 7) of rows (tid >> 3) + 32*i, i = 0..7.
  const int lrow = tid >> 3, lch = tid & 7;
  const uint32_t goff = ((uint32_t)lrow * (uint32_t)a.ld + (uint32_t)lch * 8u) * 2u;
  const uint32_t gstep = 32u * (uint32_t)a.ld * 2u;
  const uint32_t swz_w = (uint32_t)lrow * 128u + ((uint32_t)(lch ^ (lrow & 7)) << 4);

  // Fragment reader: lane reads row (lane & 31) of a 32-row block, logical
  // chunk 2*ks + (lane >> 5).
  const uint32_t rdP = (uint32_t)(wi * 128 + (lane & 31)) * 128u;
  const uint32_t rdQ = (uint32_t)BM * 128u + (uint32_t)(wj * 128 + (lane & 31)) * 128u;
  const int rsw = lane & 7, rhi = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

  u32x4_t regP[8], regQ[8];
  const int nk = (int)((a.kred + BK - 1) / BK);

  auto gload = [&](int kt) {
    const uint32_t soff = (uint32_t)kt * BK * 2u;
    const bool ok = (int64_t)kt * BK + lch * 8 < a.kred;
    const uint32_t base = ok ? goff : kOOB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      regP[i] = __builtin_amdgcn_raw_buffer_load_b128(bufP, base + (ok ? i * gstep : 0u), soff, 0);
      regQ[i] = __builtin_amdgcn_raw_buffer_load_b128(bufQ, base + (ok ? i * gstep : 0u), soff, 0);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* s = lds + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4_t*>(s + swz_w + i * 4096) = regP[i];
      *reinterpret_cast<u32x4_t*>(s + BM * 128 + swz_w + i * 4096) = regQ[i];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* s = lds + cur * STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t ch = (uint32_t)(((2 * ks + rhi) ^ rsw) << 4);
      bf16x8_t pf[4], qf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        pf[b] = *reinterpret_cast<const bf16x8_t*>(s + rdP + b * 32 * 128 + ch);
        qf[b] = *reinterpret_cast<const bf16x8_t*>(s + rdQ + b * 32 * 128 + ch);
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[bi], qf[bj], acc[bi][bj], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  epi(acc, i0, j0, wi, wj, lane, lds, ti * a.tilesJ + tj);
}

// Accumulator element (bi, bj, r) of a lane sits at
//   i = i0 + wi*128 + bi*32 + 8*(r >> 2) + 4*(lane >> 5) + (r & 3)
//   j = j0 + wj*128 + bj*32 + (lane & 31)
// (v_mfma_f32_32x32x* output layout).

// Forward epilogue: i = token t, j = output feature n. R = Y' - Y_true,
// dYᵀ[n, t] = bf16(R), per-workgroup sum of R² (fixed order).
template <typename YT>
struct EpiFwd {
  const YT* yT;      // [N, Tb] targets of this minibatch, transposed
  uint16_t* dyT;     // [N, Tb]
  float* partials;   // [tiles]
  int64_t N, Tb;

  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int64_t i0, int64_t j0, int wi,
                                             int wj, int lane, uint8_t* lds, int tile) const {
    float sq = 0.0f;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int64_t n = j0 + wj * 128 + bj * 32 + (lane & 31);
      if (n < N) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t t = i0 + wi * 128 + bi * 32 + q * 8 + (lane >> 5) * 4;
            if (t < Tb) {
              float y[4];
              if constexpr (sizeof(YT) == 2) {
                u32x2_t v = *reinterpret_cast<const u32x2_t*>(yT + n * Tb + t);
                y[0] = __uint_as_float(v[0] << 16);
                y[1] = __uint_as_float(v[0] & 0xFFFF0000u);
                y[2] = __uint_as_float(v[1] << 16);
                y[3] = __uint_as_float(v[1] & 0xFFFF0000u);
              } else {
                f32x4_t v = *reinterpret_cast<const f32x4_t*>(yT + n * Tb + t);
                y[0] = v[0]; y[1] = v[1]; y[2] = v[2]; y[3] = v[3];
              }
              float r[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                r[e] = acc[bi][bj][q * 4 + e] - y[e];
                sq += r[e] * r[e];
              }
              u32x2_t o;
              o[0] = bf16_bits(r[0]) | (bf16_bits(r[1]) << 16);
              o[1] = bf16_bits(r[2]) | (bf16_bits(r[3]) << 16);
              *reinterpret_cast<u32x2_t*>(dyT + n * Tb + t) = o;
            }
          }
        }
      }
    }
    // workgroup sum: wave butterfly, then the 4 wave sums in order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    float* red = reinterpret_cast<float*>(lds);
    const int wave = wi * 2 + wj;
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (wave == 0 && lane == 0) partials[tile] = ((red[0] + red[1]) + red[2]) + red[3];
  }
};

// Gradient epilogue: i = output feature n, j = input feature k; G = scale * acc.
struct EpiWgrad {
  float* G;   // [N, K]
  int64_t N, K;
  float scale;

  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int64_t i0, int64_t j0, int wi,
                                             int wj, int lane, uint8_t*, int) const {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int64_t k = j0 + wj * 128 + bj * 32 + (lane & 31);
      if (k < K) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t n = i0 + wi * 128 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (n < N) G[n * K + k] = acc[bi][bj][r] * scale;
          }
        }
      }
    }
  }
};

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

int ar_fwd_tiles(int64_t Tb, int64_t N) { return ceil_div(Tb, BM) * ceil_div(N, BN); }

ar_status ar_launch_gemm_fwd(const uint16_t* Xb, const uint16_t* Wq, const void* yT, int ydt,
                             uint16_t* dyT, float* partials, int64_t Tb, int64_t N, int64_t K,
                             hipStream_t st) {
  GemmArgs a;
  a.P = Xb; a.Q = Wq; a.ld = K; a.rowsP = Tb; a.rowsQ = N; a.kred = K;
  a.tilesI = ceil_div(Tb, BM); a.tilesJ = ceil_div(N, BN);
  const int nwg = a.tilesI * a.tilesJ;
  if (ydt == AR_BF16) {
    EpiFwd<uint16_t> e{static_cast<const uint16_t*>(yT), dyT, partials, N, Tb};
    hipLaunchKernelGGL(k_gemm_nt<EpiFwd<uint16_t>>, dim3(nwg), dim3(NTHR), 0, st, a, e);
  } else {
    EpiFwd<float> e{static_cast<const float*>(yT), dyT, partials, N, Tb};
    hipLaunchKernelGGL(k_gemm_nt<EpiFwd<float>>, dim3(nwg), dim3(NTHR), 0, st, a, e);
  }
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

ar_status ar_launch_gemm_wgrad(const uint16_t* dyT, const uint16_t* XTb, float* G, int64_t N,
                               int64_t K, int64_t Tb, float scale, hipStream_t st) {
  GemmArgs a;
  a.P = dyT; a.Q = XTb; a.ld = Tb; a.rowsP = N; a.rowsQ = K; a.kred = Tb;
  a.tilesI = ceil_div(N, BM); a.tilesJ = ceil_div(K, BN);
  EpiWgrad e{G, N, K, scale};
  hipLaunchKernelGGL(k_gemm_nt<EpiWgrad>, dim3(a.tilesI * a.tilesJ), dim3(NTHR), 0, st, a, e);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
