// W{2,3,4,8} x bf16 product on the packed format (gfx950): Y = X·bf16(Ŵ)ᵀ with
// Ŵ = s·(q − zp) taken straight from qweight / qzeros / scale, the deployment
// side of the codes the tuning loop produces (SGLang AutoRound page, "설계 근거":
// checkpoints reuse GPTQ/AWQ packing; the dequantisation of the llm-compressor
// page's _fake_quantize_with_offset). The bf16 operand is the one the tuning
// loop's forward product uses.
//
// Layout (as ar_pack writes it): qweight [K·b/32, N] int32, column n holds row
// n's codes along K, LSB first (3-bit codes straddle words); qzeros [G, N·b/32]
// the same along N (NULL: the symmetric grid, zp = 2^(b−1)); scale [N, G] f32.
//
// Small M (decode) is bound by reading the packed weight: a split-K GEMV reads
// each column's words once, coalesced along N, and keeps M ≤ 16 accumulators
// per lane; slices are summed in a fixed order. Larger M dequantizes once into
// the blocked bf16 operand and runs the MFMA GEMM.
#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"

namespace {

constexpr int NT = 256;

inline ar_status last_status() { return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP; }

struct DqArgs {
  const uint32_t* qw;   // [K·BITS/32, N]
  const uint32_t* qz;   // [G, N·BITS/32] or NULL
  const float* scale;   // [N, G]
  int64_t N, K;
  int g, G;
};

// Bits [off, off + NB) of a packed row whose words sit `stride` apart (NB <= 33;
// the second word is read only when the bits reach into it).
template <int NB>
__device__ __forceinline__ uint64_t window(const uint32_t* base, int64_t stride, int64_t nwords,
                                           int64_t off) {
  const int64_t w = off >> 5;
  const int sh = (int)(off & 31);
  uint64_t v = base[w * stride];
  if (sh + NB > 32 && w + 1 < nwords) v |= (uint64_t)base[(w + 1) * stride] << 32;
  return v >> sh;
}

// Zero-point and scale of group j of column n.
template <int BITS>
__device__ __forceinline__ void group_sz(const DqArgs& a, int64_t n, int64_t j, float& zp,
                                         float& s) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  if (a.qz) {
    const int64_t zw = a.N * BITS / 32;
    zp = (float)(window<BITS>(a.qz + j * zw, 1, zw, n * BITS) & MASK);
  } else {
    zp = (float)(1 << (BITS - 1));
  }
  s = a.scale[n * a.G + j];
}

// bf16 Ŵ = s·(q − zp) of the 8 codes in the low 8·BITS bits of v (round to
// nearest even; the product of a finite scale and a small integer is finite).
template <int BITS>
__device__ __forceinline__ void dequant_bits(uint64_t v, float zp, float s, float (&o)[8]) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = (float)((uint32_t)(v >> (i * BITS)) & MASK);
    const uint32_t u = __float_as_uint(s * (q - zp));
    o[i] = __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
  }
}

// Ŵ of 8 consecutive codes (one group: g % 8 == 0) of column n starting at k0.
template <int BITS>
__device__ __forceinline__ void dequant8(const DqArgs& a, int64_t n, int64_t k0, float (&o)[8]) {
  const uint64_t v = window<8 * BITS>(a.qw + n, a.N, a.K * BITS / 32, k0 * BITS);
  float zp, s;
  group_sz<BITS>(a, n, k0 / a.g, zp, s);
  dequant_bits<BITS>(v, zp, s, o);
}

// ------------------------------------------------------------------ dequant to the blocked operand
template <int BITS>
__global__ __launch_bounds__(NT) void k_dequant_blocked(DqArgs a, uint16_t* WB, int64_t nkb) {
  const int64_t cpr = a.K / 8;
  const int64_t total = a.N * cpr;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int64_t c = i / a.N, n = i - c * a.N;   // consecutive threads: consecutive columns
    float o[8];
    dequant8<BITS>(a, n, c * 8, o);
    store8(WB + arblk::chunk_offset(n, c * 8, nkb), o);
  }
}

// ------------------------------------------------------------------ small-M product
constexpr int GEMV_COLS = 64;      // columns per workgroup (one per lane)
constexpr int GEMV_MMAX = 16;
constexpr int GEMV_BATCH = 16;     // chunks whose packed words are in flight together
// Bytes of LDS for the X slice of a workgroup with at most MT rows: small
// buckets keep it small so that many workgroups share a CU.
__host__ __device__ constexpr int gemv_xlds(int MT) { return MT >= 4 ? 65536 : 16384 * MT; }

// One workgroup: 64 columns x one K slice. The slice of X (M rows) is staged in
// LDS once; each wave takes every 4th chunk of 8 codes and issues the packed
// words, zero-points and scales of GEMV_BATCH chunks before using any, so one
// memory round trip covers a batch. MT >= M is the compile-time row count.
// Index arithmetic is 32-bit (the host keeps the packed arrays below 2^31
// elements). The four waves' sums are added in wave order; slices are added by
// k_dq_reduce in slice order.
template <int BITS, int MT>
__global__ __launch_bounds__(NT) void k_dq_gemv(DqArgs a, const uint16_t* X, int M, float* part,
                                                int chunks_per_slice) {
  __shared__ float red[4][MT][GEMV_COLS];
  __shared__ __attribute__((aligned(16))) uint16_t xs[gemv_xlds(MT) / 2];
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = (int)a.N, K = (int)a.K;
  const int n = blockIdx.x * GEMV_COLS + lane;
  const int c_begin = blockIdx.y * chunks_per_slice;
  const int c_end = min(c_begin + chunks_per_slice, K / 8);
  const int nc = c_end - c_begin;   // chunks in this slice (nc * M * 16 <= gemv_xlds(MT))
  for (int i = threadIdx.x; i < nc * M; i += NT) {
    const int m = i / nc, c = i - m * nc;
    *reinterpret_cast<u32x4_t*>(xs + (m * nc + c) * 8) =
        *reinterpret_cast<const u32x4_t*>(X + (int64_t)m * K + (c_begin + c) * 8);
  }
  __syncthreads();
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  if (n < N) {
    const uint32_t nwords = (uint32_t)(K * BITS / 32);
    const int g8 = a.g / 8;                       // chunks per group
    const uint32_t zw = (uint32_t)((int64_t)N * BITS / 32);
    for (int c0 = wave; c0 < nc; c0 += 4 * GEMV_BATCH) {
      uint32_t lo[GEMV_BATCH], hi[GEMV_BATCH], zlo[GEMV_BATCH], zhi[GEMV_BATCH];
      float sc[GEMV_BATCH];
#pragma unroll
      for (int u = 0; u < GEMV_BATCH; ++u) {
        const int c = c0 + 4 * u;
        if (c < nc) {
          const uint32_t off = (uint32_t)(c_begin + c) * (8 * BITS);
          const uint32_t w = off >> 5, sh = off & 31;
          lo[u] = a.qw[w * (uint32_t)N + n];
          hi[u] = (sh + 8 * BITS > 32 && w + 1 < nwords) ? a.qw[(w + 1) * (uint32_t)N + n] : 0u;
          const uint32_t j = (uint32_t)(c_begin + c) / (uint32_t)g8;
          sc[u] = a.scale[(uint32_t)n * (uint32_t)a.G + j];
          if (a.qz) {
            const uint32_t zo = (uint32_t)n * BITS, zwi = zo >> 5;
            zlo[u] = a.qz[j * zw + zwi];
            zhi[u] = ((zo & 31) + BITS > 32 && zwi + 1 < zw) ? a.qz[j * zw + zwi + 1] : 0u;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < GEMV_BATCH; ++u) {
        const int c = c0 + 4 * u;
        if (c < nc) {
          const uint32_t sh = ((uint32_t)(c_begin + c) * (8 * BITS)) & 31;
          const uint64_t v = ((uint64_t)hi[u] << 32 | lo[u]) >> sh;
          float zp;
          if (a.qz) {
            const uint32_t zs = ((uint32_t)n * BITS) & 31;
            zp = (float)((uint32_t)(((uint64_t)zhi[u] << 32 | zlo[u]) >> zs) & MASK);
          } else {
            zp = (float)(1 << (BITS - 1));
          }
          float w[8];
          dequant_bits<BITS>(v, zp, sc[u], w);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            if (MT == 1 || m < M) {
              float x[8];
              load8(xs + (m * nc + c) * 8, x);
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[m] = fmaf(x[i], w[i], acc[m]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m < M) red[wave][m][lane] = acc[m];
  __syncthreads();
  for (int t = threadIdx.x; t < M * GEMV_COLS; t += NT) {
    const int m = t / GEMV_COLS, l = t % GEMV_COLS;
    const int64_t nn = (int64_t)blockIdx.x * GEMV_COLS + l;
    if (nn < a.N)
      part[((int64_t)blockIdx.y * M + m) * a.N + nn] =
          ((red[0][m][l] + red[1][m][l]) + red[2][m][l]) + red[3][m][l];
  }
}

// Y[m, n] = sum over slices, in slice order.
__global__ __launch_bounds__(NT) void k_dq_reduce(const float* part, int S, int64_t MN, void* Y,
                                                  int ydt) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < MN; i += (int64_t)gridDim.x * NT) {
    float s = 0.0f;
    for (int k = 0; k < S; ++k) s += part[(int64_t)k * MN + i];
    if (ydt == AR_BF16)
      static_cast<uint16_t*>(Y)[i] = (uint16_t)bf16_bits(s);
    else
      static_cast<float*>(Y)[i] = s;
  }
}

template <int BITS>
ar_status dq_blocked(const DqArgs& a, uint16_t* WB, int64_t nkb, hipStream_t st) {
  const int64_t total = a.N * (a.K / 8);
  const int64_t nb = (total + NT - 1) / NT;
  hipLaunchKernelGGL(k_dequant_blocked<BITS>, dim3((unsigned)(nb < 65536 ? nb : 65536)), dim3(NT),
                     0, st, a, WB, nkb);
  return last_status();
}

template <int BITS, int MT>
ar_status dq_gemv_m(const DqArgs& a, const uint16_t* X, int M, float* part, int S, int cps,
                    hipStream_t st) {
  const dim3 grid((unsigned)((a.N + GEMV_COLS - 1) / GEMV_COLS), (unsigned)S);
  hipLaunchKernelGGL((k_dq_gemv<BITS, MT>), grid, dim3(NT), 0, st, a, X, M, part, cps);
  return last_status();
}

template <int BITS>
ar_status dq_gemv(const DqArgs& a, const uint16_t* X, int M, float* part, int S, int cps,
                  hipStream_t st) {
  if (M <= 1) return dq_gemv_m<BITS, 1>(a, X, M, part, S, cps, st);
  if (M <= 2) return dq_gemv_m<BITS, 2>(a, X, M, part, S, cps, st);
  if (M <= 4) return dq_gemv_m<BITS, 4>(a, X, M, part, S, cps, st);
  if (M <= 8) return dq_gemv_m<BITS, 8>(a, X, M, part, S, cps, st);
  return dq_gemv_m<BITS, 16>(a, X, M, part, S, cps, st);
}

DqArgs dq_args(const int32_t* qweight, const int32_t* qzeros, const float* scale, int64_t N,
               int64_t K, int g) {
  DqArgs a;
  a.qw = reinterpret_cast<const uint32_t*>(qweight);
  a.qz = reinterpret_cast<const uint32_t*>(qzeros);
  a.scale = scale;
  a.N = N;
  a.K = K;
  a.g = g;
  a.G = (int)(K / g);
  return a;
}

}  // namespace

// Row bucket of the small-M product.
static int gemv_bucket(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// Slices of the small-M product: about two workgroups per CU, at least 16
// chunks of 8 codes per slice, and few enough chunks that the X slice fits
// the bucket's LDS stage.
int ar_dq_slices(int64_t N, int64_t K, int64_t M) {
  const int64_t colblocks = (N + GEMV_COLS - 1) / GEMV_COLS;
  const int64_t chunks = K / 8;
  int64_t S = (512 + colblocks - 1) / colblocks;
  const int64_t maxS = chunks / 16;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  const int64_t max_cps = gemv_xlds(gemv_bucket(M)) / (16 * (M > 0 ? M : 1));
  while ((chunks + S - 1) / S > max_cps) ++S;
  return (int)S;
}

ar_status ar_launch_dequant_blocked(int bits, const int32_t* qweight, const int32_t* qzeros,
                                    const float* scale, int64_t N, int64_t K, int g, uint16_t* WB,
                                    hipStream_t st) {
  const DqArgs a = dq_args(qweight, qzeros, scale, N, K, g);
  const int64_t nkb = arblk::k_blocks(K);
  switch (bits) {
    case 2: return dq_blocked<2>(a, WB, nkb, st);
    case 3: return dq_blocked<3>(a, WB, nkb, st);
    case 4: return dq_blocked<4>(a, WB, nkb, st);
    case 8: return dq_blocked<8>(a, WB, nkb, st);
    default: return AR_ERR_UNSUPPORTED;
  }
}

ar_status ar_launch_dq_gemv(int bits, const int32_t* qweight, const int32_t* qzeros,
                            const float* scale, int64_t N, int64_t K, int g, const uint16_t* X,
                            int M, float* part, void* Y, int ydt, hipStream_t st) {
  const DqArgs a = dq_args(qweight, qzeros, scale, N, K, g);
  const int S = ar_dq_slices(N, K, M);
  const int64_t chunks = K / 8;
  const int cps = (int)((chunks + S - 1) / S);
  ar_status s;
  switch (bits) {
    case 2: s = dq_gemv<2>(a, X, M, part, S, cps, st); break;
    case 3: s = dq_gemv<3>(a, X, M, part, S, cps, st); break;
    case 4: s = dq_gemv<4>(a, X, M, part, S, cps, st); break;
    case 8: s = dq_gemv<8>(a, X, M, part, S, cps, st); break;
    default: return AR_ERR_UNSUPPORTED;
  }
  if (s != AR_OK) return s;
  const int64_t MN = (int64_t)M * N;
  const int64_t nb = (MN + NT - 1) / NT;
  hipLaunchKernelGGL(k_dq_reduce, dim3((unsigned)(nb < 65536 ? nb : 65536)), dim3(NT), 0, st, part,
                     S, MN, Y, ydt);
  return last_status();
}
