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

// Bits [off, off + 8·BITS) of a packed row whose words sit `stride` apart.
template <int BITS>
__device__ __forceinline__ uint64_t window(const uint32_t* base, int64_t stride, int64_t nwords,
                                           int64_t off) {
  const int64_t w = off >> 5;
  uint64_t v = base[w * stride];
  if (w + 1 < nwords) v |= (uint64_t)base[(w + 1) * stride] << 32;
  return v >> (off & 31);
}

// Ŵ of 8 consecutive codes (one group: g % 8 == 0) of column n starting at k0.
template <int BITS>
__device__ __forceinline__ void dequant8(const DqArgs& a, int64_t n, int64_t k0, float (&o)[8]) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const uint64_t v = window<BITS>(a.qw + n, a.N, a.K * BITS / 32, k0 * BITS);
  const int64_t j = k0 / a.g;
  float zp;
  if (a.qz) {
    const int64_t zw = a.N * BITS / 32;
    zp = (float)(window<BITS>(a.qz + j * zw, 1, zw, n * BITS) & MASK);
  } else {
    zp = (float)(1 << (BITS - 1));
  }
  const float s = a.scale[n * a.G + j];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = (float)((v >> (i * BITS)) & MASK);
    o[i] = bf16_val(bf16_bits(s * (q - zp)));
  }
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
constexpr int GEMV_COLS = 64;   // columns per workgroup (one per lane)
constexpr int GEMV_MMAX = 16;

template <int BITS>
__global__ __launch_bounds__(NT) void k_dq_gemv(DqArgs a, const uint16_t* X, int M, float* part,
                                                int64_t chunks_per_slice) {
  __shared__ float red[4][GEMV_MMAX][GEMV_COLS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * GEMV_COLS + lane;
  const int64_t c_begin = (int64_t)blockIdx.y * chunks_per_slice;
  const int64_t c_end = min(c_begin + chunks_per_slice, a.K / 8);
  float acc[GEMV_MMAX];
#pragma unroll
  for (int m = 0; m < GEMV_MMAX; ++m) acc[m] = 0.0f;
  if (n < a.N) {
    for (int64_t c = c_begin + wave; c < c_end; c += 4) {
      float w[8];
      dequant8<BITS>(a, n, c * 8, w);
#pragma unroll
      for (int m = 0; m < GEMV_MMAX; ++m) {
        if (m < M) {
          float x[8];
          load8(X + (int64_t)m * a.K + c * 8, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[m] += x[i] * w[i];
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < GEMV_MMAX; ++m)
    if (m < M) red[wave][m][lane] = acc[m];
  __syncthreads();
  // the four waves' sums, in wave order; one thread per (m, column)
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

template <int BITS>
ar_status dq_gemv(const DqArgs& a, const uint16_t* X, int M, float* part, int S,
                  int64_t cps, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + GEMV_COLS - 1) / GEMV_COLS), (unsigned)S);
  hipLaunchKernelGGL(k_dq_gemv<BITS>, grid, dim3(NT), 0, st, a, X, M, part, cps);
  return last_status();
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

// Slices of the small-M product: about two workgroups per CU, at least 4 chunks
// of 8 codes per wave.
int ar_dq_slices(int64_t N, int64_t K) {
  const int64_t colblocks = (N + GEMV_COLS - 1) / GEMV_COLS;
  int64_t S = (512 + colblocks - 1) / colblocks;
  const int64_t maxS = (K / 8) / 16;
  if (S > maxS) S = maxS;
  return (int)(S < 1 ? 1 : S);
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
  const int S = ar_dq_slices(N, K);
  const int64_t chunks = K / 8;
  const int64_t cps = (chunks + S - 1) / S;
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
