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
// Small M (decode) streams the packed words once: each code is dequantized
// once and the M <= 16 rows of X share it through the MFMA unit; K slices are
// summed in a fixed order. Larger M dequantizes once into the blocked bf16
// operand and runs the MFMA GEMM.
#include <mutex>
#include <vector>

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
// The packed words are streamed once and every code is dequantized once; the
// M <= 16 rows of X share it through v_mfma_f32_16x16x32_bf16 (rows beyond M
// repeat row M - 1 and are discarded), so the arithmetic per code is only the
// dequantization.
//
// Workgroup: 256 columns (64 per wave) x one K slice. Lane l of a wave owns
// the four adjacent columns c = 4·(l % 16) .. +3 of its wave's 64, read as one
// 16-byte load per packed word, and in each 32-wide step the chunk of 8 codes
// at k = 32·step + 8·(l / 16). Those 8 codes of column c + i are the lane's B
// operand of MFMA i, whose output column l % 16 is therefore column c + i; the
// A operand is the same 8 k of X row l % 16, read from an LDS copy of the
// slice. (A and B take one k assignment per lane, so the sum is over the
// chunk's k whatever order the unit adds them in.)
//
// bf16 Ŵ = s·(q − zp) costs three VALU operations per code at 4 bits: bytes
// q + 128 − zp are formed four at a time (mask, add of a per-group constant;
// no carries, as q + 128 − zp lies in [113, 143]), converted by
// v_cvt_f32_ubyte, and fma(q + 128 − zp, s, −128·s) gives s·(q − zp) rounded
// once, as the product of an exact integer and s is; v_cvt_pk_bf16_f32 rounds
// two to bf16 (nearest even). 2-bit codes reach the same byte form through one
// v_perm; 3-bit codes are extracted one by one with a bit-field extract; 8-bit
// codes are bytes, converted and then s·(q − zp).
constexpr int DQ_COLS = 256;        // columns per workgroup
constexpr int DQ_GSTRIDE = DQ_COLS + 4;   // floats per staged group row (bank spread)
constexpr int DQ_WG_COST = 96;      // fixed cost of a workgroup (staging), in units of k
constexpr int DQ_X_LDS = 32768;     // bytes for the X slice
constexpr int DQ_G_LDS = 32768;     // bytes for the group constants (s, −128·s, zero-point term)
constexpr int DQ_MAX_LK = 4096;     // longest slice (group-row table of Lk / 8 entries)

// Per-(group, column) zero-point term of the dequantization below.
template <int BITS>
__device__ __forceinline__ uint32_t zp_term(uint32_t zp) {
  if constexpr (BITS == 4 || BITS == 2) return (128u - zp) * 0x01010101u;
  else if constexpr (BITS == 8) return __float_as_uint((float)zp);
  else return 128u - zp;
}

// 8 codes of one column (bits [sh, sh + 8·BITS) of hi:lo) → 8 bf16 Ŵ
// (nb = −128·s, exact).
template <int BITS>
__device__ __forceinline__ bf16x8_t dq_chunk(uint32_t lo, uint32_t hi, uint32_t sh, float s,
                                             float nb, uint32_t z) {
  bf16x8_t b;
  if constexpr (BITS == 4) {
    const uint32_t L = (lo & 0x0F0F0F0Fu) + z, H = ((lo >> 4) & 0x0F0F0F0Fu) + z;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      b[2 * p] = (__bf16)fmaf((float)((L >> (8 * p)) & 0xFFu), s, nb);
      b[2 * p + 1] = (__bf16)fmaf((float)((H >> (8 * p)) & 0xFFu), s, nb);
    }
  } else if constexpr (BITS == 2) {
    // x = c0..c7 (2 bits each); w = x >> 4 puts c2 at bit 0 of its low byte.
    // perm gathers [x.b0, w.b0, x.b1, w.b1] = bytes starting at c0, c2, c4, c6.
    const uint32_t x = (lo >> sh) & 0xFFFFu, w = x >> 4;
    const uint32_t t = __builtin_amdgcn_perm(w, x, 0x05010400u);
    const uint32_t E = (t & 0x03030303u) + z, O = ((t >> 2) & 0x03030303u) + z;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      b[2 * p] = (__bf16)fmaf((float)((E >> (8 * p)) & 0xFFu), s, nb);
      b[2 * p + 1] = (__bf16)fmaf((float)((O >> (8 * p)) & 0xFFu), s, nb);
    }
  } else if constexpr (BITS == 8) {
    const float zf = __uint_as_float(z);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      b[p] = (__bf16)(s * ((float)((lo >> (8 * p)) & 0xFFu) - zf));
      b[4 + p] = (__bf16)(s * ((float)((hi >> (8 * p)) & 0xFFu) - zf));
    }
  } else {
    const uint32_t v = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      b[i] = (__bf16)fmaf((float)(__builtin_amdgcn_ubfe(v, i * BITS, BITS) + z), s, nb);
  }
  return b;
}

// Four adjacent words at columns col .. col + 3 of packed row p + r·N (VEC:
// one 16-byte load, N % 4 == 0 and all four in range; else per column, zero
// past N).
template <bool VEC>
__device__ __forceinline__ u32x4_t load_cols(const uint32_t* p, uint32_t r, int N, int col) {
  if constexpr (VEC) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + r * (uint32_t)N + col));
  } else {
    u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (col + i < N) v[i] = p[r * (uint32_t)N + col + i];
    return v;
  }
}

// Steps of 32 k whose packed words are loaded together: two such batches are
// in flight per wave (the next one is loaded while the current one is used).
template <int BITS>
__host__ __device__ constexpr int dq_batch() { return BITS == 4 ? 8 : BITS == 3 ? 2 : 4; }

// Slice k0 .. k0 + Lk of K (Lk % 32 == 0, Lk <= DQ_MAX_LK; the last slice
// ends at K), computed as whole batches over Lp = Lk rounded up to 32·B.
// LDS: X rows [M][Lp + 8] bf16, zero from the slice's end; scale, −128·scale
// and zero-point term [groups][DQ_GSTRIDE]; the group-row offset of each
// chunk [Lp / 8].
// The launch bound caps registers at 128 VGPRs, for 4 waves per SIMD.
template <int BITS, bool VEC>
__global__ __launch_bounds__(NT, 4) void k_dq_mfma(DqArgs a, const uint16_t* X, int M, float* part,
                                                   int Lk) {
  constexpr int B = dq_batch<BITS>();
  extern __shared__ __attribute__((aligned(16))) uint8_t dq_lds[];
  const int N = (int)a.N, K = (int)a.K, g = a.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = blockIdx.x * DQ_COLS;
  const int k0 = blockIdx.y * Lk, k1 = min(k0 + Lk, K);
  const int Lp = (Lk + 32 * B - 1) / (32 * B) * (32 * B);
  const int j0 = k0 / g, ng = (k1 - 1) / g - j0 + 1;
  const int xstride = Lp + 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(dq_lds);
  float* gs = reinterpret_cast<float*>(dq_lds + ((M * xstride * 2 + 15) & ~15));
  float* gn = gs + ng * DQ_GSTRIDE;
  uint32_t* gz = reinterpret_cast<uint32_t*>(gn + ng * DQ_GSTRIDE);
  int* grow = reinterpret_cast<int*>(gz + ng * DQ_GSTRIDE);

  const int lcol = 64 * wave + 4 * (lane & 15);   // first of the lane's columns in the workgroup
  const int col = cb + lcol;
  const int q = lane >> 4;
  const bool live = col < N;   // columns past N have s = 0 (so B = 0) and are not stored
  // Step t reads packed word w0 + t·BITS of each column at the same bit offset
  // (32 codes are 32·BITS bits = BITS words).
  const uint32_t off0 = (uint32_t)(k0 + 8 * q) * BITS, sh = off0 & 31;
  // the chunk reaches into the next word: never at 2 and 4 bits, always at 8
  const bool two = BITS == 8 || (BITS == 3 && sh + 8 * BITS > 32);
  // Chunks past the slice meet X = 0, so any finite B will do there: their
  // loads are redirected to the lane's last chunk inside K (to row 0 if it has
  // none), and columns past N (their s is 0) to the last four columns. Inside
  // K the chunk's bits end inside the packed column (k + 8 <= K), so a second
  // word exists when it is read.
  const bool has = k0 + 8 * q + 8 <= K;
  const int tmax = has ? (K - k0 - 8 * q - 8) / 32 : 0;
  const uint32_t* qcol = a.qw + (has ? off0 >> 5 : 0u) * (uint32_t)N;
  const int colc = VEC ? (live ? col : N - 4) : col;
  auto issue = [&](int b, u32x4_t (&lo)[B], u32x4_t (&hi)[B]) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int t = min(b * B + u, tmax);
      const uint32_t* p = qcol + (uint32_t)(t * BITS) * (uint32_t)N;
      lo[u] = load_cols<VEC>(p, 0, N, colc);
      if constexpr (BITS == 8) {
        hi[u] = load_cols<VEC>(p, 1, N, colc);
      } else if constexpr (BITS == 3) {
        hi[u] = u32x4_t{0u, 0u, 0u, 0u};
        if (two) hi[u] = load_cols<VEC>(p, 1, N, colc);
      } else {
        hi[u] = lo[u];   // unused
      }
    }
  };
  u32x4_t la[B], ha[B], lb[B], hb[B];
  issue(0, la, ha);   // in flight while the workgroup stages its LDS

  // X slice, zero from the slice's end (K % 8 == 0: a chunk is wholly in or out).
  const int cx = Lp / 8;
  for (int i = threadIdx.x; i < M * cx; i += NT) {
    const int m = i / cx, c = i - m * cx, k = k0 + 8 * c;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (k < k1) v = *reinterpret_cast<const u32x4_t*>(X + (int64_t)m * K + k);
    *reinterpret_cast<u32x4_t*>(xs + m * xstride + 8 * c) = v;
  }
  // Scale and zero-point term of each (group, column); columns past N get s = 0.
  for (int i = threadIdx.x; i < ng * DQ_COLS; i += NT) {
    const int cl = i / ng, jj = i - cl * ng, n = cb + cl, j = j0 + jj;
    float sv = 0.0f;
    uint32_t zp = 1u << (BITS - 1);
    if (n < N) {
      sv = a.scale[(uint32_t)n * (uint32_t)a.G + j];
      if (a.qz) {
        const uint32_t zw = (uint32_t)(N * BITS / 32), zo = (uint32_t)n * BITS, zi = zo >> 5;
        uint64_t v = a.qz[j * zw + zi];
        if ((zo & 31) + BITS > 32) v |= (uint64_t)a.qz[j * zw + zi + 1] << 32;
        zp = (uint32_t)(v >> (zo & 31)) & ((1u << BITS) - 1u);
      }
    }
    gs[jj * DQ_GSTRIDE + cl] = sv;
    gn[jj * DQ_GSTRIDE + cl] = -128.0f * sv;
    gz[jj * DQ_GSTRIDE + cl] = zp_term<BITS>(zp);
  }
  // Chunk c of the slice (k = k0 + 8c; past the slice: its last group) → group row.
  for (int c = threadIdx.x; c < Lp / 8; c += NT)
    grow[c] = (min(k0 + 8 * c, k1 - 1) / g - j0) * DQ_GSTRIDE;
  __syncthreads();

  const uint16_t* xrow = xs + min(lane & 15, M - 1) * xstride + 8 * q;
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int b, const u32x4_t (&lo)[B], const u32x4_t (&hi)[B]) {
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int t = b * B + u;
      const int go = grow[4 * t + q];
      const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(gs + go + lcol);
      const f32x4_t nv = *reinterpret_cast<const f32x4_t*>(gn + go + lcol);
      const u32x4_t zv = *reinterpret_cast<const u32x4_t*>(gz + go + lcol);
      const bf16x8_t xa = *reinterpret_cast<const bf16x8_t*>(xrow + 32 * t);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            xa, dq_chunk<BITS>(lo[u][i], hi[u][i], sh, sv[i], nv[i], zv[i]), acc[i], 0, 0, 0);
    }
  };
  // Batches alternate between the two register sets; the loop leaves only
  // after a whole batch, so no branch separates the MFMAs of one.
  const int nb = ((k1 - k0 + 31) / 32 + B - 1) / B;
  for (int b = 0;;) {
    if (b + 1 < nb) issue(b + 1, lb, hb);
    compute(b, la, ha);
    if (++b == nb) break;
    if (b + 1 < nb) issue(b + 1, la, ha);
    compute(b, lb, hb);
    if (++b == nb) break;
  }
  // Output rows 4·(l / 16) + r of the lane's columns.
  if (live) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * q + r;
      if (m < M) {
        float* dst = part + ((int64_t)blockIdx.y * M + m) * N + col;
        if constexpr (VEC) {
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (col + i < N) dst[i] = acc[i][r];
        }
      }
    }
  }
}

// Y[m, n] = sum over slices, in slice order; the partials of up to 8 slices
// are loaded together before they are added.
__global__ __launch_bounds__(NT) void k_dq_reduce(const float* part, int S, int64_t MN, void* Y,
                                                  int ydt) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < MN; i += (int64_t)gridDim.x * NT) {
    float s = 0.0f;
    for (int k0 = 0; k0 < S; k0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = k0 + u < S ? part[(int64_t)(k0 + u) * MN + i] : 0.0f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < S) s += v[u];
    }
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

struct DqPlan {
  int S, Lk;
  size_t lds;
};

template <int BITS>
const void* dq_kernel(bool vec) {
  return vec ? reinterpret_cast<const void*>(&k_dq_mfma<BITS, true>)
             : reinterpret_cast<const void*>(&k_dq_mfma<BITS, false>);
}

// Workgroups of the small-M kernel resident at once on the current device with
// `lds` bytes of LDS each (a fixed guess if the runtime cannot say); the
// answers are remembered per device, bit width, load form and LDS size.
int dq_capacity(int bits, bool vec, size_t lds) {
  struct Entry {
    int dev, bits, vec;
    size_t lds;
    int cap;
  };
  static std::mutex mu;
  static std::vector<Entry> seen;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256 * 3;
  }
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& e : seen)
      if (e.dev == dev && e.bits == bits && e.vec == (int)vec && e.lds == lds) return e.cap;
  }
  const void* f = bits == 2 ? dq_kernel<2>(vec) : bits == 3 ? dq_kernel<3>(vec)
                : bits == 4 ? dq_kernel<4>(vec) : dq_kernel<8>(vec);
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, f, NT, lds) != hipSuccess ||
      cus <= 0 || per <= 0) {
    (void)hipGetLastError();
    return 256 * 3;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (seen.size() < 4096) seen.push_back(Entry{dev, bits, (int)vec, lds, cus * per});
  return cus * per;
}

size_t dq_lds_bytes(int64_t M, int64_t Lp, int64_t L, int64_t g, int64_t K) {
  const int64_t G = K / g;
  int64_t ng = (L - 1) / g + 2;   // groups a slice of L can touch
  if (ng > G) ng = G;
  return (size_t)((M * (Lp + 8) * 2 + 15) / 16 * 16 + ng * DQ_GSTRIDE * 12 + Lp / 8 * 4);
}

// Slices of the small-M product. Lk is a multiple of 32 no longer than the X
// budget (M rows), the group budget and DQ_MAX_LK allow; the kernel runs
// whole batches of 32·B, so a slice costs its length rounded up to that, plus
// DQ_WG_COST, plus its partial sums. Among slice counts, the one with the least
// (waves of resident workgroups) x (cost of a slice) wins, the fewest slices
// on ties.
DqPlan dq_plan(int bits, bool vec, int64_t N, int64_t K, int64_t M, int64_t g) {
  const int64_t unit = 32 * (bits == 4 ? 8 : bits == 3 ? 2 : 4);
  const int64_t colblocks = (N + DQ_COLS - 1) / DQ_COLS;
  const int64_t Mr = M > 0 ? M : 1;
  const int64_t Kr = (K + 31) / 32 * 32;
  const int64_t Lx = (DQ_X_LDS / Mr / 2 - 8) / 32 * 32;
  const int64_t maxg = DQ_G_LDS / (DQ_GSTRIDE * 12);                // group rows that fit
  const int64_t Lg = g >= K ? Kr : (maxg - 2) * g / 32 * 32;          // slice touches <= L/g + 2
  int64_t Lmax = Kr < DQ_MAX_LK ? Kr : DQ_MAX_LK;
  if (Lx < Lmax) Lmax = Lx;
  if (Lg < Lmax) Lmax = Lg;
  if (Lmax < 32) Lmax = 32;
  DqPlan best{0, 0, 0};
  int64_t best_cost = -1;
  int cap = -1;
  size_t cap_lds = 0;
  for (int64_t s = (K + Lmax - 1) / Lmax; s <= (K + 31) / 32; ++s) {
    int64_t L = ((K + s - 1) / s + 31) / 32 * 32;
    if (L >= unit && L % unit != 0) {   // whole batches when the budget allows
      const int64_t Lu = (L + unit - 1) / unit * unit;
      if (Lu <= Lmax) L = Lu;
    }
    if (L > Lmax) continue;
    const int64_t S = (K + L - 1) / L;
    if (S != s) continue;               // the same plan as a smaller count
    const int64_t Lp = (L + unit - 1) / unit * unit;
    const size_t lds = dq_lds_bytes(Mr, Lp, L, g, K);
    if (cap < 0 || lds != cap_lds) {
      cap = dq_capacity(bits, vec, lds);
      cap_lds = lds;
    }
    // the slice's partial sums (written, then read by the reduction) cost as
    // many HBM bytes as 64·M/BITS k of packed words
    const int64_t waves = (colblocks * S + cap - 1) / cap;
    const int64_t cost = waves * (Lp + DQ_WG_COST + (S > 1 ? 64 * Mr / bits : 0));
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = DqPlan{(int)S, (int)L, lds};
    }
    if (L <= 32) break;
  }
  return best;
}

template <int BITS>
ar_status dq_small(const DqArgs& a, const uint16_t* X, int M, float* part, const DqPlan& p,
                   bool vec, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + DQ_COLS - 1) / DQ_COLS), (unsigned)p.S);
  if (vec)
    hipLaunchKernelGGL((k_dq_mfma<BITS, true>), grid, dim3(NT), p.lds, st, a, X, M, part, p.Lk);
  else
    hipLaunchKernelGGL((k_dq_mfma<BITS, false>), grid, dim3(NT), p.lds, st, a, X, M, part, p.Lk);
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

// 16-byte packed-word loads need N % 4 == 0 and an aligned qweight.
static bool dq_vec(const int32_t* qweight, int64_t N) {
  return N % 4 == 0 && (reinterpret_cast<uintptr_t>(qweight) & 15) == 0;
}

int ar_dq_slices(int bits, int64_t N, int64_t K, int64_t M, int64_t g) {
  return dq_plan(bits, N % 4 == 0, N, K, M, g).S;
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
  const bool vec = dq_vec(qweight, N);
  const DqPlan p = dq_plan(bits, N % 4 == 0, N, K, M, g);   // as the workspace size assumed
  ar_status s;
  switch (bits) {
    case 2: s = dq_small<2>(a, X, M, part, p, vec, st); break;
    case 3: s = dq_small<3>(a, X, M, part, p, vec, st); break;
    case 4: s = dq_small<4>(a, X, M, part, p, vec, st); break;
    case 8: s = dq_small<8>(a, X, M, part, p, vec, st); break;
    default: return AR_ERR_UNSUPPORTED;
  }
  if (s != AR_OK) return s;
  const int64_t MN = (int64_t)M * N;
  const int64_t nb = (MN + NT - 1) / NT;
  hipLaunchKernelGGL(k_dq_reduce, dim3((unsigned)(nb < 65536 ? nb : 65536)), dim3(NT), 0, st, part,
                     p.S, MN, Y, ydt);
  return last_status();
}
