// Quantizer-side kernels of the tuning step (gfx950): fake-quant, the
// straight-through fold + SignSGD update that follows the gradient product,
// staging of the GEMM operands into their blocked layout, and int32 packing.
// All HBM-bound; every group of g
// contiguous input channels of one output row is handled by LPG consecutive
// lanes, each lane streaming 8-element chunks (16 B of bf16 / 32 B of float32)
// so that a wave reads contiguous, coalesced spans.
//
// Sources: llm-compressor AutoRound page (paper-core equations for RTN, the
// learnable offset and SignSGD; _fake_quantize_with_offset; the per-module
// tuning loop), Introducing AutoRound page section 2 (clip range tuned with
// the rounding), SGLang AutoRound page "1. AutoRoundConfig" (pack_factor).
#include <math.h>

#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"
#include "ar_ste.h"

void ar_group_layout(int g, int* lpg, int* chunks_per_lane) {
  const int chunks = g / 8;
  int l = 1;
  while (l < 64 && chunks % (2 * l) == 0) l *= 2;
  *lpg = l;
  *chunks_per_lane = chunks / l;
}

namespace {

constexpr int NT = 256;

// ------------------------------------------------------------------ initial scale
// The MSE shrink of one group (see ArInit): for every candidate p the group is
// quantized with V = 0 and alpha = beta = p; the float32 errors w - Ŵ are
// squared in float32 and summed in float64 (each lane over its chunks in
// order, then a butterfly, so every lane of the group sees the same sums).
template <typename WT, int LPG>
__device__ __forceinline__ float mse_search(const WT* W, int64_t base, int lig, int E, float mn,
                                            float mx, const Grid& gr, const ArInit& in) {
  double best = INFINITY;
  float bp = 1.0f;
  for (int j = in.j0; j <= in.j1; ++j) {
    const float p = (float)(1.0 - (double)j / (double)in.grid);
    const QP q = group_qparams(mn, mx, p, p, gr);
    double err = 0.0;
    for (int e = 0; e < E; ++e) {
      float w[8];
      load8(W + base + 8 * (lig + LPG * e), w);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = w[i] - quant_elem(w[i], 0.0f, q, gr).what;
        err += (double)(d * d);
      }
    }
    err = group_sum_f64<LPG>(err);
    if (err < best) {
      best = err;
      bp = p;
    }
  }
  return bp;
}

template <typename WT>
struct InitArgs {
  const WT* W;
  int64_t ngroups, K;
  int g, Gn, E;
  ArGrid gr;
  ArInit init;
  float* alpha;
  float* beta;
};

template <typename WT, int LPG>
__global__ __launch_bounds__(NT) void k_init_clip(InitArgs<WT> a) {
  const int64_t gid = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPG;
  const int lig = threadIdx.x % LPG;
  if (gid >= a.ngroups) return;
  const Grid gr = grid_of(a.gr);
  const int64_t n = gid / a.Gn;
  const int64_t base = n * a.K + (gid - n * a.Gn) * a.g;
  float p = a.init.shrink;
  if (a.init.mse) {
    float mn = INFINITY, mx = -INFINITY;
    for (int e = 0; e < a.E; ++e) {
      float w[8];
      load8(a.W + base + 8 * (lig + LPG * e), w);
#pragma unroll
      for (int i = 0; i < 8; ++i) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
    }
    mn = group_min<LPG>(mn);
    mx = group_max<LPG>(mx);
    p = mse_search<WT, LPG>(a.W, base, lig, a.E, mn, mx, gr, a.init);
  }
  if (lig == 0) {
    a.alpha[gid] = p;
    a.beta[gid] = p;
  }
}

// ------------------------------------------------------------------ fake-quant
template <typename WT, typename OT>
struct FQArgs {
  const WT* W;
  const float* V;
  const float* alpha;
  const float* beta;
  ArInit init;
  int64_t ngroups, K;
  int g, Gn, E;
  ArGrid gr;
  OT* Wq;
  int64_t wq_nkb;   // > 0: Wq in the blocked GEMM layout with this many k-blocks
  uint8_t* codes;
  float* scale;
  uint8_t* zp;
};

template <typename WT, typename OT, int LPG>
__global__ __launch_bounds__(NT) void k_fakequant(FQArgs<WT, OT> a) {
  const int64_t gid = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPG;
  const int lig = threadIdx.x % LPG;
  if (gid >= a.ngroups) return;
  const Grid gr = grid_of(a.gr);
  const int64_t n = gid / a.Gn;
  const int64_t base = n * a.K + (gid - n * a.Gn) * a.g;

  float mn = INFINITY, mx = -INFINITY;
  for (int e = 0; e < a.E; ++e) {
    float w[8];
    load8(a.W + base + 8 * (lig + LPG * e), w);
#pragma unroll
    for (int i = 0; i < 8; ++i) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
  }
  mn = group_min<LPG>(mn);
  mx = group_max<LPG>(mx);
  float p0 = a.init.shrink;
  if ((!a.alpha || !a.beta) && a.init.mse)
    p0 = mse_search<WT, LPG>(a.W, base, lig, a.E, mn, mx, gr, a.init);
  const float al = a.alpha ? a.alpha[gid] : p0;
  const float be = a.beta ? a.beta[gid] : p0;
  const QP p = group_qparams(mn, mx, al, be, gr);
  if (lig == 0) {
    if (a.scale) a.scale[gid] = p.s;
    if (a.zp) a.zp[gid] = (uint8_t)(int)p.zp;
  }
  for (int e = 0; e < a.E; ++e) {
    const int64_t off = base + 8 * (lig + LPG * e);
    float w[8], v[8], q[8], wh[8];
    load8(a.W + off, w);
    if (a.V) {
      load8(a.V + off, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const QE qe = quant_elem(w[i], v[i], p, gr);
      q[i] = qe.q;
      wh[i] = qe.what;
    }
    if (a.Wq) {
      if (a.wq_nkb > 0)
        store8(a.Wq + arblk::chunk_offset(n, off - n * a.K, a.wq_nkb), wh);
      else
        store8(a.Wq + off, wh);
    }
    if (a.codes) store8_u8(a.codes + off, q);
  }
}

// ONE: each lane holds exactly one chunk of its group (the whole step runs on
// registers); otherwise chunks are re-read per phase.
template <typename WT, int LPG, bool ONE>
__global__ __launch_bounds__(NT) void k_ste_update(SteK<WT> a) {
  const int64_t gid = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPG;
  const int lig = threadIdx.x % LPG;
  if (gid >= a.ngroups) return;
  const int64_t n = gid / a.Gn;
  const int64_t base = n * a.K + (gid - n * a.Gn) * a.g;
  const int64_t off0 = base + 8 * lig;
  if (ONE) {
    // the chunk, the clip factors and the snapshot flag are all requested
    // before the first wait: one round trip to memory for a small layer (the
    // flag as a vector load, which the compiler keeps where it stands)
    float w[8], v[8], g[8];
    load8(a.W + off0, w);
    load8(a.V + off0, v);
    load8(a.G + off0, g);
    const float al = a.alpha[gid], be = a.beta[gid];
    const bool snap =
        __hip_atomic_load(a.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    ste_one<WT, LPG>(a, snap, gid, n, off0, lig, w, v, g, al, be, true);
    return;
  }
  const bool snap = *a.flag != 0;
  const Grid gr = grid_of(a.gr);

  // phase 1: group min / max (the Min-Max range)
  float mn = INFINITY, mx = -INFINITY;
  for (int e = 0; e < a.E; ++e) {
    float w[8];
    load8(a.W + off0 + 8 * LPG * e, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn = fminf(mn, w[i]);
      mx = fmaxf(mx, w[i]);
    }
  }
  mn = group_min<LPG>(mn);
  mx = group_max<LPG>(mx);
  const float al = a.alpha[gid], be = a.beta[gid];
  const QP p = group_qparams(mn, mx, al, be, gr);

  // phase 2: straight-through sums over the group
  float A = 0.0f, Bs = 0.0f;
  for (int e = 0; e < a.E; ++e) {
    float w[8], v[8], g[8];
    const int64_t off = off0 + 8 * LPG * e;
    load8(a.W + off, w);
    load8(a.V + off, v);
    load8(a.G + off, g);
    ste_accum(w, v, g, p, gr, A, Bs);
  }
  A = group_sum<LPG>(A);
  Bs = group_sum<LPG>(Bs);
  float an, bn;
  clip_update(a, snap, gid, lig, mn, mx, al, be, p, A, Bs, true, an, bn);
  const QP pn = group_qparams(mn, mx, an, bn, gr);

  // phase 3: offsets, snapshot, next fake-quant
  for (int e = 0; e < a.E; ++e) {
    float w[8], v[8], g[8];
    const int64_t off = off0 + 8 * LPG * e;
    load8(a.W + off, w);
    load8(a.V + off, v);
    load8(a.G + off, g);
    ste_finish(a, n, off, w, v, g, p, pn, gr, snap);
  }
}

__global__ __launch_bounds__(NT) void k_fill_f32(float* p, float v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    p[i] = v;
}

// ------------------------------------------------------------------ non-finite scan
// *flag = 1 when any of the nbytes / EB elements at p (float32: EB = 4, bf16:
// EB = 2) is NaN or infinite (all exponent bits set); *flag is left as it is
// otherwise. vec: p is 16-byte aligned and the bulk is read 16 bytes at a time.
template <int EB>
__device__ __forceinline__ bool word_nonfinite(uint32_t w) {
  if (EB == 4) return (w & 0x7F800000u) == 0x7F800000u;
  return (w & 0x7F80u) == 0x7F80u || (w & 0x7F800000u) == 0x7F800000u;
}

template <int EB>
__global__ __launch_bounds__(NT) void k_nonfinite(const uint8_t* __restrict__ p, int64_t nbytes,
                                                  int vec, int* flag) {
  const int64_t tid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * NT;
  const int64_t nvec = vec ? nbytes / 16 : 0;
  bool bad = false;
  const uint4* v = reinterpret_cast<const uint4*>(p);
  for (int64_t i = tid; i < nvec; i += stride) {
    const uint4 q = v[i];
    bad |= word_nonfinite<EB>(q.x) | word_nonfinite<EB>(q.y) | word_nonfinite<EB>(q.z) |
           word_nonfinite<EB>(q.w);
  }
  for (int64_t b = nvec * 16 + tid * EB; b < nbytes; b += stride * EB) {
    const uint32_t w = EB == 4 ? *reinterpret_cast<const uint32_t*>(p + b)
                               : (uint32_t)*reinterpret_cast<const uint16_t*>(p + b);
    bad |= word_nonfinite<EB>(w);
  }
  if (bad) *flag = 1;
}

// ------------------------------------------------------------------ GEMM operand staging
// Row-major src [R, KR] (row stride KR) -> blocked dst (rows R, reduction KR),
// zero padding to whole blocks. One workgroup per 256 rows x 64 reduction
// elements (two blocks): eight lanes read a row's 128 bytes, and the 8 rows of
// one instruction land as two 512-byte runs, one per block.
__global__ __launch_bounds__(NT) void k_block_copy(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, int64_t R,
                                                   int64_t KR, int64_t nkb, int64_t src_batch,
                                                   int64_t dst_batch) {
  const int64_t npair = (nkb + 1) / 2;
  const int64_t rt = blockIdx.x / npair, kp = blockIdx.x - rt * npair;
  const int64_t b = blockIdx.y;
  src += b * src_batch;
  dst += b * dst_batch;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int local = it * NT + threadIdx.x;          // 0 .. 2047
    const int64_t r = rt * arblk::ROWS + (local >> 3);
    const int64_t k = kp * 2 * arblk::KB + (local & 7) * 8;
    if (k >= nkb * arblk::KB) continue;               // odd nkb: the pair's second block is absent
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < R && k < KR) v = *reinterpret_cast<const u32x4_t*>(src + r * KR + k);
    *reinterpret_cast<u32x4_t*>(dst + arblk::chunk_offset(r, k, nkb)) = v;
  }
}

// Transposed staging: src [R rows, C cols] row-major -> blocked with C rows and
// reduction R (dst row c holds src column c), zero padding. One workgroup per
// destination block (256 dst rows x 32 reduction elements, contiguous in dst):
// the 32 x 256 source tile is read with 16-byte loads along its rows into LDS,
// and the block is written out linearly, 16 bytes per lane, each chunk
// gathered from a tile column. With rdst, the same tile also goes to the
// untransposed blocked copy (rows R, reduction C, rnkb k-blocks): its 8
// k-blocks of 32 rows, 2 KiB contiguous each, so src is read once for both.
template <typename T>
__global__ __launch_bounds__(NT) void k_block_transpose(const T* __restrict__ src, T* __restrict__ dst,
                                                        int64_t R, int64_t C, int64_t nkb,
                                                        int64_t src_batch, int64_t dst_batch,
                                                        int vec, T* __restrict__ rdst, int64_t rnkb,
                                                        int64_t rdst_batch) {
  constexpr int EPC = 16 / (int)sizeof(T);            // elements per 16-byte piece
  constexpr int TS = arblk::ROWS + 16 / (int)sizeof(T); // tile row stride (elements)
  __shared__ __attribute__((aligned(16))) T tile[arblk::KB * TS];
  const int64_t rt = blockIdx.x, kb = blockIdx.y, b = blockIdx.z;
  src += b * src_batch;
  dst += b * dst_batch + ((rt * nkb + kb) << 13);   // the block: 8192 elements of T
  const int64_t c0 = rt * arblk::ROWS, r0 = kb * arblk::KB;
  constexpr int PPR = arblk::ROWS / EPC;               // pieces per tile row
  for (int i = threadIdx.x; i < arblk::KB * PPR; i += NT) {
    const int rk = i / PPR, pc = i - rk * PPR;
    const int64_t r = r0 + rk, c = c0 + (int64_t)pc * EPC;
    T v[EPC];
    if (vec && r < R && c + EPC <= C) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + r * C + c);
      *reinterpret_cast<u32x4_t*>(v) = w;
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = (r < R && c + e < C) ? src[r * C + c + e] : T(0);
    }
    *reinterpret_cast<u32x4_t*>(tile + rk * TS + pc * EPC) = *reinterpret_cast<const u32x4_t*>(v);
  }
  __syncthreads();
  if (rdst != nullptr) {
    // piece (j, rk, lc): k-block c0/32 + j, row r0 + rk, logical chunk lc (8 elements)
    T* rd = rdst + b * rdst_batch;
    for (int q = threadIdx.x; q < 8 * arblk::KB * 4; q += NT) {
      const int j = q >> 7, rk = (q >> 2) & 31, lc = q & 3;
      const int64_t k = c0 + 32 * j + 8 * lc;
      if (k >= rnkb * arblk::KB) continue;
      T v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[rk * TS + 32 * j + 8 * lc + e];
      T* d = rd + arblk::chunk_offset(r0 + rk, k, rnkb);
#pragma unroll
      for (int h = 0; h < 8 / EPC; ++h)
        reinterpret_cast<u32x4_t*>(d)[h] = *reinterpret_cast<const u32x4_t*>(v + h * EPC);
    }
  }
  // chunk q of the block: dst row q / 4, stored chunk q % 4 = logical chunk ^ swizzle
  for (int q = threadIdx.x; q < arblk::ROWS * 4; q += NT) {
    const int rr = q >> 2, lc = (q & 3) ^ ((rr >> 2) & 3);
    T v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[(8 * lc + e) * TS + rr];
    T* d = dst + (int64_t)q * 8;
#pragma unroll
    for (int h = 0; h < 8 / EPC; ++h)
      reinterpret_cast<u32x4_t*>(d)[h] = *reinterpret_cast<const u32x4_t*>(v + h * EPC);
  }
}

// ------------------------------------------------------------------ packing
// A block of CB codes (CB*BITS bits) fills WB whole words: 3-bit codes go 32
// per 3 words; 2/4/8-bit codes 16/8/4 per word.
template <int BITS>
struct PackShape {
  static constexpr int WB = (BITS == 3) ? 3 : 1;
  static constexpr int CB = 32 * WB / BITS;
  static constexpr uint32_t MASK = (1u << BITS) - 1u;
};

template <int BITS>
__device__ __forceinline__ void put_code(uint32_t* out, int c, uint32_t code) {
  const int pos = c * BITS, w = pos >> 5, off = pos & 31;
  out[w] |= code << off;
  if (off + BITS > 32) out[w + 1] |= code >> (32 - off);
}
template <int BITS>
__device__ __forceinline__ uint32_t get_code(const uint32_t* in, int c) {
  const int pos = c * BITS, w = pos >> 5, off = pos & 31;
  uint32_t v = in[w] >> off;
  if (off + BITS > 32) v |= in[w + 1] << (32 - off);
  return v & PackShape<BITS>::MASK;
}

// codes [N, K] -> qweight [K*BITS/32, N]. A workgroup stages a 64 x 256 code
// tile in LDS (coalesced row reads), then each thread packs one block of one
// row and the stores of consecutive threads hit consecutive columns.
// The WB words of one block of CB codes, one code per byte at b (16-byte
// aligned LDS), each masked to BITS bits, LSB first. 4- and 2-bit codes are
// merged within each 32-bit word by shifts, then gathered with v_perm.
template <int BITS>
__device__ __forceinline__ void pack_block(const uint8_t* b, uint32_t (&out)[PackShape<BITS>::WB]) {
  if constexpr (BITS == 8) {
    out[0] = *reinterpret_cast<const uint32_t*>(b);
  } else if constexpr (BITS == 4) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(b);
    const uint32_t x = v[0] & 0x0F0F0F0Fu, y = v[1] & 0x0F0F0F0Fu;
    // bytes 0 and 2 of x | x >> 4 hold codes (0,1) and (2,3)
    out[0] = __builtin_amdgcn_perm(y | (y >> 4), x | (x >> 4), 0x06040200u);
  } else if constexpr (BITS == 2) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(b);
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = v[i] & 0x03030303u;
      const uint32_t t = (x | (x >> 6)) & 0x000F000Fu;   // codes (0,1) at bit 0, (2,3) at 16
      u[i] = t | (t >> 12);                               // four codes in byte 0
    }
    out[0] = __builtin_amdgcn_perm(u[1], u[0], 0x0C0C0400u) |
             (__builtin_amdgcn_perm(u[3], u[2], 0x0C0C0400u) << 16);
  } else {
    const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(b);
    const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(b + 16);
    uint32_t o[PackShape<BITS>::WB + 1] = {};
#pragma unroll
    for (int c = 0; c < PackShape<BITS>::CB; ++c) {
      const uint32_t w = c < 16 ? v0[(c >> 2) & 3] : v1[(c >> 2) & 3];
      put_code<BITS>(o, c, (w >> (8 * (c & 3))) & PackShape<BITS>::MASK);
    }
#pragma unroll
    for (int w = 0; w < PackShape<BITS>::WB; ++w) out[w] = o[w];
  }
}

// codes [N, K] -> qweight [K*BITS/32, N] through an LDS tile of 64 rows x 256
// codes: coalesced 16-byte loads along K (4-byte loads when K % 16 != 0), and
// word stores coalesced along N. (bx, by) = (256-code block along K, 64-row
// block along N).
constexpr int PK_ROW = 256 + 16;   // LDS bytes per tile row
template <int BITS, bool V16>
__device__ __forceinline__ void pack_w_tile(uint8_t* tile, const uint8_t* __restrict__ codes,
                                            uint32_t* __restrict__ qw, int64_t N, int64_t K,
                                            int64_t bx, int64_t by) {
  using S = PackShape<BITS>;
  const int64_t n0 = by * 64, k0 = bx * 256;
  if constexpr (V16) {
    for (int i = threadIdx.x; i < 64 * 16; i += NT) {
      const int r = i >> 4, c = i & 15;
      const int64_t n = n0 + r, k = k0 + 16 * c;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (n < N && k < K) v = *reinterpret_cast<const u32x4_t*>(codes + n * K + k);
      *reinterpret_cast<u32x4_t*>(tile + r * PK_ROW + 16 * c) = v;
    }
  } else {
    for (int i = threadIdx.x; i < 64 * 64; i += NT) {
      const int r = i >> 6, c = i & 63;
      const int64_t n = n0 + r, k = k0 + 4 * c;
      uint32_t v = 0;
      if (n < N && k < K) v = *reinterpret_cast<const uint32_t*>(codes + n * K + k);
      *reinterpret_cast<uint32_t*>(tile + r * PK_ROW + 4 * c) = v;
    }
  }
  __syncthreads();
  constexpr int NB = 256 / S::CB;
  const int64_t wrow0 = k0 * BITS / 32;
  for (int it = threadIdx.x; it < 64 * NB; it += NT) {
    const int r = it & 63, blk = it >> 6;
    const int64_t n = n0 + r, kb = k0 + (int64_t)blk * S::CB;
    if (n >= N || kb >= K) continue;
    uint32_t out[S::WB];
    pack_block<BITS>(tile + r * PK_ROW + blk * S::CB, out);
#pragma unroll
    for (int w = 0; w < S::WB; ++w) qw[(wrow0 + (int64_t)blk * S::WB + w) * N + n] = out[w];
  }
}

// zp [N, G] -> qzeros [G, N*BITS/32]: the same bit layout along N. A workgroup
// takes 256 columns and PZ_G groups into an LDS tile transposed to
// [group][column], then stores each group's words contiguously. When one chunk
// holds every group, the workgroup's zero-points are one contiguous run of
// rows·G bytes (16-byte aligned with zp: 256·G is a multiple of 16), read in
// 16-byte pieces whatever G is. (bx, by) = (256-column block, PZ_G-group chunk).
constexpr int PZ_G = 64;    // groups per zero-point tile: its LDS equals the code tile's (64 rows)
template <int BITS>
__device__ __forceinline__ void pack_z_tile(uint8_t* tile, const uint8_t* __restrict__ zp,
                                            uint32_t* __restrict__ qz, int64_t N, int64_t G,
                                            int64_t bx, int64_t by) {
  using S = PackShape<BITS>;
  const int64_t n0 = bx * 256, j0 = by * PZ_G;
  const int gc = (int)(G - j0 < PZ_G ? G - j0 : PZ_G);
  const int rows = (int)(N - n0 < 256 ? N - n0 : 256);
  const int64_t words = N * BITS / 32;
  constexpr int NB = 256 / S::CB;
  if (gc == G && (reinterpret_cast<uintptr_t>(zp) & 15) == 0) {
    const uint8_t* run = zp + n0 * G;
    const int len = rows * (int)G, full = len / 16;
    for (int i = threadIdx.x; i < full; i += NT) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(run + 16 * i);
      int r = 16 * i / (int)G, c = 16 * i - r * (int)G;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        tile[c * PK_ROW + r] = (uint8_t)(v[e >> 2] >> (8 * (e & 3)));
        if (++c == (int)G) {
          c = 0;
          ++r;
        }
      }
    }
    for (int o = 16 * full + threadIdx.x; o < len; o += NT) {
      const int r = o / (int)G, c = o - r * (int)G;
      tile[c * PK_ROW + r] = run[o];
    }
  } else {
    for (int i = threadIdx.x; i < rows * gc; i += NT) {
      const int r = i / gc, c = i - r * gc;
      tile[c * PK_ROW + r] = zp[(n0 + r) * G + j0 + c];
    }
  }
  for (int i = threadIdx.x; i < (256 - rows) * gc; i += NT) {   // past N: zero
    const int r = rows + i / gc, c = i % gc;
    tile[c * PK_ROW + r] = 0;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < gc * NB; it += NT) {
    const int jj = it / NB, blk = it - jj * NB;
    if (blk * S::CB >= rows) continue;
    uint32_t out[S::WB];
    pack_block<BITS>(tile + jj * PK_ROW + blk * S::CB, out);
#pragma unroll
    for (int w = 0; w < S::WB; ++w)
      qz[(j0 + jj) * words + (n0 / S::CB + blk) * S::WB + w] = out[w];
  }
}

// Both packs in one launch (they share nothing): workgroups [0, nw) pack the
// codes, the pack_w grid walked along K first; the rest pack the zero-points.
template <int BITS, bool V16>
__global__ __launch_bounds__(NT) void k_pack(const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ zp,
                                             uint32_t* __restrict__ qw, uint32_t* __restrict__ qz,
                                             int64_t N, int64_t K, int64_t G, int64_t wx,
                                             int64_t nw, int64_t zx) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[PZ_G * PK_ROW];
  const int64_t b = blockIdx.x;
  if (b < nw) {
    pack_w_tile<BITS, V16>(tile, codes, qw, N, K, b % wx, b / wx);
  } else {
    const int64_t z = b - nw;
    pack_z_tile<BITS>(tile, zp, qz, N, G, z % zx, z / zx);
  }
}

template <int BITS>
__global__ __launch_bounds__(NT) void k_unpack_w(const uint32_t* __restrict__ qw,
                                                 uint8_t* __restrict__ codes, int64_t N, int64_t K) {
  using S = PackShape<BITS>;
  const int64_t nblk = K / S::CB;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= N * nblk) return;
  const int64_t blk = idx / N, n = idx - blk * N;
  uint32_t in[S::WB + 1] = {};
#pragma unroll
  for (int w = 0; w < S::WB; ++w) in[w] = qw[(blk * S::WB + w) * N + n];
  for (int c = 0; c < S::CB; ++c) codes[n * K + blk * S::CB + c] = (uint8_t)get_code<BITS>(in, c);
}

template <int BITS>
__global__ __launch_bounds__(NT) void k_unpack_z(const uint32_t* __restrict__ qz,
                                                 uint8_t* __restrict__ zp, int64_t N, int64_t G) {
  using S = PackShape<BITS>;
  const int64_t nblk = N / S::CB;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= G * nblk) return;
  const int64_t j = idx / nblk, blk = idx - j * nblk;
  const int64_t words = N * BITS / 32;
  uint32_t in[S::WB + 1] = {};
#pragma unroll
  for (int w = 0; w < S::WB; ++w) in[w] = qz[j * words + blk * S::WB + w];
  for (int c = 0; c < S::CB; ++c) zp[(blk * S::CB + c) * G + j] = (uint8_t)get_code<BITS>(in, c);
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + NT - 1) / NT); }
inline ar_status last_status() { return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP; }

template <typename WT, typename OT>
ar_status fq_dispatch(FQArgs<WT, OT> a, int lpg, hipStream_t st) {
  const unsigned nb = blocks_for(a.ngroups * lpg);
  switch (lpg) {
#define AR_FQ_CASE(L) \
  case L: hipLaunchKernelGGL((k_fakequant<WT, OT, L>), dim3(nb), dim3(NT), 0, st, a); break;
    AR_FQ_CASE(1) AR_FQ_CASE(2) AR_FQ_CASE(4) AR_FQ_CASE(8) AR_FQ_CASE(16) AR_FQ_CASE(32)
    AR_FQ_CASE(64)
#undef AR_FQ_CASE
    default: return AR_ERR_INVALID_ARG;
  }
  return last_status();
}

template <typename WT, typename OT>
ar_status fq_make(const void* W, const float* V, const float* alpha, const float* beta,
                  const ArInit& init, int64_t N, int64_t K, int g, ArGrid gr, void* Wq,
                  int64_t wq_nkb, uint8_t* codes, float* scale, uint8_t* zp, hipStream_t st) {
  int lpg, E;
  ar_group_layout(g, &lpg, &E);
  FQArgs<WT, OT> a{static_cast<const WT*>(W), V, alpha, beta, init, N * (K / g), K, g,
                   (int)(K / g), E, gr, static_cast<OT*>(Wq), wq_nkb, codes, scale, zp};
  return fq_dispatch(a, lpg, st);
}

template <typename WT>
ar_status init_make(const void* W, int64_t N, int64_t K, int g, ArGrid gr, const ArInit& init,
                    float* alpha, float* beta, hipStream_t st) {
  int lpg, E;
  ar_group_layout(g, &lpg, &E);
  InitArgs<WT> a{static_cast<const WT*>(W), N * (K / g), K, g, (int)(K / g), E, gr, init, alpha,
                 beta};
  const unsigned nb = blocks_for(a.ngroups * lpg);
  switch (lpg) {
#define AR_IC_CASE(L) \
  case L: hipLaunchKernelGGL((k_init_clip<WT, L>), dim3(nb), dim3(NT), 0, st, a); break;
    AR_IC_CASE(1) AR_IC_CASE(2) AR_IC_CASE(4) AR_IC_CASE(8) AR_IC_CASE(16) AR_IC_CASE(32)
    AR_IC_CASE(64)
#undef AR_IC_CASE
    default: return AR_ERR_INVALID_ARG;
  }
  return last_status();
}

template <typename WT>
ar_status ste_make(const ArSteArgs& s, hipStream_t st) {
  int lpg, E;
  ar_group_layout(s.g, &lpg, &E);
  const SteK<WT> a = ste_args<WT>(s, E);
  const unsigned nb = blocks_for(a.ngroups * lpg);
  switch (lpg * 2 + (E == 1 ? 1 : 0)) {
#define AR_STE_CASE(L)                                                                          \
  case 2 * L + 1:                                                                               \
    hipLaunchKernelGGL((k_ste_update<WT, L, true>), dim3(nb), dim3(NT), 0, st, a); break;       \
  case 2 * L:                                                                                   \
    hipLaunchKernelGGL((k_ste_update<WT, L, false>), dim3(nb), dim3(NT), 0, st, a); break;
    AR_STE_CASE(1) AR_STE_CASE(2) AR_STE_CASE(4) AR_STE_CASE(8) AR_STE_CASE(16)
    AR_STE_CASE(32) AR_STE_CASE(64)
#undef AR_STE_CASE
    default: return AR_ERR_INVALID_ARG;
  }
  return last_status();
}

}  // namespace

ar_status ar_launch_fakequant(int wdt, const void* W, const float* V, const float* alpha,
                              const float* beta, const ArInit& init, int64_t N, int64_t K, int g,
                              ArGrid gr, int out_dt, void* Wq, int64_t wq_nkb, uint8_t* codes,
                              float* scale, uint8_t* zp, hipStream_t st) {
  if (wq_nkb > 0 && out_dt != AR_BF16) return AR_ERR_INVALID_ARG;
  if (wdt == AR_BF16) {
    if (out_dt == AR_BF16)
      return fq_make<uint16_t, uint16_t>(W, V, alpha, beta, init, N, K, g, gr, Wq, wq_nkb, codes, scale, zp, st);
    return fq_make<uint16_t, float>(W, V, alpha, beta, init, N, K, g, gr, Wq, wq_nkb, codes, scale, zp, st);
  }
  if (out_dt == AR_BF16)
    return fq_make<float, uint16_t>(W, V, alpha, beta, init, N, K, g, gr, Wq, wq_nkb, codes, scale, zp, st);
  return fq_make<float, float>(W, V, alpha, beta, init, N, K, g, gr, Wq, wq_nkb, codes, scale, zp, st);
}

ar_status ar_launch_init_clip(int wdt, const void* W, int64_t N, int64_t K, int g, ArGrid gr,
                              const ArInit& init, float* alpha, float* beta, hipStream_t st) {
  return wdt == AR_BF16 ? init_make<uint16_t>(W, N, K, g, gr, init, alpha, beta, st)
                        : init_make<float>(W, N, K, g, gr, init, alpha, beta, st);
}

ar_status ar_launch_block_copy(const uint16_t* src, uint16_t* dst, int64_t batch, int64_t R,
                               int64_t KR, int64_t nkb, hipStream_t st) {
  if (batch <= 0 || R <= 0 || nkb <= 0) return AR_OK;
  const int64_t wgs = arblk::row_tiles(R) * ((nkb + 1) / 2);
  if (wgs > 0x7FFFFFFF || batch > 65535) return AR_ERR_SHAPE;
  hipLaunchKernelGGL(k_block_copy, dim3((unsigned)wgs, (unsigned)batch), dim3(NT), 0, st, src,
                     dst, R, KR, nkb, R * KR, arblk::row_tiles(R) * nkb * arblk::BLOCK_ELEMS);
  return last_status();
}

ar_status ar_launch_block_transpose(const void* src, void* dst, int64_t batch, int64_t R,
                                    int64_t C, int64_t nkb, int elem_bytes, hipStream_t st) {
  if (batch <= 0 || R <= 0 || C <= 0) return AR_OK;
  if (nkb > 65535 || batch > 65535) return AR_ERR_SHAPE;   // grid y / z
  const int64_t dst_batch = arblk::row_tiles(C) * nkb * arblk::BLOCK_ELEMS;
  // one workgroup per destination block; every block, padding included, is written
  const dim3 grid((unsigned)arblk::row_tiles(C), (unsigned)nkb, (unsigned)batch);
  const int epc = 16 / elem_bytes;
  const int vec = C % epc == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                  ((R * C * elem_bytes) & 15) == 0;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_block_transpose<uint16_t>, grid, dim3(NT), 0, st,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), R, C, nkb,
                       R * C, dst_batch, vec, (uint16_t*)nullptr, (int64_t)0, (int64_t)0);
  else
    hipLaunchKernelGGL(k_block_transpose<uint32_t>, grid, dim3(NT), 0, st,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), R, C, nkb,
                       R * C, dst_batch, vec, (uint32_t*)nullptr, (int64_t)0, (int64_t)0);
  return last_status();
}

ar_status ar_launch_stage_x(const uint16_t* X, uint16_t* XTB, uint16_t* XB, int64_t batch,
                            int64_t Tb, int64_t K, int64_t nkbT, int64_t nkbK, hipStream_t st) {
  if (batch <= 0 || Tb <= 0 || K <= 0) return AR_OK;
  if (nkbT > 65535 || batch > 65535) return AR_ERR_SHAPE;   // grid y / z
  // the transpose's blocks cover every XB row (nkbT·32 = row_tiles(Tb)·256) and k-block
  if (nkbT * arblk::KB != arblk::row_tiles(Tb) * arblk::ROWS ||
      nkbK > arblk::row_tiles(K) * (arblk::ROWS / arblk::KB))
    return AR_ERR_SHAPE;
  const int64_t xtb_batch = arblk::row_tiles(K) * nkbT * arblk::BLOCK_ELEMS;
  const int64_t xb_batch = arblk::row_tiles(Tb) * nkbK * arblk::BLOCK_ELEMS;
  const dim3 grid((unsigned)arblk::row_tiles(K), (unsigned)nkbT, (unsigned)batch);
  const int vec = K % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  hipLaunchKernelGGL(k_block_transpose<uint16_t>, grid, dim3(NT), 0, st, X, XTB, Tb, K, nkbT,
                     Tb * K, xtb_batch, vec, XB, nkbK, xb_batch);
  return last_status();
}

ar_status ar_launch_ste_update(const ArSteArgs& s, hipStream_t st) {
  if (s.flag == nullptr) return AR_ERR_INVALID_ARG;
  return s.wdt == AR_BF16 ? ste_make<uint16_t>(s, st) : ste_make<float>(s, st);
}


ar_status ar_launch_fill_f32(float* p, float v, int64_t n, hipStream_t st) {
  if (n <= 0) return AR_OK;
  const int64_t want = (n + NT - 1) / NT;
  const unsigned nb = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_fill_f32, dim3(nb), dim3(NT), 0, st, p, v, n);
  return last_status();
}

ar_status ar_launch_nonfinite(const void* p, int64_t n, int dt, int* flag, hipStream_t st) {
  if (n <= 0) return AR_OK;
  const int eb = dt == AR_BF16 ? 2 : 4;
  const int64_t nbytes = n * eb;
  const int vec = (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
  const int64_t units = vec ? (nbytes + 15) / 16 : n;
  int64_t nb = (units + NT - 1) / NT;
  if (nb > 4096) nb = 4096;
  const uint8_t* b = static_cast<const uint8_t*>(p);
  if (eb == 2)
    hipLaunchKernelGGL(k_nonfinite<2>, dim3((unsigned)nb), dim3(NT), 0, st, b, nbytes, vec, flag);
  else
    hipLaunchKernelGGL(k_nonfinite<4>, dim3((unsigned)nb), dim3(NT), 0, st, b, nbytes, vec, flag);
  return last_status();
}

ar_status ar_launch_pack(int bits, const uint8_t* codes, const uint8_t* zp, int64_t N, int64_t K,
                         int64_t G, int32_t* qweight, int32_t* qzeros, hipStream_t st) {
  const int64_t wx = (K + 255) / 256, nw = wx * ((N + 63) / 64);
  const int64_t zx = (N + 255) / 256, nz = zp ? zx * ((G + PZ_G - 1) / PZ_G) : 0;
  if (nw + nz > 0x7FFFFFFF) return AR_ERR_SHAPE;
  const dim3 grid((unsigned)(nw + nz));
  uint32_t* qw = reinterpret_cast<uint32_t*>(qweight);
  uint32_t* qz = reinterpret_cast<uint32_t*>(qzeros);
  switch (bits) {
#define AR_PACK_CASE(B)                                                                       \
  case B:                                                                                     \
    if (K % 16 == 0)                                                                          \
      hipLaunchKernelGGL((k_pack<B, true>), grid, dim3(NT), 0, st, codes, zp, qw, qz, N, K, G, \
                         wx, nw, zx);                                                         \
    else                                                                                      \
      hipLaunchKernelGGL((k_pack<B, false>), grid, dim3(NT), 0, st, codes, zp, qw, qz, N, K,  \
                         G, wx, nw, zx);                                                      \
    break;
    AR_PACK_CASE(2) AR_PACK_CASE(3) AR_PACK_CASE(4) AR_PACK_CASE(8)
#undef AR_PACK_CASE
    default: return AR_ERR_UNSUPPORTED;
  }
  return last_status();
}

ar_status ar_launch_unpack(int bits, const int32_t* qweight, const int32_t* qzeros, int64_t N,
                           int64_t K, int64_t G, uint8_t* codes, uint8_t* zp, hipStream_t st) {
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  switch (bits) {
#define AR_UNPACK_CASE(B)                                                                       \
  case B:                                                                                       \
    hipLaunchKernelGGL(k_unpack_w<B>, dim3(blocks_for(N * (K / PackShape<B>::CB))), dim3(NT),   \
                       0, st, qw, codes, N, K);                                                 \
    if (zp)                                                                                     \
      hipLaunchKernelGGL(k_unpack_z<B>, dim3(blocks_for(G * (N / PackShape<B>::CB))), dim3(NT), \
                         0, st, qz, zp, N, G);                                                  \
    break;
    AR_UNPACK_CASE(2) AR_UNPACK_CASE(3) AR_UNPACK_CASE(4) AR_UNPACK_CASE(8)
#undef AR_UNPACK_CASE
    default: return AR_ERR_UNSUPPORTED;
  }
  return last_status();
}
