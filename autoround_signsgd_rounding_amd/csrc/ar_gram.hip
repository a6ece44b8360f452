// Gram-form tuning step (gfx950). For a Linear whose quantized and reference
// outputs see the same tokens, the minibatch loss and its Ŵ-gradient depend on
// the tokens only through H = X_bᵀX_b, Cn = (X_b·Wᵀ − Y_b)ᵀX_b and
// e2 = |X_b·Wᵀ − Y_b|²:
//   sum R² = Σ D∘(D·H) + 2·Σ D∘Cn + e2,   dL/dŴ = (2/(T_b·N))·(D·H + Cn),
// with D = bf16(Ŵ) − W. H is the Hessian weight of the layer objective on the
// ADMM-Q page ("1. 문제 공식화"); the loss is the output-reconstruction loss of
// the llm-compressor AutoRound page's tuning loop, evaluated without rounding
// the residual.
//
// One step is one bf16 MFMA product P = D·H and one update kernel. The product
// keeps float32 accuracy through a hi/lo bf16 split over a 3K reduction:
//   P ≈ D_hi·H_hi + D_hi·H_lo + D_lo·H_hi
// (operands [D_hi | D_hi | D_lo] and [H_hi | H_lo | H_hi] in the blocked GEMM
// layout). The update kernel reads P and Cn, forms G = (2/(T_b·N))·(P + Cn) and
// the loss term D·(P + 2·Cn), runs the straight-through fold and SignSGD step
// of the standard path, and writes the next D operand. The new state goes to
// the other half of a ping-pong pair, so the state a loss was taken at is still
// intact when the next product's workgroup 0 has reduced that loss; the best
// state is then copied one step late.
#include <math.h>

#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"
#include "ar_loss.h"
#include "ar_ste.h"

namespace {

constexpr int NT = 256;

inline unsigned grid_for(int64_t threads) {
  const int64_t b = (threads + NT - 1) / NT;
  return (unsigned)(b < 65536 ? b : 65536);
}
inline ar_status last_status() { return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP; }

// ------------------------------------------------------------------ operand placement
// Row-major src [R, C] (C % 8 == 0) into the blocked operand dst (rows R,
// nkb reduction blocks) at reduction offset k_off: lo = 0 stores bf16(x),
// lo = 1 stores bf16(x − bf16(x)). Padding is left as it is (cleared by the caller).
template <typename T>
__global__ __launch_bounds__(NT) void k_place(const T* __restrict__ src, uint16_t* __restrict__ dst,
                                              int64_t R, int64_t C, int64_t nkb, int64_t k_off,
                                              int lo) {
  const int64_t cpr = C / 8;
  const int64_t total = R * cpr;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int64_t r = i / cpr, k = (i - r * cpr) * 8;
    float v[8];
    load8(src + r * C + k, v);
    if (lo) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] - bf16_val(bf16_bits(v[e]));
    }
    store8(dst + arblk::chunk_offset(r, k + k_off, nkb), v);
  }
}

// D = bf16(Ŵ) − W of one chunk, split and stored as [D_hi | D_lo] (each part Kp =
// K rounded up to whole k-blocks wide; the product reads D_hi against both H_hi
// and H_lo).
__device__ __forceinline__ void store_d(uint16_t* DB, int64_t nkbD, int64_t Kp, int64_t n,
                                        int64_t k, const float (&w)[8], const float (&wq)[8]) {
  u32x4_t h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t q = bf16_pair(wq[2 * i], wq[2 * i + 1]);
    const float d0 = __uint_as_float(q << 16) - w[2 * i];
    const float d1 = __uint_as_float(q & 0xFFFF0000u) - w[2 * i + 1];
    h[i] = bf16_pair(d0, d1);
    l[i] = bf16_pair(d0 - __uint_as_float(h[i] << 16), d1 - __uint_as_float(h[i] & 0xFFFF0000u));
  }
  *reinterpret_cast<u32x4_t*>(DB + arblk::chunk_offset(n, k, nkbD)) = h;
  *reinterpret_cast<u32x4_t*>(DB + arblk::chunk_offset(n, Kp + k, nkbD)) = l;
}

// ------------------------------------------------------------------ D of a state
template <typename WT>
struct GramD {
  const WT* W;
  const float* V;
  const float* A;
  const float* B;
  int64_t ngroups, K;
  int g, Gn, E;
  ArGrid gr;
  uint16_t* DB;
  int64_t nkbD, Kp;     // D's k-blocks (two parts) and the width of one part
};

template <typename WT, int LPG>
__global__ __launch_bounds__(NT) void k_gram_d(GramD<WT> a) {
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
  const QP p = group_qparams(mn, mx, a.A[gid], a.B[gid], gr);
  for (int e = 0; e < a.E; ++e) {
    const int64_t off = base + 8 * (lig + LPG * e);
    float w[8], v[8], wq[8];
    load8(a.W + off, w);
    load8(a.V + off, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) wq[i] = quant_elem(w[i], v[i], p, gr).what;
    store_d(a.DB, a.nkbD, a.Kp, n, off - n * a.K, w, wq);
  }
}

// ------------------------------------------------------------------ update step
template <typename WT>
struct GramK {
  const WT* W;
  const float* Vc;      // state the product was taken at
  float* Vn;            // next state (holds the previous state on entry)
  const float* Ac;
  const float* Bc;
  float* An;
  float* Bn;
  const float* P;       // D·H, row-major [N, K]
  const float* Cn;      // (X_b·Wᵀ − Y_b)ᵀ·X_b, row-major [N, K]
  int64_t ngroups, K;
  int g, Gn, E;
  ArGrid gr;
  float lr, mlr, clip_lo, clip_hi, scale;
  int apply;
  const int* flag_prev;  // nullable; 1 = copy the previous state (in Vn/An/Bn) to best
  float* bestV;
  float* bestA;
  float* bestB;
  uint16_t* DB;          // next D operand
  int64_t nkbD, Kp;     // D's k-blocks (two parts) and the width of one part
  float* partials;       // per workgroup: sum of D·(P + 2·Cn) over its elements
  float* gV;
  float* gA;
  float* gB;
};

template <typename WT>
__device__ __forceinline__ void gram_load(const GramK<WT>& a, int64_t off, float (&w)[8],
                                          float (&v)[8], float (&p)[8], float (&c)[8]) {
  load8(a.W + off, w);
  load8(a.Vc + off, v);
  load8(a.P + off, p);
  load8(a.Cn + off, c);
}

// G and the loss term of one chunk at the current state.
__device__ __forceinline__ void gram_grad(const float (&w)[8], const float (&v)[8],
                                          const float (&pp)[8], const float (&cc)[8], const QP& p,
                                          const Grid& gr, float scale, float (&g)[8],
                                          float& lsum) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = bf16_val(bf16_bits(quant_elem(w[i], v[i], p, gr).what)) - w[i];
    lsum += d * (pp[i] + 2.0f * cc[i]);
    g[i] = (pp[i] + cc[i]) * scale;
  }
}

// ONE: each lane holds exactly one chunk of its group (kept in registers);
// otherwise chunks are re-read per phase. Lanes past the last group take part
// in the reductions only.
template <typename WT, int LPG, bool ONE>
__global__ __launch_bounds__(NT) void k_ste_gram(GramK<WT> a) {
  __shared__ float red[NT / 64];
  const int64_t gid = ((int64_t)blockIdx.x * NT + threadIdx.x) / LPG;
  const int lig = threadIdx.x % LPG;
  const bool live = gid < a.ngroups;
  const Grid gr = grid_of(a.gr);
  const int64_t n = live ? gid / a.Gn : 0;
  const int64_t off0 = live ? n * a.K + (gid - n * a.Gn) * a.g + 8 * lig : 0;
  const int E = ONE ? 1 : a.E;
  const bool snap = a.flag_prev != nullptr && *a.flag_prev != 0;
  float lsum = 0.0f;

  // phase 1: group min / max
  float w0[8], v0[8], p0[8], c0[8];
  float mn = INFINITY, mx = -INFINITY;
  if (live) {
    for (int e = 0; e < E; ++e) {
      float w[8];
      if (ONE) {
        gram_load(a, off0, w0, v0, p0, c0);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = w0[i];
      } else {
        load8(a.W + off0 + 8 * LPG * e, w);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) { mn = fminf(mn, w[i]); mx = fmaxf(mx, w[i]); }
    }
  }
  mn = group_min<LPG>(mn);
  mx = group_max<LPG>(mx);
  const float al = live ? a.Ac[gid] : 1.0f, be = live ? a.Bc[gid] : 1.0f;
  const QP p = group_qparams(live ? mn : -1.0f, live ? mx : 1.0f, al, be, gr);

  // phase 2: gradient, loss term, straight-through sums
  float A = 0.0f, Bs = 0.0f;
  uint32_t mbits = 0u;   // ONE: element i's straight-through mask under p, kept for phase 3
  if (live && ONE) {
    // gram_grad and ste_accum fused: one quantization per element; each sum
    // (loss term, A, Bs) still adds its terms in element order
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const QE q = quant_elem(w0[i], v0[i], p, gr);
      const float d = __uint_as_float(bf16_pair(q.what, 0.0f) << 16) - w0[i];
      lsum += d * (p0[i] + 2.0f * c0[i]);
      g[i] = (p0[i] + c0[i]) * a.scale;
      const float dd = (q.q - p.zp) - (q.m ? q.t : 0.0f);
      A += g[i] * dd;
      if (!q.m) Bs += g[i];
      mbits |= (uint32_t)q.m << i;
    }
  } else if (live) {
    for (int e = 0; e < E; ++e) {
      float w[8], v[8], pp[8], cc[8], g[8];
      if (ONE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { w[i] = w0[i]; v[i] = v0[i]; pp[i] = p0[i]; cc[i] = c0[i]; }
      } else {
        gram_load(a, off0 + 8 * LPG * e, w, v, pp, cc);
      }
      gram_grad(w, v, pp, cc, p, gr, a.scale, g, lsum);
      ste_accum(w, v, g, p, gr, A, Bs);
    }
  }
  A = group_sum<LPG>(A);
  Bs = group_sum<LPG>(Bs);
  float ga, gb;
  clip_grads(gr, p, mn, mx, al, be, A, Bs, ga, gb);
  float an = al, bn = be;
  if (a.apply) {
    an = fminf(fmaxf(al - a.mlr * sgnf(ga), a.clip_lo), a.clip_hi);
    bn = fminf(fmaxf(be - a.mlr * sgnf(gb), a.clip_lo), a.clip_hi);
  }
  if (live && lig == 0) {
    if (a.gA) a.gA[gid] = ga;
    if (a.gB) a.gB[gid] = gb;
    if (snap) { a.bestA[gid] = a.An[gid]; a.bestB[gid] = a.Bn[gid]; }
    a.An[gid] = an;
    a.Bn[gid] = bn;
  }
  const QP pn = group_qparams(live ? mn : -1.0f, live ? mx : 1.0f, an, bn, gr);

  // phase 3: offsets, the previous state's snapshot, the next D operand
  if (live && ONE) {
    float g[8], gv[8], vn[8], wq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = (p0[i] + c0[i]) * a.scale;
    ste_chunk_update_m(w0, v0, g, mbits, p, pn, gr, a.lr, a.apply, gv, vn, wq);
    if (a.gV) store8(a.gV + off0, gv);
    if (snap) {
      float vo[8];
      load8(a.Vn + off0, vo);
      store8(a.bestV + off0, vo);
    }
    store8(a.Vn + off0, vn);
    store_d(a.DB, a.nkbD, a.Kp, n, off0 - n * a.K, w0, wq);
  } else if (live) {
    for (int e = 0; e < E; ++e) {
      const int64_t off = off0 + 8 * LPG * e;
      float w[8], v[8], pp[8], cc[8], g[8];
      if (ONE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { w[i] = w0[i]; v[i] = v0[i]; pp[i] = p0[i]; cc[i] = c0[i]; }
      } else {
        gram_load(a, off, w, v, pp, cc);
      }
      float dummy = 0.0f;
      gram_grad(w, v, pp, cc, p, gr, a.scale, g, dummy);
      float gv[8], vn[8], wq[8];
      ste_chunk_update(w, v, g, p, pn, gr, a.lr, a.apply, gv, vn, wq);
      if (a.gV) store8(a.gV + off, gv);
      if (snap) {
        float vo[8];
        load8(a.Vn + off, vo);
        store8(a.bestV + off, vo);
      }
      store8(a.Vn + off, vn);
      store_d(a.DB, a.nkbD, a.Kp, n, off - n * a.K, w, wq);
    }
  }

  // the workgroup's loss term, summed in a fixed order
  lsum = wave_sum64(lsum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lsum;
  __syncthreads();
  if (threadIdx.x == 0) a.partials[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ------------------------------------------------------------------ loop tail
__global__ __launch_bounds__(NT) void k_loss_reduce(ArLossIn L) {
  __shared__ double sh[NT];
  loss_reduce_block(L, sh);
}

// Copy a state to the best slots when *flag is set.
__global__ __launch_bounds__(NT) void k_gram_snapshot(const int* flag, const float* V,
                                                      const float* A, const float* B,
                                                      float* bestV, float* bestA, float* bestB,
                                                      int64_t nV, int64_t nG) {
  if (*flag == 0) return;
  const int64_t stride = (int64_t)gridDim.x * NT;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < nV; i += stride) bestV[i] = V[i];
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < nG; i += stride) {
    bestA[i] = A[i];
    bestB[i] = B[i];
  }
}

// ------------------------------------------------------------------ launchers
template <typename WT>
ar_status gram_d_make(const void* W, const float* V, const float* A, const float* B, int64_t N,
                      int64_t K, int g, ArGrid gr, uint16_t* DB, hipStream_t st) {
  int lpg, E;
  ar_group_layout(g, &lpg, &E);
  GramD<WT> a{static_cast<const WT*>(W), V, A, B, N * (K / g), K, g, (int)(K / g), E, gr, DB,
              2 * arblk::k_blocks(K), arblk::k_blocks(K) * arblk::KB};
  const unsigned nb = (unsigned)((a.ngroups * lpg + NT - 1) / NT);
  switch (lpg) {
#define AR_GD_CASE(L) \
  case L: hipLaunchKernelGGL((k_gram_d<WT, L>), dim3(nb), dim3(NT), 0, st, a); break;
    AR_GD_CASE(1) AR_GD_CASE(2) AR_GD_CASE(4) AR_GD_CASE(8) AR_GD_CASE(16) AR_GD_CASE(32)
    AR_GD_CASE(64)
#undef AR_GD_CASE
    default: return AR_ERR_INVALID_ARG;
  }
  return last_status();
}

template <typename WT>
ar_status ste_gram_make(const ArGramArgs& s, hipStream_t st) {
  int lpg, E;
  ar_group_layout(s.g, &lpg, &E);
  GramK<WT> a{static_cast<const WT*>(s.W), s.Vc, s.Vn, s.Ac, s.Bc, s.An, s.Bn, s.P, s.Cn,
              s.N * (s.K / s.g), s.K, s.g, (int)(s.K / s.g), E, s.gr, s.lr, s.mlr, s.clip_lo,
              s.clip_hi, s.scale, s.apply, s.flag_prev, s.bestV, s.bestA, s.bestB, s.DB,
              2 * arblk::k_blocks(s.K), arblk::k_blocks(s.K) * arblk::KB, s.partials, s.gV, s.gA,
              s.gB};
  const unsigned nb = (unsigned)ar_gram_partials(s.N, s.K, s.g);
  switch (lpg * 2 + (E == 1 ? 1 : 0)) {
#define AR_SG_CASE(L)                                                                       \
  case 2 * L + 1:                                                                           \
    hipLaunchKernelGGL((k_ste_gram<WT, L, true>), dim3(nb), dim3(NT), 0, st, a); break;     \
  case 2 * L:                                                                               \
    hipLaunchKernelGGL((k_ste_gram<WT, L, false>), dim3(nb), dim3(NT), 0, st, a); break;
    AR_SG_CASE(1) AR_SG_CASE(2) AR_SG_CASE(4) AR_SG_CASE(8) AR_SG_CASE(16) AR_SG_CASE(32)
    AR_SG_CASE(64)
#undef AR_SG_CASE
    default: return AR_ERR_INVALID_ARG;
  }
  return last_status();
}

// H [K, K] float32 into its operand [H_hi | H_lo | H_hi] (rows K, nkb blocks,
// parts Kp apart) in one pass: each element read once, its three bf16 values
// written where k_place's three launches would put them.
__global__ __launch_bounds__(NT) void k_place_h(const float* __restrict__ H, uint16_t* __restrict__ dst,
                                                int64_t K, int64_t nkb, int64_t Kp) {
  const int64_t cpr = K / 8;
  const int64_t total = K * cpr;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int64_t r = i / cpr, k = (i - r * cpr) * 8;
    float v[8], l[8];
    load8(H + r * K + k, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) l[e] = v[e] - bf16_val(bf16_bits(v[e]));
    store8(dst + arblk::chunk_offset(r, k, nkb), v);
    store8(dst + arblk::chunk_offset(r, Kp + k, nkb), l);
    store8(dst + arblk::chunk_offset(r, 2 * Kp + k, nkb), v);
  }
}

}  // namespace

ar_status ar_launch_place_h(const float* H, int64_t K, uint16_t* dst, int64_t nkb, int64_t Kp,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_place_h, dim3(grid_for(K * (K / 8))), dim3(NT), 0, st, H, dst, K, nkb, Kp);
  return last_status();
}

int64_t ar_gram_partials(int64_t N, int64_t K, int g) {
  int lpg, E;
  ar_group_layout(g, &lpg, &E);
  return (N * (K / g) * lpg + NT - 1) / NT;
}

ar_status ar_launch_place(const void* src, int src_dt, int64_t R, int64_t C, uint16_t* dst,
                          int64_t nkb, int64_t k_off, int lo, hipStream_t st) {
  const dim3 grid(grid_for(R * (C / 8)));
  if (src_dt == AR_BF16)
    hipLaunchKernelGGL(k_place<uint16_t>, grid, dim3(NT), 0, st, static_cast<const uint16_t*>(src),
                       dst, R, C, nkb, k_off, lo);
  else
    hipLaunchKernelGGL(k_place<float>, grid, dim3(NT), 0, st, static_cast<const float*>(src), dst,
                       R, C, nkb, k_off, lo);
  return last_status();
}

ar_status ar_launch_gram_d(int wdt, const void* W, const float* V, const float* A, const float* B,
                           int64_t N, int64_t K, int g, ArGrid gr, uint16_t* DB, hipStream_t st) {
  return wdt == AR_BF16 ? gram_d_make<uint16_t>(W, V, A, B, N, K, g, gr, DB, st)
                        : gram_d_make<float>(W, V, A, B, N, K, g, gr, DB, st);
}

ar_status ar_launch_ste_gram(const ArGramArgs& a, hipStream_t st) {
  return a.wdt == AR_BF16 ? ste_gram_make<uint16_t>(a, st) : ste_gram_make<float>(a, st);
}

ar_status ar_launch_loss_reduce(const ArLossIn& L, hipStream_t st) {
  hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(NT), 0, st, L);
  return last_status();
}

ar_status ar_launch_gram_snapshot(const int* flag, const float* V, const float* A, const float* B,
                                  float* bestV, float* bestA, float* bestB, int64_t nV, int64_t nG,
                                  hipStream_t st) {
  hipLaunchKernelGGL(k_gram_snapshot, dim3(grid_for(nV)), dim3(NT), 0, st, flag, V, A, B, bestV,
                     bestA, bestB, nV, nG);
  return last_status();
}
