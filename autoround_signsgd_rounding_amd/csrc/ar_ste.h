// Straight-through fold and SignSGD update of one weight group, used by the
// update kernel that runs after the gradient product (k_ste_update) and by the
// Gram form's update kernel.
//
// Per element (float32): t = W/s, c = rint(t + V) + zp, q = clamp(c, 0, maxq),
// m = [0 <= c <= maxq]; the rounding is passed straight through, so
//   dL/dV = G*s*m,
// and per group A = sum G*((q - zp) - m*t), Bs = sum over clipped elements of G.
// Asymmetric grid: with B = -s*Bs and D = A + B*lo/s^2,
//   dL/dlo = -D/maxq - B/s,  dL/dhi = D/maxq,
//   dL/dalpha = dL/dlo * wmin (wmin < 0),  dL/dbeta = dL/dhi * wmax (wmax > 0).
// Symmetric grid: dL/damax = 2A/maxq, routed to whichever of |alpha*wmin| and
// |beta*wmax| is the larger (ties to beta). SignSGD then moves every learnable
// by its step times the sign of its gradient (sgn 0 = 0) and clamps V to
// [-0.5, 0.5], alpha and beta to [clip_lo, clip_hi].
//
// Sources: llm-compressor AutoRound page (paper-core offset and SignSGD
// equations, the tuning loop's sign update and clamp, minmax_lr), Introducing
// AutoRound page section 2 (the clipping range is tuned with the rounding).
#pragma once

#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"

__device__ __forceinline__ Grid grid_of(const ArGrid& g) { return Grid{g.maxq, g.half, g.sym}; }

template <typename WT>
struct SteK {
  const WT* W;
  float* V;
  float* alpha;
  float* beta;
  const float* G;
  int64_t ngroups, K;
  int g, Gn, E;
  ArGrid gr;
  float lr, mlr, clip_lo, clip_hi;
  const int* flag;
  float* bestV;
  float* bestA;
  float* bestB;
  float* gV;
  float* gA;
  float* gB;
  int apply;
  uint16_t* Wq_next;   // blocked GEMM layout (wq_nkb k-blocks)
  int64_t wq_nkb;
};

// Straight-through sums of one chunk: A += G·((q - zp) - m·t), Bs += G·[not m].
__device__ __forceinline__ void ste_accum(const float (&w)[8], const float (&v)[8],
                                          const float (&g)[8], const QP& p, const Grid& gr,
                                          float& A, float& Bs) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const QE e = quant_elem(w[i], v[i], p, gr);
    const float d = (e.q - p.zp) - (e.m ? e.t : 0.0f);
    A += g[i] * d;
    if (!e.m) Bs += g[i];
  }
}

// Per element of one chunk: dL/dV = G·s·m, V <- clamp(V - lr·sgn(dL/dV), -0.5,
// 0.5) (unchanged when apply = 0), and the fake-quant Ŵ of the updated offset
// under the updated group parameters pn.
__device__ __forceinline__ void ste_chunk_update(const float (&w)[8], const float (&v)[8],
                                                 const float (&g)[8], const QP& p, const QP& pn,
                                                 const Grid& gr, float lr, int apply,
                                                 float (&gv)[8], float (&vn)[8], float (&wq)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const QE e = quant_elem(w[i], v[i], p, gr);
    gv[i] = e.m ? g[i] * p.s : 0.0f;
    const float sg = e.m ? sgnf(g[i]) : 0.0f;
    vn[i] = apply ? fminf(fmaxf(v[i] - lr * sg, -0.5f), 0.5f) : v[i];
    wq[i] = quant_elem(w[i], vn[i], pn, gr).what;
  }
}

// The update above for a chunk whose straight-through masks m (bit i for
// element i) were already found under p: no second quantization under p.
__device__ __forceinline__ void ste_chunk_update_m(const float (&w)[8], const float (&v)[8],
                                                   const float (&g)[8], uint32_t mbits,
                                                   const QP& p, const QP& pn, const Grid& gr,
                                                   float lr, int apply, float (&gv)[8],
                                                   float (&vn)[8], float (&wq)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool m = (mbits >> i) & 1u;
    gv[i] = m ? g[i] * p.s : 0.0f;
    const float sg = m ? sgnf(g[i]) : 0.0f;
    vn[i] = apply ? fminf(fmaxf(v[i] - lr * sg, -0.5f), 0.5f) : v[i];
    wq[i] = quant_elem(w[i], vn[i], pn, gr).what;
  }
}

// One step for the elements of one chunk: the update above, an optional
// snapshot of the pre-update offset, and the bf16 fake-quant of the updated
// state for the next forward product.
template <typename WT>
__device__ __forceinline__ void ste_finish(const SteK<WT>& a, int64_t n, int64_t off, const float (&w)[8],
                                           const float (&v)[8], const float (&g)[8], const QP& p,
                                           const QP& pn, const Grid& gr, bool snap) {
  float gv[8], vn[8], wq[8];
  ste_chunk_update(w, v, g, p, pn, gr, a.lr, a.apply, gv, vn, wq);
  if (a.gV) store8(a.gV + off, gv);
  if (snap) store8(a.bestV + off, v);
  if (a.apply) store8(a.V + off, vn);
  if (a.Wq_next) store8(a.Wq_next + arblk::chunk_offset(n, off - n * a.K, a.wq_nkb), wq);
}

// Clip-factor gradients of one group from its straight-through sums (zero for
// a zero-range group).
__device__ __forceinline__ void clip_grads(const Grid& gr, const QP& p, float mn, float mx,
                                           float al, float be, float A, float Bs, float& ga,
                                           float& gb) {
  ga = 0.0f;
  gb = 0.0f;
  if (p.zero) return;
  if (gr.sym) {
    const float damax = 2.0f * A / gr.maxq;
    const bool to_alpha = fabsf(al * mn) > fabsf(be * mx);
    ga = to_alpha ? damax * fabsf(mn) : 0.0f;
    gb = to_alpha ? 0.0f : damax * fabsf(mx);
  } else {
    const float B = -p.s * Bs;
    const float D = A + B * p.lo / (p.s * p.s);
    const float dlo = -D / gr.maxq - B / p.s;
    const float dhi = D / gr.maxq;
    ga = (mn < 0.0f) ? dlo * mn : 0.0f;
    gb = (mx > 0.0f) ? dhi * mx : 0.0f;
  }
}

// The clip-factor gradients, their SignSGD step, and the per-group writes done
// by the group's first lane: optional gradients, the pre-update snapshot, the
// updated factors.
template <typename WT>
__device__ __forceinline__ void clip_update(const SteK<WT>& a, bool snap, int64_t gid, int lig,
                                            float mn, float mx, float al, float be, const QP& p,
                                            float A, float Bs, bool live, float& an, float& bn) {
  float ga, gb;
  clip_grads(grid_of(a.gr), p, mn, mx, al, be, A, Bs, ga, gb);
  an = al;
  bn = be;
  if (a.apply) {
    an = fminf(fmaxf(al - a.mlr * sgnf(ga), a.clip_lo), a.clip_hi);
    bn = fminf(fmaxf(be - a.mlr * sgnf(gb), a.clip_lo), a.clip_hi);
  }
  if (live && lig == 0) {
    if (a.gA) a.gA[gid] = ga;
    if (a.gB) a.gB[gid] = gb;
    if (snap) { a.bestA[gid] = al; a.bestB[gid] = be; }
    if (a.apply) { a.alpha[gid] = an; a.beta[gid] = bn; }
  }
}

// One step for a group whose LPG lanes hold one 8-element chunk each (w, v, g
// in registers; off = element offset of the chunk in [N, K], row n; al, be the
// group's clip factors). Lanes of a group with live = false (padding outside
// the matrix) take part in the group reductions but touch no memory.
template <typename WT, int LPG>
__device__ __forceinline__ void ste_one(const SteK<WT>& a, bool snap, int64_t gid, int64_t n,
                                        int64_t off, int lig, const float (&w)[8],
                                        const float (&v)[8], const float (&g)[8], float al,
                                        float be, bool live) {
  const Grid gr = grid_of(a.gr);
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mn = fminf(mn, w[i]);
    mx = fmaxf(mx, w[i]);
  }
  mn = group_min<LPG>(mn);
  mx = group_max<LPG>(mx);
  if (!live) al = be = 1.0f;
  const QP p = group_qparams(mn, mx, al, be, gr);
  float A = 0.0f, Bs = 0.0f;
  ste_accum(w, v, g, p, gr, A, Bs);
  A = group_sum<LPG>(A);
  Bs = group_sum<LPG>(Bs);
  float an, bn;
  clip_update(a, snap, gid, lig, mn, mx, al, be, p, A, Bs, live, an, bn);
  const QP pn = group_qparams(mn, mx, an, bn, gr);
  if (live) ste_finish(a, n, off, w, v, g, p, pn, gr, snap);
}

// Device-side argument block from the host description (E = chunks per lane).
template <typename WT>
inline SteK<WT> ste_args(const ArSteArgs& s, int E) {
  return SteK<WT>{static_cast<const WT*>(s.W), s.V, s.alpha, s.beta, s.G, s.N * (s.K / s.g),
                  s.K, s.g, (int)(s.K / s.g), E, s.gr, s.lr, s.mlr, s.clip_lo, s.clip_hi,
                  s.flag, s.bestV, s.bestA, s.bestB, s.gV, s.gA, s.gB, s.apply, s.Wq_next,
                  s.wq_nkb};
}
