// C ABI of the AutoRound tuning library: argument validation (before any HIP
// call, so an error leaves nothing enqueued), workspace carving, and the order
// of kernel launches for one step and for the whole per-Linear loop.
#include <math.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <vector>

#include "ar_blocked.h"
#include "ar_launch.h"

namespace {

constexpr int64_t kMaxLd = int64_t(1) << 22;  // reduction length / row length bound (buffer offsets)

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool a8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
inline size_t pad256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool finite(float x) { return isfinite(x) != 0; }

ArGrid grid_of(const ar_config* c) {
  ArGrid g;
  g.maxq = (float)((1 << c->bits) - 1);
  g.half = (float)(1 << (c->bits - 1));
  g.sym = c->sym;
  return g;
}

// Candidate range of the MSE initial scale: j0..j1 with p_j = float32(1 - j/grid)
// inside [clip_lo, clip_hi]. False when there is none.
bool mse_range(const ar_config* c, int* j0, int* j1) {
  *j0 = -1;
  *j1 = -1;
  for (int j = 0;; ++j) {
    const float p = (float)(1.0 - (double)j / (double)c->mse_grid);
    if (p < c->clip_lo) break;
    if (p <= c->clip_hi) {
      if (*j0 < 0) *j0 = j;
      *j1 = j;
    }
  }
  return *j0 >= 0;
}

ArInit init_of(const ar_config* c) {
  ArInit in{};
  in.shrink = c->minmax_shrink;
  in.grid = c->mse_grid;
  in.mse = c->init_scale == 1 && mse_range(c, &in.j0, &in.j1);
  return in;
}

// bits / group / sym / shape checks shared by every quantizing entry point.
// *g = group size in elements (0 when N*K == 0).
ar_status check_quant(const ar_config* c, int64_t N, int64_t K, int* g) {
  if (!c) return AR_ERR_INVALID_ARG;
  if (!(c->bits == 2 || c->bits == 3 || c->bits == 4 || c->bits == 8)) return AR_ERR_UNSUPPORTED;
  if (c->sym != 0 && c->sym != 1) return AR_ERR_INVALID_ARG;
  if (c->group_size != -1 && c->group_size <= 0) return AR_ERR_INVALID_ARG;
  if (!finite(c->minmax_shrink) || c->minmax_shrink <= 0.0f) return AR_ERR_INVALID_ARG;
  if (c->init_scale != 0 && c->init_scale != 1) return AR_ERR_INVALID_ARG;
  if (c->check_finite != 0 && c->check_finite != 1) return AR_ERR_INVALID_ARG;
  if (c->init_scale == 1) {
    int j0, j1;
    if (!finite(c->clip_lo) || !finite(c->clip_hi) || c->clip_lo <= 0.0f ||
        c->clip_hi < c->clip_lo || c->mse_grid < 1 || c->mse_grid > 100000 ||
        !mse_range(c, &j0, &j1))
      return AR_ERR_INVALID_ARG;
  }
  if (N < 0 || K < 0) return AR_ERR_SHAPE;
  *g = 0;
  if (N == 0 || K == 0) return AR_OK;
  if (K % 8 != 0 || K >= kMaxLd) return AR_ERR_SHAPE;
  const int64_t gs = c->group_size == -1 ? K : c->group_size;
  if (gs % 8 != 0) return AR_ERR_UNSUPPORTED;
  if (K % gs != 0) return AR_ERR_SHAPE;
  if (N >= (int64_t(1) << 31) / 256) return AR_ERR_SHAPE;
  *g = (int)gs;
  return AR_OK;
}

// extra checks for the tuning entry points
ar_status check_tune(const ar_config* c) {
  if (!finite(c->lr) || c->lr < 0.0f) return AR_ERR_INVALID_ARG;
  if (!finite(c->minmax_lr)) return AR_ERR_INVALID_ARG;
  if (!finite(c->clip_lo) || !finite(c->clip_hi) || c->clip_lo <= 0.0f || c->clip_hi < c->clip_lo)
    return AR_ERR_INVALID_ARG;
  if (c->minmax_shrink < c->clip_lo || c->minmax_shrink > c->clip_hi) return AR_ERR_INVALID_ARG;
  return AR_OK;
}

float minmax_lr_of(const ar_config* c) { return c->minmax_lr < 0.0f ? c->lr : c->minmax_lr; }

bool dtype_ok(int32_t d) { return d == AR_F32 || d == AR_BF16; }
size_t dsize(int32_t d) { return d == AR_BF16 ? 2 : 4; }

// workspace carving
struct Carver {
  uint8_t* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += pad256(bytes);
    return p;
  }
};

// Element counts of the blocked GEMM operands (ar_blocked.h) for one minibatch.
struct BlkSizes {
  int64_t nkbK, nkbT;        // k-blocks along K and along Tb (Tb padded to whole tiles)
  int64_t xb, xtb, yb, wb;   // elements of XB, XTB, YB, WB / dyB
  BlkSizes(int64_t N, int64_t K, int64_t Tb) {
    nkbK = arblk::k_blocks(K);
    nkbT = arblk::row_tiles(Tb) * (arblk::ROWS / arblk::KB);
    xb = arblk::row_tiles(Tb) * nkbK * arblk::BLOCK_ELEMS;
    xtb = arblk::row_tiles(K) * nkbT * arblk::BLOCK_ELEMS;
    yb = arblk::row_tiles(N) * nkbT * arblk::BLOCK_ELEMS;
    wb = arblk::row_tiles(N) * nkbK * arblk::BLOCK_ELEMS;
  }
};

struct StepWs {
  uint16_t* XB;
  uint16_t* XTB;
  void* YB;
  uint16_t* dyB;
  uint16_t* WB;
  float* G;
  float* partials;
  int* flag;
};
StepWs carve_step(void* ws, int64_t N, int64_t K, int64_t Tb, int32_t ydt, size_t* bytes) {
  Carver c{static_cast<uint8_t*>(ws)};
  const BlkSizes z(N, K, Tb);
  StepWs w;
  w.XB = c.take<uint16_t>((size_t)z.xb * 2);
  w.XTB = c.take<uint16_t>((size_t)z.xtb * 2);
  w.YB = c.take<uint8_t>((size_t)z.yb * dsize(ydt));
  w.dyB = c.take<uint16_t>((size_t)z.yb * 2);
  w.WB = c.take<uint16_t>((size_t)z.wb * 2);
  w.G = c.take<float>((size_t)N * K * 4);
  w.partials = c.take<float>((size_t)ar_fwd_tiles(Tb, N) * 4);
  w.flag = c.take<int>(16);
  *bytes = c.off;
  return w;
}

struct LoopWs {
  uint16_t* XB;   // nb minibatches
  uint16_t* XTB;  // nb minibatches
  void* YB;       // nb minibatches
  uint16_t* dyB;
  uint16_t* WB;   // bf16 forward operand Ŵ
  float* G;
  float *V, *bestV;
  float *alpha, *beta, *bestA, *bestB;
  float* partials;
  float* best_loss;
  int* flag;
};
LoopWs carve_loop(void* ws, int64_t N, int64_t K, int64_t nb, int64_t Tb, int64_t Gn, int32_t ydt,
                  size_t* bytes) {
  Carver c{static_cast<uint8_t*>(ws)};
  const BlkSizes z(N, K, Tb);
  LoopWs w;
  w.XB = c.take<uint16_t>((size_t)nb * z.xb * 2);
  w.XTB = c.take<uint16_t>((size_t)nb * z.xtb * 2);
  w.YB = c.take<uint8_t>((size_t)nb * z.yb * dsize(ydt));
  w.dyB = c.take<uint16_t>((size_t)z.yb * 2);
  w.WB = c.take<uint16_t>((size_t)z.wb * 2);
  w.G = c.take<float>((size_t)N * K * 4);
  w.V = c.take<float>((size_t)N * K * 4);
  w.bestV = c.take<float>((size_t)N * K * 4);
  w.alpha = c.take<float>((size_t)N * Gn * 4);
  w.beta = c.take<float>((size_t)N * Gn * 4);
  w.bestA = c.take<float>((size_t)N * Gn * 4);
  w.bestB = c.take<float>((size_t)N * Gn * 4);
  w.partials = c.take<float>((size_t)ar_fwd_tiles(Tb, N) * 4);
  w.best_loss = c.take<float>(16);
  w.flag = c.take<int>(16);
  *bytes = c.off;
  return w;
}

// Gram form: blocked element counts and workspace.
struct GramSizes {
  int nred;              // 1 (bf16 W) or 2 (float32 W as W_hi + W_lo) reduction segments of K
  int64_t nkbR;          // k-blocks of the statistics product (nred·K)
  // D·H runs over three parts of Kp = K rounded up to whole k-blocks: H is stored
  // [H_hi | H_lo | H_hi] (nkbH k-blocks), D as [D_hi | D_lo] (nkbD), the product
  // reading D's first part for both of H's first two.
  int64_t Kp, nkbH, nkbD;
  int64_t xb2, wb2, hb, db, fsz;
  GramSizes(int wdt, int64_t N, int64_t K, int64_t Tb) {
    nred = wdt == AR_F32 ? 2 : 1;
    nkbR = arblk::k_blocks(nred * K);
    Kp = arblk::k_blocks(K) * arblk::KB;
    nkbH = 3 * arblk::k_blocks(K);
    nkbD = 2 * arblk::k_blocks(K);
    xb2 = arblk::row_tiles(Tb) * nkbR * arblk::BLOCK_ELEMS;
    wb2 = arblk::row_tiles(N) * nkbR * arblk::BLOCK_ELEMS;
    hb = arblk::row_tiles(K) * nkbH * arblk::BLOCK_ELEMS;
    db = arblk::row_tiles(N) * nkbD * arblk::BLOCK_ELEMS;
    fsz = (N > K ? N : K) * K;
  }
};

struct GramWs {
  uint16_t* XTB;   // nb minibatches, rows K, reduction Tb
  uint16_t* HB;    // nb x [H_hi | H_lo | H_hi]
  float* Cn;       // nb x [N, K]
  double* e2;      // nb
  uint16_t* XB2;   // staging: [X_b] or [X_b | X_b], rows Tb
  void* YB;        // staging: Y_b, rows N, reduction Tb
  uint16_t* dyB;   // staging: bf16(X_b·Wᵀ - Y_b), rows N, reduction Tb
  uint16_t* WB2;   // [W] or [W_hi | W_lo], rows N
  float* F;        // H of a minibatch (staging), then P = D·H (loop)
  float* fwd_partials;
  uint16_t* DB;    // [D_hi | D_lo], rows N
  float *V[2], *A[2], *B[2];
  float *bestV, *bestA, *bestB;
  float* partials;
  float* best_loss;
  int* flag;
};
GramWs carve_gram(void* ws, int wdt, int64_t N, int64_t K, int64_t nb, int64_t Tb, int64_t Gn,
                  int g, int32_t ydt, size_t* bytes) {
  Carver c{static_cast<uint8_t*>(ws)};
  const BlkSizes z(N, K, Tb);
  const GramSizes q(wdt, N, K, Tb);
  GramWs w;
  w.XTB = c.take<uint16_t>((size_t)nb * z.xtb * 2);
  w.HB = c.take<uint16_t>((size_t)nb * q.hb * 2);
  w.Cn = c.take<float>((size_t)nb * N * K * 4);
  w.e2 = c.take<double>((size_t)nb * 8);
  w.XB2 = c.take<uint16_t>((size_t)q.xb2 * 2);
  w.YB = c.take<uint8_t>((size_t)z.yb * dsize(ydt));
  w.dyB = c.take<uint16_t>((size_t)z.yb * 2);
  w.WB2 = c.take<uint16_t>((size_t)q.wb2 * 2);
  w.F = c.take<float>((size_t)q.fsz * 4);
  w.fwd_partials = c.take<float>((size_t)ar_fwd_tiles(Tb, N) * 4);
  w.DB = c.take<uint16_t>((size_t)q.db * 2);
  for (int i = 0; i < 2; ++i) {
    w.V[i] = c.take<float>((size_t)N * K * 4);
    w.A[i] = c.take<float>((size_t)N * Gn * 4);
    w.B[i] = c.take<float>((size_t)N * Gn * 4);
  }
  w.bestV = c.take<float>((size_t)N * K * 4);
  w.bestA = c.take<float>((size_t)N * Gn * 4);
  w.bestB = c.take<float>((size_t)N * Gn * 4);
  w.partials = c.take<float>((size_t)ar_gram_partials(N, K, g) * 4);
  w.best_loss = c.take<float>(16);
  w.flag = c.take<int>(16);
  *bytes = c.off;
  return w;
}

ar_status check_loop_shape(const ar_config* c, int64_t N, int64_t K, int* g, int64_t* M,
                           int64_t* Tb) {
  ar_status s = check_quant(c, N, K, g);
  if (s != AR_OK) return s;
  if ((s = check_tune(c)) != AR_OK) return s;
  if (c->iters < 0 || c->nsamples <= 0 || c->seqlen <= 0 || c->batch_samples <= 0)
    return AR_ERR_INVALID_ARG;
  if (c->nsamples % c->batch_samples != 0) return AR_ERR_SHAPE;
  if (N == 0 || K == 0) return AR_ERR_SHAPE;
  *M = (int64_t)c->nsamples * c->seqlen;
  *Tb = (int64_t)c->batch_samples * c->seqlen;
  if (*Tb % 8 != 0 || *Tb >= kMaxLd) return AR_ERR_SHAPE;
  return AR_OK;
}

#define AR_TRY(expr)                   \
  do {                                 \
    ar_status _s = (expr);             \
    if (_s != AR_OK) return _s;        \
  } while (0)

// Launches of one SignSGD step once the transposed minibatch is in place:
// forward product (residual, dY, per-tile sums of R²), gradient product (with
// the loss and best-loss decision), straight-through update.
ar_status enqueue_step(const ar_config* c, int wdt, const void* W, int64_t N, int64_t K, int g,
                       const uint16_t* XB, const uint16_t* XTB, const void* YB, int32_t ydt,
                       int64_t Tb, uint16_t* WB, uint16_t* dyB, float* G, float* partials,
                       int* flag, float* loss_out, float* loss_slot, float* best_loss,
                       float* V, float* alpha, float* beta, float* bestV,
                       float* bestA, float* bestB, float* gV, float* gA, float* gB, int apply,
                       bool write_next, hipStream_t st, hipEvent_t* ev /* 6 events or NULL */) {
  const double inv_count = 1.0 / ((double)Tb * (double)N);
  auto rec = [&](int k) {
    return (!ev || hipEventRecord(ev[k], st) == hipSuccess) ? AR_OK : AR_ERR_HIP;
  };
  ArSteArgs s;
  s.wdt = wdt; s.W = W; s.V = V; s.alpha = alpha; s.beta = beta; s.G = G;
  s.N = N; s.K = K; s.g = g; s.gr = grid_of(c);
  s.lr = c->lr; s.mlr = minmax_lr_of(c); s.clip_lo = c->clip_lo; s.clip_hi = c->clip_hi;
  s.flag = flag; s.bestV = bestV; s.bestA = bestA; s.bestB = bestB;
  s.gV = gV; s.gA = gA; s.gB = gB; s.apply = apply;
  s.Wq_next = write_next ? WB : nullptr;
  s.wq_nkb = arblk::k_blocks(K);
  ArLossIn li{};
  li.partials = partials; li.nparts = ar_fwd_tiles(Tb, N); li.inv_count = inv_count;
  li.loss_out = loss_out; li.loss_slot = loss_slot; li.best_loss = best_loss; li.flag = flag;

  AR_TRY(rec(0));
  AR_TRY(ar_launch_gemm_fwd(XB, WB, YB, ydt, dyB, partials, Tb, N, K, st));
  AR_TRY(rec(1));
  AR_TRY(rec(2));
  AR_TRY(ar_launch_gemm_wgrad(dyB, XTB, G, N, K, Tb, (float)(2.0 * inv_count), li, st));
  AR_TRY(rec(3));
  AR_TRY(rec(4));
  AR_TRY(ar_launch_ste_update(s, st));
  AR_TRY(rec(5));
  return AR_OK;
}

// Statistics of minibatch b (H_b, Cn_b, e2_b) from its token-major rows Xb,
// transposed rows XTB_b and targets Yb; XB2 / HB_b padding must already be zero.
ar_status stage_gram_minibatch(const GramWs& w, const GramSizes& q, int64_t N, int64_t K,
                               int64_t Tb, const uint16_t* Xb, const uint16_t* XTBb,
                               const void* Yb, int32_t ydt, uint16_t* HBb, float* Cnb, double* e2b,
                               hipStream_t st) {
  const int64_t nkbT = arblk::row_tiles(Tb) * (arblk::ROWS / arblk::KB);
  for (int r = 0; r < q.nred; ++r)
    AR_TRY(ar_launch_place(Xb, AR_BF16, Tb, K, w.XB2, q.nkbR, r * K, 0, st));
  AR_TRY(ar_launch_block_transpose(Yb, w.YB, 1, Tb, N, nkbT, (int)dsize(ydt), st));
  // dY = bf16(X_b·Wᵀ - Y_b), per-tile sums of its square
  AR_TRY(ar_launch_gemm_fwd(w.XB2, w.WB2, w.YB, ydt, w.dyB, w.fwd_partials, Tb, N, q.nred * K,
                            st));
  // Cn = dYᵀ·X_b; e2 reduced by the product's workgroup 0
  ArLossIn le{};
  le.partials = w.fwd_partials; le.nparts = ar_fwd_tiles(Tb, N); le.inv_count = 1.0;
  le.sum_out = e2b;
  AR_TRY(ar_launch_gemm_f32out(w.dyB, XTBb, Cnb, N, K, nkbT, 1.0f, le, st));
  // H = X_bᵀ·X_b, then its hi/lo operand [H_hi | H_lo | H_hi]
  ArLossIn none{};
  AR_TRY(ar_launch_gemm_f32out(XTBb, XTBb, w.F, K, K, nkbT, 1.0f, none, st));
  AR_TRY(ar_launch_place_h(w.F, K, HBb, q.nkbH, q.Kp, st));
  return AR_OK;
}

// [W] or [W_hi | W_lo] operand of the statistics product (padding cleared).
ar_status stage_gram_weight(const GramWs& w, const GramSizes& q, int wdt, const void* W,
                            int64_t N, int64_t K, hipStream_t st) {
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.WB2), 0.0f, q.wb2 / 2, st));
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.XB2), 0.0f, q.xb2 / 2, st));
  AR_TRY(ar_launch_place(W, wdt, N, K, w.WB2, q.nkbR, 0, 0, st));
  if (q.nred == 2) AR_TRY(ar_launch_place(W, wdt, N, K, w.WB2, q.nkbR, K, 1, st));
  return AR_OK;
}

// Every check of ar_tune_step except the workspace's; *need = its workspace bytes.
ar_status check_step(const ar_config* c, const ar_state* s, const uint16_t* Xb, const void* Yb,
                     int32_t ydt, int64_t Tb, const float* loss_out, const float* gV, int* g,
                     size_t* need) {
  if (!s) return AR_ERR_INVALID_ARG;
  AR_TRY(check_quant(c, s->N, s->K, g));
  AR_TRY(check_tune(c));
  if (!dtype_ok(s->wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  if (*g == 0 || Tb <= 0 || Tb % 8 != 0 || Tb >= kMaxLd) return AR_ERR_SHAPE;
  const int nbest = (s->best_V != nullptr) + (s->best_alpha != nullptr) +
                    (s->best_beta != nullptr) + (s->best_loss != nullptr);
  if (nbest != 0 && nbest != 4) return AR_ERR_INVALID_ARG;
  if (!s->W || !s->V || !s->alpha || !s->beta || !Xb || !Yb || !loss_out)
    return AR_ERR_INVALID_ARG;
  if (!a16(s->W) || !a16(s->V) || !a16(s->best_V) || !a16(Xb) || !a16(Yb) || !a16(gV))
    return AR_ERR_INVALID_ARG;
  carve_step(nullptr, s->N, s->K, Tb, ydt, need);
  return AR_OK;
}

// check_finite: AR_ERR_NONFINITE when any element of the given arrays is NaN or
// infinite. Clears *dflag (device), scans on the stream, and waits for the
// result on the host.
struct ScanItem {
  const void* p;
  int64_t n;
  int dt;
};
ar_status scan_finite(std::initializer_list<ScanItem> items, int* dflag, hipStream_t st) {
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(dflag), 0.0f, 1, st));
  for (const ScanItem& it : items) AR_TRY(ar_launch_nonfinite(it.p, it.n, it.dt, dflag, st));
  int found = 0;
  if (hipMemcpyAsync(&found, dflag, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return AR_ERR_HIP;
  return found ? AR_ERR_NONFINITE : AR_OK;
}

// One SignSGD step of ar_tune_step on validated arguments, scratch at ws.
// Everything the step reads from ws is written first by the same call (the
// staged minibatch, Ŵ with its zero padding, the products, the loss
// partials and the improvement flag), so ws may hold anything on entry.
ar_status run_step(const ar_config* c, const ar_state* s, int g, const uint16_t* Xb,
                   const void* Yb, int32_t ydt, int64_t Tb, float* loss_out, float* gV,
                   float* galpha, float* gbeta, int32_t apply_update, void* ws, hipStream_t st) {
  const int64_t N = s->N, K = s->K;
  size_t need;
  StepWs w = carve_step(ws, N, K, Tb, ydt, &need);
  const BlkSizes z(N, K, Tb);
  if (c->check_finite) {
    const int64_t Gn = K / g;
    AR_TRY(scan_finite({{s->W, N * K, s->wdt}, {s->V, N * K, AR_F32}, {s->alpha, N * Gn, AR_F32},
                        {s->beta, N * Gn, AR_F32}, {Xb, Tb * K, AR_BF16}, {Yb, Tb * N, ydt}},
                       w.flag + 1, st));
  }

  // stage the minibatch into the blocked GEMM layouts, Ŵ of the current state
  AR_TRY(ar_launch_stage_x(Xb, w.XTB, w.XB, 1, Tb, K, z.nkbT, z.nkbK, st));
  AR_TRY(ar_launch_block_transpose(Yb, w.YB, 1, Tb, N, z.nkbT, (int)dsize(ydt), st));
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.WB), 0.0f, z.wb / 2, st));
  AR_TRY(ar_launch_fakequant(s->wdt, s->W, s->V, s->alpha, s->beta, init_of(c), N, K, g,
                             grid_of(c), AR_BF16, w.WB, z.nkbK, nullptr, nullptr, nullptr, st));
  return enqueue_step(c, s->wdt, s->W, N, K, g, w.XB, w.XTB, w.YB, ydt, Tb, w.WB, w.dyB, w.G,
                      w.partials, w.flag, loss_out, nullptr, s->best_loss, s->V, s->alpha,
                      s->beta, s->best_V, s->best_alpha, s->best_beta, gV, galpha, gbeta,
                      apply_update != 0, false, st, nullptr);
}

// Scratch of ar_tune_step_noalloc: a fixed array in every GPU's memory, held
// until the process ends. In host code `scratch` is a host-side stand-in, not
// a device address; the address of a device's copy comes from
// hipGetSymbolAddress with that device current, once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ar_status scratch_of_current_device(void** out);

ArGramArgs gram_args(const ar_config* c, int wdt, const void* W, int64_t N, int64_t K, int g,
                     int64_t Tb) {
  ArGramArgs a{};
  a.wdt = wdt; a.W = W; a.N = N; a.K = K; a.g = g; a.gr = grid_of(c);
  a.lr = c->lr; a.mlr = minmax_lr_of(c); a.clip_lo = c->clip_lo; a.clip_hi = c->clip_hi;
  a.scale = (float)(2.0 / ((double)Tb * (double)N));
  a.apply = 1;
  return a;
}

}  // namespace

static __device__ __align__(256) uint8_t scratch[AR_NOALLOC_SCRATCH_BYTES];

namespace {
ar_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();   // leave no error behind for the caller's next HIP call
      return AR_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AR_OK;
}
}  // namespace

extern "C" {

ar_status ar_config_default(ar_config* c) {
  if (!c) return AR_ERR_INVALID_ARG;
  c->bits = 4;
  c->group_size = 128;
  c->sym = 0;
  c->nsamples = 128;
  c->seqlen = 2048;
  c->batch_samples = 8;
  c->iters = 200;
  c->lr = 0.005f;
  c->minmax_lr = -1.0f;
  c->minmax_shrink = 1.0f;
  c->clip_lo = 0.5f;
  c->clip_hi = 1.0f;
  c->init_scale = 0;
  c->mse_grid = 100;
  c->check_finite = 0;
  return AR_OK;
}

const char* ar_status_string(int32_t s) {
  switch (s) {
    case AR_OK: return "ok";
    case AR_ERR_INVALID_ARG: return "invalid argument (null pointer, bad hyper-parameter or misaligned pointer)";
    case AR_ERR_UNSUPPORTED: return "unsupported (bits must be 2, 3, 4 or 8; group_size a multiple of 8; dtype f32/bf16)";
    case AR_ERR_SHAPE: return "shape constraint violated";
    case AR_ERR_WORKSPACE: return "workspace too small (ar_tune_step_noalloc: the problem needs more than its fixed scratch)";
    case AR_ERR_NONFINITE: return "an input holds NaN or Inf (check_finite)";
    case AR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

ar_status ar_workspace_size(const ar_config* c, int64_t N, int64_t K, int32_t ydt, size_t* bytes) {
  int g;
  int64_t M, Tb;
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_loop_shape(c, N, K, &g, &M, &Tb));
  if (!dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  carve_loop(nullptr, N, K, M / Tb, Tb, K / g, ydt, bytes);
  return AR_OK;
}

ar_status ar_step_workspace_size(const ar_config* c, int64_t N, int64_t K, int64_t Tb,
                                 int32_t ydt, size_t* bytes) {
  int g;
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_quant(c, N, K, &g));
  if (N == 0 || K == 0 || Tb <= 0 || Tb % 8 != 0 || Tb >= kMaxLd) return AR_ERR_SHAPE;
  if (!dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  carve_step(nullptr, N, K, Tb, ydt, bytes);
  return AR_OK;
}

ar_status ar_init_clip(const ar_config* c, int32_t wdt, const void* W, int64_t N, int64_t K,
                       float* alpha, float* beta, void* stream) {
  int g;
  AR_TRY(check_quant(c, N, K, &g));
  if (!dtype_ok(wdt)) return AR_ERR_UNSUPPORTED;
  if (g == 0) return AR_OK;
  if (!W || !alpha || !beta || !a16(W)) return AR_ERR_INVALID_ARG;
  return ar_launch_init_clip(wdt, W, N, K, g, grid_of(c), init_of(c), alpha, beta,
                             static_cast<hipStream_t>(stream));
}

ar_status ar_rtn_quant(const ar_config* c, int32_t wdt, const void* W, int64_t N, int64_t K,
                       uint8_t* codes, float* scale, uint8_t* zp, void* Wq, void* stream) {
  int g;
  AR_TRY(check_quant(c, N, K, &g));
  if (!dtype_ok(wdt)) return AR_ERR_UNSUPPORTED;
  if (g == 0) return AR_OK;
  if (!W || !a16(W) || !a16(Wq) || !a8(codes)) return AR_ERR_INVALID_ARG;
  return ar_launch_fakequant(wdt, W, nullptr, nullptr, nullptr, init_of(c), N, K, g,
                             grid_of(c), wdt, Wq, 0, codes, scale, zp,
                             static_cast<hipStream_t>(stream));
}

ar_status ar_fakequant_fwd(const ar_config* c, int32_t wdt, const void* W, int64_t N, int64_t K,
                           const float* V, const float* alpha, const float* beta,
                           uint16_t* Wq_bf16, uint8_t* codes, float* scale, uint8_t* zp,
                           void* stream) {
  int g;
  AR_TRY(check_quant(c, N, K, &g));
  if (!dtype_ok(wdt)) return AR_ERR_UNSUPPORTED;
  if (g == 0) return AR_OK;
  if (!W || !V || !alpha || !beta) return AR_ERR_INVALID_ARG;
  if (!a16(W) || !a16(V) || !a16(Wq_bf16) || !a8(codes)) return AR_ERR_INVALID_ARG;
  return ar_launch_fakequant(wdt, W, V, alpha, beta, init_of(c), N, K, g, grid_of(c),
                             AR_BF16, Wq_bf16, 0, codes, scale, zp,
                             static_cast<hipStream_t>(stream));
}

ar_status ar_tune_step(const ar_config* c, const ar_state* s, const uint16_t* Xb, const void* Yb,
                       int32_t ydt, int64_t Tb, float* loss_out, float* gV, float* galpha,
                       float* gbeta, int32_t apply_update, void* ws, size_t ws_bytes,
                       void* stream) {
  int g;
  size_t need;
  AR_TRY(check_step(c, s, Xb, Yb, ydt, Tb, loss_out, gV, &g, &need));
  if (!ws || !a16(ws)) return AR_ERR_INVALID_ARG;
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  return run_step(c, s, g, Xb, Yb, ydt, Tb, loss_out, gV, galpha, gbeta, apply_update, ws,
                  static_cast<hipStream_t>(stream));
}

ar_status ar_tune_step_noalloc(const ar_config* c, const ar_state* s, const uint16_t* Xb,
                               const void* Yb, int32_t ydt, int64_t Tb, float* loss_out,
                               float* gV, float* galpha, float* gbeta, int32_t apply_update,
                               void* stream) {
  int g;
  size_t need;
  AR_TRY(check_step(c, s, Xb, Yb, ydt, Tb, loss_out, gV, &g, &need));
  if (need > AR_NOALLOC_SCRATCH_BYTES) return AR_ERR_WORKSPACE;
  void* ws = nullptr;
  AR_TRY(scratch_of_current_device(&ws));
  return run_step(c, s, g, Xb, Yb, ydt, Tb, loss_out, gV, galpha, gbeta, apply_update, ws,
                  static_cast<hipStream_t>(stream));
}

ar_status ar_tune_linear(const ar_config* c, int32_t wdt, const void* W, int64_t N, int64_t K,
                         const uint16_t* X, const void* Y, int32_t ydt, uint8_t* codes,
                         float* scale, uint8_t* zp, void* Wq, float* V_out, float* alpha_out,
                         float* beta_out, float* losses, void* ws, size_t ws_bytes,
                         ar_kernel_times* times, void* stream) {
  int g;
  int64_t M, Tb;
  AR_TRY(check_loop_shape(c, N, K, &g, &M, &Tb));
  if (!dtype_ok(wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  if (!W || !X || !Y || !codes || !scale || !zp || !ws) return AR_ERR_INVALID_ARG;
  if (!a16(W) || !a16(X) || !a16(Y) || !a8(codes) || !a16(Wq) || !a16(V_out) || !a16(ws))
    return AR_ERR_INVALID_ARG;
  const int64_t Gn = K / g;
  const int64_t nb = c->nsamples / c->batch_samples;
  size_t need;
  carve_loop(nullptr, N, K, nb, Tb, Gn, ydt, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  LoopWs w = carve_loop(ws, N, K, nb, Tb, Gn, ydt, &need);
  const BlkSizes z(N, K, Tb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t ysz = dsize(ydt);

  // events around the kernels of every `every`-th step (6 per timed step)
  const int every = (times && times->sample_every > 1) ? times->sample_every : 1;
  const int ntimed = (times && c->iters > 0) ? (c->iters + every - 1) / every : 0;
  std::vector<hipEvent_t> ev;
  if (ntimed > 0) {
    ev.resize((size_t)ntimed * 6);
    for (auto& e : ev) {
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        for (auto& d : ev)
          if (d) (void)hipEventDestroy(d);
        return AR_ERR_HIP;
      }
    }
  }
  auto cleanup = [&](ar_status s) {
    for (auto& e : ev) (void)hipEventDestroy(e);
    return s;
  };
#define AR_TRY_C(expr)                   \
  do {                                   \
    ar_status _s = (expr);               \
    if (_s != AR_OK) return cleanup(_s); \
  } while (0)

  if (c->check_finite)
    AR_TRY_C(scan_finite({{W, N * K, wdt}, {X, M * K, AR_BF16}, {Y, M * N, ydt}}, w.flag + 1, st));
  // one-time staging of every minibatch into the blocked GEMM layouts
  AR_TRY_C(ar_launch_stage_x(X, w.XTB, w.XB, nb, Tb, K, z.nkbT, z.nkbK, st));
  AR_TRY_C(ar_launch_block_transpose(Y, w.YB, nb, Tb, N, z.nkbT, (int)ysz, st));
  AR_TRY_C(ar_launch_fill_f32(reinterpret_cast<float*>(w.WB), 0.0f, z.wb / 2, st));
  // initial state: V = 0, the initial clip factors, best = initial, best loss = +inf
  AR_TRY_C(ar_launch_fill_f32(w.V, 0.0f, N * K, st));
  AR_TRY_C(ar_launch_fill_f32(w.bestV, 0.0f, N * K, st));
  AR_TRY_C(ar_launch_init_clip(wdt, W, N, K, g, grid_of(c), init_of(c), w.alpha, w.beta, st));
  AR_TRY_C(ar_launch_init_clip(wdt, W, N, K, g, grid_of(c), init_of(c), w.bestA, w.bestB, st));
  AR_TRY_C(ar_launch_fill_f32(w.best_loss, INFINITY, 1, st));
  const ArGrid gr = grid_of(c);
  if (c->iters > 0)
    AR_TRY_C(ar_launch_fakequant(wdt, W, w.V, w.alpha, w.beta, init_of(c), N, K, g, gr,
                                 AR_BF16, w.WB, z.nkbK, nullptr, nullptr, nullptr, st));
  for (int i = 0; i < c->iters; ++i) {
    const int64_t b = i % nb;
    AR_TRY_C(enqueue_step(
        c, wdt, W, N, K, g, w.XB + b * z.xb, w.XTB + b * z.xtb,
        static_cast<const uint8_t*>(w.YB) + (size_t)b * z.yb * ysz, ydt, Tb, w.WB, w.dyB, w.G,
        w.partials, w.flag, nullptr, losses ? losses + i : nullptr, w.best_loss, w.V, w.alpha,
        w.beta, w.bestV, w.bestA, w.bestB, nullptr, nullptr, nullptr, 1, true, st,
        (ntimed > 0 && i % every == 0) ? &ev[(size_t)(i / every) * 6] : nullptr));
  }
  // restore the best state and quantize it (the initial state when iters = 0)
  AR_TRY_C(ar_launch_fakequant(wdt, W, w.bestV, w.bestA, w.bestB, init_of(c), N, K, g, gr,
                               wdt, Wq, 0, codes, scale, zp, st));
  if (V_out && hipMemcpyAsync(V_out, w.bestV, (size_t)N * K * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (alpha_out &&
      hipMemcpyAsync(alpha_out, w.bestA, (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (beta_out &&
      hipMemcpyAsync(beta_out, w.bestB, (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (times) {
    const int32_t sample = times->sample_every;
    memset(times, 0, sizeof(*times));
    times->sample_every = sample;
    if (ntimed > 0) {
      if (hipStreamSynchronize(st) != hipSuccess) return cleanup(AR_ERR_HIP);
      for (int i = 0; i < ntimed; ++i) {
        float ms[3];
        for (int k = 0; k < 3; ++k)
          if (hipEventElapsedTime(&ms[k], ev[(size_t)i * 6 + 2 * k], ev[(size_t)i * 6 + 2 * k + 1]) !=
              hipSuccess)
            return cleanup(AR_ERR_HIP);
        times->fwd_gemm_ms += ms[0];
        times->wgrad_gemm_ms += ms[1];
        times->ste_update_ms += ms[2];
      }
      times->steps = ntimed;
    }
  }
#undef AR_TRY_C
  return cleanup(AR_OK);
}

ar_status ar_gram_workspace_size(const ar_config* c, int32_t wdt, int64_t N, int64_t K,
                                 int32_t ydt, size_t* bytes) {
  int g;
  int64_t M, Tb;
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_loop_shape(c, N, K, &g, &M, &Tb));
  if (!dtype_ok(wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  carve_gram(nullptr, wdt, N, K, M / Tb, Tb, K / g, g, ydt, bytes);
  return AR_OK;
}

ar_status ar_gram_step_workspace_size(const ar_config* c, int32_t wdt, int64_t N, int64_t K,
                                      int64_t Tb, int32_t ydt, size_t* bytes) {
  int g;
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_quant(c, N, K, &g));
  if (N == 0 || K == 0 || Tb <= 0 || Tb % 8 != 0 || Tb >= kMaxLd) return AR_ERR_SHAPE;
  if (!dtype_ok(wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  carve_gram(nullptr, wdt, N, K, 1, Tb, K / g, g, ydt, bytes);
  return AR_OK;
}

ar_status ar_tune_step_gram(const ar_config* c, const ar_state* s, const uint16_t* Xb,
                            const void* Yb, int32_t ydt, int64_t Tb, float* loss_out, float* gV,
                            float* galpha, float* gbeta, int32_t apply_update, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!s) return AR_ERR_INVALID_ARG;
  int g;
  AR_TRY(check_quant(c, s->N, s->K, &g));
  AR_TRY(check_tune(c));
  if (!dtype_ok(s->wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  if (g == 0 || Tb <= 0 || Tb % 8 != 0 || Tb >= kMaxLd) return AR_ERR_SHAPE;
  const int nbest = (s->best_V != nullptr) + (s->best_alpha != nullptr) +
                    (s->best_beta != nullptr) + (s->best_loss != nullptr);
  if (nbest != 0 && nbest != 4) return AR_ERR_INVALID_ARG;
  if (!s->W || !s->V || !s->alpha || !s->beta || !Xb || !Yb || !loss_out || !ws)
    return AR_ERR_INVALID_ARG;
  if (!a16(s->W) || !a16(s->V) || !a16(s->best_V) || !a16(Xb) || !a16(Yb) || !a16(gV) || !a16(ws))
    return AR_ERR_INVALID_ARG;
  const int64_t N = s->N, K = s->K, Gn = K / g;
  size_t need;
  carve_gram(nullptr, s->wdt, N, K, 1, Tb, Gn, g, ydt, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  GramWs w = carve_gram(ws, s->wdt, N, K, 1, Tb, Gn, g, ydt, &need);
  const GramSizes q(s->wdt, N, K, Tb);
  const BlkSizes z(N, K, Tb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (c->check_finite)
    AR_TRY(scan_finite({{s->W, N * K, s->wdt}, {s->V, N * K, AR_F32}, {s->alpha, N * Gn, AR_F32},
                        {s->beta, N * Gn, AR_F32}, {Xb, Tb * K, AR_BF16}, {Yb, Tb * N, ydt}},
                       w.flag + 1, st));

  AR_TRY(stage_gram_weight(w, q, s->wdt, s->W, N, K, st));
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.HB), 0.0f, q.hb / 2, st));
  AR_TRY(ar_launch_block_transpose(Xb, w.XTB, 1, Tb, K, z.nkbT, 2, st));
  AR_TRY(stage_gram_minibatch(w, q, N, K, Tb, Xb, w.XTB, Yb, ydt, w.HB, w.Cn, w.e2, st));
  // D of the current state, P = D·H, then the update into scratch buffers so the
  // current state stays intact for the snapshot
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.DB), 0.0f, q.db / 2, st));
  AR_TRY(ar_launch_gram_d(s->wdt, s->W, s->V, s->alpha, s->beta, N, K, g, grid_of(c), w.DB, st));
  ArLossIn none{};
  AR_TRY(ar_launch_gemm_gram(w.DB, w.HB, w.F, N, K, none, st));
  ArGramArgs a = gram_args(c, s->wdt, s->W, N, K, g, Tb);
  a.Vc = s->V; a.Vn = w.V[0]; a.Ac = s->alpha; a.Bc = s->beta; a.An = w.A[0]; a.Bn = w.B[0];
  a.P = w.F; a.Cn = w.Cn; a.apply = apply_update != 0; a.DB = w.DB; a.partials = w.partials;
  a.gV = gV; a.gA = galpha; a.gB = gbeta;
  AR_TRY(ar_launch_ste_gram(a, st));
  ArLossIn li{};
  li.partials = w.partials; li.nparts = (int)ar_gram_partials(N, K, g);
  li.inv_count = 1.0 / ((double)Tb * (double)N); li.add = w.e2; li.loss_out = loss_out;
  li.best_loss = s->best_loss; li.flag = w.flag;
  AR_TRY(ar_launch_loss_reduce(li, st));
  if (s->best_loss)
    AR_TRY(ar_launch_gram_snapshot(w.flag, s->V, s->alpha, s->beta, s->best_V, s->best_alpha,
                                   s->best_beta, N * K, N * Gn, st));
  if (apply_update) {
    if (hipMemcpyAsync(s->V, w.V[0], (size_t)N * K * 4, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(s->alpha, w.A[0], (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st) ||
        hipMemcpyAsync(s->beta, w.B[0], (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st))
      return AR_ERR_HIP;
  }
  return AR_OK;
}

ar_status ar_tune_linear_gram(const ar_config* c, int32_t wdt, const void* W, int64_t N,
                              int64_t K, const uint16_t* X, const void* Y, int32_t ydt,
                              uint8_t* codes, float* scale, uint8_t* zp, void* Wq, float* V_out,
                              float* alpha_out, float* beta_out, float* losses, void* ws,
                              size_t ws_bytes, ar_kernel_times* times, void* stream) {
  int g;
  int64_t M, Tb;
  AR_TRY(check_loop_shape(c, N, K, &g, &M, &Tb));
  if (!dtype_ok(wdt) || !dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  if (!W || !X || !Y || !codes || !scale || !zp || !ws) return AR_ERR_INVALID_ARG;
  if (!a16(W) || !a16(X) || !a16(Y) || !a8(codes) || !a16(Wq) || !a16(V_out) || !a16(ws))
    return AR_ERR_INVALID_ARG;
  const int64_t Gn = K / g;
  const int64_t nb = c->nsamples / c->batch_samples;
  size_t need;
  carve_gram(nullptr, wdt, N, K, nb, Tb, Gn, g, ydt, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  GramWs w = carve_gram(ws, wdt, N, K, nb, Tb, Gn, g, ydt, &need);
  const GramSizes q(wdt, N, K, Tb);
  const BlkSizes z(N, K, Tb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t ysz = dsize(ydt);
  const double inv_count = 1.0 / ((double)Tb * (double)N);
  const int nparts = (int)ar_gram_partials(N, K, g);

  // events around the two kernels of every `every`-th step
  const int every = (times && times->sample_every > 1) ? times->sample_every : 1;
  const int ntimed = (times && c->iters > 0) ? (c->iters + every - 1) / every : 0;
  std::vector<hipEvent_t> ev;
  if (ntimed > 0) {
    ev.resize((size_t)ntimed * 4);
    for (auto& e : ev) {
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        for (auto& d : ev)
          if (d) (void)hipEventDestroy(d);
        return AR_ERR_HIP;
      }
    }
  }
  auto cleanup = [&](ar_status s) {
    for (auto& e : ev) (void)hipEventDestroy(e);
    return s;
  };
#define AR_TRY_C(expr)                   \
  do {                                   \
    ar_status _s = (expr);               \
    if (_s != AR_OK) return cleanup(_s); \
  } while (0)

  if (c->check_finite)
    AR_TRY_C(scan_finite({{W, N * K, wdt}, {X, M * K, AR_BF16}, {Y, M * N, ydt}}, w.flag + 1, st));
  // once per Linear: the statistics of every minibatch
  AR_TRY_C(stage_gram_weight(w, q, wdt, W, N, K, st));
  AR_TRY_C(ar_launch_fill_f32(reinterpret_cast<float*>(w.HB), 0.0f, nb * q.hb / 2, st));
  AR_TRY_C(ar_launch_block_transpose(X, w.XTB, nb, Tb, K, z.nkbT, 2, st));
  for (int64_t b = 0; b < nb; ++b)
    AR_TRY_C(stage_gram_minibatch(w, q, N, K, Tb, X + b * Tb * K, w.XTB + b * z.xtb,
                                  static_cast<const uint8_t*>(Y) + (size_t)b * Tb * N * ysz, ydt,
                                  w.HB + b * q.hb, w.Cn + b * N * K, w.e2 + b, st));
  // initial state, its D operand
  AR_TRY_C(ar_launch_fill_f32(w.V[0], 0.0f, N * K, st));
  AR_TRY_C(ar_launch_fill_f32(w.V[1], 0.0f, N * K, st));
  AR_TRY_C(ar_launch_fill_f32(w.bestV, 0.0f, N * K, st));
  for (int k = 0; k < 3; ++k) {
    float* A = k < 2 ? w.A[k] : w.bestA;
    float* B = k < 2 ? w.B[k] : w.bestB;
    AR_TRY_C(ar_launch_init_clip(wdt, W, N, K, g, grid_of(c), init_of(c), A, B, st));
  }
  AR_TRY_C(ar_launch_fill_f32(w.best_loss, INFINITY, 1, st));
  AR_TRY_C(ar_launch_fill_f32(reinterpret_cast<float*>(w.flag), 0.0f, 1, st));
  AR_TRY_C(ar_launch_fill_f32(reinterpret_cast<float*>(w.DB), 0.0f, q.db / 2, st));
  const ArGrid gr = grid_of(c);
  if (c->iters > 0)
    AR_TRY_C(ar_launch_gram_d(wdt, W, w.V[0], w.A[0], w.B[0], N, K, g, gr, w.DB, st));

  ArGramArgs a = gram_args(c, wdt, W, N, K, g, Tb);
  a.P = w.F; a.DB = w.DB; a.partials = w.partials;
  a.bestV = w.bestV; a.bestA = w.bestA; a.bestB = w.bestB;
  for (int i = 0; i < c->iters; ++i) {
    const int64_t b = i % nb, bp = (i + nb - 1) % nb;
    const int cur = i & 1;
    hipEvent_t* e = (ntimed > 0 && i % every == 0) ? &ev[(size_t)(i / every) * 4] : nullptr;
    // P = D·H; workgroup 0 settles the previous step's loss and best-loss decision
    ArLossIn li{};
    if (i > 0) {
      li.partials = w.partials; li.nparts = nparts; li.inv_count = inv_count;
      li.add = w.e2 + bp; li.loss_slot = losses ? losses + (i - 1) : nullptr;
      li.best_loss = w.best_loss; li.flag = w.flag;
    }
    if (e && hipEventRecord(e[0], st) != hipSuccess) return cleanup(AR_ERR_HIP);
    AR_TRY_C(ar_launch_gemm_gram(w.DB, w.HB + b * q.hb, w.F, N, K, li, st));
    if (e && hipEventRecord(e[1], st) != hipSuccess) return cleanup(AR_ERR_HIP);
    // update into the other half of the pair, copying the previous state to best
    // first when its loss improved
    a.Vc = w.V[cur]; a.Vn = w.V[1 - cur]; a.Ac = w.A[cur]; a.Bc = w.B[cur];
    a.An = w.A[1 - cur]; a.Bn = w.B[1 - cur]; a.Cn = w.Cn + b * N * K;
    a.flag_prev = i > 0 ? w.flag : nullptr;
    if (e && hipEventRecord(e[2], st) != hipSuccess) return cleanup(AR_ERR_HIP);
    AR_TRY_C(ar_launch_ste_gram(a, st));
    if (e && hipEventRecord(e[3], st) != hipSuccess) return cleanup(AR_ERR_HIP);
  }
  if (c->iters > 0) {
    // the last step's loss and snapshot (its state is still in its half of the pair)
    const int last = (c->iters - 1) & 1;
    ArLossIn li{};
    li.partials = w.partials; li.nparts = nparts; li.inv_count = inv_count;
    li.add = w.e2 + (c->iters - 1) % nb; li.loss_slot = losses ? losses + (c->iters - 1) : nullptr;
    li.best_loss = w.best_loss; li.flag = w.flag;
    AR_TRY_C(ar_launch_loss_reduce(li, st));
    AR_TRY_C(ar_launch_gram_snapshot(w.flag, w.V[last], w.A[last], w.B[last], w.bestV, w.bestA,
                                     w.bestB, N * K, N * Gn, st));
  }
  // restore the best state and quantize it (the initial state when iters = 0)
  AR_TRY_C(ar_launch_fakequant(wdt, W, w.bestV, w.bestA, w.bestB, init_of(c), N, K, g, gr,
                               wdt, Wq, 0, codes, scale, zp, st));
  if (V_out && hipMemcpyAsync(V_out, w.bestV, (size_t)N * K * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (alpha_out &&
      hipMemcpyAsync(alpha_out, w.bestA, (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (beta_out &&
      hipMemcpyAsync(beta_out, w.bestB, (size_t)N * Gn * 4, hipMemcpyDeviceToDevice, st))
    return cleanup(AR_ERR_HIP);
  if (times) {
    const int32_t sample = times->sample_every;
    memset(times, 0, sizeof(*times));
    times->sample_every = sample;
    if (ntimed > 0) {
      if (hipStreamSynchronize(st) != hipSuccess) return cleanup(AR_ERR_HIP);
      for (int i = 0; i < ntimed; ++i) {
        float ms[2];
        for (int k = 0; k < 2; ++k)
          if (hipEventElapsedTime(&ms[k], ev[(size_t)i * 4 + 2 * k], ev[(size_t)i * 4 + 2 * k + 1]) !=
              hipSuccess)
            return cleanup(AR_ERR_HIP);
        times->fwd_gemm_ms += ms[0];
        times->ste_update_ms += ms[1];
      }
      times->steps = ntimed;
    }
  }
#undef AR_TRY_C
  return cleanup(AR_OK);
}

// ---- W-bit x bf16 product
static constexpr int64_t kGemvMaxM = 16;

static size_t dequant_ws(int bits, int64_t M, int64_t N, int64_t K, int64_t g) {
  if (M <= kGemvMaxM) return pad256((size_t)ar_dq_slices(bits, N, K, M, g) * M * N * 4);
  Carver c{nullptr};
  c.take<uint16_t>((size_t)arblk::row_tiles(M) * arblk::k_blocks(K) * arblk::BLOCK_ELEMS * 2);
  c.take<uint16_t>((size_t)arblk::row_tiles(N) * arblk::k_blocks(K) * arblk::BLOCK_ELEMS * 2);
  return c.off;
}

static ar_status check_dequant(int32_t bits, int64_t M, int64_t N, int64_t K) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return AR_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxLd * 64 || N >= (int64_t(1) << 31) / 256)
    return AR_ERR_SHAPE;
  if (K != 0 && (K % 8 != 0 || (K * bits) % 32 != 0 || K >= kMaxLd)) return AR_ERR_SHAPE;
  return AR_OK;
}

static ar_status dequant_group(int32_t group_size, int64_t K, int64_t* g) {
  if (group_size != -1 && group_size <= 0) return AR_ERR_INVALID_ARG;
  *g = group_size == -1 ? K : group_size;
  if (*g % 8 != 0) return AR_ERR_UNSUPPORTED;
  if (K % *g != 0) return AR_ERR_SHAPE;
  return AR_OK;
}

ar_status ar_dequant_gemm_workspace_size(int32_t bits, int32_t group_size, int64_t M, int64_t N,
                                         int64_t K, size_t* bytes) {
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_dequant(bits, M, N, K));
  if (M == 0 || N == 0 || K == 0) {
    *bytes = 0;
    return AR_OK;
  }
  int64_t g = 0;
  AR_TRY(dequant_group(group_size, K, &g));
  *bytes = dequant_ws(bits, M, N, K, g);
  return AR_OK;
}

ar_status ar_dequant_gemm(int32_t bits, int32_t group_size, const uint16_t* X, int64_t M,
                          int64_t K, const int32_t* qweight, const int32_t* qzeros,
                          const float* scale, int64_t N, void* Y, int32_t ydt, void* ws,
                          size_t ws_bytes, void* stream) {
  AR_TRY(check_dequant(bits, M, N, K));
  if (!dtype_ok(ydt)) return AR_ERR_UNSUPPORTED;
  if (group_size != -1 && group_size <= 0) return AR_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return AR_OK;
  if (K == 0) return AR_ERR_SHAPE;
  int64_t g = 0;
  AR_TRY(dequant_group(group_size, K, &g));
  if (qzeros && (N * bits) % 32 != 0) return AR_ERR_SHAPE;
  if (K * bits / 32 * N >= (int64_t(1) << 31) || (K / g) * N >= (int64_t(1) << 31))
    return AR_ERR_SHAPE;   // packed arrays are indexed with 32-bit offsets
  if (!X || !qweight || !scale || !Y || !ws) return AR_ERR_INVALID_ARG;
  if (!a16(X) || !a16(ws) || !a8(qweight)) return AR_ERR_INVALID_ARG;
  if (ws_bytes < dequant_ws(bits, M, N, K, g)) return AR_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M <= kGemvMaxM)
    return ar_launch_dq_gemv(bits, qweight, qzeros, scale, N, K, (int)g, X, (int)M,
                             static_cast<float*>(ws), Y, ydt, st);
  Carver c{static_cast<uint8_t*>(ws)};
  uint16_t* XB = c.take<uint16_t>((size_t)arblk::row_tiles(M) * arblk::k_blocks(K) *
                                  arblk::BLOCK_ELEMS * 2);
  uint16_t* WB = c.take<uint16_t>((size_t)arblk::row_tiles(N) * arblk::k_blocks(K) *
                                  arblk::BLOCK_ELEMS * 2);
  const int64_t nkb = arblk::k_blocks(K);
  AR_TRY(ar_launch_block_copy(X, XB, 1, M, K, nkb, st));
  // the dequantization writes every element of [N, K]; only padding rows and
  // reduction elements need clearing
  if (N % arblk::ROWS != 0 || K % arblk::KB != 0)
    AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(WB),
                              0.0f, arblk::row_tiles(N) * nkb * arblk::BLOCK_ELEMS / 2, st));
  AR_TRY(ar_launch_dequant_blocked(bits, qweight, qzeros, scale, N, K, (int)g, WB, st));
  return ar_launch_gemm_out(XB, WB, Y, ydt, M, N, K, st);
}

ar_status ar_pack(int32_t bits, const uint8_t* codes, const uint8_t* zp, int64_t N, int64_t K,
                  int64_t G, int32_t* qweight, int32_t* qzeros, void* stream) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return AR_ERR_UNSUPPORTED;
  if (N < 0 || K < 0) return AR_ERR_SHAPE;
  if (N == 0 || K == 0) return AR_OK;
  if ((K * bits) % 32 != 0 || K % 4 != 0) return AR_ERR_SHAPE;
  if (!codes || !qweight || !a16(codes)) return AR_ERR_INVALID_ARG;
  if ((zp == nullptr) != (qzeros == nullptr)) return AR_ERR_INVALID_ARG;
  if (zp && (G <= 0 || (N * bits) % 32 != 0)) return AR_ERR_SHAPE;
  return ar_launch_pack(bits, codes, zp, N, K, G, qweight, qzeros,
                        static_cast<hipStream_t>(stream));
}

ar_status ar_unpack(int32_t bits, const int32_t* qweight, const int32_t* qzeros, int64_t N,
                    int64_t K, int64_t G, uint8_t* codes, uint8_t* zp, void* stream) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return AR_ERR_UNSUPPORTED;
  if (N < 0 || K < 0) return AR_ERR_SHAPE;
  if (N == 0 || K == 0) return AR_OK;
  if ((K * bits) % 32 != 0 || K % 4 != 0) return AR_ERR_SHAPE;
  if (!codes || !qweight) return AR_ERR_INVALID_ARG;
  if ((zp == nullptr) != (qzeros == nullptr)) return AR_ERR_INVALID_ARG;
  if (zp && (G <= 0 || (N * bits) % 32 != 0)) return AR_ERR_SHAPE;
  return ar_launch_unpack(bits, qweight, qzeros, N, K, G, codes, zp,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"
