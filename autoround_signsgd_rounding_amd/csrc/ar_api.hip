// C ABI of the AutoRound tuning library: argument validation (before any HIP
// call, so an error leaves nothing enqueued), workspace carving, and the order
// of kernel launches for one step and for the whole per-Linear loop.
#include <math.h>
#include <string.h>

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

// bits / group / sym / shape checks shared by every quantizing entry point.
// *g = group size in elements (0 when N*K == 0).
ar_status check_quant(const ar_config* c, int64_t N, int64_t K, int* g) {
  if (!c) return AR_ERR_INVALID_ARG;
  if (!(c->bits == 2 || c->bits == 3 || c->bits == 4 || c->bits == 8)) return AR_ERR_UNSUPPORTED;
  if (c->sym != 0 && c->sym != 1) return AR_ERR_INVALID_ARG;
  if (c->group_size != -1 && c->group_size <= 0) return AR_ERR_INVALID_ARG;
  if (!finite(c->minmax_shrink) || c->minmax_shrink <= 0.0f) return AR_ERR_INVALID_ARG;
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
  ArLossIn li;
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
  return AR_OK;
}

const char* ar_status_string(int32_t s) {
  switch (s) {
    case AR_OK: return "ok";
    case AR_ERR_INVALID_ARG: return "invalid argument (null pointer, bad hyper-parameter or misaligned pointer)";
    case AR_ERR_UNSUPPORTED: return "unsupported (bits must be 2, 3, 4 or 8; group_size a multiple of 8; dtype f32/bf16)";
    case AR_ERR_SHAPE: return "shape constraint violated";
    case AR_ERR_WORKSPACE: return "workspace too small";
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

ar_status ar_rtn_quant(const ar_config* c, int32_t wdt, const void* W, int64_t N, int64_t K,
                       uint8_t* codes, float* scale, uint8_t* zp, void* Wq, void* stream) {
  int g;
  AR_TRY(check_quant(c, N, K, &g));
  if (!dtype_ok(wdt)) return AR_ERR_UNSUPPORTED;
  if (g == 0) return AR_OK;
  if (!W || !a16(W) || !a16(Wq) || !a8(codes)) return AR_ERR_INVALID_ARG;
  return ar_launch_fakequant(wdt, W, nullptr, nullptr, nullptr, c->minmax_shrink, N, K, g,
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
  return ar_launch_fakequant(wdt, W, V, alpha, beta, c->minmax_shrink, N, K, g, grid_of(c),
                             AR_BF16, Wq_bf16, 0, codes, scale, zp,
                             static_cast<hipStream_t>(stream));
}

ar_status ar_tune_step(const ar_config* c, const ar_state* s, const uint16_t* Xb, const void* Yb,
                       int32_t ydt, int64_t Tb, float* loss_out, float* gV, float* galpha,
                       float* gbeta, int32_t apply_update, void* ws, size_t ws_bytes,
                       void* stream) {
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
  const int64_t N = s->N, K = s->K;
  size_t need;
  carve_step(nullptr, N, K, Tb, ydt, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  StepWs w = carve_step(ws, N, K, Tb, ydt, &need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BlkSizes z(N, K, Tb);

  // stage the minibatch into the blocked GEMM layouts, Ŵ of the current state
  AR_TRY(ar_launch_block_copy(Xb, w.XB, 1, Tb, K, z.nkbK, st));
  AR_TRY(ar_launch_block_transpose(Xb, w.XTB, 1, Tb, K, z.nkbT, 2, st));
  AR_TRY(ar_launch_block_transpose(Yb, w.YB, 1, Tb, N, z.nkbT, (int)dsize(ydt), st));
  AR_TRY(ar_launch_fill_f32(reinterpret_cast<float*>(w.WB), 0.0f, z.wb / 2, st));
  AR_TRY(ar_launch_fakequant(s->wdt, s->W, s->V, s->alpha, s->beta, c->minmax_shrink, N, K, g,
                             grid_of(c), AR_BF16, w.WB, z.nkbK, nullptr, nullptr, nullptr, st));
  return enqueue_step(c, s->wdt, s->W, N, K, g, w.XB, w.XTB, w.YB, ydt, Tb, w.WB, w.dyB, w.G,
                      w.partials, w.flag, loss_out, nullptr, s->best_loss, s->V, s->alpha,
                      s->beta, s->best_V, s->best_alpha, s->best_beta, gV, galpha, gbeta,
                      apply_update != 0, false, st, nullptr);
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

  // one-time staging of every minibatch into the blocked GEMM layouts
  AR_TRY_C(ar_launch_block_copy(X, w.XB, nb, Tb, K, z.nkbK, st));
  AR_TRY_C(ar_launch_block_transpose(X, w.XTB, nb, Tb, K, z.nkbT, 2, st));
  AR_TRY_C(ar_launch_block_transpose(Y, w.YB, nb, Tb, N, z.nkbT, (int)ysz, st));
  AR_TRY_C(ar_launch_fill_f32(reinterpret_cast<float*>(w.WB), 0.0f, z.wb / 2, st));
  // initial state: V = 0, alpha = beta = minmax_shrink, best = initial, best loss = +inf
  AR_TRY_C(ar_launch_fill_f32(w.V, 0.0f, N * K, st));
  AR_TRY_C(ar_launch_fill_f32(w.bestV, 0.0f, N * K, st));
  AR_TRY_C(ar_launch_fill_f32(w.alpha, c->minmax_shrink, N * Gn, st));
  AR_TRY_C(ar_launch_fill_f32(w.beta, c->minmax_shrink, N * Gn, st));
  AR_TRY_C(ar_launch_fill_f32(w.bestA, c->minmax_shrink, N * Gn, st));
  AR_TRY_C(ar_launch_fill_f32(w.bestB, c->minmax_shrink, N * Gn, st));
  AR_TRY_C(ar_launch_fill_f32(w.best_loss, INFINITY, 1, st));
  const ArGrid gr = grid_of(c);
  if (c->iters > 0)
    AR_TRY_C(ar_launch_fakequant(wdt, W, w.V, w.alpha, w.beta, c->minmax_shrink, N, K, g, gr,
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
  AR_TRY_C(ar_launch_fakequant(wdt, W, w.bestV, w.bestA, w.bestB, c->minmax_shrink, N, K, g, gr,
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
