// Sequential block-wise tuning with quantized inputs (gfx950): the forward of a
// Llama-style decoder block and the driver that tunes its seven Linears in
// order, each on its input in the quantized pipeline (the block with the
// Linears tuned so far) and its full-precision target (llm-compressor AutoRound
// page: the per-subgraph loop; enable_quanted_input uses the previous layers'
// quantized output as input; design point 3, layer by layer).
//
// The block (the pages do not show one; LLaMA-2-7B is their model):
//   a = RMSNorm(h); q, k, v = a·W{q,k,v}ᵀ; rotary (rotate-half) on q, k;
//   attn = causal softmax(q·kᵀ/sqrt(Dh))·v per sequence and head;
//   h1 = h + attn·Woᵀ; m = RMSNorm(h1); z = SiLU(m·Wgᵀ)·(m·Wuᵀ); out = h1 + z·Wdᵀ.
// Activations are bf16 between operations. Each operation rounds its float32
// result to bf16 (RNE): RMSNorm sums squares in float64, the rotary table is
// float64 rounded to float32, SiLU·mul is float64, additions float32, the
// Linears float32 MFMA accumulation, attention float32 with an online softmax.
#include <math.h>
#include <string.h>

#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"

namespace {

constexpr int NT = 256;

inline ar_status last_status() { return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP; }
inline unsigned grid_for(int64_t n) {
  const int64_t b = (n + NT - 1) / NT;
  return (unsigned)(b < 65536 ? b : 65536);
}

// ------------------------------------------------------------------ elementwise
// y = x / sqrt(mean(x²) + eps) · w per row (one workgroup per row).
__global__ __launch_bounds__(NT) void k_rmsnorm(const uint16_t* __restrict__ x,
                                                const uint16_t* __restrict__ w,
                                                uint16_t* __restrict__ y, int64_t D, float eps) {
  __shared__ double sh[NT];
  const uint16_t* xr = x + (int64_t)blockIdx.x * D;
  uint16_t* yr = y + (int64_t)blockIdx.x * D;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < D; i += NT) {
    const double v = (double)bf16_val(xr[i]);
    acc += v * v;
  }
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const float r = (float)(1.0 / sqrt(sh[0] / (double)D + (double)eps));
  for (int64_t i = threadIdx.x; i < D; i += NT)
    yr[i] = (uint16_t)bf16_bits((bf16_val(xr[i]) * r) * bf16_val(w[i]));
}

// cos/sin [S, Dh/2] of p·theta^(-2j/Dh), float64 rounded to float32.
__global__ __launch_bounds__(NT) void k_rope_table(float* cs, float* sn, int S, int Dh,
                                                   double theta) {
  const int half = Dh / 2;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < (int64_t)S * half;
       e += (int64_t)gridDim.x * NT) {
    const int p = (int)(e / half), j = (int)(e % half);
    const double ang = (double)p * pow(theta, -2.0 * (double)j / (double)Dh);
    cs[e] = (float)cos(ang);
    sn[e] = (float)sin(ang);
  }
}

// Rotate-half rotary embedding of x [M, D] into y (heads of Dh, position = row mod S).
__global__ __launch_bounds__(NT) void k_rope(const uint16_t* __restrict__ x,
                                             uint16_t* __restrict__ y, const float* cs,
                                             const float* sn, int64_t M, int D, int Dh, int S) {
  const int half = Dh / 2, H = D / Dh;
  const int64_t total = M * H * half;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * NT) {
    const int64_t row = e / (H * half);
    const int r = (int)(e - row * H * half), h = r / half, j = r % half;
    const int p = (int)(row % S);
    const int64_t ia = row * D + h * Dh + j, ib = ia + half;
    const float a = bf16_val(x[ia]), b = bf16_val(x[ib]);
    const float c = cs[p * half + j], s = sn[p * half + j];
    y[ia] = (uint16_t)bf16_bits(a * c - b * s);
    y[ib] = (uint16_t)bf16_bits(b * c + a * s);
  }
}

__global__ __launch_bounds__(NT) void k_silu_mul(const uint16_t* g, const uint16_t* u, uint16_t* z,
                                                 int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const double gv = (double)bf16_val(g[i]);
    z[i] = (uint16_t)bf16_bits((float)(gv / (1.0 + exp(-gv)) * (double)bf16_val(u[i])));
  }
}

__global__ __launch_bounds__(NT) void k_add(const uint16_t* a, const uint16_t* b, uint16_t* c,
                                            int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    c[i] = (uint16_t)bf16_bits(bf16_val(a[i]) + bf16_val(b[i]));
}

// ------------------------------------------------------------------ attention
// Causal attention for one (sequence, head) and 256 queries per workgroup, one
// query per thread: keys and values go through LDS in tiles of KT; per tile
// the scores are formed first, then the running max, the rescale of the
// running sums, and the weighted values (online softmax, float32).
template <int DH>
__global__ __launch_bounds__(NT) void k_attention(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  uint16_t* __restrict__ out, int D, int S,
                                                  int H, float scale) {
  constexpr int KT = 32;
  __shared__ float ks[KT][DH];
  __shared__ float vs[KT][DH];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int q0 = blockIdx.y * NT;
  const int i = q0 + threadIdx.x;
  const bool live = i < S;
  const int64_t base = (int64_t)b * S;
  float qv[DH], o[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = live ? bf16_val(q[(base + i) * D + h * DH + d]) : 0.0f;
    o[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int kend = min(S, q0 + NT);
  for (int t0 = 0; t0 < kend; t0 += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * DH; e += NT) {
      const int j = e / DH, d = e % DH, key = t0 + j;
      const bool ok = key < S;
      ks[j][d] = ok ? bf16_val(k[(base + key) * D + h * DH + d]) : 0.0f;
      vs[j][d] = ok ? bf16_val(v[(base + key) * D + h * DH + d]) : 0.0f;
    }
    __syncthreads();
    if (live && t0 <= i) {
      float s[KT];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DH; ++d) dot = fmaf(qv[d], ks[j][d], dot);
        s[j] = (t0 + j <= i) ? dot * scale : -INFINITY;
        tmax = fmaxf(tmax, s[j]);
      }
      const float mn = fmaxf(m, tmax);
      const float corr = expf(m - mn);
      l *= corr;
#pragma unroll
      for (int d = 0; d < DH; ++d) o[d] *= corr;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const float p = (t0 + j <= i) ? expf(s[j] - mn) : 0.0f;
        l += p;
#pragma unroll
        for (int d = 0; d < DH; ++d) o[d] = fmaf(p, vs[j][d], o[d]);
      }
      m = mn;
    }
  }
  if (live) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DH; ++d)
      out[(base + i) * D + h * DH + d] = (uint16_t)bf16_bits(o[d] * inv);
  }
}

struct Carve {
  uint8_t* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t n) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (n * sizeof(T) + 255) & ~size_t(255);
    return p;
  }
};

#define AR_TRY(expr)                   \
  do {                                 \
    ar_status _s = (expr);             \
    if (_s != AR_OK) return _s;        \
  } while (0)

struct Dims {
  int64_t D, H, Dh, F, S, B, M;
  float eps;
  double theta;
};

// Linear y = x·Wᵀ (x [M, K], W [N, K] bf16 row-major) through the blocked MFMA product.
struct LinearWs {
  uint16_t* XB;
  uint16_t* WB;
};

ar_status linear(const LinearWs& w, const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M,
                 int64_t N, int64_t K, hipStream_t st) {
  const int64_t nkb = arblk::k_blocks(K);
  AR_TRY(ar_launch_block_copy(x, w.XB, 1, M, K, nkb, st));
  AR_TRY(ar_launch_block_copy(W, w.WB, 1, N, K, nkb, st));
  return ar_launch_gemm_out(w.XB, w.WB, y, AR_BF16, M, N, K, st);
}

ar_status attention(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    uint16_t* out, hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.H), (unsigned)((d.S + NT - 1) / NT));
  const float scale = (float)(1.0 / sqrt((double)d.Dh));
  if (d.Dh == 64)
    hipLaunchKernelGGL(k_attention<64>, grid, dim3(NT), 0, st, q, k, v, out, (int)d.D, (int)d.S,
                       (int)d.H, scale);
  else if (d.Dh == 128)
    hipLaunchKernelGGL(k_attention<128>, grid, dim3(NT), 0, st, q, k, v, out, (int)d.D, (int)d.S,
                       (int)d.H, scale);
  else
    return AR_ERR_UNSUPPORTED;
  return last_status();
}

// Activations of one pipeline.
struct Acts {
  uint16_t *a, *q, *k, *v, *qr, *kr, *attn, *o, *h1, *m, *g, *u, *z, *dn, *out;
};

Acts carve_acts(Carve& c, const Dims& d) {
  Acts t;
  const size_t MD = (size_t)(d.M * d.D), MF = (size_t)(d.M * d.F);
  t.a = c.take<uint16_t>(MD); t.q = c.take<uint16_t>(MD); t.k = c.take<uint16_t>(MD);
  t.v = c.take<uint16_t>(MD); t.qr = c.take<uint16_t>(MD); t.kr = c.take<uint16_t>(MD);
  t.attn = c.take<uint16_t>(MD); t.o = c.take<uint16_t>(MD); t.h1 = c.take<uint16_t>(MD);
  t.m = c.take<uint16_t>(MD); t.g = c.take<uint16_t>(MF); t.u = c.take<uint16_t>(MF);
  t.z = c.take<uint16_t>(MF); t.dn = c.take<uint16_t>(MD); t.out = c.take<uint16_t>(MD);
  return t;
}

struct BlockWs {
  Acts fp, qp;
  LinearWs lin;
  float *cs, *sn;
  uint8_t* tune;
  size_t tune_bytes;
};

const int64_t kLinN[7] = {0, 0, 0, 0, 1, 1, 0};   // out features: 0 = D, 1 = F
const int64_t kLinK[7] = {0, 0, 0, 0, 0, 0, 1};   // in features: 0 = D, 1 = F

BlockWs carve_block(void* ws, const Dims& d, size_t tune_bytes, size_t* bytes) {
  Carve c{static_cast<uint8_t*>(ws)};
  BlockWs w;
  w.fp = carve_acts(c, d);
  w.qp = carve_acts(c, d);
  const int64_t Kmax = d.F > d.D ? d.F : d.D;
  w.lin.XB = c.take<uint16_t>((size_t)(arblk::row_tiles(d.M) * arblk::k_blocks(Kmax) *
                                       arblk::BLOCK_ELEMS));
  w.lin.WB = c.take<uint16_t>((size_t)(arblk::row_tiles(Kmax) * arblk::k_blocks(Kmax) *
                                       arblk::BLOCK_ELEMS));
  w.cs = c.take<float>((size_t)(d.S * d.Dh / 2));
  w.sn = c.take<float>((size_t)(d.S * d.Dh / 2));
  w.tune = c.take<uint8_t>(tune_bytes);
  w.tune_bytes = tune_bytes;
  *bytes = c.off;
  return w;
}

ar_status check_dims(const ar_block_dims* bd, Dims* d) {
  if (!bd) return AR_ERR_INVALID_ARG;
  d->D = bd->hidden; d->H = bd->heads; d->F = bd->inter; d->S = bd->seqlen; d->B = bd->nsamples;
  if (d->D <= 0 || d->H <= 0 || d->F <= 0 || d->S <= 0 || d->B <= 0) return AR_ERR_SHAPE;
  if (d->D % d->H != 0) return AR_ERR_SHAPE;
  d->Dh = d->D / d->H;
  if (d->Dh != 64 && d->Dh != 128) return AR_ERR_UNSUPPORTED;
  if (d->D % 8 != 0 || d->F % 8 != 0) return AR_ERR_SHAPE;
  d->M = d->S * d->B;
  if (!(bd->rms_eps >= 0.0f) || !(bd->rope_theta > 0.0f)) return AR_ERR_INVALID_ARG;
  d->eps = bd->rms_eps;
  d->theta = bd->rope_theta;
  return AR_OK;
}

const uint16_t* weight_of(const ar_block_weights* w, int i) {
  const uint16_t* all[7] = {w->Wq, w->Wk, w->Wv, w->Wo, w->Wg, w->Wu, w->Wd};
  return all[i];
}

// The block from h up to (and including) the stage that produces Linear `upto`'s
// input; stage order: 0 a, 1 q/k/v + rotary + attention, 2 o/h1/m, 3 gate/up/z,
// 4 down/out. W[i] are the weights to use.
ar_status forward_stages(const Dims& d, const BlockWs& w, const Acts& t, const uint16_t* h,
                         const uint16_t* const W[7], const uint16_t* n1, const uint16_t* n2,
                         int from, int to, hipStream_t st) {
  const int64_t MD = d.M * d.D, MF = d.M * d.F;
  for (int s = from; s <= to; ++s) {
    switch (s) {
      case 0:
        hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)d.M), dim3(NT), 0, st, h, n1, t.a, d.D,
                           d.eps);
        AR_TRY(last_status());
        break;
      case 1:
        AR_TRY(linear(w.lin, t.a, W[0], t.q, d.M, d.D, d.D, st));
        AR_TRY(linear(w.lin, t.a, W[1], t.k, d.M, d.D, d.D, st));
        AR_TRY(linear(w.lin, t.a, W[2], t.v, d.M, d.D, d.D, st));
        hipLaunchKernelGGL(k_rope, dim3(grid_for(MD / 2)), dim3(NT), 0, st, t.q, t.qr, w.cs, w.sn,
                           d.M, (int)d.D, (int)d.Dh, (int)d.S);
        hipLaunchKernelGGL(k_rope, dim3(grid_for(MD / 2)), dim3(NT), 0, st, t.k, t.kr, w.cs, w.sn,
                           d.M, (int)d.D, (int)d.Dh, (int)d.S);
        AR_TRY(last_status());
        AR_TRY(attention(d, t.qr, t.kr, t.v, t.attn, st));
        break;
      case 2:
        AR_TRY(linear(w.lin, t.attn, W[3], t.o, d.M, d.D, d.D, st));
        hipLaunchKernelGGL(k_add, dim3(grid_for(MD)), dim3(NT), 0, st, h, t.o, t.h1, MD);
        AR_TRY(last_status());
        hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)d.M), dim3(NT), 0, st, t.h1, n2, t.m, d.D,
                           d.eps);
        AR_TRY(last_status());
        break;
      case 3:
        AR_TRY(linear(w.lin, t.m, W[4], t.g, d.M, d.F, d.D, st));
        AR_TRY(linear(w.lin, t.m, W[5], t.u, d.M, d.F, d.D, st));
        hipLaunchKernelGGL(k_silu_mul, dim3(grid_for(MF)), dim3(NT), 0, st, t.g, t.u, t.z, MF);
        AR_TRY(last_status());
        break;
      case 4:
        AR_TRY(linear(w.lin, t.z, W[6], t.dn, d.M, d.D, d.F, st));
        hipLaunchKernelGGL(k_add, dim3(grid_for(MD)), dim3(NT), 0, st, t.h1, t.dn, t.out, MD);
        AR_TRY(last_status());
        break;
    }
  }
  return AR_OK;
}

ar_status rope_table(const Dims& d, const BlockWs& w, hipStream_t st) {
  hipLaunchKernelGGL(k_rope_table, dim3(grid_for(d.S * d.Dh / 2)), dim3(NT), 0, st, w.cs, w.sn,
                     (int)d.S, (int)d.Dh, d.theta);
  return last_status();
}

bool weights_ok(const ar_block_weights* w) {
  if (!w || !w->norm_attn || !w->norm_mlp) return false;
  for (int i = 0; i < 7; ++i)
    if (!weight_of(w, i) || (reinterpret_cast<uintptr_t>(weight_of(w, i)) & 15u)) return false;
  return true;
}

// Largest ar_tune_linear workspace over the block's Linear shapes.
ar_status tune_ws(const ar_config* c, const Dims& d, size_t* bytes) {
  *bytes = 0;
  for (int i = 0; i < 7; ++i) {
    size_t b;
    const int64_t N = kLinN[i] ? d.F : d.D, K = kLinK[i] ? d.F : d.D;
    AR_TRY(ar_workspace_size(c, N, K, AR_BF16, &b));
    if (b > *bytes) *bytes = b;
  }
  return AR_OK;
}

}  // namespace

extern "C" {

ar_status ar_block_workspace_size(const ar_config* cfg, const ar_block_dims* bd, size_t* bytes) {
  Dims d;
  if (!bytes) return AR_ERR_INVALID_ARG;
  AR_TRY(check_dims(bd, &d));
  size_t tb = 0;
  if (cfg) {
    if ((int64_t)cfg->nsamples * cfg->seqlen != d.M || cfg->seqlen != d.S) return AR_ERR_SHAPE;
    AR_TRY(tune_ws(cfg, d, &tb));
  }
  carve_block(nullptr, d, tb, bytes);
  return AR_OK;
}

ar_status ar_block_forward(const ar_block_dims* bd, const ar_block_weights* wts,
                           const uint16_t* h, uint16_t* out, void* ws, size_t ws_bytes,
                           void* stream) {
  Dims d;
  AR_TRY(check_dims(bd, &d));
  if (!weights_ok(wts) || !h || !out || !ws) return AR_ERR_INVALID_ARG;
  size_t need;
  carve_block(nullptr, d, 0, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  BlockWs w = carve_block(ws, d, 0, &need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* W[7];
  for (int i = 0; i < 7; ++i) W[i] = weight_of(wts, i);
  AR_TRY(rope_table(d, w, st));
  AR_TRY(forward_stages(d, w, w.fp, h, W, wts->norm_attn, wts->norm_mlp, 0, 4, st));
  if (hipMemcpyAsync(out, w.fp.out, (size_t)(d.M * d.D) * 2, hipMemcpyDeviceToDevice, st))
    return AR_ERR_HIP;
  return AR_OK;
}

ar_status ar_tune_block(const ar_config* cfg, const ar_block_dims* bd,
                        const ar_block_weights* wts, const uint16_t* h, const uint16_t* h_q,
                        int32_t quanted_input, const ar_block_outputs* outs, void* ws,
                        size_t ws_bytes, void* stream) {
  Dims d;
  AR_TRY(check_dims(bd, &d));
  if (!cfg || !weights_ok(wts) || !h || !outs || !ws) return AR_ERR_INVALID_ARG;
  if ((int64_t)cfg->nsamples * cfg->seqlen != d.M || cfg->seqlen != d.S) return AR_ERR_SHAPE;
  for (int i = 0; i < 7; ++i)
    if (!outs->codes[i] || !outs->scale[i] || !outs->zp[i] || !outs->Wq[i])
      return AR_ERR_INVALID_ARG;
  size_t tb, need;
  AR_TRY(tune_ws(cfg, d, &tb));
  carve_block(nullptr, d, tb, &need);
  if (ws_bytes < need) return AR_ERR_WORKSPACE;
  BlockWs w = carve_block(ws, d, tb, &need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* hq = h_q ? h_q : h;

  const uint16_t* Wfp[7];
  const uint16_t* Wqp[7];
  for (int i = 0; i < 7; ++i) Wfp[i] = Wqp[i] = weight_of(wts, i);
  AR_TRY(rope_table(d, w, st));
  // full-precision pipeline: every Linear's target and (without quantized inputs) input
  AR_TRY(forward_stages(d, w, w.fp, h, Wfp, wts->norm_attn, wts->norm_mlp, 0, 4, st));
  const uint16_t* fp_out[7] = {w.fp.q, w.fp.k, w.fp.v, w.fp.o, w.fp.g, w.fp.u, w.fp.dn};
  const uint16_t* fp_in[7] = {w.fp.a, w.fp.a, w.fp.a, w.fp.attn, w.fp.m, w.fp.m, w.fp.z};
  const uint16_t* q_in[7] = {w.qp.a, w.qp.a, w.qp.a, w.qp.attn, w.qp.m, w.qp.m, w.qp.z};
  // stage that produces each Linear's input in the quantized pipeline
  const int stage_of[7] = {0, 0, 0, 1, 2, 2, 3};
  int done = -1;   // last quantized-pipeline stage computed
  for (int i = 0; i < 7; ++i) {
    const int64_t N = kLinN[i] ? d.F : d.D, K = kLinK[i] ? d.F : d.D;
    if (quanted_input && stage_of[i] > done) {
      AR_TRY(forward_stages(d, w, w.qp, hq, Wqp, wts->norm_attn, wts->norm_mlp, done + 1,
                            stage_of[i], st));
      done = stage_of[i];
    }
    const uint16_t* X = quanted_input ? q_in[i] : fp_in[i];
    AR_TRY(ar_tune_linear(cfg, AR_BF16, Wfp[i], N, K, X, fp_out[i], AR_BF16, outs->codes[i],
                          outs->scale[i], outs->zp[i], outs->Wq[i], nullptr, nullptr, nullptr,
                          outs->losses[i], w.tune, w.tune_bytes, nullptr, stream));
    Wqp[i] = outs->Wq[i];
  }
  // the quantized block's output with every Linear tuned
  if (!quanted_input) done = -1;
  AR_TRY(forward_stages(d, w, w.qp, hq, Wqp, wts->norm_attn, wts->norm_mlp, done + 1, 4, st));
  if (outs->out_q &&
      hipMemcpyAsync(outs->out_q, w.qp.out, (size_t)(d.M * d.D) * 2, hipMemcpyDeviceToDevice, st))
    return AR_ERR_HIP;
  if (outs->out_fp &&
      hipMemcpyAsync(outs->out_fp, w.fp.out, (size_t)(d.M * d.D) * 2, hipMemcpyDeviceToDevice, st))
    return AR_ERR_HIP;
  return AR_OK;
}

}  // extern "C"
