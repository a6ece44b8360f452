// Sequential block-wise tuning with quantized inputs (gfx950): the forward of a
// Llama-style decoder block and the host routine that tunes its seven Linears in
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
// Linears float32 MFMA accumulation, attention float32 MFMA accumulation with
// an online softmax.
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
// Causal attention on v_mfma_f32_16x16x32_bf16, for one (sequence, head) and
// 64 queries per workgroup (16 per wave). Keys and values pass through LDS in
// tiles of 64: K row-major, V transposed (Vᵀ[dh][key]).
//
// Scores are formed transposed, Sᵀ = K·Qᵀ (A: 8 dh of a key row, B: the same
// 8 dh of a query), so lane l holds query l % 16 at keys 16j + 4·(l/16) + r of
// the tile. The online softmax therefore keeps one running max and sum per
// lane, exchanged across the four lanes of a query only for the tile max and
// the final sum. P = exp(s − max) is split into three bf16 parts whose sum is
// the float32 weight to its last bit or so, and Oᵀ = Vᵀ·Pᵀ takes each part as
// the B operand in the same registers it was computed in; the A operand reads
// Vᵀ at the lane's keys.
// Float32 throughout; exp is exp2 of scores pre-scaled by log2(e)/sqrt(Dh).
template <int DH>
__global__ __launch_bounds__(NT) void k_attention(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  uint16_t* __restrict__ out, int D, int S,
                                                  int H, float scale_log2e) {
  constexpr int KT = 64;            // keys per tile
  constexpr int KS = DH + 8;        // K row stride (elements): rows 16 banks apart
  constexpr int VS = KT + 8;        // Vᵀ row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t ks[KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[DH * VS];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;
  const int qb = blockIdx.y * 64;          // first query of the workgroup
  const int qw = qb + 16 * wave;           // first query of the wave
  const int qi = qw + (lane & 15);         // the lane's query
  const int64_t base = (int64_t)b * S;
  const uint16_t* kh = k + base * D + h * DH;
  const uint16_t* vh = v + base * D + h * DH;

  bf16x8_t qf[DH / 32];                    // B operand: Q[qi][32c + 8·g4 .. +8]
#pragma unroll
  for (int c = 0; c < DH / 32; ++c) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (qi < S) w = *reinterpret_cast<const u32x4_t*>(q + (base + qi) * D + h * DH + 32 * c + 8 * g4);
    qf[c] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x4_t o[DH / 16];                      // Oᵀ[16d + 4·g4 + r][qi]
#pragma unroll
  for (int d = 0; d < DH / 16; ++d) o[d] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  const int kend = min(S, qb + 64);
  for (int t0 = 0; t0 < kend; t0 += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * DH / 8; e += NT) {
      // K: consecutive threads along a key row
      const int key = e / (DH / 8), c = e % (DH / 8);
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (t0 + key < S) w = *reinterpret_cast<const u32x4_t*>(kh + (int64_t)(t0 + key) * D + 8 * c);
      *reinterpret_cast<u32x4_t*>(ks + key * KS + 8 * c) = w;
      // Vᵀ: consecutive threads along keys, so the transposed writes are adjacent
      const int vk = e % KT, vc = e / KT;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (t0 + vk < S) x = *reinterpret_cast<const u32x4_t*>(vh + (int64_t)(t0 + vk) * D + 8 * vc);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vt[(8 * vc + i) * VS + vk] = (uint16_t)(x[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();
    if (t0 > qw + 15) continue;            // every key after every query of the wave

    f32x4_t sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < DH / 32; ++c) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t*>(ks + (16 * j + (lane & 15)) * KS + 32 * c + 8 * g4);
        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[c], sc[j], 0, 0, 0);
      }
    }
    float s[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t0 + 16 * j + 4 * g4 + r;
        const float x = (key <= qi && key < S) ? sc[j][r] * scale_log2e : -INFINITY;
        s[4 * j + r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);       // finite: key 0 is in every query's first tile
    const float corr = exp2f(m - mn);
    m = mn;
    l *= corr;
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) o[d] *= corr;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {       // keys 32·h2 .. +31 of the tile
      bf16x8_t ph, pm, pl;
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {     // e2 < 4: block 2·h2, else block 2·h2 + 1
        const float p = exp2f(s[8 * h2 + e2] - mn);
        l += p;
        const __bf16 hi = (__bf16)p;
        const float r1 = p - (float)hi;    // exact
        const __bf16 mid = (__bf16)r1;
        ph[e2] = hi;
        pm[e2] = mid;
        pl[e2] = (__bf16)(r1 - (float)mid);
      }
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) {
        const uint16_t* vr = vt + (16 * d + (lane & 15)) * VS + 32 * h2 + 4 * g4;
        const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(vr);
        const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(vr + 16);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, u32x4_t{v0[0], v0[1], v1[0], v1[1]});
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pm, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, o[d], 0, 0, 0);
      }
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qi < S) {
    const float inv = 1.0f / l;
    uint16_t* orow = out + (base + qi) * D + h * DH + 4 * g4;
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) {
      const uint32_t lo = bf16_bits(o[d][0] * inv) | (bf16_bits(o[d][1] * inv) << 16);
      const uint32_t hi = bf16_bits(o[d][2] * inv) | (bf16_bits(o[d][3] * inv) << 16);
      *reinterpret_cast<u32x2_t*>(orow + 16 * d) = u32x2_t{lo, hi};
    }
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
  const dim3 grid((unsigned)(d.B * d.H), (unsigned)((d.S + 63) / 64));
  const float sl = (float)(1.4426950408889634 / sqrt((double)d.Dh));   // log2(e)/sqrt(Dh)
  if (d.Dh == 64)
    hipLaunchKernelGGL(k_attention<64>, grid, dim3(NT), 0, st, q, k, v, out, (int)d.D, (int)d.S,
                       (int)d.H, sl);
  else if (d.Dh == 128)
    hipLaunchKernelGGL(k_attention<128>, grid, dim3(NT), 0, st, q, k, v, out, (int)d.D, (int)d.S,
                       (int)d.H, sl);
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

ar_status ar_attention(const ar_block_dims* bd, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, uint16_t* out, void* stream) {
  Dims d;
  AR_TRY(check_dims(bd, &d));
  if (!q || !k || !v || !out) return AR_ERR_INVALID_ARG;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (!a16(q) || !a16(k) || !a16(v) || !a16(out)) return AR_ERR_INVALID_ARG;
  return attention(d, q, k, v, out, static_cast<hipStream_t>(stream));
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
