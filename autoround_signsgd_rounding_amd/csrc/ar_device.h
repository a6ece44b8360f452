// Device-side helpers for the gfx950 AutoRound kernels: bf16 rounding, buffer
// resources, group reductions and the float32 quantizer step sequence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
// float32 -> bf16 bit pattern, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

// Two values to bf16 in one v_cvt_pk_bf16_f32 (lo in bits 0..15): nearest
// even, the same bits as bf16_bits for every non-NaN value (a NaN stays a
// NaN, its payload aside).
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2_hw_t h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer descriptor: loads at byte offsets >= num_bytes return zero, which
// gives free zero-fill for ragged tiles (rows past the end of a panel).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
static constexpr uint32_t kOOB = 0x80000000u;  // offset that always lies past a panel

// ---------------------------------------------------------------- 8-element chunks
__device__ __forceinline__ void load8(const uint16_t* p, float (&o)[8]) {
  u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(v[i] << 16);
    o[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
  f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
  f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4_t a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  reinterpret_cast<f32x4_t*>(p)[0] = a;
  reinterpret_cast<f32x4_t*>(p)[1] = b;
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16_bits(v[2 * i]) | (bf16_bits(v[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(p) = o;
}
__device__ __forceinline__ void store8_u8(uint8_t* p, const float (&q)[8]) {
  u32x2_t o;
  o[0] = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
  o[1] = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
  *reinterpret_cast<u32x2_t*>(p) = o;
}

// ---------------------------------------------------------------- group reductions
// Butterfly over LPG consecutive lanes (LPG a power of two <= 64). Every lane
// of the group ends with the same value and the order is fixed.
template <int LPG>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = LPG / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
template <int LPG>
__device__ __forceinline__ double group_sum_f64(double x) {
#pragma unroll
  for (int o = LPG / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
template <int LPG>
__device__ __forceinline__ float group_min(float x) {
#pragma unroll
  for (int o = LPG / 2; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
template <int LPG>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int o = LPG / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// ---------------------------------------------------------------- quantizer
// Static description of the integer grid.
struct Grid {
  float maxq;   // 2^bits - 1
  float half;   // 2^(bits-1): symmetric zero-point
  int sym;
};

// Group scale / zero-point from the clipped min/max. float32, in this order:
//   asym: lo = min(alpha*wmin, 0); hi = max(beta*wmax, 0); s = (hi - lo)/maxq;
//         zp = clamp(rint(-lo/s), 0, maxq)
//   sym:  amax = max(|alpha*wmin|, |beta*wmax|); s = (2*amax)/maxq; zp = 2^(bits-1)
// A zero-range group gets s = 1 (flagged in `zero`).
struct QP {
  float s, zp, lo;
  bool zero;
};
__device__ __forceinline__ QP group_qparams(float wmin, float wmax, float alpha, float beta,
                                            const Grid& gr) {
  QP r;
  if (gr.sym) {
    float amax = fmaxf(fabsf(alpha * wmin), fabsf(beta * wmax));
    float s = (2.0f * amax) / gr.maxq;
    r.zero = (s == 0.0f);
    r.s = r.zero ? 1.0f : s;
    r.zp = gr.half;
    r.lo = 0.0f;
  } else {
    float lo = fminf(alpha * wmin, 0.0f);
    float hi = fmaxf(beta * wmax, 0.0f);
    float s = (hi - lo) / gr.maxq;
    r.zero = (s == 0.0f);
    r.s = r.zero ? 1.0f : s;
    r.zp = fminf(fmaxf(rintf(-lo / r.s), 0.0f), gr.maxq);
    r.lo = lo;
  }
  return r;
}

// One element: t = w/s (IEEE division); r = rint(t + v) (half to even);
// c = r + zp; q = clamp(c, 0, maxq); m = [0 <= c <= maxq]; what = s*(q - zp).
struct QE {
  float t, q, what;
  bool m;
};
__device__ __forceinline__ QE quant_elem(float w, float v, const QP& p, const Grid& gr) {
  QE e;
  e.t = w / p.s;
  float u = e.t + v;
  float c = rintf(u) + p.zp;
  e.q = fminf(fmaxf(c, 0.0f), gr.maxq);
  e.m = (c >= 0.0f) && (c <= gr.maxq);
  e.what = p.s * (e.q - p.zp);
  return e;
}

// Sum over the 64 lanes of a wave (butterfly, fixed order; every lane gets it).
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---------------------------------------------------------------- loss reduction
// Sum of n float32 partials in float64 by a block of 256 threads, in a fixed
// order: thread t adds partials t, t+256, ... in turn, then a pairwise tree
// over the 256 sums. Every thread of the block calls it; all get the total.
// sh: 256 doubles of LDS.
__device__ __forceinline__ double block_sum_f64(const float* partials, int n, double* sh) {
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int i = t; i < n; i += 256) acc += (double)partials[i];
  sh[t] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) sh[t] += sh[t + s];
    __syncthreads();
  }
  return sh[0];
}

__device__ __forceinline__ float sgnf(float x) {
  return (x > 0.0f) ? 1.0f : ((x < 0.0f) ? -1.0f : 0.0f);
}
