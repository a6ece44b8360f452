// Internal host-side launchers (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/autoround_hip.h"

struct ArGrid {
  float maxq, half;
  int sym;
};

// Lanes per group and 8-element chunks per lane for a group of g elements.
void ar_group_layout(int g, int* lpg, int* chunks_per_lane);

// GEMMs (ar_gemm.hip)
// Operands in the blocked layout of ar_blocked.h:
//   XB  rows Tb, reduction K      WB  rows N, reduction K
//   YB  rows N,  reduction Tb (padded to whole 256-row tiles of Tb), dtype ydt
//   dyB rows N,  reduction Tb (same padding)     XTB rows K, reduction Tb (same padding)
int ar_fwd_tiles(int64_t Tb, int64_t N);
ar_status ar_launch_gemm_fwd(const uint16_t* XB, const uint16_t* WB, const void* yB, int ydt,
                             uint16_t* dyB, float* partials, int64_t Tb, int64_t N, int64_t K,
                             hipStream_t st);
// Loss of the step from the forward product's per-tile sums of R², reduced by
// the gradient product's workgroup 0 (float64, fixed order) while its first
// loads are in flight: loss = sum * inv_count, written to loss_out / loss_slot
// (nullable); flag = (loss < *best_loss) with *best_loss lowered on
// improvement, or flag = 0 when best_loss is NULL.
struct ArLossIn {
  const float* partials;
  int nparts;
  double inv_count;     // 1 / (Tb * N)
  float* loss_out;
  float* loss_slot;
  float* best_loss;
  int* flag;
};
// G = scale * dYᵀ·X_b, row-major [N, K].
ar_status ar_launch_gemm_wgrad(const uint16_t* dyB, const uint16_t* XTB, float* G, int64_t N,
                               int64_t K, int64_t Tb, float scale, const ArLossIn& loss,
                               hipStream_t st);
// blocked staging: batch of row-major [R, KR] -> blocked (rows R, reduction KR)
ar_status ar_launch_block_copy(const uint16_t* src, uint16_t* dst, int64_t batch, int64_t R,
                               int64_t KR, int64_t nkb, hipStream_t st);
// batch of row-major [R, C] -> blocked (rows C, reduction R); elem_bytes 2 or 4
ar_status ar_launch_block_transpose(const void* src, void* dst, int64_t batch, int64_t R,
                                    int64_t C, int64_t nkb, int elem_bytes, hipStream_t st);

// Quantizer / update kernels (ar_quant.hip)
// out_dt: dtype of Wq (AR_BF16 or AR_F32); alpha/beta NULL means the constant `shrink`,
// V NULL means zero.
// wq_nkb > 0 writes Wq (bf16 only) in the blocked GEMM layout (rows N, reduction K).
ar_status ar_launch_fakequant(int wdt, const void* W, const float* V, const float* alpha,
                              const float* beta, float shrink, int64_t N, int64_t K, int g,
                              ArGrid gr, int out_dt, void* Wq, int64_t wq_nkb, uint8_t* codes,
                              float* scale, uint8_t* zp, hipStream_t st);

struct ArSteArgs {
  int wdt;
  const void* W;
  float* V;
  float* alpha;
  float* beta;
  const float* G;
  int64_t N, K;
  int g;
  ArGrid gr;
  float lr, mlr, clip_lo, clip_hi;
  const int* flag;       // device: 1 = snapshot the current state
  float* bestV;
  float* bestA;
  float* bestB;
  float* gV;             // nullable debug outputs
  float* gA;
  float* gB;
  int apply;             // update V, alpha, beta in place
  uint16_t* Wq_next;     // nullable: bf16 Ŵ of the updated state, blocked GEMM layout
  int64_t wq_nkb;        // k-blocks of Wq_next
};
ar_status ar_launch_ste_update(const ArSteArgs& a, hipStream_t st);

ar_status ar_launch_fill_f32(float* p, float v, int64_t n, hipStream_t st);
ar_status ar_launch_pack(int bits, const uint8_t* codes, const uint8_t* zp, int64_t N, int64_t K,
                         int64_t G, int32_t* qweight, int32_t* qzeros, hipStream_t st);
ar_status ar_launch_unpack(int bits, const int32_t* qweight, const int32_t* qzeros, int64_t N,
                           int64_t K, int64_t G, uint8_t* codes, uint8_t* zp, hipStream_t st);
