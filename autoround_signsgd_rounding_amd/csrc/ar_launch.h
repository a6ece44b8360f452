// Internal host-side launchers (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/autoround_hip.h"

struct ArGrid {
  float maxq, half;
  int sym;
};

// Initial clip factors: alpha = beta = shrink (mse = 0), or per group the shrink
// p_j = float32(1 - j/grid), j0 <= j <= j1, with the smallest sum of squared
// round-to-nearest weight errors (float32 errors, float64 sum, first minimum).
struct ArInit {
  int mse;
  int j0, j1, grid;
  float shrink;
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
// Loss of a step from per-workgroup partial sums of squared residuals, reduced
// in float64 in a fixed order (ar_loss.h): total = sum(partials) + (*add when
// add), *sum_out = total, loss = total * inv_count written to loss_out /
// loss_slot, flag = (loss < *best_loss) with *best_loss lowered on
// improvement (flag = 0 without best_loss). Every pointer but partials is
// nullable; partials = NULL skips the reduction.
struct ArLossIn {
  const float* partials;
  int nparts;
  double inv_count;     // 1 / (Tb * N)
  const double* add;
  double* sum_out;
  float* loss_out;
  float* loss_slot;
  float* best_loss;
  int* flag;
};
// out[rowsP, rowsQ] (row-major float32) = scale * P·Qᵀ over nkb reduction
// blocks (P rows rowsP, Q rows rowsQ, both blocked with nkb blocks per row
// tile). `loss` (the previous forward's) is reduced in the same launch.
ar_status ar_launch_gemm_f32out(const uint16_t* P, const uint16_t* Q, float* out, int64_t rowsP,
                                int64_t rowsQ, int64_t nkb, float scale, const ArLossIn& loss,
                                hipStream_t st);
// P = D·H, row-major [N, K]: DB rows N and HB rows K, both with k_blocks(3K)
// reduction blocks (the Gram-form product).
ar_status ar_launch_gemm_gram(const uint16_t* DB, const uint16_t* HB, float* P, int64_t N,
                              int64_t K, const ArLossIn& loss, hipStream_t st);
// G = scale * dYᵀ·X_b, row-major [N, K] (the weight-gradient product).
ar_status ar_launch_gemm_wgrad(const uint16_t* dyB, const uint16_t* XTB, float* G, int64_t N,
                               int64_t K, int64_t Tb, float scale, const ArLossIn& loss,
                               hipStream_t st);
// Small products (ar_gemm_small.hip), taken by the launchers above when the
// product has at most four 256 x 256 tiles (ar_small_product): one one-wave
// workgroup per 64 x 64 output tile (32 x 32 for the smallest products), the
// same MFMA order per element as the 256 x 256 kernels. The forward writes one
// partial per tile (ar_small_fwd_tiles of them); the float32-output product
// reads P block s at step s < foldP and s - foldP after it, with nkP blocks per
// P panel.
bool ar_small_product(int64_t rowsP, int64_t rowsQ);
int ar_small_fwd_tiles(int64_t Tb, int64_t N);
ar_status ar_launch_small_fwd(const uint16_t* XB, const uint16_t* WB, const void* yB, int ydt,
                              uint16_t* dyB, float* partials, int64_t Tb, int64_t N, int64_t K,
                              hipStream_t st);
ar_status ar_launch_small_f32out(const uint16_t* P, const uint16_t* Q, float* out, int64_t N,
                                 int64_t K, int64_t nkb, float scale, const ArLossIn& loss,
                                 int64_t nkP, int64_t foldP, hipStream_t st);
// Y[M, N] = XB·WBᵀ (XB rows M, WB rows N, reduction K), row-major f32 or bf16.
ar_status ar_launch_gemm_out(const uint16_t* XB, const uint16_t* WB, void* Y, int ydt, int64_t M,
                             int64_t N, int64_t K, hipStream_t st);
// blocked staging: batch of row-major [R, KR] -> blocked (rows R, reduction KR)
ar_status ar_launch_block_copy(const uint16_t* src, uint16_t* dst, int64_t batch, int64_t R,
                               int64_t KR, int64_t nkb, hipStream_t st);
// batch of row-major [R, C] -> blocked (rows C, reduction R); elem_bytes 2 or 4
ar_status ar_launch_block_transpose(const void* src, void* dst, int64_t batch, int64_t R,
                                    int64_t C, int64_t nkb, int elem_bytes, hipStream_t st);
// X [batch][Tb, K] bf16 -> XTB (rows K, reduction Tb) and XB (rows Tb, reduction K),
// both blocked, from one read of X.
ar_status ar_launch_stage_x(const uint16_t* X, uint16_t* XTB, uint16_t* XB, int64_t batch,
                            int64_t Tb, int64_t K, int64_t nkbT, int64_t nkbK, hipStream_t st);

// Quantizer / update kernels (ar_quant.hip)
// out_dt: dtype of Wq (AR_BF16 or AR_F32); alpha/beta NULL means the initial clip
// factor of `init`, V NULL means zero.
// wq_nkb > 0 writes Wq (bf16 only) in the blocked GEMM layout (rows N, reduction K).
ar_status ar_launch_fakequant(int wdt, const void* W, const float* V, const float* alpha,
                              const float* beta, const ArInit& init, int64_t N, int64_t K, int g,
                              ArGrid gr, int out_dt, void* Wq, int64_t wq_nkb, uint8_t* codes,
                              float* scale, uint8_t* zp, hipStream_t st);
// alpha = beta = the initial clip factor of every group.
ar_status ar_launch_init_clip(int wdt, const void* W, int64_t N, int64_t K, int g, ArGrid gr,
                              const ArInit& init, float* alpha, float* beta, hipStream_t st);

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
  const int* flag;       // device, not null: 1 = snapshot the current state
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
// *flag = 1 when any of the n elements at p (dtype dt: AR_F32 or AR_BF16) is NaN
// or infinite; *flag is not touched otherwise (the caller clears it first).
ar_status ar_launch_nonfinite(const void* p, int64_t n, int dt, int* flag, hipStream_t st);

// W-bit x bf16 product on the packed format (ar_dequant.hip). g % 8 == 0.
// Dequantized bf16 Ŵ into the blocked operand (rows N, reduction K).
ar_status ar_launch_dequant_blocked(int bits, const int32_t* qweight, const int32_t* qzeros,
                                    const float* scale, int64_t N, int64_t K, int g, uint16_t* WB,
                                    hipStream_t st);
// Split-K slices of the small-M product; its workspace is slices*M*N floats.
int ar_dq_slices(int bits, int64_t N, int64_t K, int64_t M, int64_t g);
// Y[M, N] = X·bf16(Ŵ)ᵀ for M <= 16.
ar_status ar_launch_dq_gemv(int bits, const int32_t* qweight, const int32_t* qzeros,
                            const float* scale, int64_t N, int64_t K, int g, const uint16_t* X,
                            int M, float* part, void* Y, int ydt, hipStream_t st);

// Gram-form step (ar_gram.hip). D operands are blocked with rows N and reduction
// 3K ([D_hi | D_hi | D_lo]); H operands with rows K and reduction 3K
// ([H_hi | H_lo | H_hi]).
// Row-major src [R, C] (dtype src_dt, C % 8 == 0) into blocked dst (nkb blocks)
// at reduction offset k_off; lo = 0: bf16(x), lo = 1: bf16(x - bf16(x)).
ar_status ar_launch_place(const void* src, int src_dt, int64_t R, int64_t C, uint16_t* dst,
                          int64_t nkb, int64_t k_off, int lo, hipStream_t st);
// H [K, K] float32 row-major (K % 8 == 0) into [H_hi | H_lo | H_hi] at reduction
// offsets 0, Kp and 2·Kp of dst (nkb blocks): the three ar_launch_place calls
// in one pass.
ar_status ar_launch_place_h(const float* H, int64_t K, uint16_t* dst, int64_t nkb, int64_t Kp,
                            hipStream_t st);
// D operand of the state (V, A, B).
ar_status ar_launch_gram_d(int wdt, const void* W, const float* V, const float* A, const float* B,
                           int64_t N, int64_t K, int g, ArGrid gr, uint16_t* DB, hipStream_t st);
struct ArGramArgs {
  int wdt;
  const void* W;
  const float* Vc;       // state the product P was taken at
  float* Vn;             // next state; on entry the previous state
  const float* Ac;
  const float* Bc;
  float* An;
  float* Bn;
  const float* P;        // D·H [N, K]
  const float* Cn;       // target correction [N, K]
  int64_t N, K;
  int g;
  ArGrid gr;
  float lr, mlr, clip_lo, clip_hi;
  float scale;           // 2 / (Tb * N)
  int apply;
  const int* flag_prev;  // nullable: copy the previous state to best when set
  float* bestV;
  float* bestA;
  float* bestB;
  uint16_t* DB;          // next D operand
  float* partials;       // ar_gram_partials() floats: per-workgroup sums of D·(P + 2·Cn)
  float* gV;             // nullable gradient outputs
  float* gA;
  float* gB;
};
int64_t ar_gram_partials(int64_t N, int64_t K, int g);
ar_status ar_launch_ste_gram(const ArGramArgs& a, hipStream_t st);
// One-workgroup loss reduction (see ArLossIn).
ar_status ar_launch_loss_reduce(const ArLossIn& L, hipStream_t st);
// Copy (V, A, B) to (bestV, bestA, bestB) when *flag is set.
ar_status ar_launch_gram_snapshot(const int* flag, const float* V, const float* A, const float* B,
                                  float* bestV, float* bestA, float* bestB, int64_t nV, int64_t nG,
                                  hipStream_t st);
ar_status ar_launch_pack(int bits, const uint8_t* codes, const uint8_t* zp, int64_t N, int64_t K,
                         int64_t G, int32_t* qweight, int32_t* qzeros, hipStream_t st);
ar_status ar_launch_unpack(int bits, const int32_t* qweight, const int32_t* qzeros, int64_t N,
                           int64_t K, int64_t G, uint8_t* codes, uint8_t* zp, hipStream_t st);
