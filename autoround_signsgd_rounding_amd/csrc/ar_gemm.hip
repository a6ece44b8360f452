// bf16 MFMA contractions of the tuning step (gfx950).
//
// Both products are one "NT" GEMM, C[i, j] = sum_k P[i, k] * Q[j, k], over
// operands stored in the blocked layout of ar_blocked.h:
//   forward   Y'[t, n] = sum_k X_b[t, k] * Ŵ[n, k]       P = X_b  (rows t),  Q = Ŵ   (rows n)
//   gradient  G[n, k]  = sum_t dY[t, n] * X_b[t, k]      P = dYᵀ (rows n),  Q = X_bᵀ (rows k)
// (the loss and its weight gradient in the per-module loop of the llm-compressor
// AutoRound page: F.linear forward, mean-squared error, backward). The forward
// epilogue writes dYᵀ straight into the blocked layout the gradient product
// reads; X_b and Xᵀ_b are staged once per Linear.
//
// Tile 256 x 256 per workgroup of 4 waves (2 x 2), each wave 128 x 128 as 4 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (float32 accumulators). The reduction
// advances 32 elements per step through 4 LDS stages (4 x 32 KiB) filled by
// direct global->LDS buffer loads (1 KiB per wave instruction, contiguous in
// the blocked layout). One barrier per step, placed between the two 16-element
// substeps: after it the stage just consumed is refilled four steps ahead and
// the first fragments of the next step are read while the second substep's
// MFMAs run. Fragments are double-buffered in registers and every MFMA is
// followed by at most one LDS read or one global load (explicit order).
//
// Two kernels share that step. k_gemm runs one tile per workgroup with a
// pluggable epilogue (forward with float32 targets or short reductions, the
// weight gradient, the Gram-form product, the plain product).
// k_fwd_stream is the forward with bf16 targets: one workgroup per CU runs its
// tiles in turn and moves the targets and residuals under the MFMAs. Both
// produce the same bits. Products of at most four tiles go to the one-wave
// kernel of ar_gemm_small.hip instead.
#include "ar_blocked.h"
#include "ar_device.h"
#include "ar_launch.h"
#include "ar_loss.h"

#include <mutex>

namespace {

constexpr int BM = 256, BN = 256, BK = arblk::KB, NTHR = 256, NSTAGE = 4;
constexpr int ROWB = BK * 2;                        // 64 B per LDS row
constexpr int OPB = BM * ROWB;                      // 16 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * OPB;                // 32 KiB
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;     // 128 KiB
constexpr int IPW = OPB / 1024 / 4;                 // 1 KiB loads per operand per wave (4)
constexpr int LPI = 2 * IPW;                        // loads per wave per step (8)
// LDS past the stages: per-wave sums of the forward epilogue (16 B), the loss
// reduction's 256 doubles (at +64)
constexpr int EXTRA_BYTES = 64 + 256 * 8;

__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt vmcnt(n) leaving the other counters unconstrained
  switch (n) {
#define AR_W(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8)); break;
    AR_W(0) AR_W(8) AR_W(16) AR_W(24)
#undef AR_W
    default: __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  }
}

// Workgroup -> tile. The dispatcher places workgroup w on XCD (w mod 8); give
// each XCD one contiguous range of the tile sequence, walked in groups of GI
// tile rows, so the ~32 tiles resident on one XCD share a few panels in its L2.
__device__ __forceinline__ void tile_of(int w, int nwg, int tilesI, int tilesJ, int& ti, int& tj) {
  const int xcd = w & 7, local = w >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  const int L = xcd * q + min(xcd, r) + local;
  constexpr int GI = 4;
  const int per_group = GI * tilesJ;
  const int grp = L / per_group;
  const int first = grp * GI;
  const int gsize = min(tilesI - first, GI);
  const int inner = L - grp * per_group;
  ti = first + inner % gsize;
  tj = inner / gsize;
}

struct GemmArgs {
  const uint16_t* P;   // blocked, tilesI panels of nkb blocks (nkP with a folded P)
  const uint16_t* Q;   // blocked, tilesJ panels of nkb blocks
  int nkb;
  int tilesI, tilesJ;
  // Folded P (epilogues with kFoldP): P panels hold nkP blocks and reduction
  // step kt reads P block kt for kt < foldP, else kt - foldP.
  int nkP = 0, foldP = 0;
};

template <class Epi>
__global__ __launch_bounds__(NTHR, 1) void k_gemm(GemmArgs a, Epi epi) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES + EXTRA_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  int ti, tj;
  tile_of(blockIdx.x, gridDim.x, a.tilesI, a.tilesJ, ti, tj);
  const int nk = a.nkb;
  const int nkP = Epi::kFoldP ? a.nkP : nk;
  const __amdgpu_buffer_rsrc_t bufP =
      make_rsrc(a.P + (int64_t)ti * nkP * arblk::BLOCK_ELEMS, (uint32_t)nkP * OPB);
  const __amdgpu_buffer_rsrc_t bufQ =
      make_rsrc(a.Q + (int64_t)tj * nk * arblk::BLOCK_ELEMS, (uint32_t)nk * OPB);

  // Load j (0..LPI-1) of step kt: operand j&1, 1 KiB piece wave*IPW + j/2 of its block.
  const uint32_t lane_off = (uint32_t)(wave * IPW * 1024 + lane * 16);
  auto lds_dst = [&](int kt, int j) -> uint8_t* {
    return lds + (kt % NSTAGE) * STAGE_BYTES + ((j & 1) ? OPB : 0) + (wave * IPW + (j >> 1)) * 1024;
  };
#define AR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
  auto issue_main = [&](int kt, int j) {   // kt < nk
    const uint32_t vo = lane_off + (uint32_t)(j >> 1) * 1024u;
    const uint32_t so = (uint32_t)kt * OPB;
    if (j & 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bufQ, AR_LDS(lds_dst(kt, j)), 16, vo, so, 0, 0);
    } else {
      const uint32_t sp = Epi::kFoldP && kt >= a.foldP ? (uint32_t)(kt - a.foldP) * OPB : so;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bufP, AR_LDS(lds_dst(kt, j)), 16, vo, sp, 0, 0);
    }
  };
  // kt >= nk: the freed stage takes piece kt-nk of the epilogue's prefetch (piece j lands
  // in stage (nk + j) % NSTAGE); without a prefetch, an out-of-range load keeps the
  // per-step load count uniform (zeros land in a stage nobody reads).
  const __amdgpu_buffer_rsrc_t bufE =
      make_rsrc(epi.prefetch_base(ti, tj), Epi::kPrefetch * (uint32_t)STAGE_BYTES);
  auto issue_tail = [&](int kt, int j) {
    const bool pf = Epi::kPrefetch > 0 && kt - nk < Epi::kPrefetch;
    const uint32_t vo = pf ? lane_off + (uint32_t)(j >> 1) * 1024u + ((j & 1) ? (uint32_t)OPB : 0u)
                           : kOOB;
    const uint32_t so = pf ? (uint32_t)(kt - nk) * STAGE_BYTES : 0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(bufE, AR_LDS(lds_dst(kt, j)), 16, vo, so, 0, 0);
  };

  // fragment reads: lane reads row (lane & 31) of a 32-row block, logical chunk 2*ks + (lane >> 5)
  const uint32_t rdP = (uint32_t)(wi * 128 + (lane & 31)) * ROWB;
  const uint32_t rdQ = OPB + (uint32_t)(wj * 128 + (lane & 31)) * ROWB;
  const int sw = ((lane & 31) >> 2) & 3, rhi = lane >> 5;
  bf16x8_t pf[2][4], qf[2][4];
  auto rd = [&](int kt, int ks, int buf, int idx) {
    const uint8_t* s = lds + (kt % NSTAGE) * STAGE_BYTES;
    const uint32_t ch = (uint32_t)(((2 * ks + rhi) ^ sw) << 4);
    const int b = idx & 3;
    if (idx < 4) pf[buf][b] = *reinterpret_cast<const bf16x8_t*>(s + rdP + b * 32 * ROWB + ch);
    else qf[buf][b] = *reinterpret_cast<const bf16x8_t*>(s + rdQ + b * 32 * ROWB + ch);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

#pragma unroll
  for (int p = 0; p < NSTAGE; ++p)
#pragma unroll
    for (int j = 0; j < LPI; ++j) {
      if (p < nk) issue_main(p, j);
      else issue_tail(p, j);
    }
  epi.pre(lds + LDS_BYTES);   // runs while the first stages load
  wait_vm((NSTAGE - 1) * LPI);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int idx = 0; idx < 8; ++idx) rd(0, 0, 0, idx);
  __builtin_amdgcn_sched_barrier(0);

  // one step: substep 0 (buffer 0) reads substep 1 into buffer 1; barrier; substep 1
  // (buffer 1) reads step kt+1 substep 0 into buffer 0 and refills stage kt with step kt+4
  auto step = [&](int kt, bool tail) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      acc[m >> 2][m & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[0][m >> 2], qf[0][m & 3], acc[m >> 2][m & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (m & 1) {
        rd(kt, 1, 1, m >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // step kt+1 loaded (at most steps kt+2, kt+3 outstanding) and everyone done with stage kt
    wait_vm((NSTAGE - 2) * LPI);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      acc[m >> 2][m & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[1][m >> 2], qf[1][m & 3], acc[m >> 2][m & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (m & 1) rd(kt + 1, 0, 0, m >> 1);
      else if (tail) issue_tail(kt + NSTAGE, m >> 1);
      else issue_main(kt + NSTAGE, m >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int kt = 0;
  for (; kt < nk - NSTAGE; ++kt) step(kt, false);
  for (; kt < nk; ++kt) step(kt, true);
  wait_vm(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  epi(acc, ti, tj, wi, wj, lane, lds, nk);
#undef AR_LDS
}

// Accumulator element (bi, bj, r) of a lane sits at tile-local
//   i = wi*128 + bi*32 + 8*(r >> 2) + 4*(lane >> 5) + (r & 3)
//   j = wj*128 + bj*32 + (lane & 31)
// (v_mfma_f32_32x32x* output layout).

// Forward epilogue: i = token t, j = output feature n. R = Y' - Y_true,
// dYᵀ = bf16(R) into the blocked layout (rows n, reduction t), per-tile sum of R²
// in a fixed order. Padding rows/columns give R = 0.
//
// bf16 targets: the tile's 8 target blocks (rows n, 256 t = 128 KiB, contiguous in
// the blocked array) are prefetched into the four freed LDS stages during the last
// main-loop steps; each lane turns its accumulators into R in place (8 bytes per
// 4 tokens), then the workgroup streams the 128 KiB dYᵀ tile out with 16-byte
// coalesced stores.
struct EpiFwdBf16 {
  static constexpr int kPrefetch = NSTAGE;     // 4 x 32 KiB = the whole target tile
  static constexpr bool kFoldP = false;
  const uint16_t* yB;   // targets, blocked like dYᵀ (rows n, reduction t)
  uint16_t* dyB;
  float* partials;
  int nkbT;
  int tilesJ;

  __device__ __forceinline__ const uint16_t* tile_base(const uint16_t* base, int ti, int tj) const {
    return base + ((int64_t)tj * nkbT + (int64_t)ti * (BM / BK)) * arblk::BLOCK_ELEMS;
  }
  __device__ __forceinline__ const void* prefetch_base(int ti, int tj) const {
    return tile_base(yB, ti, tj);
  }
  __device__ __forceinline__ void pre(uint8_t*) const {}
  // LDS byte address of target/residual block q (0..7) of the tile
  __device__ __forceinline__ uint32_t blk_lds(int q, int nk) const {
    return (uint32_t)(((nk + (q >> 1)) % NSTAGE) * STAGE_BYTES + (q & 1) * OPB);
  }

  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int ti, int tj, int wi, int wj,
                                             int lane, uint8_t* lds, int nk) const {
    float* red = reinterpret_cast<float*>(lds + LDS_BYTES);
    float sq = 0.0f;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int nl = wj * 128 + bj * 32 + (lane & 31);
      const int nsw = (nl >> 2) & 3;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int tl = wi * 128 + bi * 32 + q * 8 + (lane >> 5) * 4;   // tile-local token
          const int c = (tl & 31) >> 3;
          const uint32_t a = blk_lds(tl >> 5, nk) + (uint32_t)nl * ROWB +
                             ((uint32_t)(c ^ nsw) << 4) + (uint32_t)(tl & 7) * 2u;
          u32x2_t* p = reinterpret_cast<u32x2_t*>(lds + a);
          const u32x2_t v = *p;
          float y[4] = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                        __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = acc[bi][bj][q * 4 + e] - y[e];
            sq += r[e] * r[e];
          }
          u32x2_t o;
          o[0] = bf16_bits(r[0]) | (bf16_bits(r[1]) << 16);
          o[1] = bf16_bits(r[2]) | (bf16_bits(r[3]) << 16);
          *p = o;
        }
      }
    }
    sq = wave_sum64(sq);
    const int wave = wi * 2 + wj;
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    // stream the residual tile: 8 blocks x 16 KiB, contiguous in dyB
    uint16_t* dst = const_cast<uint16_t*>(tile_base(dyB, ti, tj));
    const int tid = wave * 64 + lane;
#pragma unroll 4
    for (int u = 0; u < (8 * arblk::BLOCK_BYTES) / (16 * NTHR); ++u) {
      const int chunk = u * NTHR + tid;                 // 16-byte chunk of the tile
      const int q = chunk >> 10;                        // 1024 chunks per block
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(lds + blk_lds(q, nk) + (uint32_t)(chunk & 1023) * 16u);
      *reinterpret_cast<u32x4_t*>(dst + (int64_t)chunk * 8) = v;
    }
    if (wave == 0 && lane == 0) partials[ti * tilesJ + tj] = ((red[0] + red[1]) + red[2]) + red[3];
  }
};

// ---------------------------------------------------------------------------
// Streamed forward product (bf16 targets, reduction of at least FS_MIN_NK steps).
//
// Same tiles, operands, accumulators and per-tile arithmetic as k_gemm with
// EpiFwdBf16, but each workgroup runs a fixed sequence of tiles:
// u = blockIdx.x + r * gridDim.x for r = 0, 1, ..., mapped by tile_of exactly as
// the one-tile-per-workgroup launch maps workgroup u, so XCD placement and
// panel sharing are unchanged. What changes is when the epilogue traffic moves.
// Per lane, the 256 targets/residuals of its 128 x 128 sub-tile sit in 64
// slots of four bf16 tokens (the accumulator order, 8 bytes of one blocked row
// each): the slots of accumulator blocks 0..12 in registers, those of blocks
// 13..15 in a per-wave LDS area past the stages (two dwords per slot at
// base + 4*lane, the layout of a 4-byte global->LDS load), which keeps the
// kernel within 256 VGPRs. The main loop of tile r is cut into 16 groups; at the
// start of group g the four slots of block g are first stored as tile r-1's dYᵀ
// and then reloaded with tile r's targets (LDS slots: read back, stored, then
// refilled by global->LDS loads). The target reads and residual writes therefore
// run under the MFMAs instead of as a chip-wide burst after every tile, and the
// last four steps of tile r fill the stages with tile r+1's first four steps.
// Only the last tile's residuals leave in a burst.
//
// vmcnt accounting: a step waits for at most 16 outstanding vector-memory
// operations. The newest 16 always come after the loads of step kt+1 (steps kt+2
// and kt+3 alone are 16 loads; the slot stores and loads only add to that), and
// the counter retires in issue order, so step kt+1's stage is complete.
constexpr int FS_GROUPS = 16;
constexpr int FS_MIN_NK = FS_GROUPS + NSTAGE;   // at least one main-loop step per group
constexpr int FS_REG_G = 13;                     // blocks whose slots live in registers
constexpr int FS_WAVE_LDS = (FS_GROUPS - FS_REG_G) * 4 * 2 * 256;   // 6 KiB per wave
constexpr int FS_RED = LDS_BYTES + 4 * FS_WAVE_LDS;                // per-wave sums
constexpr int FS_LDS_TOTAL = FS_RED + 64;
static_assert(FS_LDS_TOTAL <= 160 * 1024, "LDS of one workgroup");

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// wave_sum64's butterfly (partners lane^32, ^16, ..., ^1, each lane adding its
// partner to its own value) without lane-address registers: v_permlane32_swap for
// the two halves, ds_swizzle xor patterns inside them. Of the swap's two results one
// is the lane's own value and the other its partner, so x ^ r0 ^ r1 is the partner.
__device__ __forceinline__ float wave_sum64_swz(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  x += __uint_as_float(xb ^ (uint32_t)r[0] ^ (uint32_t)r[1]);
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (16 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (8 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (4 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (2 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (1 << 10)));
  return x;
}

struct FwdStreamArgs {
  const uint16_t* P;    // X_b, blocked (rows t)
  const uint16_t* Q;    // Ŵ, blocked (rows n)
  const uint16_t* yB;   // targets, blocked like dYᵀ (rows n, reduction t)
  uint16_t* dyB;
  float* partials;      // one per tile, ti * tilesJ + tj
  int nkb, tilesI, tilesJ, nkbT, ntiles;
};

__global__ __launch_bounds__(NTHR, 1) void k_fwd_stream(FwdStreamArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[FS_LDS_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const int nk = a.nkb;
  constexpr uint32_t TILE_BYTES = 8u * arblk::BLOCK_BYTES;   // one tile of targets / dYᵀ
  auto tile_at = [&](int r, int& ti, int& tj) -> bool {
    const int u = (int)blockIdx.x + r * (int)gridDim.x;
    if (u >= a.ntiles) return false;
    tile_of(u, a.ntiles, a.tilesI, a.tilesJ, ti, tj);
    return true;
  };
  auto rsrcP = [&](int ti) {
    return make_rsrc(a.P + (int64_t)ti * nk * arblk::BLOCK_ELEMS, (uint32_t)nk * OPB);
  };
  auto rsrcQ = [&](int tj) {
    return make_rsrc(a.Q + (int64_t)tj * nk * arblk::BLOCK_ELEMS, (uint32_t)nk * OPB);
  };
  auto tile_off = [&](int ti, int tj) -> int64_t {
    return ((int64_t)tj * a.nkbT + (int64_t)ti * (BM / BK)) * arblk::BLOCK_ELEMS;
  };

#define AR_LDS(p) ((__attribute__((address_space(3))) void*)(p))
  // stage loads: piece j (0..LPI-1) of step `s` of a tile, into LDS stage `stg`
  const uint32_t lane_off = (uint32_t)(wave * IPW * 1024 + lane * 16);
  auto issue = [&](__amdgpu_buffer_rsrc_t bp, __amdgpu_buffer_rsrc_t bq, int stg, int s, int j) {
    uint8_t* dst = lds + stg * STAGE_BYTES + ((j & 1) ? OPB : 0) + (wave * IPW + (j >> 1)) * 1024;
    const uint32_t vo = lane_off + (uint32_t)(j >> 1) * 1024u;
    const uint32_t so = (uint32_t)s * OPB;
    if (j & 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(bq, AR_LDS(dst), 16, vo, so, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(bp, AR_LDS(dst), 16, vo, so, 0, 0);
  };

  const uint32_t rdP = (uint32_t)(wi * 128 + (lane & 31)) * ROWB;
  const uint32_t rdQ = OPB + (uint32_t)(wj * 128 + (lane & 31)) * ROWB;
  const int sw = ((lane & 31) >> 2) & 3, rhi = lane >> 5;
  bf16x8_t pf[2][4], qf[2][4];
  auto rd = [&](int stg, int ks, int buf, int idx) {
    const uint8_t* s = lds + stg * STAGE_BYTES;
    const uint32_t ch = (uint32_t)(((2 * ks + rhi) ^ sw) << 4);
    const int b = idx & 3;
    if (idx < 4) pf[buf][b] = *reinterpret_cast<const bf16x8_t*>(s + rdP + b * 32 * ROWB + ch);
    else qf[buf][b] = *reinterpret_cast<const bf16x8_t*>(s + rdQ + b * 32 * ROWB + ch);
  };

  // register slots: slot 4*g + q holds tokens 8q + 4*(lane>>5) .. +3 of accumulator
  // block g = 4*bj + bi; its byte offset in the tile's blocked region is the lane part
  // qv[q] (a VGPR per q) plus the block part blk_so(g) (the instruction's scalar offset)
  const uint32_t lane_base =
      (uint32_t)(wi * 4 * arblk::BLOCK_BYTES + (wj * 128 + (lane & 31)) * ROWB + (lane >> 5) * 8);
  uint32_t qv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) qv[q] = lane_base + ((uint32_t)(q ^ sw) << 4);
  auto blk_so = [](int g) -> uint32_t {
    return (uint32_t)((g & 3) * arblk::BLOCK_BYTES + (g >> 2) * 32 * ROWB);
  };
  u32x2_t slot[4 * FS_REG_G];
#pragma unroll
  for (int i = 0; i < 4 * FS_REG_G; ++i) slot[i] = u32x2_t{0u, 0u};
  // LDS slot (block g >= FS_REG_G, q): low dwords of the wave's 64 lanes, then the high ones
  auto lslot = [&](int g, int q) -> uint8_t* {
    return lds + LDS_BYTES + wave * FS_WAVE_LDS + ((g - FS_REG_G) * 4 + q) * 512;
  };
  auto lds_get = [&](int g, int q) -> u32x2_t {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(lslot(g, q)) + lane;
    return u32x2_t{p[0], p[64]};
  };
  auto lds_put = [&](int g, int q, u32x2_t v) {
    uint32_t* p = reinterpret_cast<uint32_t*>(lslot(g, q)) + lane;
    p[0] = v[0];
    p[64] = v[1];
  };

  f32x16_t acc[4][4];
  float* red = reinterpret_cast<float*>(lds + FS_RED);

  int ti, tj;
  tile_at(0, ti, tj);   // gridDim.x <= ntiles
  __amdgpu_buffer_rsrc_t bP = rsrcP(ti), bQ = rsrcQ(tj);
  // residuals pending from the previous tile (none before the first: every store drops)
  __amdgpu_buffer_rsrc_t bOut = make_rsrc(a.dyB, 0u);
  int stg0 = 0;   // stage of the current tile's step 0

#pragma unroll
  for (int s = 0; s < NSTAGE; ++s)
#pragma unroll
    for (int j = 0; j < LPI; ++j) issue(bP, bQ, s, s, j);
  wait_vm((NSTAGE - 1) * LPI);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int idx = 0; idx < 8; ++idx) rd(0, 0, 0, idx);
  __builtin_amdgcn_sched_barrier(0);

  for (int r = 0;; ++r) {
    int nti = ti, ntj = tj;
    const bool more = tile_at(r + 1, nti, ntj);
    // without a next tile the tail refills read an empty range (zeros into stages nobody reads)
    const __amdgpu_buffer_rsrc_t nP = more ? rsrcP(nti) : make_rsrc(a.P, 0u);
    const __amdgpu_buffer_rsrc_t nQ = more ? rsrcQ(ntj) : make_rsrc(a.Q, 0u);
    const __amdgpu_buffer_rsrc_t bY = make_rsrc(a.yB + tile_off(ti, tj), TILE_BYTES);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.0f;

    // one step: as in k_gemm; the refill of stage kt takes step kt+4 of this tile
    // (tail = false) or step kt+4-nk of the next tile (tail = true). The tile's last
    // step (last = true) leaves the next tile's first fragments for after the epilogue,
    // so that they are not held in registers through it.
    auto step = [&](int kt, bool tail, bool last = false) {
      const int sc = (stg0 + kt) & (NSTAGE - 1), sn = (sc + 1) & (NSTAGE - 1);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        acc[m >> 2][m & 3] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[0][m >> 2], qf[0][m & 3], acc[m >> 2][m & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (m & 1) {
          rd(sc, 1, 1, m >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_vm((NSTAGE - 2) * LPI);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        acc[m >> 2][m & 3] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[1][m >> 2], qf[1][m & 3], acc[m >> 2][m & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (m & 1) {
          if (!last) rd(sn, 0, 0, m >> 1);
        } else if (tail) issue(nP, nQ, sc, kt + NSTAGE - nk, m >> 1);
        else issue(bP, bQ, sc, kt + NSTAGE, m >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    const int S = (nk - NSTAGE) / FS_GROUPS;   // >= 1 (nk >= FS_MIN_NK)
    __builtin_assume(S >= 1);
    int kt = 0;
#pragma unroll
    for (int g = 0; g < FS_GROUPS; ++g) {
      // the previous tile's residuals of block g out, this tile's targets of block g in
      if (g < FS_REG_G) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b64(slot[4 * g + q], bOut, qv[q], blk_so(g), 0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          slot[4 * g + q] = __builtin_amdgcn_raw_buffer_load_b64(bY, qv[q], blk_so(g), 0);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b64(lds_get(g, q), bOut, qv[q], blk_so(g), 0);
        __builtin_amdgcn_sched_barrier(0);
        // (the reads above have returned: the stores consumed their data)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bY, AR_LDS(lslot(g, q)), 4, qv[q], blk_so(g), 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bY, AR_LDS(lslot(g, q) + 256), 4, qv[q],
                                                   blk_so(g) + 4u, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      int j = 0;
      do {
        step(kt, false);
        ++kt;
      } while (++j < S);
    }
    for (; kt < nk - NSTAGE; ++kt) step(kt, false);
#pragma unroll
    for (int t = 0; t < NSTAGE; ++t) step(nk - NSTAGE + t, true, t == NSTAGE - 1);

    // R = Y' - Y_true in place of the targets, tile's sum of R² in the order of EpiFwdBf16.
    // The LDS slots' target loads are complete: they were issued before the tail steps'
    // 32 loads, and the last step waited until at most 16 operations were outstanding.
    __builtin_amdgcn_sched_barrier(0);
    float sq = 0.0f;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = 4 * bj + bi;
          u32x2_t v = g < FS_REG_G ? slot[4 * g + q] : lds_get(g, q);
          const float y[4] = {__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                              __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
          float rr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rr[e] = acc[bi][bj][q * 4 + e] - y[e];
            sq += rr[e] * rr[e];
          }
          // v_cvt_pk_bf16_f32: nearest-even, the same bits as bf16_bits for every
          // non-NaN value (NaN stays NaN, payload aside); no per-element compare
          const bf16x2_t h0 = {(__bf16)rr[0], (__bf16)rr[1]};
          const bf16x2_t h1 = {(__bf16)rr[2], (__bf16)rr[3]};
          v[0] = __builtin_bit_cast(uint32_t, h0);
          v[1] = __builtin_bit_cast(uint32_t, h1);
          if (g < FS_REG_G) slot[4 * g + q] = v;
          else lds_put(g, q, v);
          __builtin_amdgcn_sched_barrier(0);   // one slot's temporaries live at a time
        }
    sq = wave_sum64_swz(sq);
    if (lane == 0) red[wave] = sq;
    // The sums pass through LDS only: wait for this wave's LDS write, then the barrier,
    // with compiler-only memory clobbers around it. A fence would also wait for the
    // next tile's global->LDS stage loads (vmcnt), which must stay in flight here.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (wave == 0 && lane == 0) a.partials[ti * a.tilesJ + tj] = ((red[0] + red[1]) + red[2]) + red[3];
    bOut = make_rsrc(a.dyB + tile_off(ti, tj), TILE_BYTES);
    if (!more) break;
    ti = nti; tj = ntj; bP = nP; bQ = nQ;
    stg0 = (stg0 + nk) & (NSTAGE - 1);
    // next tile's step 0 (stage complete and visible: the last step's wait and barrier)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) rd(stg0, 0, 0, idx);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last tile's residuals
#pragma unroll
  for (int g = 0; g < FS_GROUPS; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_buffer_store_b64(g < FS_REG_G ? slot[4 * g + q] : lds_get(g, q), bOut,
                                            qv[q], blk_so(g), 0);
#undef AR_LDS
}

// Workgroups the streamed forward product keeps resident: one per compute unit
// (its LDS allows no more), a multiple of 8 so that workgroup w's tiles stay on
// XCD w mod 8. Remembered per device.
int fwd_stream_grid(int ntiles) {
  static std::mutex mu;
  static int cus_of[64] = {0};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    cus = 256;
  } else {
    std::lock_guard<std::mutex> lk(mu);
    if (cus_of[dev] == 0) {
      int c = 0;
      if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
        (void)hipGetLastError();
        c = 256;
      }
      cus_of[dev] = c;
    }
    cus = cus_of[dev];
  }
  int g = cus >= 8 ? cus / 8 * 8 : cus;
  return ntiles < g ? ntiles : g;
}

// float32 targets (float32 layers): read straight from the blocked array.
struct EpiFwdF32 {
  static constexpr int kPrefetch = 0;
  static constexpr bool kFoldP = false;
  const float* yB;
  uint16_t* dyB;
  float* partials;
  int nkbT;
  int tilesJ;

  __device__ __forceinline__ const void* prefetch_base(int, int) const { return yB; }
  __device__ __forceinline__ void pre(uint8_t*) const {}
  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int ti, int tj, int wi, int wj,
                                             int lane, uint8_t* lds, int) const {
    float* red = reinterpret_cast<float*>(lds + LDS_BYTES);
    float sq = 0.0f;
    const int64_t t0 = (int64_t)ti * BM, n0 = (int64_t)tj * BN;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int64_t n = n0 + wj * 128 + bj * 32 + (lane & 31);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t t = t0 + wi * 128 + bi * 32 + q * 8 + (lane >> 5) * 4;
          const int64_t off = arblk::offset(n, t, nkbT);
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(yB + off);
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = acc[bi][bj][q * 4 + e] - v[e];
            sq += r[e] * r[e];
          }
          u32x2_t o;
          o[0] = bf16_bits(r[0]) | (bf16_bits(r[1]) << 16);
          o[1] = bf16_bits(r[2]) | (bf16_bits(r[3]) << 16);
          *reinterpret_cast<u32x2_t*>(dyB + off) = o;
        }
      }
    }
    sq = wave_sum64(sq);
    const int wave = wi * 2 + wj;
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (wave == 0 && lane == 0) partials[ti * tilesJ + tj] = ((red[0] + red[1]) + red[2]) + red[3];
  }
};

// Loss of the previous launch's partial sums (see ArLossIn), reduced by
// workgroup 0 while its first stages load.
__device__ __forceinline__ void loss_pre(const ArLossIn& L, uint8_t* extra) {
  if (blockIdx.x != 0 || L.partials == nullptr) return;
  loss_reduce_block(L, reinterpret_cast<double*>(extra + 64));
}

// float32 epilogue (weight gradient, Gram products): i = row of P, j = row of Q;
// out[i, j] = scale * acc, rows i < N, columns j < K of a row-major [N, K].
struct EpiWgrad {
  static constexpr int kPrefetch = 0;
  static constexpr bool kFoldP = false;
  float* G;   // [N, K] row-major
  int64_t N, K;
  float scale;
  ArLossIn loss;

  __device__ __forceinline__ const void* prefetch_base(int, int) const { return G; }
  __device__ __forceinline__ void pre(uint8_t* extra) const { loss_pre(loss, extra); }
  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int ti, int tj, int wi, int wj,
                                             int lane, uint8_t*, int) const {
    const int64_t n0 = (int64_t)ti * BM, k0 = (int64_t)tj * BN;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int64_t k = k0 + wj * 128 + bj * 32 + (lane & 31);
      if (k < K) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t n = n0 + wi * 128 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (n < N) G[n * K + k] = acc[bi][bj][r] * scale;
          }
        }
      }
    }
  }
};

}  // namespace

int ar_fwd_tiles(int64_t Tb, int64_t N) {
  if (ar_small_product(Tb, N)) return ar_small_fwd_tiles(Tb, N);
  return (int)(arblk::row_tiles(Tb) * arblk::row_tiles(N));
}

ar_status ar_launch_gemm_fwd(const uint16_t* XB, const uint16_t* WB, const void* yB, int ydt,
                             uint16_t* dyB, float* partials, int64_t Tb, int64_t N, int64_t K,
                             hipStream_t st) {
  GemmArgs a;
  a.P = XB; a.Q = WB;
  a.nkb = (int)arblk::k_blocks(K);
  a.tilesI = (int)arblk::row_tiles(Tb);
  a.tilesJ = (int)arblk::row_tiles(N);
  const int nkbT = (int)(arblk::row_tiles(Tb) * (BM / BK));
  const int nwg = a.tilesI * a.tilesJ;
  if (ar_small_product(Tb, N)) {
    return ar_launch_small_fwd(XB, WB, yB, ydt, dyB, partials, Tb, N, K, st);
  } else if (ydt == AR_BF16 && a.nkb >= FS_MIN_NK) {
    FwdStreamArgs s{XB, WB, static_cast<const uint16_t*>(yB), dyB, partials,
                    a.nkb, a.tilesI, a.tilesJ, nkbT, nwg};
    hipLaunchKernelGGL(k_fwd_stream, dim3(fwd_stream_grid(nwg)), dim3(NTHR), 0, st, s);
  } else if (ydt == AR_BF16) {
    EpiFwdBf16 e{static_cast<const uint16_t*>(yB), dyB, partials, nkbT, a.tilesJ};
    hipLaunchKernelGGL(k_gemm<EpiFwdBf16>, dim3(nwg), dim3(NTHR), 0, st, a, e);
  } else {
    EpiFwdF32 e{static_cast<const float*>(yB), dyB, partials, nkbT, a.tilesJ};
    hipLaunchKernelGGL(k_gemm<EpiFwdF32>, dim3(nwg), dim3(NTHR), 0, st, a, e);
  }
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

// Plain product epilogue (the dequantized-weight GEMM): Y[i, j] = acc for
// i < M (rows of P), j < N (rows of Q), row-major, float32 or bf16.
struct EpiOut {
  static constexpr int kPrefetch = 0;
  static constexpr bool kFoldP = false;
  void* Y;
  int64_t M, N;
  int ydt;

  __device__ __forceinline__ const void* prefetch_base(int, int) const { return Y; }
  __device__ __forceinline__ void pre(uint8_t*) const {}
  __device__ __forceinline__ void operator()(f32x16_t (&acc)[4][4], int ti, int tj, int wi, int wj,
                                             int lane, uint8_t*, int) const {
    const int64_t m0 = (int64_t)ti * BM, n0 = (int64_t)tj * BN;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int64_t n = n0 + wj * 128 + bj * 32 + (lane & 31);
      if (n < N) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wi * 128 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m < M) {
              if (ydt == AR_BF16)
                static_cast<uint16_t*>(Y)[m * N + n] = (uint16_t)bf16_bits(acc[bi][bj][r]);
              else
                static_cast<float*>(Y)[m * N + n] = acc[bi][bj][r];
            }
          }
        }
      }
    }
  }
};

ar_status ar_launch_gemm_out(const uint16_t* XB, const uint16_t* WB, void* Y, int ydt, int64_t M,
                             int64_t N, int64_t K, hipStream_t st) {
  GemmArgs a;
  a.P = XB; a.Q = WB;
  a.nkb = (int)arblk::k_blocks(K);
  a.tilesI = (int)arblk::row_tiles(M);
  a.tilesJ = (int)arblk::row_tiles(N);
  EpiOut e{Y, M, N, ydt};
  hipLaunchKernelGGL(k_gemm<EpiOut>, dim3(a.tilesI * a.tilesJ), dim3(NTHR), 0, st, a, e);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

// The Gram-form product D·H: the weight-gradient epilogue, with D folded (D is
// stored [D_hi | D_lo] against H's [H_hi | H_lo | H_hi]). Its own type also
// names it apart in profiles.
struct EpiGramP : EpiWgrad {
  static constexpr bool kFoldP = true;
};

template <class Epi>
static ar_status launch_f32out(const uint16_t* P, const uint16_t* Q, float* out, int64_t rowsP,
                               int64_t rowsQ, int64_t nkb, float scale, const ArLossIn& loss,
                               hipStream_t st, int64_t nkP = 0, int64_t foldP = 0) {
  GemmArgs a;
  a.P = P; a.Q = Q;
  a.nkb = (int)nkb;
  a.nkP = (int)nkP; a.foldP = (int)foldP;
  a.tilesI = (int)arblk::row_tiles(rowsP);
  a.tilesJ = (int)arblk::row_tiles(rowsQ);
  Epi e;
  e.G = out; e.N = rowsP; e.K = rowsQ; e.scale = scale; e.loss = loss;
  hipLaunchKernelGGL(k_gemm<Epi>, dim3(a.tilesI * a.tilesJ), dim3(NTHR), 0, st, a, e);
  return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}

ar_status ar_launch_gemm_f32out(const uint16_t* P, const uint16_t* Q, float* out, int64_t rowsP,
                                int64_t rowsQ, int64_t nkb, float scale, const ArLossIn& loss,
                                hipStream_t st) {
  if (ar_small_product(rowsP, rowsQ))
    return ar_launch_small_f32out(P, Q, out, rowsP, rowsQ, nkb, scale, loss, nkb, nkb, st);
  return launch_f32out<EpiWgrad>(P, Q, out, rowsP, rowsQ, nkb, scale, loss, st);
}

ar_status ar_launch_gemm_gram(const uint16_t* DB, const uint16_t* HB, float* P, int64_t N,
                              int64_t K, const ArLossIn& loss, hipStream_t st) {
  // reduction over [H_hi | H_lo | H_hi] (3 parts of k_blocks(K) blocks); D = [D_hi | D_lo]
  const int64_t kb = arblk::k_blocks(K);
  if (ar_small_product(N, K))
    return ar_launch_small_f32out(DB, HB, P, N, K, 3 * kb, 1.0f, loss, 2 * kb, kb, st);
  return launch_f32out<EpiGramP>(DB, HB, P, N, K, 3 * kb, 1.0f, loss, st, 2 * kb, kb);
}

ar_status ar_launch_gemm_wgrad(const uint16_t* dyB, const uint16_t* XTB, float* G, int64_t N,
                               int64_t K, int64_t Tb, float scale, const ArLossIn& loss,
                               hipStream_t st) {
  const int64_t nkb = arblk::row_tiles(Tb) * (BM / BK);
  return ar_launch_gemm_f32out(dyB, XTB, G, N, K, nkb, scale, loss, st);
}
