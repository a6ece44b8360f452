// Step loss from per-workgroup partial sums of squared residuals (see ArLossIn):
// float64 sum in a fixed order, an optional float64 term added, then the
// mean-squared-error normalisation and the strict best-loss decision of the
// tuning loop's snapshot.
#pragma once

#include "ar_device.h"
#include "ar_launch.h"

// Called by all 256 threads of one workgroup; sh = 256 doubles of LDS.
__device__ __forceinline__ void loss_reduce_block(const ArLossIn& L, double* sh) {
  double total = block_sum_f64(L.partials, L.nparts, sh);
  if (threadIdx.x == 0) {
    if (L.add) total += *L.add;
    if (L.sum_out) *L.sum_out = total;
    const float loss = (float)(total * L.inv_count);
    if (L.loss_out) *L.loss_out = loss;
    if (L.loss_slot) *L.loss_slot = loss;
    int imp = 0;
    if (L.best_loss) {
      imp = loss < *L.best_loss;
      if (imp) *L.best_loss = loss;
    }
    if (L.flag) *L.flag = imp;
  }
}
