// select.hip -- binary64 second stage of the two-level Gumbel-max draws: the
// draft token of position k (summary page §3.1), the corrective token drawn
// from max(0, p^t - p^d) at the first rejection and the bonus token drawn from
// p^t after full acceptance (standard speculative rejection sampling, notes
// page 배경).
//
// A draw picks a 32-entry block by Gumbel-max over the blocks' log-masses, then
// a member of that block by Gumbel-max over its log-weights; exact ties go to
// the lowest block / entry.  The split passes leave, per (row, split), the
// bracket [lo, hi] of every block's binary32 score in compressed form (largest
// lo, best hi with its block, second-best hi).  One workgroup per row here:
//   1. merges the splits (draft: log-sum-exp of the logits);
//   2. L* = largest lower bound over all blocks; only a block whose upper bound
//      reaches L* can win, so each split contributes its best block if hi1 >= L*,
//      or all of its blocks if hi2 >= L* too;
//   3. rescores those blocks in binary64 from the stored inputs (the bias
//      recomputed from W1 and the packed W2) and keeps the best;
//   4. draws the member of the winning block in binary64.
#include "select_impl.h"

namespace dspark {

namespace {

template <int MODE>
__global__ __launch_bounds__(256) void k_select(const SelectArgs a, int bf16_flag) {
  __shared__ sel::SelShared sh;
  sel::select_row<MODE>(a, bf16_flag, blockIdx.x, sh, a.k);
}

// The verify's final draws in one launch, one workgroup per request: every
// request is on exactly one of the two lists (a rejection, or full acceptance
// and a bonus draw), the residual list first.
__global__ __launch_bounds__(256) void k_select_final(const SelectArgs ar, const SelectArgs ab,
                                                      int bf16_flag) {
  __shared__ sel::SelShared sh;
  const int nres = *ar.row_count;
  const int i = (int)blockIdx.x;
  if (i < nres) sel::select_row<kSelResidual>(ar, bf16_flag, i, sh, 0);
  else sel::select_row<kSelBonus>(ab, bf16_flag, i - nres, sh, 0);
}

}  // namespace

hipError_t launch_select(int mode, bool bf16, const SelectArgs& a, hipStream_t stream) {
  const int flag = bf16 ? 1 : 0;
  // each of the 256 threads holds at most RecSlots<MODE>::K split records
  const int max_splits = 256 * (mode == kSelBonus ? sel::RecSlots<kSelBonus>::K : 1);
  if (a.nsplit < 1 || a.nsplit > max_splits) return hipErrorInvalidValue;
  if (mode == kSelDraft) {
    TimingScope timing("draft_select", stream);
    hipLaunchKernelGGL(k_select<kSelDraft>, dim3(a.R), dim3(256), 0, stream, a, flag);
  } else if (mode == kSelResidual) {
    TimingScope timing("residual_select", stream);
    hipLaunchKernelGGL(k_select<kSelResidual>, dim3(a.R), dim3(256), 0, stream, a, flag);
  } else {
    TimingScope timing("bonus_select", stream);
    hipLaunchKernelGGL(k_select<kSelBonus>, dim3(a.R), dim3(256), 0, stream, a, flag);
  }
  return hipGetLastError();
}

hipError_t launch_select_final(bool bf16, const SelectArgs& ar, const SelectArgs& ab,
                               hipStream_t stream) {
  if (ar.nsplit < 1 || ar.nsplit > 256 * sel::RecSlots<kSelResidual>::K) return hipErrorInvalidValue;
  if (ab.nsplit < 1 || ab.nsplit > 256 * sel::RecSlots<kSelBonus>::K) return hipErrorInvalidValue;
  if (ar.R != ab.R) return hipErrorInvalidValue;
  TimingScope timing("final_select", stream);
  hipLaunchKernelGGL(k_select_final, dim3(ar.R), dim3(256), 0, stream, ar, ab, bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dspark
