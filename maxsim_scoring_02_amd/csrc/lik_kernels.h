// Internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lik_plan.h"

namespace lik {

// Arguments of the forward kernels (passed by value).
struct FwdArgs {
  const void* Q;
  const void* D;
  const uint8_t* q_mask;
  uint32_t* bits;     // [n_docs][nwords] tile validity words, or null (no doc mask)
  int32_t* ntiles;    // [n_docs] tiles up to the last valid token, or null
  float* scores;
  int32_t* argmax;
  // partial maxima [nchunks][n_docs][n_cg * SPW]: all-pairs by token
  // (q * Lq + i, tokens with a slot only), pairwise / kd by (slot group, slot)
  float* part_M;
  int32_t* part_J;          // partial argmaxes, same layout
  // compacted query tokens (all-pairs with a query mask): slot s holds token
  // tok[s] = q * Lq + i for s < *tok_cnt
  int32_t* tok;
  int32_t* tok_cnt;
  int compact;
  int layout;
  int SPW;
  int partial;
  int64_t Nq, Lq, n_docs, Ld, K;
  int64_t nwords, ntiles_max;
  int64_t qpw, n_cg, n_sb, nchunks, tpc, upw, n_groups, gpx, n_units;
};

bool fwd_dim_supported(int64_t dim);

// Events the caller asked to have recorded around the main forward kernel
// (null when not profiling); see lik_set_profile_events.
void profile_events(hipEvent_t* start, hipEvent_t* stop);

hipError_t run_forward(const FwdPlan& p, const void* Q, const void* D, const uint8_t* q_mask,
                       const uint8_t* d_mask, float* scores, int32_t* argmax, char* ws,
                       hipStream_t s);

hipError_t run_backward(const BwdPlan& p, const void* Q, const void* D, const uint8_t* q_mask,
                        const uint8_t* d_mask, const float* grad_scores, const int32_t* argmax,
                        float* grad_Q, float* grad_D, char* ws, hipStream_t s);

// Loss head: row cross-entropy of a score matrix (lik_loss.hip).
hipError_t run_ce_rows(const float* S, int64_t R, int64_t C, const int32_t* labels, float scale,
                       float* row_loss, float* loss, float* grad, hipStream_t s);

}  // namespace lik
