// Loss head on gfx950: softmax cross-entropy over the rows of a float32 score
// matrix, one target column per row, mean over rows, and its gradient.
//
// The colpali pull request puts its in-batch ColBERT loss and its negative-doc
// losses (over the per-query candidate layout) on top of the MaxSim scores
// ("What this PR adds"), and its "Results" benchmark that loss head with the
// operator.  The pages name the losses without defining them; the row
// cross-entropy below is the plain reading: targets on the diagonal for the
// in-batch loss, column 0 (the positive candidate) for the negative-doc loss,
// logits scaled by s:
//
//   l_r = logsumexp_c(s S[r,c]) - s S[r,t_r],   L = mean_r l_r,
//   dL/dS[r,c] = (s / R) (softmax_c(s S[r,:]) - [c == t_r]).
//
//   ce_rows_kernel   one wave per row: row max, sum of exponentials, row loss
//                    and the gradient row (three coalesced passes)
//   ce_mean_kernel   one workgroup: the mean of the row losses in a fixed
//                    order (float64 accumulation), so the loss is bitwise
//                    reproducible
#include <hip/hip_runtime.h>

#include "lik_kernels.h"

namespace lik {

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v = fmaxf(v, __shfl_xor(v, k));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
  return v;
}

// One row on one wave: returns the row loss (in every lane) and writes the
// gradient row when asked.
__device__ __forceinline__ float ce_row(const float* __restrict__ row, int64_t C, int64_t t,
                                        float scale, float k, float* __restrict__ out, int lane) {
  float m = -__builtin_inff();
  for (int64_t c = lane; c < C; c += 64) m = fmaxf(m, scale * row[c]);
  m = wave_max_f32(m);
  float sum = 0.0f;
  for (int64_t c = lane; c < C; c += 64) sum += expf(scale * row[c] - m);
  sum = wave_sum_f32(sum);
  const float lse = m + logf(sum);
  if (out) {
    for (int64_t c = lane; c < C; c += 64) {
      const float p = expf(scale * row[c] - lse);
      out[c] = k * (c == t ? p - 1.0f : p);
    }
  }
  return (t >= 0 && t < C) ? lse - scale * row[t] : __builtin_nanf("");
}

__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ S, int64_t R,
                                                      int64_t C, const int32_t* __restrict__ labels,
                                                      float scale, float* __restrict__ row_loss,
                                                      float* __restrict__ grad) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;                       // whole wave
  const int64_t t = labels ? (int64_t)labels[r] : r;
  const float l = ce_row(S + r * C, C, t, scale, scale / (float)R, grad ? grad + r * C : nullptr,
                         lane);
  if (lane == 0) row_loss[r] = l;
}

__global__ __launch_bounds__(256) void ce_mean_kernel(const float* __restrict__ row_loss,
                                                      int64_t R, float* __restrict__ loss) {
  __shared__ double part[256];
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int64_t r = tid; r < R; r += 256) acc += (double)row_loss[r];
  part[tid] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) *loss = (float)(part[0] / (double)R);
}

hipError_t run_ce_rows(const float* S, int64_t R, int64_t C, const int32_t* labels, float scale,
                       float* row_loss, float* loss, float* grad, hipStream_t s) {
  hipLaunchKernelGGL(ce_rows_kernel, dim3((unsigned)cdiv(R, 4)), dim3(256), 0, s, S, R, C, labels,
                     scale, row_loss, grad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ce_mean_kernel, dim3(1), dim3(256), 0, s, row_loss, R, loss);
  return hipGetLastError();
}

}  // namespace lik
