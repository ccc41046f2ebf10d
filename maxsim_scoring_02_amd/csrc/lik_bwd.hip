// Backward kernels of the gfx950 MaxSim scorer.
//
// At the forward's argmax a(p, i) (p = a (query, document) pair) the score is
// linear in Q and D, so (colpali pull request, "Results": only the input
// gradients are produced):
//   grad_Q[q,i,:] = sum over the pairs p of query q of g[p] * D[doc(p), a(p,i), :]
//   grad_D[e,j,:] = sum over (p, i) with doc(p) = e and a(p,i) = j of g[p] * Q[q(p), i, :]
// Masked query tokens and empty documents carry argmax -1 and contribute
// nothing.
//
//   gradq_kernel       gather: one lane group per (query token, 16-byte chunk)
//   gradd_sort_kernel  per document, a stable counting sort of its hits by
//                      row j (integer LDS histogram, ballot ranks), so that
//   gradd_rows_kernel  can give every row of grad_D one owner that sums its
//                      hits in a fixed order: deterministic, no float atomics.
#include <hip/hip_runtime.h>

#include "lik_device.h"
#include "lik_kernels.h"
#include "lik_plan.h"

namespace lik {

struct BwdArgs {
  const void* Q;
  const void* D;
  const float* g;
  const int32_t* argmax;
  float* gQ;
  float* gD;
  int32_t* sorted;   // [n_docs][H] hit ids ordered by row, then by hit id
  int32_t* roff;     // [n_docs][Ld + 1] row offsets into `sorted`
  int layout;
  int key_bits;
  int64_t Nq, Lq, n_docs, Ld, K, H;
};

// ---------------------------------------------------------------------------
// grad_Q: grid (query, token group); thread = (token, 16-byte chunk)
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradq_kernel(BwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int TPB = 256 / CPR;
  const int tid = threadIdx.x;
  const int tk = tid / CPR, c = tid - tk * CPR;
  const int64_t q = blockIdx.x;
  const int64_t i = (int64_t)blockIdx.y * TPB + tk;
  if (i >= a.Lq) return;
  const bool ap = a.layout == kAllPairs;
  const int64_t K = ap ? a.n_docs : a.K;
  const char* Db = (const char*)a.D;
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
  constexpr int U = 4;
  for (int64_t k0 = 0; k0 < K; k0 += U) {
    int jj[U];
    float gg[U];
    int64_t dd[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u;
      jj[u] = -1;
      gg[u] = 0.0f;
      dd[u] = 0;
      if (k < K) {
        const int64_t p = q * K + k;
        dd[u] = ap ? k : p;
        jj[u] = a.argmax[p * a.Lq + i];
        gg[u] = a.g[p];
      }
    }
    u32x4 ch[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = jj[u] >= 0 && jj[u] < a.Ld;
      u32x4 z = {0u, 0u, 0u, 0u};
      ch[u] = ok ? ld_global_16(Db + (dd[u] * a.Ld + jj[u]) * (int64_t)G::kRowBytes + c * 16) : z;
      if (!ok) gg[u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[EPC];
      chunk_to_float<E>(ch[u], f);
#pragma unroll
      for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(gg[u], f[k], acc[k]);
    }
  }
  float* out = a.gQ + (q * a.Lq + i) * DIM + c * EPC;
#pragma unroll
  for (int k = 0; k < EPC; k += 4)
    *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
}

// ---------------------------------------------------------------------------
// grad_D, step 1: per document, hits sorted by row (stable)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int hit_row(const BwdArgs& a, int64_t e, int64_t h) {
  int64_t p, i;
  if (a.layout == kAllPairs) {
    const int64_t q = h / a.Lq;
    i = h - q * a.Lq;
    p = q * a.n_docs + e;
  } else {
    p = e;
    i = h;
  }
  const int j = a.argmax[p * a.Lq + i];
  return (j >= 0 && j < a.Ld) ? j : -1;
}

__global__ __launch_bounds__(256) void gradd_sort_kernel(BwdArgs a) {
  extern __shared__ int smem[];
  const int Ld = (int)a.Ld;
  int* cur = smem;             // counts, then (in place) the running row cursors
  int* wtot = smem + Ld;       // 4 wave totals
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t e = blockIdx.x;
  const int64_t H = a.H;

  for (int j = tid; j < Ld; j += 256) cur[j] = 0;
  __syncthreads();
  for (int64_t h = tid; h < H; h += 256) {
    const int j = hit_row(a, e, h);
    if (j >= 0) atomicAdd(&cur[j], 1);
  }
  __syncthreads();

  // exclusive scan of the counts, in place; each thread owns a segment
  const int seg = (Ld + 255) / 256;
  const int lo = min(tid * seg, Ld), hi = min(lo + seg, Ld);
  int local = 0;
  for (int j = lo; j < hi; ++j) local += cur[j];
  int incl = local;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int t = __shfl_up(incl, k);
    if (lane >= k) incl += t;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = incl - local;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  int32_t* roff = a.roff + e * (a.Ld + 1);
  for (int j = lo; j < hi; ++j) {
    const int c = cur[j];
    cur[j] = base;
    roff[j] = base;
    base += c;
  }
  if (tid == 0) roff[Ld] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();

  // stable placement: waves take turns over each group of 256 hits
  int32_t* out = a.sorted + e * H;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int64_t h0 = 0; h0 < H; h0 += 256) {
    for (int w = 0; w < 4; ++w) {
      if (wave == w) {
        const int64_t h = h0 + w * 64 + lane;
        const int j = h < H ? hit_row(a, e, h) : -1;
        const bool v = j >= 0;
        uint64_t same = __ballot(v);
        for (int b = 0; b < a.key_bits; ++b) {
          const bool bit = v && ((j >> b) & 1);
          const uint64_t bb = __ballot(bit);
          same &= bit ? bb : ~bb;
        }
        const int rank = __popcll(same & below);
        const int count = __popcll(same);
        const int pos = v ? cur[j] : 0;
        __asm__ volatile("" ::: "memory");
        if (v && pos + rank < H) out[pos + rank] = (int32_t)h;
        if (v && rank == count - 1) cur[j] = pos + count;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// grad_D, step 2: one lane group per row sums its hits in sorted order
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradd_rows_kernel(BwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int RPB = 256 / CPR;
  const int tid = threadIdx.x;
  const int rk = tid / CPR, c = tid - rk * CPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + rk;
  if (row >= a.n_docs * a.Ld) return;
  const int64_t e = row / a.Ld;
  const int64_t j = row - e * a.Ld;
  const int32_t* roff = a.roff + e * (a.Ld + 1);
  const int s = max(0, min(roff[j], (int)a.H));
  const int t = max(s, min(roff[j + 1], (int)a.H));
  const int32_t* lst = a.sorted + e * a.H;
  const bool ap = a.layout == kAllPairs;
  const char* Qb = (const char*)a.Q;
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
  constexpr int U = 4;
  for (int k0 = s; k0 < t; k0 += U) {
    float gg[U];
    int64_t qrow[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      gg[u] = 0.0f;
      qrow[u] = 0;
      if (k0 + u < t) {
        const int64_t h = min(max((int64_t)lst[k0 + u], (int64_t)0), a.H - 1);
        int64_t p;
        if (ap) {
          const int64_t q = h / a.Lq;
          p = q * a.n_docs + e;
          qrow[u] = h;
        } else {
          p = e;
          qrow[u] = (e / a.K) * a.Lq + h;
        }
        gg[u] = a.g[p];
      }
    }
    u32x4 ch[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ch[u] = ld_global_16(Qb + qrow[u] * (int64_t)G::kRowBytes + c * 16);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[EPC];
      chunk_to_float<E>(ch[u], f);
#pragma unroll
      for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(gg[u], f[k], acc[k]);
    }
  }
  float* out = a.gD + row * DIM + c * EPC;
#pragma unroll
  for (int k = 0; k < EPC; k += 4)
    *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
}

__global__ void zero_kernel(float4* p, int64_t n4) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n4) p[k] = make_float4(0.f, 0.f, 0.f, 0.f);
}

static hipError_t zero_fill(float* p, int64_t n, hipStream_t s) {
  // n is a multiple of 4 for every supported dim
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)cdiv(n4, 256)), dim3(256), 0, s,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

template <Elem E, int DIM>
static hipError_t launch_grads(const BwdArgs& a, bool want_q, bool want_d, hipStream_t s) {
  using G = Geo<E, DIM>;
  constexpr int CPR = G::kCPR;
  if (want_q) {
    const int64_t tpb = 256 / CPR;
    hipLaunchKernelGGL((gradq_kernel<E, DIM>), dim3((unsigned)a.Nq, (unsigned)cdiv(a.Lq, tpb)),
                       dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (want_d) {
    const size_t lds = (size_t)(a.Ld + 4) * sizeof(int);
    hipLaunchKernelGGL(gradd_sort_kernel, dim3((unsigned)a.n_docs), dim3(256), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rpb = 256 / CPR;
    hipLaunchKernelGGL((gradd_rows_kernel<E, DIM>), dim3((unsigned)cdiv(a.n_docs * a.Ld, rpb)),
                       dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <Elem E>
static hipError_t grads_dim(int dim, const BwdArgs& a, bool wq, bool wd, hipStream_t s) {
  switch (dim) {
    case 64: return launch_grads<E, 64>(a, wq, wd, s);
    case 128: return launch_grads<E, 128>(a, wq, wd, s);
    case 256: return launch_grads<E, 256>(a, wq, wd, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_backward(const BwdPlan& p, const void* Q, const void* D, const uint8_t* q_mask,
                        const uint8_t* d_mask, const float* grad_scores, const int32_t* argmax,
                        float* grad_Q, float* grad_D, char* ws, hipStream_t s) {
  const FwdPlan& f = p.fwd;
  if (f.Nq == 0 || f.n_docs == 0) return hipSuccess;
  const int64_t dim = f.dim;
  if (f.Lq == 0) {
    // no query tokens: every gradient is zero (grad_Q is empty)
    return grad_D ? zero_fill(grad_D, f.n_docs * f.Ld * dim, s) : hipSuccess;
  }
  if (f.Ld == 0) {
    return grad_Q ? zero_fill(grad_Q, f.Nq * f.Lq * dim, s) : hipSuccess;
  }
  const int32_t* am = argmax;
  if (p.recompute) {
    int32_t* am_ws = reinterpret_cast<int32_t*>(ws + p.off_argmax);
    float* sc_ws = reinterpret_cast<float*>(ws + p.off_scores);
    hipError_t e = run_forward(f, Q, D, q_mask, d_mask, sc_ws, am_ws, ws + p.off_fwd, s);
    if (e != hipSuccess) return e;
    am = am_ws;
  }
  BwdArgs a{};
  a.Q = Q;
  a.D = D;
  a.g = grad_scores;
  a.argmax = am;
  a.gQ = grad_Q;
  a.gD = grad_D;
  a.sorted = reinterpret_cast<int32_t*>(ws + p.off_sorted);
  a.roff = reinterpret_cast<int32_t*>(ws + p.off_roff);
  a.layout = f.layout;
  a.key_bits = p.key_bits;
  a.Nq = f.Nq;
  a.Lq = f.Lq;
  a.n_docs = f.n_docs;
  a.Ld = f.Ld;
  a.K = f.K;
  a.H = p.H;
  switch (f.elem) {
    case 0: return grads_dim<Elem::F16>(f.dim, a, grad_Q != nullptr, grad_D != nullptr, s);
    case 1: return grads_dim<Elem::BF16>(f.dim, a, grad_Q != nullptr, grad_D != nullptr, s);
    default: return grads_dim<Elem::F32>(f.dim, a, grad_Q != nullptr, grad_D != nullptr, s);
  }
}

}  // namespace lik
