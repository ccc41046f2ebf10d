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

// documents up to this length use the per-wave histogram sort (4 * Ld ints of LDS)
constexpr int64_t kSortWavesMaxLd = 3840;

struct BwdArgs {
  const void* Q;
  const void* D;
  const float* g;
  const int32_t* argmax;
  float* gQ;
  float* gD;
  int32_t* sorted;   // [n_docs][H] Q-row index of each hit, ordered by doc row, then hit id
  float* sorted_g;   // [n_docs][H] upstream gradient g[pair] of each sorted hit
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
  // 16 gathered rows in flight per thread: the loop is bound by memory
  // latency, not bandwidth, at the usual few-thousand-thread grids
  constexpr int U = 16;
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
// grad_Q, sliced: one workgroup per (query, token); its threads are CPR
// chunk lanes x NS document slices.  Every thread gathers its slice's rows
// with all loads independent (one latency round trip for the indices, one
// for the rows), and the NS slice partials of each chunk are added in slice
// order through LDS: deterministic, and tens of thousands of rows in flight.
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradq_sliced_kernel(BwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int NS = 256 / CPR;            // document slices
  constexpr int U = 16;                    // rows per round
  __shared__ float part[NS][CPR * EPC];
  const int tid = threadIdx.x;
  const int c = tid % CPR, sl = tid / CPR;
  const int64_t qi = blockIdx.x;           // q * Lq + i
  const int64_t q = qi / a.Lq, i = qi - q * a.Lq;
  const bool ap = a.layout == kAllPairs;
  const int64_t K = ap ? a.n_docs : a.K;
  const int64_t per = (K + NS - 1) / NS;
  const int64_t k_lo = min(sl * per, K), k_hi = min(k_lo + per, K);
  const char* Db = (const char*)a.D;
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += U) {
    int jj[U];
    float gg[U];
    int64_t dd[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u;
      jj[u] = -1;
      gg[u] = 0.0f;
      dd[u] = 0;
      if (k < k_hi) {
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
#pragma unroll
  for (int k = 0; k < EPC; ++k) part[sl][c * EPC + k] = acc[k];
  __syncthreads();
  // thread t < CPR*EPC/4 sums one float4 of the row over the slices in order
  constexpr int NV = CPR * EPC / 4;
  if (tid < NV) {
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int x = 0; x < NS; ++x) {
      const float4 v = *reinterpret_cast<const float4*>(&part[x][tid * 4]);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    *reinterpret_cast<float4*>(a.gQ + qi * DIM + tid * 4) = sum;
  }
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

// Q row and score (pair) index of hit h of document e.
__device__ __forceinline__ void hit_qrow_pair(const BwdArgs& a, int64_t e, int64_t h,
                                              int64_t& qrow, int64_t& p) {
  if (a.layout == kAllPairs) {
    qrow = h;
    p = (h / a.Lq) * a.n_docs + e;
  } else {
    qrow = (e / a.K) * a.Lq + h;
    p = e;
  }
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
        if (v && pos + rank < H) {
          int64_t qrow, p;
          hit_qrow_pair(a, e, h, qrow, p);
          out[pos + rank] = (int32_t)qrow;
          a.sorted_g[e * H + pos + rank] = a.g[p];
        }
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

// ---------------------------------------------------------------------------
// grad_D, step 1 (parallel form): each of the 4 waves owns a contiguous
// quarter of the document's hits and its own row histogram, so the stable
// placement needs no cross-wave turns: a hit's slot is the row's start, plus
// the row's hits in earlier waves, plus its ballot rank inside its wave.
// LDS: 4 * Ld + 4 ints.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gradd_sort_waves_kernel(BwdArgs a) {
  extern __shared__ int smem[];
  const int Ld = (int)a.Ld;
  int* cnt = smem;               // [4][Ld] counts, then running cursors
  int* wtot = smem + 4 * Ld;     // 4 wave totals of the scan
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t e = blockIdx.x;
  const int64_t H = a.H;
  const int64_t Hq = ((H + 255) / 256) * 64;   // hits per wave, a multiple of 64
  const int64_t h0 = min(wave * Hq, H), h1 = min(h0 + Hq, H);

  for (int j = tid; j < 4 * Ld; j += 256) cnt[j] = 0;
  __syncthreads();
  int* mine = cnt + wave * Ld;
  // 16 independent argmax loads in flight per lane before any is consumed
  constexpr int UH = 16;
  for (int64_t hb = h0 + lane; hb < h1; hb += 64 * UH) {
    int jj[UH];
#pragma unroll
    for (int u = 0; u < UH; ++u) {
      const int64_t h = hb + 64 * u;
      jj[u] = h < h1 ? hit_row(a, e, h) : -1;
    }
#pragma unroll
    for (int u = 0; u < UH; ++u)
      if (jj[u] >= 0) atomicAdd(&mine[jj[u]], 1);
  }
  __syncthreads();

  // exclusive scan over rows of the per-row totals; per-wave cursors
  const int seg = (Ld + 255) / 256;
  const int lo = min(tid * seg, Ld), hi = min(lo + seg, Ld);
  int local = 0;
  for (int j = lo; j < hi; ++j) local += cnt[j] + cnt[Ld + j] + cnt[2 * Ld + j] + cnt[3 * Ld + j];
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
    roff[j] = base;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w * Ld + j];
      cnt[w * Ld + j] = base;
      base += c;
    }
  }
  if (tid == 0) roff[Ld] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();

  int32_t* out = a.sorted + e * H;
  float* outg = a.sorted_g + e * H;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  // rows of the next chunk of 64 hits are loaded while this chunk is placed
  int jn = (h0 + lane < h1) ? hit_row(a, e, h0 + lane) : -1;
  for (int64_t hb = h0; hb < h1; hb += 64) {
    const int64_t h = hb + lane;
    const int j = jn;
    jn = (hb + 64 + lane < h1) ? hit_row(a, e, hb + 64 + lane) : -1;
    const bool v = j >= 0;
    uint64_t same = __ballot(v);
    for (int b = 0; b < a.key_bits; ++b) {
      const bool bit = v && ((j >> b) & 1);
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & below);
    const int count = __popcll(same);
    const int pos = v ? mine[j] : 0;
    __asm__ volatile("" ::: "memory");
    if (v && pos + rank < H) {
      int64_t qrow, p;
      hit_qrow_pair(a, e, h, qrow, p);
      out[pos + rank] = (int32_t)qrow;
      outg[pos + rank] = a.g[p];
    }
    if (v && rank == count - 1) mine[j] = pos + count;
  }
}

// ---------------------------------------------------------------------------
// grad_D, step 2 (wave per row): the wave's lanes form 64/CPR entry groups;
// group k takes the row's entries k, k + groups, ... (in sorted order) and the
// group partials are added by a fixed xor tree, so the sum order depends only
// on the row's entry list: deterministic, and long rows are spread over the
// whole wave.  Each wave walks `rpw` consecutive rows.
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradd_rows_wave_kernel(BwdArgs a, int rpw) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int EG = CPR >= 64 ? 1 : 64 / CPR;    // entry groups per wave
  constexpr int U = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = CPR >= 64 ? 0 : lane / CPR, c = CPR >= 64 ? lane : lane - grp * CPR;
  const int64_t n_rows = a.n_docs * a.Ld;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * rpw;
  const bool ap = a.layout == kAllPairs;
  const char* Qb = (const char*)a.Q;
  for (int rr = 0; rr < rpw; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= n_rows) break;
    const int64_t e = row / a.Ld;
    const int64_t j = row - e * a.Ld;
    const int32_t* roff = a.roff + e * (a.Ld + 1);
    const int s = max(0, min(roff[j], (int)a.H));
    const int t = max(s, min(roff[j + 1], (int)a.H));
    const int32_t* lst = a.sorted + e * a.H;
    float acc[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
    for (int k0 = s; k0 < t; k0 += EG * U) {
      float gg[U];
      int64_t qrow[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * EG + grp;
        gg[u] = 0.0f;
        qrow[u] = 0;
        if (k < t) {
          const int64_t h = min(max((int64_t)lst[k], (int64_t)0), a.H - 1);
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
      for (int u = 0; u < U; ++u)
        ch[u] = ld_global_16(Qb + qrow[u] * (int64_t)G::kRowBytes + c * 16);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[EPC];
        chunk_to_float<E>(ch[u], f);
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(gg[u], f[k], acc[k]);
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int k = 0; k < EPC; ++k) acc[k] += __shfl_xor(acc[k], off);
    if (grp == 0) {
      float* out = a.gD + row * DIM + c * EPC;
#pragma unroll
      for (int k = 0; k < EPC; k += 4)
        *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// grad_D, step 2 (lane group per row): a group of CPR lanes (one 16-byte
// chunk of the row each) owns `rpg` consecutive rows.  The rows' offsets come
// in one load; a row's (Q row, g) pairs come 16 at a time, the next 16
// prefetched while the current 16 Q rows are in flight; partial sums are
// added in the sorted order, so every row has one owner and a fixed order.
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradd_rows_group_kernel(BwdArgs a, int rpg) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;                  // lanes per group
  constexpr int GPB = 256 / CPR;                // groups per workgroup
  constexpr int B = CPR < 16 ? CPR : 16;        // entries per batch (one pair per lane)
  const int tid = threadIdx.x;
  const int c = tid % CPR;
  const int64_t gid = (int64_t)blockIdx.x * GPB + tid / CPR;
  const int64_t n_rows = a.n_docs * a.Ld;
  const int64_t row0 = gid * rpg;
  if (row0 >= n_rows) return;
  const char* Qb = (const char*)a.Q;
  // lane c < rpg: offsets [s, t) of row row0 + c
  int my_s = 0, my_t = 0;
  if (c < rpg && row0 + c < n_rows) {
    const int64_t row = row0 + c;
    const int64_t e = row / a.Ld, j = row - e * a.Ld;
    const int32_t* roff = a.roff + e * (a.Ld + 1);
    my_s = max(0, min(roff[j], (int)a.H));
    my_t = max(my_s, min(roff[j + 1], (int)a.H));
  }
  for (int r = 0; r < rpg; ++r) {
    const int64_t row = row0 + r;
    if (row >= n_rows) break;
    const int s = __shfl(my_s, r, CPR), t = __shfl(my_t, r, CPR);
    const int64_t e = row / a.Ld;
    const int32_t* lq = a.sorted + e * a.H;
    const float* lg = a.sorted_g + e * a.H;
    float acc[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
    // pairs of the first batch
    int pq = 0;
    float pg = 0.0f;
    if (s + c < t && c < B) {
      pq = lq[s + c];
      pg = lg[s + c];
    }
    for (int k0 = s; k0 < t; k0 += B) {
      const int cq = pq;
      const float cg = pg;
      // prefetch the next batch's pairs
      if (k0 + B + c < t && c < B) {
        pq = lq[k0 + B + c];
        pg = lg[k0 + B + c];
      }
      const int nb = min(B, t - k0);
      u32x4 ch[B];
      float gg[B];
#pragma unroll
      for (int m = 0; m < B; ++m) {
        const int64_t qrow = min(max(__shfl(cq, m, CPR), 0), (int)(a.Nq * a.Lq) - 1);
        gg[m] = m < nb ? __shfl(cg, m, CPR) : 0.0f;
        ch[m] = ld_global_16(Qb + qrow * (int64_t)G::kRowBytes + c * 16);
      }
#pragma unroll
      for (int m = 0; m < B; ++m) {
        float f[EPC];
        chunk_to_float<E>(ch[m], f);
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(gg[m], f[k], acc[k]);
      }
    }
    float* out = a.gD + row * DIM + c * EPC;
#pragma unroll
    for (int k = 0; k < EPC; k += 4)
      *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
  }
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
    const int64_t K = a.layout == kAllPairs ? a.n_docs : a.K;
    if (K >= 64) {
      // many documents per query: split each (query, token) over slices
      hipLaunchKernelGGL((gradq_sliced_kernel<E, DIM>), dim3((unsigned)(a.Nq * a.Lq)), dim3(256), 0,
                         s, a);
    } else {
      const int64_t tpb = 256 / CPR;
      hipLaunchKernelGGL((gradq_kernel<E, DIM>), dim3((unsigned)a.Nq, (unsigned)cdiv(a.Lq, tpb)),
                         dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (want_d) {
    hipError_t e;
    if (a.Ld <= kSortWavesMaxLd) {
      const size_t lds = (size_t)(4 * a.Ld + 4) * sizeof(int);
      hipLaunchKernelGGL(gradd_sort_waves_kernel, dim3((unsigned)a.n_docs), dim3(256), lds, s, a);
    } else {
      const size_t lds = (size_t)(a.Ld + 4) * sizeof(int);
      hipLaunchKernelGGL(gradd_sort_kernel, dim3((unsigned)a.n_docs), dim3(256), lds, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // rows per group: one while groups are scarce; up to 16 (one offsets
    // load) when the output is large and mostly empty rows
    const int64_t n_rows = a.n_docs * a.Ld;
    int rpg = (int)cdiv(n_rows, 256 * 256);
    const int max_rpg = CPR < 16 ? CPR : 16;   // one offsets load per group
    rpg = rpg < 1 ? 1 : (rpg > max_rpg ? max_rpg : rpg);
    const int64_t gpb = 256 / CPR;
    hipLaunchKernelGGL((gradd_rows_group_kernel<E, DIM>),
                       dim3((unsigned)cdiv(cdiv(n_rows, rpg), gpb)), dim3(256), 0, s, a, rpg);
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
  a.sorted_g = reinterpret_cast<float*>(ws + p.off_sorted_g);
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
