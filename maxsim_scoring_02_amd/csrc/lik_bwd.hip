// Backward kernels of the gfx950 MaxSim scorer.
//
// At the forward's argmax a(p, i) (p = a (query, document) pair) the score is
// linear in Q and D, so (colpali pull request, "Results": only the input
// gradients are produced):
//   grad_Q[q,i,:] = sum over the pairs p of query q of g[p] * D[doc(p), a(p,i), :]
//   grad_D[e,j,:] = sum over (p, i) with doc(p) = e and a(p,i) = j of g[p] * Q[q(p), i, :]
// Masked query tokens and empty documents carry argmax -1 and contribute
// nothing.  No floating-point atomics anywhere: every output row has one
// owner that adds its terms in an order fixed by the inputs alone.
//
//   grad_Q
//     gradq_ap_kernel      all-pairs with many documents: a token's lanes take
//                          16 documents per round, each lane preparing one
//                          (row offset, weight) that the others read by a lane
//                          broadcast; with several document slices (workgroup
//                          b runs on XCD b % 8 and takes slice b % slices)
//                          the partials are added in slice order at the start
//                          of the sorted grad_D kernel that follows, or by
//                          gradq_reduce_kernel when that kernel does not run
//     gradq_kernel         few documents per query (pairwise, kd, small Nd)
//   grad_D
//     gradd_sorted_kernel  all-pairs: per document, one workgroup sorts its
//                          hits by row (stable counting sort in LDS), then
//                          lane groups sum equal shares of the sorted hits,
//                          16 hits per round prepared one per lane; rows cut by
//                          a share boundary are finished by the group where
//                          they start
//     gradd_pairs_kernel   pairwise / kd: waves per document stream its rows
//                          as zeros, then store the few rows with hits again
//                          with their sums (grads_pairs_kernel runs it beside
//                          the grad_Q gather in one launch)
//     gradd_sort_*_kernel + gradd_rows_group_kernel
//                          general fallback through the workspace
#include <hip/hip_runtime.h>

#include <utility>

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
  float* gq_part;    // [gq_slices][Nq * Lq][dim] grad_Q partials per document slice
  int layout;
  int key_bits;
  int gq_slices;
  int gq_ap;                                // grad_Q by gradq_ap_kernel (else gradq_kernel)
  int gs_sw, gs_split;                      // sorted grad_D: sorting waves, workgroups per doc
  int gd_parts;                             // pairwise / kd grad_D: waves per document
  int gs_masks;                             // sorted grad_D: ranks from LDS match masks
  int gs_off_sorted, gs_off_start, gs_off_gl, gs_off_keys, gs_off_hist, gs_off_masks,
      gs_off_part;                          // LDS layout
  uint64_t lq_magic;                        // ceil(2^32 / Lq): h / Lq for h < 2^16
  int64_t Nq, Lq, n_docs, Ld, K, H;
  int64_t e0, nb;                           // workspace sort: first document and documents of a batch
  int gq_red;                               // the sorted grad_D kernel also adds the grad_Q partials
};

// ---------------------------------------------------------------------------
// grad_Q: grid (query, token group); thread = (token, 16-byte chunk)
// ---------------------------------------------------------------------------
// U gathered rows in flight per thread.
template <Elem E, int DIM, int U>
__device__ __forceinline__ void gradq_body(const BwdArgs& a, int64_t q, int64_t iblk) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int TPB = 256 / CPR;
  const int tid = threadIdx.x;
  const int tk = tid / CPR, c = tid - tk * CPR;
  const int64_t i = iblk * TPB + tk;
  if (i >= a.Lq) return;
  const bool ap = a.layout == kAllPairs;
  const int64_t K = ap ? a.n_docs : a.K;
  const char* Db = (const char*)a.D;
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
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

template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradq_kernel(BwdArgs a) {
  // 16 gathered rows in flight per thread: the loop is bound by memory
  // latency, not bandwidth, at the usual few-thousand-thread grids
  gradq_body<E, DIM, 16>(a, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// Lane broadcasts inside a lane group of CPR lanes (one row chunk each): with
// 16-lane groups a DPP row_newbcast (a VALU move, folded by the compiler into
// the instruction that consumes it), otherwise a lane swap.
// ---------------------------------------------------------------------------
template <int CPR, int U>
__device__ __forceinline__ int grp_bcast(int v, int base_lane) {
  if constexpr (CPR == 16) {
    (void)base_lane;
    // every lane reads a valid source lane, so bound_ctrl needs no old value
    return __builtin_amdgcn_update_dpp(0, v, 0x150 + U, 0xf, 0xf, true);
  } else {
    return __shfl(v, base_lane + U);
  }
}
template <int CPR, int U>
__device__ __forceinline__ float grp_bcast_f(float v, int base_lane) {
  return __int_as_float(grp_bcast<CPR, U>(__float_as_int(v), base_lane));
}

template <int... U, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}
// f(integral_constant<0>) ... f(integral_constant<N-1>), fully unrolled
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ u32x4 ld_buf_16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
}

// Buffer descriptor over `bytes` bytes at `p` (bytes < 2^32): loads outside
// it return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// grad_Q, all-pairs.  Thread = (query token, 16-byte chunk c of the row).
// Documents are taken R at a time: lane c of a token looks up document k0 + c
// (its argmax row, turned into a byte offset inside the document slice, and
// its weight g[q, d]; row 0 and weight 0 when the document gives this token
// nothing), then the token's lanes issue the R row gathers with those values
// broadcast from lane u, and add g * row in document order.  With several
// slices, workgroup b runs on XCD b % 8 and gathers only from slice
// b % slices, so each XCD's L2 serves a fraction of D; partials go to gq_part.
// ---------------------------------------------------------------------------
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradq_ap_kernel(BwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int TPB = 256 / CPR;           // query tokens per workgroup
  constexpr int R = CPR < 16 ? CPR : 16;   // documents per round (one per lane)
  const int ns = a.gq_slices;
  const int sl = (int)(blockIdx.x % ns);
  const int64_t tb = blockIdx.x / ns;
  const int tid = threadIdx.x, lane = tid & 63;
  const int t = tid / CPR, c = tid - t * CPR;
  const int base_lane = lane - c;          // lane of chunk 0 of this token
  const int64_t n_tok = a.Nq * a.Lq;
  const int64_t qi = min(tb * TPB + t, n_tok - 1);  // a clamped token computes, never stores
  const bool tok_ok = tb * TPB + t < n_tok;
  const int64_t q = qi / a.Lq, i = qi - q * a.Lq;
  const int64_t Nd = a.n_docs;
  const int64_t d0 = Nd * sl / ns, d1 = Nd * (sl + 1) / ns;
  // the slice's rows, read through a buffer descriptor (the plan keeps a
  // slice below 2^32 bytes)
  const char* Ds = (const char*)a.D + d0 * a.Ld * (int64_t)G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(Ds, (uint32_t)((d1 - d0) * a.Ld * G::kRowBytes));
  const int32_t* am = a.argmax + q * Nd * a.Lq + i;     // + d * Lq
  const float* gq = a.g + q * Nd;
  const uint32_t my_chunk = (uint32_t)c * 16u;
  auto prep = [&](int64_t k0, uint32_t& off, float& w) {
    const int64_t d = k0 + c;
    off = 0;
    w = 0.0f;
    if (c < R && d < d1) {
      const int j = am[d * a.Lq];
      if (j >= 0 && j < a.Ld) {
        off = (uint32_t)(((d - d0) * a.Ld + j) * G::kRowBytes);
        w = gq[d];
      }
    }
  };
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
  uint32_t on;
  float wn;
  prep(d0, on, wn);
  for (int64_t k0 = d0; k0 < d1; k0 += R) {
    const uint32_t oc = on;
    const float wc = wn;
    prep(k0 + R, on, wn);                  // next round's lookups in flight
    u32x4 ch[R];
    float gg[R];
    static_for<R>([&](auto u) {
      // a looked-up offset is the row's start; add this lane's chunk
      const uint32_t o = (uint32_t)grp_bcast<CPR, u>((int)oc, base_lane);
      ch[u] = ld_buf_16(rs, o + my_chunk);
      gg[u] = grp_bcast_f<CPR, u>(wc, base_lane);
    });
#pragma unroll
    for (int u = 0; u < R; ++u) {
      float f[EPC];
      chunk_to_float<E>(ch[u], f);
#pragma unroll
      for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(gg[u], f[k], acc[k]);
    }
  }
  if (!tok_ok) return;
  float* out = (ns > 1 ? a.gq_part + (int64_t)sl * n_tok * DIM : a.gQ) + qi * DIM + c * EPC;
#pragma unroll
  for (int k = 0; k < EPC; k += 4)
    *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
}

// grad_Q element group k (four floats) = sum of the slice partials, added in
// slice order.
__device__ __forceinline__ void gradq_reduce_at(const float4* __restrict__ part, int ns, int64_t n4,
                                                float4* __restrict__ gQ, int64_t k) {
  float4 s = part[k];
  for (int x = 1; x < ns; ++x) {
    const float4 v = part[(int64_t)x * n4 + k];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  gQ[k] = s;
}

__global__ __launch_bounds__(256) void gradq_reduce_kernel(const float4* __restrict__ part, int ns,
                                                           int64_t n4, float4* __restrict__ gQ) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < n4) gradq_reduce_at(part, ns, n4, gQ, k);
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

// Rows are taken in windows of at most kSortWin (one int of LDS per row), so
// documents of any length sort in 64 KB of LDS: per window, the hits on its
// rows are counted, their row starts follow the hits of earlier windows, and
// they are placed in hit order.  Every window reads the hits' rows again.
constexpr int kSortWin = 16000;

__global__ __launch_bounds__(256) void gradd_sort_kernel(BwdArgs a) {
  extern __shared__ int smem[];
  const int Ld = (int)a.Ld;
  const int W = Ld < kSortWin ? Ld : kSortWin;
  int* cur = smem;             // counts, then (in place) the running row cursors of a window
  int* wtot = smem + W;        // 4 wave totals
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t el = blockIdx.x;          // document of the batch (workspace index)
  const int64_t e = a.e0 + el;            // document
  const int64_t H = a.H;
  int32_t* roff = a.roff + el * (a.Ld + 1);
  int32_t* out = a.sorted + el * H;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  int placed = 0;              // hits on the rows of earlier windows

  for (int r0 = 0; r0 < Ld; r0 += W) {
    const int nw = min(W, Ld - r0);
    for (int j = tid; j < nw; j += 256) cur[j] = 0;
    __syncthreads();
    for (int64_t h = tid; h < H; h += 256) {
      const int j = hit_row(a, e, h) - r0;
      if (j >= 0 && j < nw) atomicAdd(&cur[j], 1);
    }
    __syncthreads();

    // exclusive scan of the window's counts, in place; each thread owns a segment
    const int seg = (nw + 255) / 256;
    const int lo = min(tid * seg, nw), hi = min(lo + seg, nw);
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
    int base = placed + incl - local;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    for (int j = lo; j < hi; ++j) {
      const int c = cur[j];
      cur[j] = base;
      roff[r0 + j] = base;
      base += c;
    }
    placed += wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();

    // stable placement: waves take turns over each group of 256 hits
    for (int64_t h0 = 0; h0 < H; h0 += 256) {
      for (int w = 0; w < 4; ++w) {
        if (wave == w) {
          const int64_t h = h0 + w * 64 + lane;
          const int jr = h < H ? hit_row(a, e, h) : -1;
          const bool v = jr >= r0 && jr < r0 + nw;
          const int j = v ? jr - r0 : 0;
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
            a.sorted_g[el * H + pos + rank] = a.g[p];
          }
          if (v && rank == count - 1) cur[j] = pos + count;
        }
        __syncthreads();
      }
    }
  }
  if (tid == 0) roff[Ld] = placed;
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
  const int64_t el = blockIdx.x;          // document of the batch (workspace index)
  const int64_t e = a.e0 + el;            // document
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
  int32_t* roff = a.roff + el * (a.Ld + 1);
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

  int32_t* out = a.sorted + el * H;
  float* outg = a.sorted_g + el * H;
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
  const int64_t n_rows = a.nb * a.Ld;      // rows of the batch's documents
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
    float* out = a.gD + (a.e0 * a.Ld + row) * DIM + c * EPC;
#pragma unroll
    for (int k = 0; k < EPC; k += 4)
      *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
  }
}
// ---------------------------------------------------------------------------
// grad_D, all-pairs, sorted: workgroup (document e, split s) of kGsThreads.
//
//  1. sorting wave w takes the hits [w*Hw, (w+1)*Hw) in chunks of 64: the key
//     of hit h = q*Lq + i is its row a(q,e,i) (none for masked tokens).  The
//     lanes of a chunk holding the same row find each other through an LDS
//     word per row that each ORs its lane bit into (OR is order-free, so the
//     word is exact; long documents use ballots over the key bits instead); a
//     hit's rank is the number of such lanes below it, and the last of them
//     adds their count to the wave's row histogram.  Key, rank and count are
//     kept per hit;
//  2. row starts (exclusive scan over rows of all waves' counts) and per-wave
//     cursors; the document's hits are cut into gs_split equal shares at row
//     boundaries and this workgroup owns the rows [c0, c1) of share s; its
//     rows without hits are written as zeros now;
//  3. placement in chunk order: slot = the wave's cursor of the row + rank,
//     so the sorted list is ordered by row, then by h (a stable sort);
//  4. the sorted hits of [c0, c1) are cut into NG equal ranges, one per lane
//     group of CPR lanes (16 bytes of the row each).  A group takes R hits per
//     round: lane u of the group reads sorted entry u and prepares its Q-row
//     offset, weight g[q, e] and row; the group's lanes gather the R rows with
//     those values broadcast from lane u and add g * Q[h] in sorted order.  A
//     round inside one row (the usual case) needs no row checks; a row that
//     ends is stored whole, kept as the range's head (begun in an earlier
//     range) or, at the range's end, left as a partial in LDS, and after a
//     barrier the group where that row starts adds the later groups' partials
//     in group order.
// The sums depend only on the sorted list, so results are bitwise stable.
// ---------------------------------------------------------------------------
constexpr int kGsWaves = kGsThreads / kWave;

// h / Lq for 0 <= h < 2^16 and 1 <= Lq <= 2^16, with magic = ceil(2^32 / Lq):
// the rounding error of the product is below 2^-16 <= 1/Lq, so the floor is exact.
__device__ __forceinline__ int div_lq(int h, uint64_t magic) {
  return (int)(((uint64_t)(uint32_t)h * magic) >> 32);
}

// rank of this lane among the valid lanes holding the same key, and their
// count (keys of `bits` bits; every lane takes part in the ballots)
__device__ __forceinline__ void match_rank(int key, bool valid, int bits, uint64_t below,
                                           int& rank, int& count) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool bit = valid && ((key >> b) & 1);
    const uint64_t bb = __ballot(bit);
    same &= bit ? bb : ~bb;
  }
  rank = __popcll(same & below);
  count = __popcll(same);
}

template <Elem E, int DIM>
__global__ __launch_bounds__(kGsThreads) void gradd_sorted_kernel(BwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int EPC = ElemInfo<E>::kPerChunk;
  constexpr int CPR = G::kCPR;
  constexpr int NG = kGsThreads / CPR;     // lane groups
  constexpr int R = CPR < 16 ? CPR : 16;   // hits per round (one prepared per lane)
  constexpr int F4 = DIM / 4;              // float4 per gradient row
  constexpr uint32_t kNoKey = 0xffffu;
  extern __shared__ __attribute__((aligned(16))) char gs_smem[];
  uint32_t* sorted = reinterpret_cast<uint32_t*>(gs_smem + a.gs_off_sorted);  // [H]: row << 16 | h
  int32_t* start = reinterpret_cast<int32_t*>(gs_smem + a.gs_off_start);      // [Ld + 1]
  float* gl = reinterpret_cast<float*>(gs_smem + a.gs_off_gl);                // [Nq]
  uint32_t* keys = reinterpret_cast<uint32_t*>(gs_smem + a.gs_off_keys);      // [H] (steps 1-3)
  int32_t* hist = reinterpret_cast<int32_t*>(gs_smem + a.gs_off_hist);        // [SW][Ld] (steps 1-3)
  unsigned long long* masks =
      reinterpret_cast<unsigned long long*>(gs_smem + a.gs_off_masks);        // [SW][Ld] (step 1)
  float* part = reinterpret_cast<float*>(gs_smem + a.gs_off_part);            // [NG][2][DIM] (step 4)
  __shared__ int wtot[kGsWaves];
  __shared__ int cut[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = a.gs_split;
  const int64_t e = blockIdx.x / split;
  const int s = (int)(blockIdx.x - e * split);
  const int Ld = (int)a.Ld, H = (int)a.H, Lq = (int)a.Lq, Nq = (int)a.Nq;
  const int SW = a.gs_sw;
  const int Hw = ((H + SW * 64 - 1) / (SW * 64)) * 64;   // hits per sorting wave
  const int64_t Nd = a.n_docs;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const bool use_masks = a.gs_masks != 0;
  float* __restrict__ gD_doc = a.gD + e * (int64_t)Ld * DIM;

  // The grad_Q slice partials (written by the previous launch on this
  // stream) are added here, spread over the grid, instead of in a kernel of
  // their own.
  if (a.gq_red) {
    const int64_t n4 = a.Nq * a.Lq * (DIM / 4);
    for (int64_t k = (int64_t)blockIdx.x * kGsThreads + tid; k < n4;
         k += (int64_t)gridDim.x * kGsThreads)
      gradq_reduce_at(reinterpret_cast<const float4*>(a.gq_part), a.gq_slices, n4,
                      reinterpret_cast<float4*>(a.gQ), k);
  }

  // 0. clear the histograms and match words; this document's upstream grads
  for (int k = tid; k < SW * Ld; k += kGsThreads) {
    hist[k] = 0;
    if (use_masks) masks[k] = 0ull;
  }
  for (int q = tid; q < Nq; q += kGsThreads) gl[q] = a.g[(int64_t)q * Nd + e];
  __syncthreads();

  // 1. keys, ranks inside each 64-hit chunk, per-wave row histograms
  const int h0 = min(wave * Hw, H), h1 = min(h0 + Hw, H);
  if (wave < SW) {
    int* hw = hist + wave * Ld;
    unsigned long long* mw = masks + wave * Ld;
    constexpr int UL = 8;                        // chunks whose argmax loads are in flight together
    // argmax[(q * Nd + e) * Lq + i] for hit h = q * Lq + i is
    // argmax[q * (Nd - 1) * Lq + e * Lq + h]
    const uint64_t q_stride = (uint64_t)(Nd - 1) * (uint64_t)Lq;
    const int32_t* am_e = a.argmax + e * (int64_t)Lq;
    for (int hb = h0; hb < h1; hb += 64 * UL) {
      // every load is issued before any is used: hits past the range read
      // the range's last hit and are dropped afterwards
      int raw[UL];
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        const int hc = min(hb + 64 * u + lane, h1 - 1);
        const uint32_t q = (uint32_t)div_lq(hc, a.lq_magic);
        raw[u] = am_e[q * q_stride + (uint32_t)hc];
      }
      int jj[UL];
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        const bool ok = hb + 64 * u + lane < h1 && raw[u] >= 0 && raw[u] < Ld;
        jj[u] = ok ? raw[u] : (int)kNoKey;
      }
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        if (hb + 64 * u >= h1) break;            // wave-uniform
        const int h = hb + 64 * u + lane;
        const bool v = jj[u] != (int)kNoKey;
        int rank, count;
        if (use_masks) {
          // OR, read back and clear: LDS runs one wave's operations in order
          if (v) atomicOr(&mw[jj[u]], 1ull << lane);
          const uint64_t same = v ? (uint64_t)mw[jj[u]] : 0ull;
          if (v) mw[jj[u]] = 0ull;
          rank = __popcll(same & below);
          count = __popcll(same);
        } else {
          match_rank(jj[u], v, a.key_bits, below, rank, count);
        }
        if (h < h1) keys[h] = (uint32_t)jj[u] | ((uint32_t)rank << 16) | ((uint32_t)count << 22);
        if (v && rank == count - 1) atomicAdd(&hw[jj[u]], count);
      }
    }
  }
  __syncthreads();

  // 2. row starts and per-wave cursors (each thread scans a segment of rows)
  {
    const int seg = (Ld + kGsThreads - 1) / kGsThreads;
    const int lo = min(tid * seg, Ld), hi = min(lo + seg, Ld);
    int local = 0;
    for (int j = lo; j < hi; ++j)
      for (int w = 0; w < SW; ++w) local += hist[w * Ld + j];
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
    for (int j = lo; j < hi; ++j) {
      start[j] = base;
      for (int w = 0; w < SW; ++w) {
        const int cnt = hist[w * Ld + j];
        hist[w * Ld + j] = base;
        base += cnt;
      }
    }
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kGsWaves; ++w) tot += wtot[w];
      start[Ld] = tot;
    }
  }
  __syncthreads();
  if (tid < 2) {
    // share boundary k: the first row whose hits reach past position Hv*k/split
    const int k = s + tid;
    const int Hv = start[Ld];
    int r = (k == 0) ? 0 : Ld;
    if (k > 0 && k < split) {
      const int P = (int)((int64_t)Hv * k / split);
      int lo = 0, hi = Ld;                       // smallest r with start[r+1] > P
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (start[mid + 1] > P) hi = mid; else lo = mid + 1;
      }
      r = lo;
    }
    cut[tid] = r;
  }
  __syncthreads();
  const int c0 = cut[0], c1 = cut[1];

  // rows of [c0, c1) without hits are zeros: stored now, so that the writes
  // drain while the hits are placed and summed
  {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = tid; k < (c1 - c0) * F4; k += kGsThreads) {
      const int row = c0 + k / F4, f = k - (k / F4) * F4;
      if (start[row] == start[row + 1])
        *reinterpret_cast<float4*>(gD_doc + (int64_t)row * DIM + 4 * f) = z;
    }
  }

  // 3. placement in chunk order: slot = the wave's cursor of the row + rank;
  // the sorted list is ordered by row, then by h.  Only rows in [c0, c1).
  if (wave < SW) {
    int* cur = hist + wave * Ld;
    for (int hb = h0; hb < h1; hb += 64) {
      const int h = hb + lane;
      const uint32_t kr = h < h1 ? keys[h] : kNoKey;
      const int j = (int)(kr & 0xffffu);
      const int rank = (int)((kr >> 16) & 0x3fu), count = (int)(kr >> 22);
      const bool mine = j != (int)kNoKey && j >= c0 && j < c1;
      const int pos = mine ? cur[j] : 0;
      __asm__ volatile("" ::: "memory");
      if (mine) sorted[pos + rank] = ((uint32_t)j << 16) | (uint32_t)h;
      if (mine && rank == count - 1) cur[j] = pos + count;
    }
  }
  __syncthreads();

  // 4. row sums over equal shares of the sorted hits
  const int H0 = start[c0], H1 = start[c1];
  const int grp = tid / CPR, c = tid - grp * CPR;
  const int base_lane = lane - c;
  auto range_lo = [&](int k) { return H0 + (int)((int64_t)(H1 - H0) * k / NG); };
  const int lo = range_lo(grp), hi = range_lo(grp + 1);
  const __amdgpu_buffer_rsrc_t qrs = buf_rsrc(a.Q, (uint32_t)((int64_t)Nq * Lq * G::kRowBytes));
  const uint32_t my_chunk = (uint32_t)c * 16u;
  float acc[EPC];
#pragma unroll
  for (int k = 0; k < EPC; ++k) acc[k] = 0.0f;
  int cur_row = lo < hi ? (int)(sorted[lo] >> 16) : -1;
  bool in_head = lo < hi && start[cur_row] < lo;   // first row began in an earlier range
  auto store_row = [&](int row, const float (&v)[EPC]) {
    float* out = gD_doc + (int64_t)row * DIM + c * EPC;
#pragma unroll
    for (int k = 0; k < EPC; k += 4)
      *reinterpret_cast<float4*>(out + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  };
  // the head (a row begun in an earlier range) goes to this group's first
  // LDS partial slot, for the group where the row starts
  auto write_head = [&](const float (&v)[EPC]) {
    float* out = part + (grp * 2) * DIM + c * EPC;
#pragma unroll
    for (int k = 0; k < EPC; k += 4)
      *reinterpret_cast<float4*>(out + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
  };
  // a row ended inside the range: the head is kept, any other row is whole
  // and stored.  Only stores here: the caller clears acc with selects, so the
  // accumulators keep one register assignment on both sides of the branch.
  auto end_row = [&]() {
    if (in_head) {
      write_head(acc);
      in_head = false;
    } else {
      store_row(cur_row, acc);
    }
  };
  for (int p = lo; p < hi; p += R) {
    // lane u (< R) of the group prepares sorted entry p + u; entries past the
    // range repeat the range's last entry with weight 0 (same row, no effect)
    int row_c = 0;
    uint32_t qoff_c = 0;
    float g_c = 0.0f;
    if (c < R) {
      const int pe = min(p + c, hi - 1);
      const uint32_t ent = sorted[pe];
      const int h = (int)(ent & 0xffffu);
      row_c = (int)(ent >> 16);
      qoff_c = (uint32_t)h * (uint32_t)G::kRowBytes;
      g_c = p + c < hi ? gl[div_lq(h, a.lq_magic)] : 0.0f;
    }
    u32x4 ch[R];
    static_for<R>([&](auto u) {
      const uint32_t o = (uint32_t)grp_bcast<CPR, u>((int)qoff_c, base_lane);
      ch[u] = ld_buf_16(qrs, o + my_chunk);
    });
    // weights and rows are broadcast where they are used (few live registers)
    auto add = [&](const u32x4& x, float w) {
      float f[EPC];
      chunk_to_float<E>(x, f);
#pragma unroll
      for (int k = 0; k < EPC; ++k) acc[k] = __builtin_fmaf(w, f[k], acc[k]);
    };
    // entries are sorted by row: the round stays in the current row iff its
    // last entry does
    if (__ballot(grp_bcast<CPR, R - 1>(row_c, base_lane) != cur_row) == 0ull) {
      static_for<R>([&](auto u) { add(ch[u], grp_bcast_f<CPR, u>(g_c, base_lane)); });
    } else {
      static_for<R>([&](auto u) {
        const int r = grp_bcast<CPR, u>(row_c, base_lane);
        const bool chg = r != cur_row;
        if (chg) end_row();
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[k] = chg ? 0.0f : acc[k];
        cur_row = chg ? r : cur_row;
        add(ch[u], grp_bcast_f<CPR, u>(g_c, base_lane));
      });
    }
  }
  // the range's last row: whole, a tail (continues in later ranges), or the
  // head itself (the range lies inside one row)
  int tail_row = -1;
  if (cur_row >= 0) {
    if (in_head) {
      write_head(acc);
    } else if (start[cur_row + 1] > hi) {
      tail_row = cur_row;
      float* out = part + (grp * 2 + 1) * DIM + c * EPC;
#pragma unroll
      for (int k = 0; k < EPC; k += 4)
        *reinterpret_cast<float4*>(out + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
    } else {
      store_row(cur_row, acc);
    }
  }
  __syncthreads();

  // rows cut by range boundaries: the group where the row starts finishes it
  if (tail_row >= 0) {
    const float* own = part + (grp * 2 + 1) * DIM + c * EPC;
#pragma unroll
    for (int k = 0; k < EPC; ++k) acc[k] = own[k];
    const int rt = start[tail_row + 1];
    for (int k2 = grp + 1; k2 < NG; ++k2) {
      const int lo2 = range_lo(k2), hi2 = range_lo(k2 + 1);
      if (lo2 >= rt) break;
      if (lo2 < hi2) {
        const float* pp = part + (k2 * 2) * DIM + c * EPC;
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[k] += pp[k];
      }
    }
    store_row(tail_row, acc);
  }
}

// ---------------------------------------------------------------------------
// grad_D, pairwise / kd: four waves per document, each over a contiguous
// quarter of its rows.  A document has only Lq hits (one per query token), so
// its gradient is Ld rows of which at most Lq are non-zero: a wave streams its
// rows in order with non-temporal stores and, for a row some hit points at,
// adds g * Q[h] over those hits in increasing h (their lanes, found by
// ballot) before storing it.
// ---------------------------------------------------------------------------

template <Elem E>
__device__ __forceinline__ void load4_as_float(const char* p, float (&f)[4]);
template <> __device__ __forceinline__ void load4_as_float<Elem::BF16>(const char* p, float (&f)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xffff0000u);
}
template <> __device__ __forceinline__ void load4_as_float<Elem::F16>(const char* p, float (&f)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  f[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x & 0xffffu));
  f[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.x >> 16));
  f[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y & 0xffffu));
  f[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.y >> 16));
}
template <> __device__ __forceinline__ void load4_as_float<Elem::F32>(const char* p, float (&f)[4]) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  f[0] = w.x;
  f[1] = w.y;
  f[2] = w.z;
  f[3] = w.w;
}


template <Elem E, int DIM>
__device__ __forceinline__ void gradd_pairs_body(const BwdArgs& a, int64_t block) {
  constexpr int F4 = DIM / 4;                 // float4 per gradient row
  constexpr int RPI = F4 >= 64 ? 1 : 64 / F4; // rows per wave store
  constexpr int NH = kPairsMaxLq / 64;        // hit registers per lane
  constexpr int ES = ElemInfo<E>::kBytes;
  constexpr int kNone = 0x7fffffff;
  static_assert(F4 <= 64, "one gradient row per wave store at most");
  const int lane = threadIdx.x & 63;
  // gd_parts waves per document, each streaming a contiguous share of its
  // rows (whole stores of RPI rows), so enough stores are in flight
  const int parts = a.gd_parts;
  const int64_t wv = block * 4 + (threadIdx.x >> 6);
  const int64_t e = wv / parts;
  const int part = (int)(wv - e * parts);
  if (e >= a.n_docs) return;
  const int Lq = (int)a.Lq, Ld = (int)a.Ld;
  const int n_st = (Ld + RPI - 1) / RPI;                  // stores per document
  const int r_begin = (int)((int64_t)n_st * part / parts) * RPI;
  const int r_end = min((int)((int64_t)n_st * (part + 1) / parts) * RPI, Ld);
  const int nh = (Lq + 63) / 64;
  // the hits' rows are requested first; the zero stream below does not
  // wait for them
  int key[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    const int h = 64 * k + lane;
    key[k] = (k < nh && h < Lq) ? a.argmax[e * a.Lq + h] : -1;
  }
  const float g = a.g[e];
  const int sub = lane / F4, f = lane - (lane / F4) * F4;
  float* out = a.gD + e * (int64_t)Ld * DIM;
  // 1. every row of the share as zeros; a row with hits is stored again
  // below, by the same lanes, so its sum lands after its zeros
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r0 = r_begin; r0 < r_end; r0 += RPI) {
    const int row = r0 + sub;
    if (sub < RPI && row < r_end) *reinterpret_cast<f32x4*>(out + (int64_t)row * DIM + 4 * f) = z;
  }
  // 2. the rows of the share that have hits, in increasing row order, each
  // the sum of g * Q[h] over its hits in increasing h
#pragma unroll
  for (int k = 0; k < NH; ++k) key[k] = (key[k] >= r_begin && key[k] < r_end) ? key[k] : kNone;
  const char* Qb = (const char*)a.Q;
  const int64_t qbase = (e / a.K) * a.Lq;     // first Q row of this document's query
  while (true) {
    int m = key[0];
#pragma unroll
    for (int k = 1; k < NH; ++k) m = min(m, key[k]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o));
    const int row = __builtin_amdgcn_readfirstlane(m);
    if (row == kNone) break;
    const bool mine = sub == (row - r_begin) % RPI;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      if (k >= nh) break;
      uint64_t mk = __ballot(key[k] == row);
      while (mk != 0ull) {
        const int b = __ffsll((unsigned long long)mk) - 1;
        mk &= mk - 1;
        if (mine) {
          float x[4];
          load4_as_float<E>(Qb + (qbase + 64 * k + b) * (int64_t)(DIM * ES) + 4 * f * ES, x);
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(g, x[t], v[t]);
        }
      }
      key[k] = key[k] == row ? kNone : key[k];
    }
    if (mine) {
      const f32x4 w = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(out + (int64_t)row * DIM + 4 * f) = w;
    }
  }
}

template <Elem E, int DIM>
__global__ __launch_bounds__(256) void gradd_pairs_kernel(BwdArgs a) {
  gradd_pairs_body<E, DIM>(a, blockIdx.x);
}

// Both gradients of the pairwise / kd layouts in one launch: the first
// n_gq blocks gather grad_Q (bound by the latency of row gathers from HBM),
// the rest stream grad_D (bound by HBM writes), so the gathers run under
// the write stream instead of before it.  The two parts share no data.
constexpr int kGqFusedRows = 4;
template <Elem E, int DIM>
__global__ __launch_bounds__(256) void grads_pairs_kernel(BwdArgs a, int64_t n_gq, int64_t n_iblk) {
  const int64_t b = blockIdx.x;
  if (b < n_gq) {
    const int64_t q = b / n_iblk;
    // fewer rows in flight than gradq_kernel: the registers stay within what
    // the grad_D part needs for its full occupancy, and the gathers' latency
    // is hidden by the write stream anyway
    gradq_body<E, DIM, kGqFusedRows>(a, q, b - q * n_iblk);
  } else {
    gradd_pairs_body<E, DIM>(a, b - n_gq);
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
static hipError_t launch_gradq(const BwdArgs& a, hipStream_t s) {
  using G = Geo<E, DIM>;
  constexpr int CPR = G::kCPR;
  constexpr int TPB = 256 / CPR;
  if (a.gq_ap) {
    const int64_t n_tok = a.Nq * a.Lq;
    hipLaunchKernelGGL((gradq_ap_kernel<E, DIM>), dim3((unsigned)(a.gq_slices * cdiv(n_tok, TPB))),
                       dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.gq_slices == 1 || a.gq_red) return e;
    const int64_t n4 = n_tok * DIM / 4;
    hipLaunchKernelGGL(gradq_reduce_kernel, dim3((unsigned)cdiv(n4, 256)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(a.gq_part), a.gq_slices, n4,
                       reinterpret_cast<float4*>(a.gQ));
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gradq_kernel<E, DIM>), dim3((unsigned)a.Nq, (unsigned)cdiv(a.Lq, TPB)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <Elem E, int DIM>
static hipError_t launch_gradd(const BwdArgs& a, int mode, size_t gs_lds, hipStream_t s) {
  using G = Geo<E, DIM>;
  constexpr int CPR = G::kCPR;
  hipError_t e;
  if (mode == kGdSorted) {
    if (gs_lds > 65536) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gradd_sorted_kernel<E, DIM>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)gs_lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gradd_sorted_kernel<E, DIM>), dim3((unsigned)(a.n_docs * a.gs_split)),
                       dim3(kGsThreads), gs_lds, s, a);
    return hipGetLastError();
  }
  if (mode == kGdPairs) {
    hipLaunchKernelGGL((gradd_pairs_kernel<E, DIM>),
                       dim3((unsigned)cdiv(a.n_docs * a.gd_parts, 4)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // documents are sorted and summed in batches that fit the workspace
  for (int64_t e0 = 0; e0 < a.n_docs; e0 += a.nb) {
    BwdArgs b = a;
    b.e0 = e0;
    b.nb = a.n_docs - e0 < a.nb ? a.n_docs - e0 : a.nb;
    if (b.Ld <= kSortWavesMaxLd) {
      const size_t lds = (size_t)(4 * b.Ld + 4) * sizeof(int);
      hipLaunchKernelGGL(gradd_sort_waves_kernel, dim3((unsigned)b.nb), dim3(256), lds, s, b);
    } else {
      const size_t lds = (size_t)((b.Ld < kSortWin ? b.Ld : kSortWin) + 4) * sizeof(int);
      hipLaunchKernelGGL(gradd_sort_kernel, dim3((unsigned)b.nb), dim3(256), lds, s, b);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // rows per group: one while groups are scarce; up to 16 (one offsets
    // load) when the output is large and mostly empty rows
    const int64_t n_rows = b.nb * b.Ld;
    int rpg = (int)cdiv(n_rows, 256 * 256);
    const int max_rpg = CPR < 16 ? CPR : 16;
    rpg = rpg < 1 ? 1 : (rpg > max_rpg ? max_rpg : rpg);
    const int64_t gpb = 256 / CPR;
    hipLaunchKernelGGL((gradd_rows_group_kernel<E, DIM>),
                       dim3((unsigned)cdiv(cdiv(n_rows, rpg), gpb)), dim3(256), 0, s, b, rpg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <Elem E, int DIM>
static hipError_t launch_grads(const BwdPlan& p, const BwdArgs& a, bool want_q, bool want_d,
                               hipStream_t s) {
  if (want_q && want_d && !a.gq_ap && p.gd_mode == kGdPairs) {
    using G = Geo<E, DIM>;
    constexpr int TPB = 256 / G::kCPR;
    const int64_t n_iblk = cdiv(a.Lq, TPB);
    const int64_t n_gq = a.Nq * n_iblk;
    const int64_t n_gd = cdiv(a.n_docs * a.gd_parts, 4);
    hipLaunchKernelGGL((grads_pairs_kernel<E, DIM>), dim3((unsigned)(n_gq + n_gd)), dim3(256), 0,
                       s, a, n_gq, n_iblk);
    return hipGetLastError();
  }
  if (want_q) {
    hipError_t e = launch_gradq<E, DIM>(a, s);
    if (e != hipSuccess) return e;
  }
  if (want_d) return launch_gradd<E, DIM>(a, p.gd_mode, p.gs_lds, s);
  return hipSuccess;
}

template <Elem E>
static hipError_t grads_dim(const BwdPlan& p, const BwdArgs& a, bool wq, bool wd, hipStream_t s) {
  switch (p.fwd.dim) {
    case 64: return launch_grads<E, 64>(p, a, wq, wd, s);
    case 128: return launch_grads<E, 128>(p, a, wq, wd, s);
    case 256: return launch_grads<E, 256>(p, a, wq, wd, s);
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
  a.gq_part = reinterpret_cast<float*>(ws + p.off_gq_part);
  a.layout = f.layout;
  a.key_bits = p.key_bits;
  a.gq_slices = p.gq_slices;
  a.gq_ap = p.gq_ap ? 1 : 0;
  a.gs_sw = p.gs_sw;
  a.gs_split = p.gs_split;
  a.gd_parts = p.gd_parts;
  a.gs_off_sorted = p.gs_off_sorted;
  a.gs_off_start = p.gs_off_start;
  a.gs_off_gl = p.gs_off_gl;
  a.gs_off_keys = p.gs_off_keys;
  a.gs_off_hist = p.gs_off_hist;
  a.gs_off_masks = p.gs_off_masks;
  a.gs_off_part = p.gs_off_part;
  a.gs_masks = p.gs_masks;
  a.lq_magic = ((uint64_t(1) << 32) + (uint64_t)f.Lq - 1) / (uint64_t)f.Lq;
  a.Nq = f.Nq;
  a.Lq = f.Lq;
  a.n_docs = f.n_docs;
  a.Ld = f.Ld;
  a.K = f.K;
  a.H = p.H;
  a.e0 = 0;
  a.nb = p.sort_batch;
  const bool wq = grad_Q != nullptr, wd = grad_D != nullptr;
  // with both gradients, the sorted grad_D kernel (launched after grad_Q on
  // the same stream) adds the grad_Q slice partials
  a.gq_red = (wq && wd && p.gq_ap && p.gq_slices > 1 && p.gd_mode == kGdSorted) ? 1 : 0;
  switch (f.elem) {
    case 0: return grads_dim<Elem::F16>(p, a, wq, wd, s);
    case 1: return grads_dim<Elem::BF16>(p, a, wq, wd, s);
    default: return grads_dim<Elem::F32>(p, a, wq, wd, s);
  }
}

}  // namespace lik
