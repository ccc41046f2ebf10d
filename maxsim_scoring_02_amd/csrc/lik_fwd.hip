// Forward kernels of the gfx950 MaxSim scorer.
//
//   mask_prep       bool document mask -> 32-bit tile words + tile count
//   allpairs_fwd    MFMA S^T tiles for every (query, doc), doc tiles shared
//                   through LDS by the workgroup's waves (compute-bound shapes)
//   pairs_fwd       pairwise / kd: one wave streams its own document
//                   (bandwidth-bound shapes), split along Ld when pairs are few
//   combine_fwd     exact merge of per-chunk (max, argmax) partials, then the
//                   sum over valid query tokens
//
// Semantics (README "Late Interaction Kernels", "Scoring interface"): masked
// document tokens never win the max, masked query tokens leave the sum, a
// document with no valid token scores -1e9, scores are float32.  The running
// max is kept in registers and the similarity grid is never stored (social
// thread, post (4/N)).
#include <hip/hip_runtime.h>

#include "lik_device.h"
#include "lik_kernels.h"
#include "lik_plan.h"

namespace lik {

constexpr float kEmptyDocScore = -1e9f;

// ---------------------------------------------------------------------------
// mask prep: one wave per document
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_prep_kernel(const uint8_t* __restrict__ d_mask,
                                                        int64_t n_docs, int64_t Ld, int64_t nwords,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t d = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (d >= n_docs) return;
  const uint8_t* m = d_mask + d * Ld;
  int last = -1;
  for (int64_t w = lane; w < nwords; w += 64) {
    uint32_t word = 0;
    const int64_t j0 = w * 32;
    for (int b = 0; b < 32; ++b) {
      const int64_t j = j0 + b;
      if (j < Ld && m[j]) word |= 1u << b;
    }
    bits[d * nwords + w] = word;
    if (word) last = (int)w;
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) last = max(last, __shfl_xor(last, k));
  if (lane == 0) ntiles[d] = last + 1;
}

// scores when no query has tokens (Lq == 0): 0, or -1e9 for empty documents
__global__ void fill_scores_no_query_tokens_kernel(float* scores, int64_t n_out, int64_t n_docs,
                                                   int layout, int64_t Ld,
                                                   const int32_t* ntiles) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n_out) return;
  int64_t e = layout == kAllPairs ? k % n_docs : k;
  bool empty = ntiles ? ntiles[e] == 0 : Ld == 0;
  scores[k] = empty ? kEmptyDocScore : 0.0f;
}

// ---------------------------------------------------------------------------
// slot mapping (all-pairs): wave gw, slot L -> (query q, token i)
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool slot_qi(int64_t gw, int L, int SPW, int64_t qpw, int64_t Nq,
                                        int64_t Lq, int64_t& q, int64_t& i) {
  if (qpw > 0) {
    int64_t k = L / Lq;
    i = L - k * Lq;
    q = gw * qpw + k;
    return k < qpw && q < Nq;
  }
  int64_t s = gw * SPW + L;
  q = s / Lq;
  i = s - q * Lq;
  return q < Nq;
}

template <Elem E, int DIM, int NB, int KS = Geo<E, DIM>::kKSteps>
__device__ __forceinline__ void load_bfrags(u32x4 (&bf)[NB][KS], const char* Qb,
                                            const int64_t (&row_of_slot)[NB], const bool (&ok)[NB],
                                            int h) {
  using G = Geo<E, DIM>;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const char* rowp = Qb + row_of_slot[b] * G::kRowBytes;
#pragma unroll
    for (int m = 0; m < G::kKSteps; ++m) {
      u32x4 z = {0u, 0u, 0u, 0u};
      bf[b][m] = ok[b] ? ld_global_16(rowp + (2 * m + h) * 16) : z;
    }
  }
}

// ---------------------------------------------------------------------------
// all-pairs forward
// ---------------------------------------------------------------------------
constexpr int kApNW = 8;                       // waves per workgroup
constexpr int kApThreads = kApNW * kWave;

template <Elem E, int DIM, int NB>
__global__ __launch_bounds__(kApThreads) void allpairs_fwd_kernel(FwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int SPW = 32 * NB;
  constexpr int kLoads = (G::kTileChunks + kApThreads - 1) / kApThreads;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;

  // Workgroups are dispatched round-robin over the 8 XCDs; give every doc
  // group a fixed XCD so its tiles stay in that XCD's L2 across slot blocks.
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid & 7, kx = bid >> 3;
  const int64_t g = xcd + 8 * (kx % a.gpx);
  const int64_t sb = kx / a.gpx;
  if (g >= a.n_groups || sb >= a.n_sb) return;
  const int64_t gw = sb * kApNW + wave;
  const bool active = gw < a.n_cg;

  // query fragments of this wave's slots (B operand), kept for all units
  u32x4 bf[NB][G::kKSteps];
  {
    int64_t rows[NB];
    bool ok[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int64_t q, i;
      ok[b] = active && slot_qi(gw, b * 32 + r, SPW, a.qpw, a.Nq, a.Lq, q, i);
      rows[b] = ok[b] ? q * a.Lq + i : 0;
    }
    load_bfrags<E, DIM, NB>(bf, (const char*)a.Q, rows, ok, h);
  }

  const int64_t n_units = a.n_docs * a.nchunks;
  const int64_t u_begin = g * a.upw;
  const int64_t u_end = min(u_begin + a.upw, n_units);
  const int64_t ntiles_full = a.ntiles_max;

  auto unit_tiles = [&](int64_t u, int64_t& d, int64_t& t0, int64_t& t1) {
    d = u / a.nchunks;
    const int64_t c = u - d * a.nchunks;
    const int64_t nt = a.ntiles ? (int64_t)a.ntiles[d] : ntiles_full;
    t0 = c * a.tpc;
    t1 = min(t0 + a.tpc, nt);
    if (t1 < t0) t1 = t0;
  };

  // load cursor: the next tile to bring into LDS, in consumption order
  int64_t pu = u_begin, pd = 0, pt = 0, pt1 = 0;
  bool have = false;
  for (; pu < u_end; ++pu) {
    unit_tiles(pu, pd, pt, pt1);
    if (pt < pt1) { have = true; break; }
  }
  auto advance = [&]() {
    ++pt;
    if (pt < pt1) return true;
    for (++pu; pu < u_end; ++pu) {
      unit_tiles(pu, pd, pt, pt1);
      if (pt < pt1) return true;
    }
    return false;
  };

  u32x4 pre[kLoads];
  auto gload = [&]() {
    const char* base = (const char*)a.D + (pd * a.Ld + pt * kTile) * (int64_t)G::kRowBytes;
    const int64_t rows_left = a.Ld - pt * kTile;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = tid + k * kApThreads;
      const int row = idx / G::kCPR;
      u32x4 z = {0u, 0u, 0u, 0u};
      pre[k] = (idx < G::kTileChunks && row < rows_left) ? ld_global_16(base + idx * 16) : z;
    }
  };
  auto lstore = [&](char* buf) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = tid + k * kApThreads;
      const int row = idx / G::kCPR, c = idx - row * G::kCPR;
      if (idx < G::kTileChunks) st_lds_16(buf, lds_off<E, DIM>(row, c), pre[k]);
    }
  };

  int cur = 0;
  if (have) {
    gload();
    lstore(lds);
  }
  __syncthreads();

  for (int64_t u = u_begin; u < u_end; ++u) {
    int64_t d, t0, t1;
    unit_tiles(u, d, t0, t1);
    const uint32_t* bits_d = a.bits ? a.bits + d * a.nwords : nullptr;
    BlockState st[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) state_init(st[b], (int)t0);

    for (int64_t t = t0; t < t1; ++t) {
      const bool nxt = advance();
      if (nxt) gload();
      if (active) {
        const uint32_t word = tile_word(bits_d, (int)t, a.Ld);
        if (word != 0u) {
          f32x16 acc[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
          const char* buf = lds + cur * G::kTileBytes;
#pragma unroll
          for (int m = 0; m < G::kKSteps; ++m) {
            const u32x4 av = ld_lds_16(buf, lds_off<E, DIM>(r, 2 * m + h));
#pragma unroll
            for (int b = 0; b < NB; ++b) mfma_chunk<E>(acc[b], av, bf[b][m]);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) state_update(st[b], acc[b], word, (int)t, h);
        }
      }
      if (nxt) lstore(lds + (cur ^ 1) * G::kTileBytes);
      __syncthreads();
      cur ^= 1;
    }

    if (!active) continue;
    // flush this unit
    float M[NB];
    int J[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) state_resolve(st[b], h, M[b], J[b]);
    float Mv;
    int Jv;
    combine_halves<NB>(M, J, lane, Mv, Jv);
    const int L = NB == 2 ? lane : (lane & 31);
    const bool writer = NB == 2 || lane < 32;
    if (a.partial) {
      const int64_t c = u - d * a.nchunks;
      const bool any = t1 > t0;
      if (writer) {
        const int64_t idx = ((c * a.n_docs + d) * a.n_cg + gw) * SPW + L;
        a.part_M[idx] = any ? Mv : -__builtin_inff();
        a.part_J[idx] = any ? Jv : -1;
      }
    } else {
      const bool empty = t1 == 0;   // single chunk: t1 is the doc's tile count
      int64_t q, i;
      const bool ok = slot_qi(gw, L, SPW, a.qpw, a.Nq, a.Lq, q, i);
      const bool tok = ok && (!a.q_mask || a.q_mask[q * a.Lq + i]);
      const float v = tok ? Mv : 0.0f;
      const int seg_start = (int)((L / a.Lq) * a.Lq);
      const float s = segmented_scan<SPW>(v, L, seg_start);
      if (ok && writer) {
        const int64_t pair = q * a.n_docs + d;
        if (i == a.Lq - 1) a.scores[pair] = empty ? kEmptyDocScore : s;
        if (a.argmax) a.argmax[pair * a.Lq + i] = (tok && !empty) ? Jv : -1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// pairwise / kd forward: one wave per (pair, slot group, chunk)
// ---------------------------------------------------------------------------
// Waves per workgroup: 4, or fewer when their private tiles would pass 64 KB.
template <Elem E, int DIM>
constexpr int pr_waves() {
  return Geo<E, DIM>::kTileBytes * 4 <= 65536 ? 4 : (Geo<E, DIM>::kTileBytes * 2 <= 65536 ? 2 : 1);
}

template <Elem E, int DIM, int NB>
__global__ __launch_bounds__(256) void pairs_fwd_kernel(FwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int kPrWaves = pr_waves<E, DIM>();
  constexpr int SPW = 32 * NB;
  constexpr int kLoads = G::kTileChunks / kWave;
  static_assert(G::kTileChunks % kWave == 0, "tile chunks must split over a wave");
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int64_t unit = (int64_t)blockIdx.x * kPrWaves + wave;
  if (unit >= a.n_units) return;          // whole wave leaves; no workgroup barriers below
  char* buf = lds + wave * G::kTileBytes;

  const int64_t c = unit % a.nchunks;
  const int64_t rest = unit / a.nchunks;
  const int64_t cg = rest % a.n_cg;
  const int64_t p = rest / a.n_cg;        // pair index = document index
  const int64_t q = p / a.K;

  u32x4 bf[NB][G::kKSteps];
  {
    int64_t rows[NB];
    bool ok[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t i = cg * SPW + b * 32 + r;
      ok[b] = i < a.Lq;
      rows[b] = ok[b] ? q * a.Lq + i : 0;
    }
    load_bfrags<E, DIM, NB>(bf, (const char*)a.Q, rows, ok, h);
  }

  const int64_t nt = a.ntiles ? (int64_t)a.ntiles[p] : a.ntiles_max;
  const int64_t t0 = c * a.tpc;
  int64_t t1 = min(t0 + a.tpc, nt);
  if (t1 < t0) t1 = t0;
  const uint32_t* bits_d = a.bits ? a.bits + p * a.nwords : nullptr;
  const char* docp = (const char*)a.D + p * a.Ld * (int64_t)G::kRowBytes;

  u32x4 pre[kLoads];
  auto gload = [&](int64_t t) {
    const char* base = docp + t * kTile * (int64_t)G::kRowBytes;
    const int64_t rows_left = a.Ld - t * kTile;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = lane + k * kWave;
      const int row = idx / G::kCPR;
      u32x4 z = {0u, 0u, 0u, 0u};
      pre[k] = row < rows_left ? ld_global_16(base + idx * 16) : z;
    }
  };

  BlockState st[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) state_init(st[b], (int)t0);

  if (t0 < t1) gload(t0);
  for (int64_t t = t0; t < t1; ++t) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = lane + k * kWave;
      const int row = idx / G::kCPR, cc = idx - row * G::kCPR;
      st_lds_16(buf, lds_off<E, DIM>(row, cc), pre[k]);
    }
    if (t + 1 < t1) gload(t + 1);
    __asm__ volatile("" ::: "memory");
    const uint32_t word = tile_word(bits_d, (int)t, a.Ld);
    if (word != 0u) {
      f32x16 acc[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
#pragma unroll
      for (int m = 0; m < G::kKSteps; ++m) {
        const u32x4 av = ld_lds_16(buf, lds_off<E, DIM>(r, 2 * m + h));
#pragma unroll
        for (int b = 0; b < NB; ++b) mfma_chunk<E>(acc[b], av, bf[b][m]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) state_update(st[b], acc[b], word, (int)t, h);
    }
    __asm__ volatile("" ::: "memory");
  }

  float M[NB];
  int J[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) state_resolve(st[b], h, M[b], J[b]);
  float Mv;
  int Jv;
  combine_halves<NB>(M, J, lane, Mv, Jv);
  const int L = NB == 2 ? lane : (lane & 31);
  const bool writer = NB == 2 || lane < 32;
  if (a.partial) {
    if (writer) {
      const bool any = t1 > t0;
      const int64_t idx = ((c * a.n_docs + p) * a.n_cg + cg) * SPW + L;
      a.part_M[idx] = any ? Mv : -__builtin_inff();
      a.part_J[idx] = any ? Jv : -1;
    }
  } else {
    const bool empty = t1 == 0;
    const int64_t i = L;
    const bool ok = writer && i < a.Lq;
    const bool tok = ok && (!a.q_mask || a.q_mask[q * a.Lq + i]);
    const float s = wave_sum(tok ? Mv : 0.0f);
    if (lane == 0) a.scores[p] = empty ? kEmptyDocScore : s;
    if (ok && a.argmax) a.argmax[p * a.Lq + i] = (tok && !empty) ? Jv : -1;
  }
}

// ---------------------------------------------------------------------------
// combine: one wave per output (query, doc) / pair
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_fwd_kernel(FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t out = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool ap = a.layout == kAllPairs;
  const int64_t n_out = ap ? a.Nq * a.n_docs : a.n_docs;
  if (out >= n_out) return;
  const int64_t q = ap ? out / a.n_docs : out / a.K;
  const int64_t e = ap ? out - q * a.n_docs : out;
  const bool empty = a.ntiles ? a.ntiles[e] == 0 : a.Ld == 0;
  float total = 0.0f;
  for (int64_t i0 = 0; i0 < a.Lq; i0 += 64) {
    const int64_t i = i0 + lane;
    const bool ok = i < a.Lq;
    int64_t cg, slot;
    if (ap) {
      if (a.qpw > 0) {
        cg = q / a.qpw;
        slot = (q - cg * a.qpw) * a.Lq + i;
      } else {
        const int64_t s = q * a.Lq + i;
        cg = s / a.SPW;
        slot = s - cg * a.SPW;
      }
    } else {
      cg = i / a.SPW;
      slot = i - cg * a.SPW;
    }
    float M = -__builtin_inff();
    int J = -1;
    if (ok) {
      for (int64_t c = 0; c < a.nchunks; ++c) {
        const int64_t idx = ((c * a.n_docs + e) * a.n_cg + cg) * a.SPW + slot;
        merge_mj(M, J, a.part_M[idx], a.part_J[idx]);
      }
    }
    const bool tok = ok && (!a.q_mask || a.q_mask[q * a.Lq + i]);
    total += wave_sum(tok ? M : 0.0f);
    if (ok && a.argmax) a.argmax[out * a.Lq + i] = (tok && !empty) ? J : -1;
  }
  if (lane == 0) a.scores[out] = empty ? kEmptyDocScore : total;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <Elem E, int DIM, int NB>
static hipError_t launch_main(const FwdPlan& p, const FwdArgs& a, hipStream_t s) {
  using G = Geo<E, DIM>;
  if (p.layout == kAllPairs) {
    const int64_t grid = 8 * p.gpx * p.n_sb;
    hipLaunchKernelGGL((allpairs_fwd_kernel<E, DIM, NB>), dim3((unsigned)grid), dim3(kApThreads),
                       2 * G::kTileBytes, s, a);
  } else {
    constexpr int W = pr_waves<E, DIM>();
    const int64_t grid = cdiv(p.n_units, W);
    hipLaunchKernelGGL((pairs_fwd_kernel<E, DIM, NB>), dim3((unsigned)grid), dim3(W * kWave),
                       W * G::kTileBytes, s, a);
  }
  return hipGetLastError();
}

template <Elem E>
static hipError_t dispatch_dim(const FwdPlan& p, const FwdArgs& a, hipStream_t s) {
  switch (p.dim) {
    case 64: return p.NB == 2 ? launch_main<E, 64, 2>(p, a, s) : launch_main<E, 64, 1>(p, a, s);
    case 128: return p.NB == 2 ? launch_main<E, 128, 2>(p, a, s) : launch_main<E, 128, 1>(p, a, s);
    case 256: return launch_main<E, 256, 1>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

bool fwd_dim_supported(int64_t dim) { return dim == 64 || dim == 128 || dim == 256; }

hipError_t run_forward(const FwdPlan& p, const void* Q, const void* D, const uint8_t* q_mask,
                       const uint8_t* d_mask, float* scores, int32_t* argmax, char* ws,
                       hipStream_t s) {
  FwdArgs a{};
  a.Q = Q;
  a.D = D;
  a.q_mask = q_mask;
  a.scores = scores;
  a.argmax = argmax;
  a.layout = p.layout;
  a.Nq = p.Nq;
  a.Lq = p.Lq;
  a.n_docs = p.n_docs;
  a.Ld = p.Ld;
  a.K = p.K;
  a.SPW = p.SPW;
  a.nwords = p.nwords;
  a.ntiles_max = p.ntiles_max;
  a.qpw = p.qpw;
  a.n_cg = p.n_cg;
  a.n_sb = p.n_sb;
  a.nchunks = p.nchunks;
  a.tpc = p.tpc;
  a.upw = p.upw;
  a.n_groups = p.n_groups;
  a.gpx = p.gpx;
  a.n_units = p.n_units;
  a.partial = p.partial ? 1 : 0;
  if (p.has_dmask && p.n_docs > 0) {
    a.bits = reinterpret_cast<uint32_t*>(ws + p.off_bits);
    a.ntiles = reinterpret_cast<int32_t*>(ws + p.off_tiles);
    if (p.nwords > 0) {
      hipLaunchKernelGGL(mask_prep_kernel, dim3((unsigned)cdiv(p.n_docs, 4)), dim3(256), 0, s,
                         d_mask, p.n_docs, p.Ld, p.nwords, a.bits, a.ntiles);
    } else {
      // Ld == 0: every document is empty
      hipLaunchKernelGGL(mask_prep_kernel, dim3((unsigned)cdiv(p.n_docs, 4)), dim3(256), 0, s,
                         d_mask, p.n_docs, p.Ld, p.nwords, a.bits, a.ntiles);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Nq == 0 || p.n_docs == 0) return hipSuccess;
  if (p.Lq == 0) {
    const int64_t n_out = p.layout == kAllPairs ? p.Nq * p.n_docs : p.n_docs;
    hipLaunchKernelGGL(fill_scores_no_query_tokens_kernel, dim3((unsigned)cdiv(n_out, 256)),
                       dim3(256), 0, s, scores, n_out, p.n_docs, p.layout, p.Ld, a.ntiles);
    return hipGetLastError();
  }
  if (p.partial) {
    a.part_M = reinterpret_cast<float*>(ws + p.off_partM);
    a.part_J = reinterpret_cast<int32_t*>(ws + p.off_partJ);
  }
  hipError_t e;
  switch (p.elem) {
    case 0: e = dispatch_dim<Elem::F16>(p, a, s); break;
    case 1: e = dispatch_dim<Elem::BF16>(p, a, s); break;
    default: e = dispatch_dim<Elem::F32>(p, a, s); break;
  }
  if (e != hipSuccess) return e;
  if (p.partial) {
    const int64_t n_out = p.layout == kAllPairs ? p.Nq * p.n_docs : p.n_docs;
    hipLaunchKernelGGL(combine_fwd_kernel, dim3((unsigned)cdiv(n_out, 4)), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace lik
