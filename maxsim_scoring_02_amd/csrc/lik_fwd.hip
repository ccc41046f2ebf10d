// Forward kernels of the gfx950 MaxSim scorer.
//
//   mask_prep       bool document mask -> 32-bit tile words + tile count
//   compact_prep    bool query mask -> list of the valid query tokens (all-pairs)
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "lik_device.h"
#include "lik_kernels.h"
#include "lik_plan.h"

namespace lik {

constexpr float kEmptyDocScore = -1e9f;

// ---------------------------------------------------------------------------
// mask prep: one workgroup of 4 waves per document; every load is issued
// before any is used, blocks past the document's end form no words (a short
// document's waves skip most of their unrolled pass: long documents
// 7.2 -> 5.9 us), and the last valid word is the maximum over the waves.
// - byte path: a wave reads 64 consecutive mask bytes (one per lane) and a
//   ballot of "byte != 0" is directly two tile words;
// - dword path (mask rows 4-byte aligned): a lane reads 4 bytes, forms their
//   4 validity bits, and the 8 lanes of a 32-byte word OR their nibbles
//   together by three lane exchanges, so a wave load covers 8 words.
// ---------------------------------------------------------------------------
template <bool DW>
__global__ __launch_bounds__(256) void mask_prep_kernel(const uint8_t* __restrict__ d_mask,
                                                        int64_t n_docs, int64_t Ld, int64_t nwords,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ ntiles) {
  constexpr int U = 16, NWV = 4;
  constexpr int kBlk = DW ? 256 : 64;             // bytes per wave load
  __shared__ int s_last[NWV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t d = blockIdx.x;
  if (d >= n_docs) return;                        // whole workgroup
  const uint8_t* m = d_mask + d * Ld;
  uint32_t* out = bits + d * nwords;
  const int64_t nblk = (Ld + kBlk - 1) / kBlk;
  int last = -1;                                  // last word with a valid row
  for (int64_t b0 = wave; b0 < nblk; b0 += (int64_t)NWV * U) {
    if constexpr (DW) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = (b0 + (int64_t)u * NWV) * kBlk + 4 * lane;   // Ld % 4 == 0: j + 3 < Ld or j >= Ld
        v[u] = j < Ld ? *reinterpret_cast<const uint32_t*>(m + j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + (int64_t)u * NWV >= nblk) break;   // uniform: past the document
        uint32_t nib = ((v[u] & 0xffu) != 0) | (((v[u] >> 8) & 0xffu) != 0) << 1 |
                       (((v[u] >> 16) & 0xffu) != 0) << 2 | ((v[u] >> 24) != 0) << 3;
        uint32_t word = nib << (4 * (lane & 7));
        word |= __shfl_xor(word, 1);
        word |= __shfl_xor(word, 2);
        word |= __shfl_xor(word, 4);
        const int64_t w = (b0 + (int64_t)u * NWV) * 8 + (lane >> 3);
        if ((lane & 7) == 0 && w < nwords) out[w] = word;
        if (word != 0u && w < nwords) last = max(last, (int)w);
      }
    } else {
      uint8_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = (b0 + (int64_t)u * NWV) * kBlk + lane;
        v[u] = j < Ld ? m[j] : (uint8_t)0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + (int64_t)u * NWV >= nblk) break;   // uniform: past the document
        const uint64_t bal = __ballot(v[u] != 0);
        const int64_t w = 2 * (b0 + (int64_t)u * NWV);
        if (lane < 2 && w + lane < nwords) out[w + lane] = (uint32_t)(bal >> (32 * lane));
        if (bal >> 32) last = max(last, (int)w + 1);
        else if (bal) last = max(last, (int)w);
      }
    }
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) last = max(last, __shfl_xor(last, k));
  if (lane == 0) s_last[wave] = last;
  __syncthreads();
  if (threadIdx.x == 0) {
    int l = s_last[0];
#pragma unroll
    for (int k = 1; k < NWV; ++k) l = max(l, s_last[k]);
    ntiles[d] = l + 1;
  }
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
// compacted query tokens: the valid (q, i) of the query mask in (q, i) order.
// One workgroup walks the mask in blocks of 1024 x 16 tokens: a thread counts
// its 16, a scan over the workgroup gives its first slot, and the running
// total carries from block to block.  n <= 2^22.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void compact_prep_kernel(const uint8_t* __restrict__ q_mask,
                                                            int64_t n, int32_t* __restrict__ tok,
                                                            int32_t* __restrict__ cnt) {
  constexpr int T = 1024, PER = 16, NWV = T / 64;
  __shared__ int wsum[NWV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int64_t base = 0; base < n; base += (int64_t)T * PER) {
    const int64_t t0 = base + (int64_t)tid * PER;
    uint8_t m[PER];
    int c = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int64_t j = t0 + k;
      m[k] = j < n ? q_mask[j] : (uint8_t)0;
      c += m[k] != 0;
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const int x = wsum[w];
      if (w < wave) wbase += x;
      total += x;
    }
    int slot = carry + wbase + incl - c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (t0 + k < n && m[k]) tok[slot++] = (int32_t)(t0 + k);
    }
    carry += total;
    __syncthreads();                       // wsum is rewritten by the next block
  }
  if (tid == 0) *cnt = carry;
}

// ---------------------------------------------------------------------------
// slot mapping (all-pairs): wave gw, slot L -> (query q, token i)
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool slot_qi(int gw, int L, int SPW, int qpw, int Nq, int Lq, int& q,
                                        int& i) {
  // 32-bit throughout: the plan keeps Nq * Lq below 2^31
  if (qpw > 0) {
    const int k = (int)((uint32_t)L / (uint32_t)Lq);
    i = L - k * Lq;
    q = gw * qpw + k;
    return k < qpw && q < Nq;
  }
  const uint32_t s = (uint32_t)gw * (uint32_t)SPW + (uint32_t)L;
  q = (int)(s / (uint32_t)Lq);
  i = (int)(s - (uint32_t)q * (uint32_t)Lq);
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

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// ---------------------------------------------------------------------------
// all-pairs forward
//
// A workgroup of 4 waves holds 4 x SPW query-token slots in registers (the
// MFMA B operand) and streams document super-tiles of 2 x 32 rows through a
// three-stage LDS ring (padded rows), one barrier per super-tile.  Tiles are
// copied global -> LDS by buffer loads whose descriptor covers only the
// unit's remaining rows, so rows past the end read as zeros (and are masked)
// with no per-lane bounds arithmetic.  Two workgroups fit on a CU, so the
// waves sharing a SIMD run in independent phases and one's MFMAs overlap the
// other's VALU work.
// ---------------------------------------------------------------------------
constexpr int kApNW = 4;                       // waves per workgroup
constexpr int kApThreads = kApNW * kWave;
constexpr int kSub = 2;                        // tiles per super-tile

// LDS buffers of super-tiles: three (loads run two super-tiles ahead) when
// they fit in 64 KB, else two (one ahead)
template <Elem E, int DIM>
constexpr int ap_stages() {
  return 3 * kSub * Pad<E, DIM>::kTileBytes <= 65536 ? 3 : 2;
}

template <Elem E, int DIM>
constexpr int ap_lds_bytes() {
  return ap_stages<E, DIM>() * kSub * Pad<E, DIM>::kTileBytes;
}

// The tile's A chunks are read from LDS up to kWin ahead of the MFMAs that
// use them, so an MFMA waits on LDS latency only at the start of a tile.  The
// order (kWin reads, then per chunk its MFMAs and the next read) is pinned for
// the scheduler, which otherwise interleaves one read per MFMA pair.
// acc = C + A * B over one tile, C the tile's initial value (zero with
// ZERO, else c0: -inf in the rows a mask removes).  The first K-step reads C
// and writes acc, so the initial value is never copied into the accumulators.
// With split float32 rows (BF16S, K-steps 0..n-1 the high parts and n..2n-1
// the low parts of both operands) the A chunk of a high K-step m meets the
// query's high and low parts (B m and m + n) and that of a low K-step meets
// the query's high part (B m - n): the three products hi*hi, hi*lo, lo*hi.
template <Elem E, int KS>
__device__ __forceinline__ constexpr int split_b(int m) {
  return (E == Elem::BF16S && m >= KS / 2) ? m - KS / 2 : m;
}
template <Elem E, int KS>
__device__ __forceinline__ constexpr bool split_second(int m) {
  return E == Elem::BF16S && m < KS / 2;
}

template <Elem E, int DIM, int NB, bool ZERO>
__device__ __forceinline__ void mfma_tile_c(f32x16 (&acc)[NB], const char* buf,
                                            const u32x4 (&bf)[NB][Geo<E, DIM>::kKSteps],
                                            int a_off, const f32x16& c0) {
  using G = Geo<E, DIM>;
  constexpr int KS = G::kKSteps;
  constexpr int kWin = KS < 8 ? KS : 8;
  constexpr int kMfmaPerChunk = NB * (E == Elem::F32 ? 4 : 1);
  u32x4 av[KS];
#pragma unroll
  for (int m = 0; m < kWin; ++m) av[m] = ld_lds_16(buf, a_off + m * 32);
  __builtin_amdgcn_sched_group_barrier(0x100, kWin, 0);
#pragma unroll
  for (int m = 0; m < KS; ++m) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (m == 0) acc[b] = mfma_first<E, ZERO>(av[0], bf[b][0], c0);
      else mfma_chunk<E>(acc[b], av[m], bf[b][split_b<E, KS>(m)]);
    }
    if (split_second<E, KS>(m)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) mfma_chunk<E>(acc[b], av[m], bf[b][m + KS / 2]);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kMfmaPerChunk, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerChunk, 0);
    }
    if (m + kWin < KS) {
      av[m + kWin] = ld_lds_16(buf, a_off + (m + kWin) * 32);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
}

// Both tiles of a super-tile at once: four independent accumulator chains
// (two tiles x NB), so an MFMA never waits on the result of the one issued
// just before it.  Chunks of both tiles are read kWin steps ahead.  With
// ZERO the chains start from zero, else from ca / cb (the masked-row init).
template <Elem E, int DIM, int NB, bool ZERO>
__device__ __forceinline__ void mfma_pair_run(f32x16 (&xa)[NB], f32x16 (&xb)[NB],
                                              const char* bufa, const char* bufb,
                                              const u32x4 (&bf)[NB][Geo<E, DIM>::kKSteps],
                                              int a_off, const f32x16& ca, const f32x16& cb,
                                              bool twob = true) {
  using G = Geo<E, DIM>;
  constexpr int KS = G::kKSteps;
  constexpr int kWin = E == Elem::F32 ? 2 : (KS < 4 ? KS : 4);
  constexpr int kMfmaPerChunk = NB * (E == Elem::F32 ? 4 : 1);
  u32x4 aa[KS], ab[KS];
#pragma unroll
  for (int m = 0; m < kWin; ++m) {
    aa[m] = ld_lds_16(bufa, a_off + m * 32);
    ab[m] = ld_lds_16(bufb, a_off + m * 32);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kWin, 0);
#pragma unroll
  for (int m = 0; m < KS; ++m) {
    constexpr int kH = KS / 2;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (m == 0) xa[b] = mfma_first<E, ZERO>(aa[0], bf[b][0], ca);
      else mfma_chunk<E>(xa[b], aa[m], bf[b][split_b<E, KS>(m)]);
    }
    // without a second tile, its chains stop after the first K-step: every
    // row started at -inf (cb), so -inf is already their final value
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (m == 0) xb[b] = mfma_first<E, ZERO>(ab[0], bf[b][0], cb);
      else if (twob) mfma_chunk<E>(xb[b], ab[m], bf[b][split_b<E, KS>(m)]);
    }
    if (split_second<E, KS>(m)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) mfma_chunk<E>(xa[b], aa[m], bf[b][m + kH]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (twob) mfma_chunk<E>(xb[b], ab[m], bf[b][m + kH]);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kMfmaPerChunk, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kMfmaPerChunk, 0);
    }
    if (m + kWin < KS) {
      aa[m + kWin] = ld_lds_16(bufa, a_off + (m + kWin) * 32);
      ab[m + kWin] = ld_lds_16(bufb, a_off + (m + kWin) * 32);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
}

// Workgroup barrier that waits for this wave's LDS operations only:
// __syncthreads() would also wait for every global load still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt left at their maxima
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// KEEP: the caller wants the argmax; without it only running maxima are kept.
template <Elem E, int DIM, int NB, bool MASK, bool KEEP>
__global__ __launch_bounds__(kApThreads) void allpairs_fwd_kernel(FwdArgs a) {
  using G = Geo<E, DIM>;
  using PD = Pad<E, DIM>;
  constexpr int SPW = 32 * NB;
  constexpr int kSTRows = kSub * kTile;
  constexpr int kSTBytes = kSub * PD::kTileBytes;
  constexpr int kSTChunks = kSTRows * G::kCPR;
  static_assert(kSTChunks % kApThreads == 0 && kApThreads % G::kCPR == 0,
                "super-tile chunks must split evenly over the workgroup");
  constexpr uint32_t kFull = 0xffffffffu;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform: held in a scalar register, the load issue and
  // its LDS addresses below need no per-lane branches or lane reads
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;

  // Workgroups are dispatched round-robin over the 8 XCDs.  Every doc group
  // has a fixed XCD, and its slot blocks are dispatched back to back there,
  // so they run together and each tile comes from HBM once, then from L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, kx = bid >> 3;
  const int n_sb = (int)a.n_sb;
  const int g = xcd + 8 * (kx / n_sb);
  const int sb = kx - (kx / n_sb) * n_sb;
  if (g >= a.n_groups || sb >= a.n_sb) return;
  const int gw = sb * kApNW + wave;
  // compacted query tokens: slots past the last valid token hold nothing, and
  // a workgroup with none of its slots below it leaves at once
  const int64_t n_valid = a.compact ? (int64_t)*a.tok_cnt : 0;
  if (a.compact && (int64_t)sb * kApNW * SPW >= n_valid) return;
  const bool active = gw < a.n_cg && (!a.compact || (int64_t)gw * SPW < n_valid);
  // slot L of this wave -> (query q, token i); false for an empty slot
  const int Lq32 = (int)a.Lq;
  auto slot_of = [&](int L, int64_t& q, int64_t& i) -> bool {
    if (a.compact) {
      const int64_t s2 = (int64_t)gw * SPW + L;
      if (!active || s2 >= n_valid) {
        q = i = 0;
        return false;
      }
      const uint32_t t = (uint32_t)a.tok[s2];
      const uint32_t q32 = t / (uint32_t)Lq32;
      q = q32;
      i = t - q32 * (uint32_t)Lq32;
      return true;
    }
    int q32 = 0, i32 = 0;
    const bool ok = active && slot_qi(gw, L, SPW, (int)a.qpw, (int)a.Nq, Lq32, q32, i32);
    q = q32;
    i = i32;
    return ok;
  };

  // ---- the workgroup's units (document, chunk) and their super-tiles ----
  // A flat schedule in LDS: entry e = one super-tile (or one empty unit),
  // with its tile index, validity words and start/end-of-unit flags, so the
  // hot loop below holds no cursor arithmetic and no global index loads.
  const int nchunks = (int)a.nchunks, tpc = (int)a.tpc;
  const int64_t n_units = a.n_docs * a.nchunks;
  // Units are numbered chunk-major (u = chunk * n_docs + document) and dealt
  // out strided (unit k of this workgroup is g + k * n_groups), so every
  // workgroup gets about as many units of each chunk index: a mix of long,
  // partial and empty chunks.
  // unit numbers stay below 2^31 (documents < 2^23, chunks < 256): 32-bit
  // arithmetic, and no division at all when documents are not split
  const uint32_t n_grp = (uint32_t)a.n_groups, n_docs32 = (uint32_t)a.n_docs;
  const int n_my = (int)min((uint32_t)a.upw, ((uint32_t)n_units - g + n_grp - 1) / n_grp);
  auto unit_dc = [&](int k, int& d, int& c) {
    const uint32_t u = (uint32_t)g + (uint32_t)k * n_grp;
    if (nchunks == 1) {
      c = 0;
      d = (int)u;
    } else {
      const uint32_t cu = u / n_docs32;
      c = (int)cu;
      d = (int)(u - cu * n_docs32);
    }
  };
  const int Ld = (int)a.Ld;
  // Super-tiles are copied global -> LDS directly (no registers): the padded
  // super-tile is kBlocks blocks of 1 KB, block q written by wave q % 4 as its
  // (q / 4)-th load, lane l landing at byte 16 l of the block.  A lane's
  // global offset inside the super-tile follows from that LDS position;
  // lanes that land on row padding re-read offset 0.  One buffer descriptor
  // per super-tile bounds the reads to the unit's rows (the rest read zero).
  constexpr int kBlocks = kSTBytes / 1024;
  static_assert(kSTBytes % 1024 == 0, "padded super-tile must be whole 1 KB blocks");
  constexpr int kMyLoads = (kBlocks + kApNW - 1) / kApNW;   // per wave, at most
  const int my_loads = (kBlocks - wave + kApNW - 1) / kApNW;
  uint32_t voff[kMyLoads];
#pragma unroll
  for (int i = 0; i < kMyLoads; ++i) {
    const int q = i * kApNW + wave;
    const int bt = q * 1024 + lane * 16;                // byte in the padded super-tile
    const int tile = bt / PD::kTileBytes, o = bt - tile * PD::kTileBytes;
    const int row = o / PD::kStride, cb = o - row * PD::kStride;
    voff[i] = (q < kBlocks && cb < G::kRowBytes)
                  ? (uint32_t)((tile * kTile + row) * G::kRowBytes + cb)
                  : 0u;
  }
  auto gload = [&](int meta, int unit, int stage) {
    const int d = unit >> 8, c = unit & 0xff;
    const int t = meta & 0xffffff;
    const int t1 = min(c * tpc + tpc, (int)a.ntiles_max);
    const char* base = (const char*)a.D + ((int64_t)d * Ld + (int64_t)t * kTile) * G::kRowBytes;
    const int rows = min(t1 * kTile, Ld) - t * kTile;
    const int nbytes = ((meta >> 27) & 1) ? min(rows, kSTRows) * G::kRowBytes : 0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
    char* dst = lds + stage * kSTBytes;
#pragma unroll
    for (int i = 0; i < kMyLoads; ++i) {
      if (i < my_loads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + (i * kApNW + wave) * 1024), 16,
            (int)voff[i], 0, 0, 0);
    }
  };
  constexpr int NST = ap_stages<E, DIM>();
  // wait until this wave's loads for the next entry are in LDS (with three
  // stages the loads issued this step, for the entry after, stay in flight)
  auto wait_stage = [&]() {
    if constexpr (NST == 3) {
      if (my_loads == kMyLoads) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMyLoads));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMyLoads - 1));
      }
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  };


  // Before the set-up: the first unit's first super-tile (the schedule's
  // first entry is always that tile; when the unit turns out empty the
  // entry does not read it) and this wave's query fragments, so their
  // latency overlaps the set-up's reads.
  {
    int d0, c0;
    unit_dc(0, d0, c0);
    gload((c0 * tpc) | (1 << 27), (d0 << 8) | c0, 0);
  }
  u32x4 bf[NB][G::kKSteps];
  {
    int64_t rows[NB];
    bool ok[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int64_t q, i;
      ok[b] = slot_of(b * 32 + r, q, i);
      rows[b] = ok[b] ? q * a.Lq + i : 0;
    }
    load_bfrags<E, DIM, NB>(bf, (const char*)a.Q, rows, ok, h);
  }
  __shared__ int s_meta[kApMaxST];     // t | two << 24 | start << 25 | end << 26 | has << 27
  __shared__ int s_unit[kApMaxST];     // d << 8 | chunk
  __shared__ uint32_t s_w0[kApMaxST], s_w1[kApMaxST];
  __shared__ int s_uoff[kApMaxDocs + 1], s_ut0[kApMaxDocs], s_ut1[kApMaxDocs];

  // Set-up in two rounds of global reads.  First the units' tile counts and
  // every validity word of the schedule, all issued before any is used
  // (words past a document's last valid tile are zero, so they are read
  // before the counts are known, bounded only by the document's word count).
  // Schedule entry x = (unit x / 32, pair j = x % 32), kSetupIt per thread.
  int unit_nt = 0;                      // wave 0, lane k: tile count of unit k's document
  if (MASK && wave == 0 && lane < n_my) {
    int d, c;
    unit_dc(lane, d, c);
    unit_nt = a.ntiles[d];
  }
  constexpr int kSetupIt = kApMaxDocs * 32 / kApThreads;
  uint32_t pw0[kSetupIt], pw1[kSetupIt];
#pragma unroll
  for (int it = 0; it < kSetupIt; ++it) {
    const int x = tid + it * kApThreads;
    pw0[it] = pw1[it] = 0u;
    if (MASK && x < n_my * 32) {
      const int k = x >> 5, j = x & 31;
      int d, c;
      unit_dc(k, d, c);
      const int t = c * tpc + 2 * j;
      const uint32_t* wd = a.bits + (int64_t)d * a.nwords;
      if (2 * j < tpc && t < a.nwords) pw0[it] = wd[t];
      if (2 * j + 1 < tpc && t + 1 < a.nwords) pw1[it] = wd[t + 1];
    }
  }

  if (wave == 0) {
    int nst = 0, t0 = 0, t1 = 0;
    if (lane < n_my) {
      int d, c;
      unit_dc(lane, d, c);
      const int nt = MASK ? unit_nt : (int)a.ntiles_max;
      t0 = c * tpc;
      t1 = min(t0 + tpc, nt);
      if (t1 < t0) t1 = t0;
      nst = t1 > t0 ? (t1 - t0 + 1) / 2 : 1;    // an empty unit still flushes
    }
    int incl = nst;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane < n_my) {
      s_uoff[lane] = incl - nst;
      s_ut0[lane] = t0;
      s_ut1[lane] = t1;
    }
    if (lane == 63) s_uoff[kApMaxDocs] = incl;
  }
  lds_barrier();
#pragma unroll
  for (int it = 0; it < kSetupIt; ++it) {
    const int x = tid + it * kApThreads;
    if (x < n_my * 32) {
      const int k = x >> 5, j = x & 31;
      const int t0 = s_ut0[k], t1 = s_ut1[k], off = s_uoff[k];
      const int nst = t1 > t0 ? (t1 - t0 + 1) / 2 : 1;
      if (j < nst) {
        int d, c;
        unit_dc(k, d, c);
        const int t = t0 + 2 * j;
        const bool has = t < t1, two = t + 1 < t1;
        uint32_t w0 = 0u, w1 = 0u;
        if (has) w0 = MASK ? pw0[it] : tile_word(nullptr, t, Ld);
        if (two) w1 = MASK ? pw1[it] : tile_word(nullptr, t + 1, Ld);
        s_w0[off + j] = w0;
        s_w1[off + j] = w1;
        s_meta[off + j] = t | ((int)two << 24) | ((int)(j == 0) << 25) | ((int)(j == nst - 1) << 26) |
                          ((int)has << 27);
        s_unit[off + j] = (d << 8) | c;
      }
    }
  }
  lds_barrier();
  const int S = s_uoff[kApMaxDocs];

  // prologue: the second entry's tiles go out now; the first entry's
  // tiles and the query fragments, requested before the set-up, are older
  // than them, so waiting with only the second entry's loads in flight
  // covers both
  const bool second = NST == 3 && S > 1;
  if (second)
    gload(__builtin_amdgcn_readfirstlane(s_meta[1]), __builtin_amdgcn_readfirstlane(s_unit[1]), 1);
  // this lane's output slot, fixed for the whole kernel
  const int L = NB == 2 ? lane : (lane & 31);
  const bool writer = NB == 2 || lane < 32;
  int64_t slot_q = 0, slot_i = 0;
  const bool slot_ok = slot_of(L, slot_q, slot_i);
  const bool slot_tok = slot_ok && (!a.q_mask || a.q_mask[slot_q * a.Lq + slot_i]);
  const int seg_start = a.qpw > 0 ? (int)(((uint32_t)L / (uint32_t)Lq32) * (uint32_t)Lq32) : 0;
  const bool seg_last = slot_ok && slot_i == a.Lq - 1;
  // queries of 32 tokens two to a wave: their sums are lane-aligned halves
  const bool fast_sum = a.qpw > 0 && a.Lq == 32;
  const int64_t score_base = slot_q * a.n_docs;
  if (second) {
    if (my_loads == kMyLoads) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMyLoads));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMyLoads - 1));
    }
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  lds_barrier();

  const int a_off = r * PD::kStride + h * 16;
  f32x16 Xa[NB], Xb[NB];
  // One tile's similarities; a tile that is not fully valid starts its
  // masked rows at -inf (-inf plus finite products stays -inf, so they
  // never win a max), a full tile starts from zero.
  auto tile_mfma = [&](f32x16 (&X)[NB], const char* tb, uint32_t w) {
    if (w == kFull) {
      mfma_tile_c<E, DIM, NB, true>(X, tb, bf, a_off, X[0]);
    } else {
      f32x16 c0;
      tile_init_uniform(c0, w);
      mfma_tile_c<E, DIM, NB, false>(X, tb, bf, a_off, c0);
    }
  };
  BlockState st[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    state_init(st[b], 0);
    Xa[b] = f32x16{};
    Xb[b] = f32x16{};
  }
  // a lone tile runs as a pair in these kernels (see the step below)
  constexpr bool kPairsOnly = KEEP && NB == 2;
  int cur = 0;                                   // stage of entry e
  // schedule words are read one step ahead, so no LDS round trip stands
  // between a step's start and its first load or MFMA
  const int last = S > 0 ? S - 1 : 0;
  int n_meta = s_meta[0], n_unit = s_unit[0];
  uint32_t n_w0 = s_w0[0], n_w1 = s_w1[0];
  int l_meta = s_meta[min(NST - 1, last)], l_unit = s_unit[min(NST - 1, last)];
  for (int e = 0; e < S; ++e) {
    const int meta = __builtin_amdgcn_readfirstlane(n_meta);
    const int unit = __builtin_amdgcn_readfirstlane(n_unit);
    const uint32_t word0 = __builtin_amdgcn_readfirstlane(n_w0);
    const uint32_t word1 = __builtin_amdgcn_readfirstlane(n_w1);
    const int ld_meta = __builtin_amdgcn_readfirstlane(l_meta);
    const int ld_unit = __builtin_amdgcn_readfirstlane(l_unit);
    {
      const int en = min(e + 1, last), el = min(e + NST, last);
      n_meta = s_meta[en];
      n_unit = s_unit[en];
      n_w0 = s_w0[en];
      n_w1 = s_w1[en];
      l_meta = s_meta[el];
      l_unit = s_unit[el];
    }
    const int t = meta & 0xffffff;
    const bool two = (meta >> 24) & 1, ustart = (meta >> 25) & 1, uend = (meta >> 26) & 1;
    const bool has = (meta >> 27) & 1;
    // entry e+NST-1 goes to the stage entry e-1 used (every wave passed the
    // barrier after reading it); past the end the last entry is reloaded
    const int st_ld = cur == 0 ? NST - 1 : cur - 1;
    gload(ld_meta, ld_unit, st_ld);
    if (ustart) {
#pragma unroll
      for (int b = 0; b < NB; ++b) state_begin(st[b], t);
    }
    const bool step = active && has;
    // The accumulators start each step undefined (an empty statement defines
    // them): a value written in one step is never carried into the next, so
    // the paths below merge without register copies.
#pragma unroll
    for (int b = 0; b < NB; ++b) asm volatile("" : "=v"(Xa[b]), "=v"(Xb[b]));
    if (step) {
      const char* buf = lds + cur * kSTBytes;
      // With the argmax kept and two column blocks, a single-tile step runs
      // as a pair whose second tile is wholly masked (word 0: every row
      // starts at -inf and never wins): with a single-tile path the two
      // paths' accumulators met in different registers and every pair step
      // paid 32 register copies (in-batch text 111.4 -> 109.7 us, pages
      // 94.7 -> 92.8).  The max-only fold and the one-block kernels have no
      // such join cost and keep the single-tile path (long documents: 703
      // against 730 us).
      const uint32_t w1 = two ? word1 : 0u;
      if (!kPairsOnly && !two) {
        tile_mfma(Xa, buf, word0);
      } else if (word0 == kFull && w1 == kFull) {
        mfma_pair_run<E, DIM, NB, true>(Xa, Xb, buf, buf + PD::kTileBytes, bf, a_off, Xa[0],
                                        Xb[0]);
      } else {
        f32x16 ca, cb;                 // a full word gives an all-zero init
        tile_init_uniform(ca, word0);
        tile_init_uniform(cb, w1);
        mfma_pair_run<E, DIM, NB, false>(Xa, Xb, buf, buf + PD::kTileBytes, bf, a_off, ca, cb,
                                         two);
      }
    }
    // One fold per step on every path, so the argmax state has a single
    // definition in the loop and stays in its registers.  A step without
    // tiles folds nothing; a single-tile step ignores Xb.
    if constexpr (KEEP) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        state_fold_step(st[b], Xa[b], Xb[b], t, step, kPairsOnly || two);
    } else if (step) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float tb = two ? max16_lean(Xb[b]) : -__builtin_inff();
        st[b].run_max = vmax3(st[b].run_max, max16_lean(Xa[b]), tb);
      }
    }
    // entry e+1's rows (loaded one step ago) must be in LDS before the barrier
    wait_stage();
    if (uend && active) {
      // flush this unit
      const int cd = unit >> 8, cc = unit & 0xff;
      float M[NB];
      int J[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (KEEP) {
          state_resolve(st[b], h, M[b], J[b]);
        } else {
          M[b] = st[b].run_max;
          J[b] = 0;
        }
      }
      float Mv;
      int Jv;
      combine_halves<NB>(M, J, lane, Mv, Jv);
      if (a.partial) {
        if (writer && slot_ok) {
          const int64_t idx = ((int64_t)cc * a.n_docs + cd) * a.n_cg * SPW + slot_q * a.Lq + slot_i;
          a.part_M[idx] = has ? Mv : -__builtin_inff();
          if constexpr (KEEP) a.part_J[idx] = has ? Jv : -1;
        }
      } else {
        const bool empty = !has;          // single chunk: no tile means no valid token
        const float v = slot_tok ? Mv : 0.0f;
        const float sc = fast_sum ? half_sum32(v) : segmented_scan<SPW>(v, L, seg_start);
        if (slot_ok && writer) {
          const int64_t pair = score_base + cd;
          if (seg_last) a.scores[pair] = empty ? kEmptyDocScore : sc;
          if constexpr (KEEP) a.argmax[pair * a.Lq + slot_i] = (slot_tok && !empty) ? Jv : -1;
        }
      }
    }
    // A plain s_barrier: the tile data needs no memory fence (each wave has
    // waited for its own loads above), and __syncthreads() would also wait
    // for the loads still in flight for the entry after next.
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    cur = cur == NST - 1 ? 0 : cur + 1;
  }
  // drain this wave's last (redundant) loads before the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---------------------------------------------------------------------------
// pairwise / kd forward: one wave per (pair, slot group, chunk)
// ---------------------------------------------------------------------------
// Waves per workgroup: 4, or fewer when their private tiles would pass 64 KB.
template <Elem E, int DIM>
constexpr int pr_waves() {
  return Geo<E, DIM>::kTileBytes * 4 <= 65536 ? 4 : (Geo<E, DIM>::kTileBytes * 2 <= 65536 ? 2 : 1);
}

template <Elem E, int DIM, int NB, bool MASK>
__global__ __launch_bounds__(256) void pairs_fwd_kernel(FwdArgs a) {
  using G = Geo<E, DIM>;
  constexpr int kPrWaves = pr_waves<E, DIM>();
  constexpr int SPW = 32 * NB;
  constexpr int kLoads = G::kTileChunks / kWave;
  static_assert(G::kTileChunks % kWave == 0, "tile chunks must split over a wave");
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
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

  const int64_t nt = MASK ? (int64_t)a.ntiles[p] : a.ntiles_max;
  const int64_t t0 = c * a.tpc;
  int64_t t1 = min(t0 + a.tpc, nt);
  if (t1 < t0) t1 = t0;
  const uint32_t* bits_d = MASK ? a.bits + p * a.nwords : nullptr;
  const char* docp = (const char*)a.D + p * a.Ld * (int64_t)G::kRowBytes;

  // rows past the document repeat its last row (masked before any max)
  u32x4 pre[kLoads];
  auto gload = [&](int64_t t) {
    const char* base = docp + t * kTile * (int64_t)G::kRowBytes;
    const int rows_left = (int)min((int64_t)kTile, a.Ld - t * kTile);   // >= 1
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = lane + k * kWave;
      const int row = idx / G::kCPR, c = idx - row * G::kCPR;
      const int rr = min(row, rows_left - 1);
      // each document byte is used once: non-temporal loads stream faster
      pre[k] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (rr * G::kCPR + c) * 16));
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
    // The word is read before the next prefetch (loads retire in order) and
    // the prefetch is unconditional (the last tile re-reads itself from L2),
    // so the wait before the MFMAs covers only the word.
    const uint32_t word = MASK ? bits_d[t] : tile_word(nullptr, (int)t, a.Ld);
    gload(min(t + 1, t1 - 1));
    __asm__ volatile("" ::: "memory");
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
// Offset of token i's chunk-0 partials for output (q, document or pair e),
// and whether the token has partials.  The all-pairs kernel writes them in
// token order (document e, then q * Lq + i), only for tokens with a slot:
// with compacted tokens the masked ones have none, and their (never
// written) entries are read and then dropped, so the mask load and the
// partial loads issue together.  The pairwise / kd kernel writes them by
// (pair e, slot group, slot).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t partial_base(const FwdArgs& a, bool ap, int64_t q, int64_t e,
                                                int64_t i, bool ok, bool& have) {
  if (ap) {
    have = ok && (!a.compact || a.q_mask[q * a.Lq + i] != 0);
    return e * a.n_cg * a.SPW + q * a.Lq + i;
  }
  have = ok;
  const int64_t cg = i / a.SPW;
  return (e * a.n_cg + cg) * a.SPW + (i - cg * a.SPW);
}

// ---------------------------------------------------------------------------
// Many chunks: one workgroup per output.  Its 256 threads are TG query-token
// lanes (32, or 64 when Lq > 32) x G = 256 / TG chunk groups; a thread merges
// the chunks c = g, g + G, ... with all of its loads issued before any is
// used (up to 16 at a time), then group 0 merges the G group results in
// group order and sums over the valid tokens.  Merge rule: the larger max
// wins, ties to the lower index, so the result does not depend on the order
// in which chunks are merged.
__global__ __launch_bounds__(256) void combine_fwd_kernel(FwdArgs a) {
  __shared__ float sM[8][64];
  __shared__ int sJ[8][64];
  const int tid = threadIdx.x;
  const int TG = a.Lq <= 32 ? 32 : 64;       // token lanes per group
  const int G = 256 / TG;                     // chunk groups
  const int tl = tid % TG, grp = tid / TG;
  const bool ap = a.layout == kAllPairs;
  const int64_t n_out = ap ? a.Nq * a.n_docs : a.n_docs;
  const int64_t stride = a.n_docs * a.n_cg * a.SPW;      // between chunks
  for (int64_t out = blockIdx.x; out < n_out; out += gridDim.x) {
    const int64_t q = ap ? out / a.n_docs : out / a.K;
    const int64_t e = ap ? out - q * a.n_docs : out;
    const bool empty = a.ntiles ? a.ntiles[e] == 0 : a.Ld == 0;
    float total = 0.0f;
    for (int64_t i0 = 0; i0 < a.Lq; i0 += TG) {
      const int64_t i = i0 + tl;
      const bool ok = i < a.Lq;
      bool have;                             // this token has partials
      const int64_t base = partial_base(a, ap, q, e, i, ok, have);
      float M = -__builtin_inff();
      int J = -1;
      if (ok) {
        constexpr int U = 16;
        for (int64_t c0 = grp; c0 < a.nchunks; c0 += (int64_t)G * U) {
          float mm[U];
          int jj[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)G * u;
            mm[u] = -__builtin_inff();
            jj[u] = -1;
            if (c < a.nchunks) {
              mm[u] = a.part_M[c * stride + base];
              // without an argmax output the indices are not kept
              jj[u] = a.argmax ? a.part_J[c * stride + base] : 0;
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) merge_mj(M, J, mm[u], jj[u]);
        }
        if (!have) {
          M = -__builtin_inff();
          J = -1;
        }
      }
      sM[grp][tl] = M;
      sJ[grp][tl] = J;
      __syncthreads();
      if (grp == 0) {
        for (int g2 = 1; g2 < G; ++g2) merge_mj(M, J, sM[g2][tl], sJ[g2][tl]);
        const bool tok = ok && (!a.q_mask || a.q_mask[q * a.Lq + i]);
        float v = tok ? M : 0.0f;
        for (int k = TG >> 1; k >= 1; k >>= 1) v += __shfl_xor(v, k, TG);
        total += v;
        if (ok && a.argmax) a.argmax[out * a.Lq + i] = (tok && !empty) ? J : -1;
      }
      __syncthreads();
    }
    if (tid == 0) a.scores[out] = empty ? kEmptyDocScore : total;
  }
}

// Few chunks: one wave per output (two, one per 32-lane half, when Lq <= 32).
// A lane owns a query token and merges its chunks in order with independent
// loads; no LDS and no barrier.  Same merge rule as above.
constexpr int kCombineWaveMaxChunks = 16;

__global__ __launch_bounds__(256) void combine_fwd_wave_kernel(FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const bool half = a.Lq <= 32;
  const int per_wave = half ? 2 : 1;
  const int gs = half ? 32 : 64;                 // lanes per output
  const int sub = half ? lane >> 5 : 0;
  const int li = half ? (lane & 31) : lane;
  const bool ap = a.layout == kAllPairs;
  const int64_t n_out = ap ? a.Nq * a.n_docs : a.n_docs;
  const int64_t n_waves = (n_out + per_wave - 1) / per_wave;
  const int64_t stride = a.n_docs * a.n_cg * a.SPW;      // between chunks
  for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < n_waves;
       w += (int64_t)gridDim.x * 4) {
    const int64_t out_raw = w * per_wave + sub;
    const bool out_ok = out_raw < n_out;
    const int64_t out = out_ok ? out_raw : n_out - 1;    // a clamped lane never stores
    const int64_t q = ap ? out / a.n_docs : out / a.K;
    const int64_t e = ap ? out - q * a.n_docs : out;
    const bool empty = a.ntiles ? a.ntiles[e] == 0 : a.Ld == 0;
    float total = 0.0f;
    for (int64_t i0 = 0; i0 < a.Lq; i0 += gs) {
      const int64_t i = i0 + li;
      const bool ok = i < a.Lq;
      bool have;                             // this token has partials
      const int64_t base = partial_base(a, ap, q, e, i, ok, have);
      float M = -__builtin_inff();
      int J = -1;
      if (ok) {
        constexpr int U = 4;
        for (int64_t c0 = 0; c0 < a.nchunks; c0 += U) {
          float mm[U];
          int jj[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u;
            mm[u] = -__builtin_inff();
            jj[u] = -1;
            if (c < a.nchunks) {
              mm[u] = a.part_M[c * stride + base];
              jj[u] = a.argmax ? a.part_J[c * stride + base] : 0;
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) merge_mj(M, J, mm[u], jj[u]);
        }
        if (!have) {
          M = -__builtin_inff();
          J = -1;
        }
      }
      const bool tok = ok && (!a.q_mask || a.q_mask[q * a.Lq + i]);
      float v = tok ? M : 0.0f;
      for (int k = gs >> 1; k >= 1; k >>= 1) v += __shfl_xor(v, k);
      total += v;
      if (out_ok && ok && a.argmax) a.argmax[out * a.Lq + i] = (tok && !empty) ? J : -1;
    }
    if (out_ok && li == 0) a.scores[out] = empty ? kEmptyDocScore : total;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// Launch `kernel` with FwdArgs a; with the profiling events set, they are
// attached to the launch itself (hipExtLaunchKernel), so they carry the
// kernel's own start and end rather than the stream's position around it.
template <class K>
static hipError_t launch_fwd(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                             const FwdArgs& a) {
  hipEvent_t ev0, ev1;
  profile_events(&ev0, &ev1);
  if (ev0 && ev1) {
    FwdArgs copy = a;
    void* args[] = {&copy};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, s,
                              ev0, ev1, 0);
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
  return hipGetLastError();
}

template <Elem E, int DIM, int NB, bool MASK, bool KEEP>
static hipError_t launch_main_m(const FwdPlan& p, const FwdArgs& a, hipStream_t s) {
  using G = Geo<E, DIM>;
  if (E == Elem::BF16S || p.layout == kAllPairs) {
    const int64_t grid = 8 * p.gpx * p.n_sb;
    constexpr int lds = ap_lds_bytes<E, DIM>();
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&allpairs_fwd_kernel<E, DIM, NB, MASK, KEEP>),
          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    return launch_fwd(allpairs_fwd_kernel<E, DIM, NB, MASK, KEEP>, dim3((unsigned)grid),
                      dim3(kApThreads), lds, s, a);
  }
  if constexpr (E != Elem::BF16S) {   // split rows are only made for all-pairs
    constexpr int W = pr_waves<E, DIM>();
    const int64_t grid = cdiv(p.n_units, W);
    return launch_fwd(pairs_fwd_kernel<E, DIM, NB, MASK>, dim3((unsigned)grid), dim3(W * kWave),
                      W * G::kTileBytes, s, a);
  }
  return hipErrorInvalidValue;
}

template <Elem E, int DIM, int NB>
static hipError_t launch_main(const FwdPlan& p, const FwdArgs& a, hipStream_t s) {
  // the pairs kernel always tracks the argmax (it is bandwidth-bound)
  const bool keep = a.argmax != nullptr || p.layout != kAllPairs;
  if (a.bits)
    return keep ? launch_main_m<E, DIM, NB, true, true>(p, a, s)
                : launch_main_m<E, DIM, NB, true, false>(p, a, s);
  return keep ? launch_main_m<E, DIM, NB, false, true>(p, a, s)
              : launch_main_m<E, DIM, NB, false, false>(p, a, s);
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

// Split float32 rows: the kernels see bfloat16 rows of 2 * dim.
static hipError_t dispatch_split(const FwdPlan& p, const FwdArgs& a, hipStream_t s) {
  switch (p.dim) {
    case 64: return p.NB == 2 ? launch_main<Elem::BF16S, 128, 2>(p, a, s)
                              : launch_main<Elem::BF16S, 128, 1>(p, a, s);
    case 128: return launch_main<Elem::BF16S, 256, 1>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

bool fwd_dim_supported(int64_t dim) { return dim == 64 || dim == 128 || dim == 256; }

// bfloat16 bits of x rounded to nearest, ties to even (a NaN stays a NaN)
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Float32 rows of DIM values -> rows of 2 * DIM bfloat16 [hi | lo]:
// hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in float32), so that
// x = hi + lo + e with |e| <= 2^-16 |x|.  A value whose high part is not
// finite gets lo = 0.  Thread = 8 consecutive values of a row; one launch
// splits Q (groups [0, nq)) and D (groups [nq, nq + nd)).
template <int DIM>
__global__ __launch_bounds__(256) void split_f32_kernel(const float* __restrict__ xq,
                                                        uint32_t* __restrict__ yq, int64_t nq,
                                                        const float* __restrict__ xd,
                                                        uint32_t* __restrict__ yd, int64_t nd) {
  constexpr int kG = DIM / 8;   // groups of 8 per row
  const int64_t n = nq + nd;
  for (int64_t gg = (int64_t)blockIdx.x * 256 + threadIdx.x; gg < n;
       gg += (int64_t)gridDim.x * 256) {
    const bool isq = gg < nq;
    const int64_t g = isq ? gg : gg - nq;
    const float* x = isq ? xq : xd;
    uint32_t* y = isq ? yq : yd;
    const int64_t r = g / kG;
    const int c = (int)(g - r * kG);
    const float4 v0 = reinterpret_cast<const float4*>(x)[2 * g];
    const float4 v1 = reinterpret_cast<const float4*>(x)[2 * g + 1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      hb[k] = bf16_bits_rne(v[k]);
      const float h = __uint_as_float(hb[k] << 16);
      lb[k] = __builtin_isfinite(h) ? bf16_bits_rne(v[k] - h) : 0u;
    }
    u32x4 ho, lo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ho[k] = hb[2 * k] | (hb[2 * k + 1] << 16);
      lo[k] = lb[2 * k] | (lb[2 * k + 1] << 16);
    }
    // a split row is DIM 32-bit words: hi in words [0, DIM/2), lo after
    uint32_t* row = y + r * DIM;
    *reinterpret_cast<u32x4*>(row + c * 4) = ho;
    *reinterpret_cast<u32x4*>(row + DIM / 2 + c * 4) = lo;
  }
}

// Q (q_rows rows) and D (d_rows rows) into their split copies, one launch.
static hipError_t split_rows(const void* Q, int64_t q_rows, char* q_out, const void* D,
                             int64_t d_rows, char* d_out, int dim, hipStream_t s) {
  const int64_t nq = q_rows * (dim / 8), nd = d_rows * (dim / 8);
  if (nq + nd == 0) return hipSuccess;
  const int64_t blocks = cdiv(nq + nd, 256) < 8192 ? cdiv(nq + nd, 256) : 8192;
  const float* xq = static_cast<const float*>(Q);
  const float* xd = static_cast<const float*>(D);
  uint32_t* yq = reinterpret_cast<uint32_t*>(q_out);
  uint32_t* yd = reinterpret_cast<uint32_t*>(d_out);
  if (dim == 64)
    hipLaunchKernelGGL(split_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, xq, yq, nq,
                       xd, yd, nd);
  else
    hipLaunchKernelGGL(split_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, xq, yq, nq,
                       xd, yd, nd);
  return hipGetLastError();
}

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
    // (with Ld == 0 it only records that every document is empty)
    const bool dw = p.Ld % 4 == 0 && (reinterpret_cast<uintptr_t>(d_mask) & 3u) == 0;
    if (dw)
      hipLaunchKernelGGL(mask_prep_kernel<true>, dim3((unsigned)p.n_docs), dim3(256), 0, s, d_mask,
                         p.n_docs, p.Ld, p.nwords, a.bits, a.ntiles);
    else
      hipLaunchKernelGGL(mask_prep_kernel<false>, dim3((unsigned)p.n_docs), dim3(256), 0, s,
                         d_mask, p.n_docs, p.Ld, p.nwords, a.bits, a.ntiles);
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
  if (p.compact) {
    a.compact = 1;
    a.tok = reinterpret_cast<int32_t*>(ws + p.off_tok);
    a.tok_cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
    hipLaunchKernelGGL(compact_prep_kernel, dim3(1), dim3(1024), 0, s, q_mask, p.Nq * p.Lq, a.tok,
                       a.tok_cnt);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipError_t e;
  if (p.elem == 3) {   // float32 inputs scored through split bfloat16 rows
    e = split_rows(Q, p.Nq * p.Lq, ws + p.off_sq, D, p.n_docs * p.Ld, ws + p.off_sd, p.dim, s);
    if (e != hipSuccess) return e;
    a.Q = ws + p.off_sq;
    a.D = ws + p.off_sd;
  }
  switch (p.elem) {
    case 0: e = dispatch_dim<Elem::F16>(p, a, s); break;
    case 1: e = dispatch_dim<Elem::BF16>(p, a, s); break;
    case 3: e = dispatch_split(p, a, s); break;
    default: e = dispatch_dim<Elem::F32>(p, a, s); break;
  }
  if (e != hipSuccess) return e;
  if (p.partial) {
    const int64_t n_out = p.layout == kAllPairs ? p.Nq * p.n_docs : p.n_docs;
    if (p.nchunks <= kCombineWaveMaxChunks) {
      const int64_t blocks = cdiv(cdiv(n_out, p.Lq <= 32 ? 2 : 1), 4);
      hipLaunchKernelGGL(combine_fwd_wave_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                         dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(combine_fwd_kernel, dim3((unsigned)(n_out < 65536 ? n_out : 65536)),
                         dim3(256), 0, s, a);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace lik
