// Device-side building blocks of the gfx950 MaxSim kernels.
//
// MaxSim (README "Late Interaction Kernels", "What does it compute?"):
//   score(q,d) = sum_{valid i} max_{valid j} Q[q,i,:] . D[d,j,:]
//
// Orientation.  One 32x32 MFMA output tile is S^T = Dtile (32 doc rows) x
// Q^T (32 query-token columns).  In the 32x32 accumulator layout lane l owns
// column l%32 and 16 rows {8*(v/4) + 4*(l/32) + v%4 : v = 0..15}, so the max
// over document tokens is mostly a per-lane reduction; lanes l and l^32 hold
// the two row halves of the same column and meet once per (column, unit).
//
// K mapping.  Each lane feeds the MFMA 16-byte chunks of its row: lane
// (row or column r, half h = l/32) supplies chunk 2m+h at K-step m.  A and B
// use the same mapping, so every product Q[.,k]*D[.,k] is summed exactly once
// (the order of the K-sum is the only freedom taken).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lik {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = 32;   // document rows per tile (MFMA M)
constexpr int kWave = 64;

// BF16S: float32 values held as two bfloat16 parts, a row of dim values
// stored as 2 * dim bfloat16 [hi(0..dim) | lo(0..dim)] with hi = bf16(x) and
// lo = bf16(x - hi); the kernels see a bfloat16 row of twice the width and
// multiply it with three products per element pair (hi*hi, lo*hi, hi*lo).
enum class Elem { F16 = 0, BF16 = 1, F32 = 2, BF16S = 3 };

template <Elem E> struct ElemInfo;
template <> struct ElemInfo<Elem::F16>  { static constexpr int kBytes = 2; static constexpr int kPerChunk = 8; };
template <> struct ElemInfo<Elem::BF16> { static constexpr int kBytes = 2; static constexpr int kPerChunk = 8; };
template <> struct ElemInfo<Elem::F32>  { static constexpr int kBytes = 4; static constexpr int kPerChunk = 4; };
template <> struct ElemInfo<Elem::BF16S> { static constexpr int kBytes = 2; static constexpr int kPerChunk = 8; };

// Geometry of one document row / tile for an element type and embedding dim.
template <Elem E, int DIM>
struct Geo {
  static constexpr int kRowBytes = DIM * ElemInfo<E>::kBytes;
  static constexpr int kCPR = kRowBytes / 16;            // 16-byte chunks per row
  static constexpr int kKSteps = kCPR / 2;               // chunks each lane feeds
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int kTileChunks = kTile * kCPR;
  static constexpr int kSwz = kCPR < 16 ? kCPR : 16;     // XOR swizzle span
  static_assert(kCPR % 2 == 0 && kCPR >= 2, "dim must give an even chunk count");
};

// Physical LDS byte offset of (row r, chunk c) in a swizzled tile: the chunk
// index is XORed with the row so that the 32 rows read by one MFMA operand
// load fall in distinct banks.
template <Elem E, int DIM>
__device__ __forceinline__ int lds_off(int r, int c) {
  using G = Geo<E, DIM>;
  return r * G::kRowBytes + ((c ^ (r & (G::kSwz - 1))) << 4);
}

__device__ __forceinline__ u32x4 ld_global_16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_lds_16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void st_lds_16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// acc += A(32 x k) * B(k x 32) for one 16-byte chunk per lane.
template <Elem E> __device__ __forceinline__ void mfma_chunk(f32x16& acc, u32x4 a, u32x4 b);

template <> __device__ __forceinline__ void mfma_chunk<Elem::BF16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_chunk<Elem::BF16S>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_chunk<Elem::F16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
// Vector elements are read into scalars before reinterpretation: a bit-cast
// applied directly to an element lvalue of an ext_vector reads element 0.
template <> __device__ __forceinline__ void mfma_chunk<Elem::F32>(f32x16& acc, u32x4 a, u32x4 b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ae), __uint_as_float(be), acc, 0,
                                               0, 0);
  }
}

// First K-step of a tile: returns C + a*b with C = c, or 0 when ZERO, so the
// initial value is an operand and never copied into the accumulator.
template <Elem E, bool ZERO>
__device__ __forceinline__ f32x16 mfma_first(u32x4 a, u32x4 b, const f32x16& c) {
  f32x16 acc;
  if constexpr (ZERO) acc = f32x16{};
  else acc = c;
  mfma_chunk<E>(acc, a, b);
  return acc;
}

// Row of accumulator element v for a lane in half h (32x32 MFMA layout).
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// Validity word of tile t (bit r = doc row 32t+r is a valid token).
__device__ __forceinline__ uint32_t tile_word(const uint32_t* bits_d, int t, int64_t Ld) {
  if (bits_d) return bits_d[t];
  int64_t rem = Ld - (int64_t)t * kTile;
  return rem >= kTile ? 0xffffffffu : ((1u << rem) - 1u);
}

// Running state of one 32-column block: the best value seen by this lane,
// the tile it came from and that tile's 16 values (to recover the row).
struct BlockState {
  float run_max;
  int best_tile;
  float best_val[16];
};

__device__ __forceinline__ void state_init(BlockState& s, int t0) {
  s.run_max = -__builtin_inff();
  s.best_tile = t0;
#pragma unroll
  for (int v = 0; v < 16; ++v) s.best_val[v] = -__builtin_inff();
}

// Masked rows of a tile never win: set them to -inf.  `word` bit r = row r
// valid.  Call only for tiles that are not fully valid.
__device__ __forceinline__ void tile_mask(f32x16& acc, uint32_t word, int h) {
  const uint32_t w = word >> (4 * h);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int bit = 8 * (v >> 2) + (v & 3);
    if (!((w >> bit) & 1u)) acc[v] = -__builtin_inff();
  }
}

// Initial accumulator of a tile that is not fully valid: 0 in the rows the
// validity word keeps, -inf in the others (-inf + finite products stays
// -inf, so a masked row never wins a max).  `word` bit r = row r valid.
__device__ __forceinline__ void tile_init(f32x16& c, uint32_t word, int h) {
  const uint32_t w = word >> (4 * h);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int bit = 8 * (v >> 2) + (v & 3);
    const int keep = (int)(w << (31 - bit)) >> 31;     // -1 valid, 0 masked
    c[v] = __int_as_float(~keep & (int)0xff800000u);
  }
}

// The same for a wave-uniform word: element v of the lanes in half h comes
// from bit 8*(v/4) + 4*h + v%4, so each element is one select under a lane
// mask built with two scalar bit-field extracts straight into vcc (valid
// rows 0, masked rows -inf).
template <int V>
__device__ __forceinline__ float tile_init_elem(uint32_t word, float ninf, float zero) {
  constexpr int b0 = 8 * (V >> 2) + (V & 3);
  // lane mask = (bit b0 of word ? all of lanes 0-31) | (bit b0+4 ? all of
  // 32-63): two sign-extended 1-bit fields, one per half of the mask.  Each
  // element's mask is its own register pair, so the selects do not wait on
  // the next element's mask overwriting a shared condition register.
  const uint32_t lo = (uint32_t)(-(int32_t)((word >> b0) & 1u));
  const uint32_t hi = (uint32_t)(-(int32_t)((word >> (b0 + 4)) & 1u));
  const uint64_t mask = (uint64_t)lo | ((uint64_t)hi << 32);
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(ninf), "v"(zero), "s"(mask));
  return r;
}
__device__ __forceinline__ void tile_init_uniform(f32x16& c, uint32_t word) {
  const float ninf = -__builtin_inff(), zero = 0.0f;
  c[0] = tile_init_elem<0>(word, ninf, zero);
  c[1] = tile_init_elem<1>(word, ninf, zero);
  c[2] = tile_init_elem<2>(word, ninf, zero);
  c[3] = tile_init_elem<3>(word, ninf, zero);
  c[4] = tile_init_elem<4>(word, ninf, zero);
  c[5] = tile_init_elem<5>(word, ninf, zero);
  c[6] = tile_init_elem<6>(word, ninf, zero);
  c[7] = tile_init_elem<7>(word, ninf, zero);
  c[8] = tile_init_elem<8>(word, ninf, zero);
  c[9] = tile_init_elem<9>(word, ninf, zero);
  c[10] = tile_init_elem<10>(word, ninf, zero);
  c[11] = tile_init_elem<11>(word, ninf, zero);
  c[12] = tile_init_elem<12>(word, ninf, zero);
  c[13] = tile_init_elem<13>(word, ninf, zero);
  c[14] = tile_init_elem<14>(word, ninf, zero);
  c[15] = tile_init_elem<15>(word, ninf, zero);
}

// Fold one (masked) tile's accumulator into the running state, branch-free.
// Strict '>' keeps the earlier tile on ties, so tiles must come in order.
__device__ __forceinline__ void state_fold(BlockState& s, const f32x16& acc, int t) {
  const float m01 = __builtin_fmaxf(__builtin_fmaxf(acc[0], acc[1]), acc[2]);
  const float m02 = __builtin_fmaxf(__builtin_fmaxf(acc[3], acc[4]), acc[5]);
  const float m03 = __builtin_fmaxf(__builtin_fmaxf(acc[6], acc[7]), acc[8]);
  const float m04 = __builtin_fmaxf(__builtin_fmaxf(acc[9], acc[10]), acc[11]);
  const float m05 = __builtin_fmaxf(__builtin_fmaxf(acc[12], acc[13]), acc[14]);
  const float m1 = __builtin_fmaxf(__builtin_fmaxf(m01, m02), m03);
  const float m2 = __builtin_fmaxf(__builtin_fmaxf(m04, m05), acc[15]);
  const float tmax = __builtin_fmaxf(m1, m2);
  const bool better = tmax > s.run_max;
  s.run_max = better ? tmax : s.run_max;
  s.best_tile = better ? t : s.best_tile;
#pragma unroll
  for (int v = 0; v < 16; ++v) s.best_val[v] = better ? acc[v] : s.best_val[v];
}

// Padded LDS layout: each document row takes its bytes plus 16, so the 32
// rows read by one MFMA operand load start 4 banks apart (no conflicts), and
// a lane's successive K-step chunks sit at fixed immediate offsets.
template <Elem E, int DIM>
struct Pad {
  static constexpr int kStride = Geo<E, DIM>::kRowBytes + 16;
  static constexpr int kTileBytes = kTile * kStride;
};

// ---------------------------------------------------------------------------
// Lean fold for the all-pairs hot loop.  The fold's VALU work mostly runs
// while no MFMA is in flight on the SIMD (the waves sharing it tend to
// multiply and fold in step), so it is written to issue as few VALU
// instructions as possible:
// - a 3-input max tree written directly (the generic fmax path re-quiets
//   NaNs of unknown operands first; inputs are finite or -inf here);
// - the copy of the improving tile runs under an exec mask of the improving
//   lanes inside one asm statement whose operands are tied to the state's
//   registers, so the state is updated in place (a divergent branch around
//   the copy makes the compiler move all 16 values on every fold);
// - a unit starts by resetting only the running max and tile.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max16_lean(const f32x16& x) {
  const float m1 = vmax3(x[0], x[1], x[2]), m2 = vmax3(x[3], x[4], x[5]);
  const float m3 = vmax3(x[6], x[7], x[8]), m4 = vmax3(x[9], x[10], x[11]);
  const float m5 = vmax3(x[12], x[13], x[14]);
  return vmax2(vmax3(m1, m2, m3), vmax3(m4, m5, x[15]));
}

// dst[O..O+7] = (useb ? b : a)[O..O+7] in the lanes of `lanes` (a subset of
// the active lanes, from a ballot); other lanes keep dst.  exec is narrowed
// and restored inside the statement, with no SCC write.
template <int O>
__device__ __forceinline__ void sel_copy8(float (&dst)[16], const f32x16& a, const f32x16& b,
                                          uint64_t lanes, uint64_t useb) {
  uint64_t sv;
  asm("s_mov_b64 %[sv], exec\n\t"
      "s_mov_b64 exec, %[ln]\n\t"
      "v_cndmask_b32_e64 %[d0], %[a0], %[b0], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d1], %[a1], %[b1], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d2], %[a2], %[b2], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d3], %[a3], %[b3], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d4], %[a4], %[b4], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d5], %[a5], %[b5], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d6], %[a6], %[b6], %[ub]\n\t"
      "v_cndmask_b32_e64 %[d7], %[a7], %[b7], %[ub]\n\t"
      "s_mov_b64 exec, %[sv]"
      : [sv] "=&s"(sv), [d0] "+v"(dst[O + 0]), [d1] "+v"(dst[O + 1]), [d2] "+v"(dst[O + 2]),
        [d3] "+v"(dst[O + 3]), [d4] "+v"(dst[O + 4]), [d5] "+v"(dst[O + 5]),
        [d6] "+v"(dst[O + 6]), [d7] "+v"(dst[O + 7])
      : [ln] "s"(lanes), [ub] "s"(useb), [a0] "v"(a[O + 0]), [b0] "v"(b[O + 0]),
        [a1] "v"(a[O + 1]), [b1] "v"(b[O + 1]), [a2] "v"(a[O + 2]), [b2] "v"(b[O + 2]),
        [a3] "v"(a[O + 3]), [b3] "v"(b[O + 3]), [a4] "v"(a[O + 4]), [b4] "v"(b[O + 4]),
        [a5] "v"(a[O + 5]), [b5] "v"(b[O + 5]), [a6] "v"(a[O + 6]), [b6] "v"(b[O + 6]),
        [a7] "v"(a[O + 7]), [b7] "v"(b[O + 7]));
}

// (mask bit of this lane ? b : a), one select under a wave-uniform lane mask.
__device__ __forceinline__ float sel_mask(float a, float b, uint64_t mask) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}
__device__ __forceinline__ int sel_mask_i(int a, int b, uint64_t mask) {
  int r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}
// (mask bit of this lane ? 1 : 0)
__device__ __forceinline__ int mask_bit(uint64_t mask) {
  int r;
  asm("v_cndmask_b32_e64 %0, 0, 1, %1" : "=v"(r) : "s"(mask));
  return r;
}

// Start of a unit: only the running max and the tile are reset.  The 16
// values are written by the first fold that improves on -inf; a lane that
// never improves (no valid row of its half in the unit) keeps run_max = -inf,
// and its resolved row is then never used (a valid row of the other half,
// or the empty-document rule, decides).
__device__ __forceinline__ void state_begin(BlockState& s, int t0) {
  s.run_max = -__builtin_inff();
  s.best_tile = t0;
}

// Fold one step of the hot loop: tiles t and t+1 when `two`, else tile t
// alone (xb ignored); nothing when `step` is false.
__device__ __forceinline__ void state_fold_step(BlockState& s, const f32x16& xa,
                                                const f32x16& xb, int t, bool step, bool two) {
  const float ta = max16_lean(xa);
  const float tb = two ? max16_lean(xb) : -__builtin_inff();
  const float tm = vmax2(ta, tb);
  // lane masks straight from the compares (step is uniform), and the state
  // updated by selects under them
  const uint64_t lanes = step ? __builtin_amdgcn_ballot_w64(tm > s.run_max) : 0ull;
  const uint64_t ub = __builtin_amdgcn_ballot_w64(tb > ta);
  s.run_max = sel_mask(s.run_max, tm, lanes);
  s.best_tile = sel_mask_i(s.best_tile, t + mask_bit(ub), lanes);
  sel_copy8<0>(s.best_val, xa, xb, lanes, ub);
  sel_copy8<8>(s.best_val, xa, xb, lanes, ub);
}

// Fold one tile of the pairwise/kd kernel: rows the validity word masks are
// set to -inf first (a full word skips that).
__device__ __forceinline__ void state_update(BlockState& s, f32x16 acc, uint32_t word, int t, int h) {
  if (word != 0xffffffffu) tile_mask(acc, word, h);
  state_fold(s, acc, t);
}

// (max, lowest doc row reaching it) of this lane's half-column.
// (mask bit of this lane ? V : a), V an inline constant
template <int V>
__device__ __forceinline__ int sel_mask_const(int a, uint64_t mask) {
  int r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "n"(V), "s"(mask));
  return r;
}
template <int V>
__device__ __forceinline__ int lowest_equal(const uint64_t (&eq)[15], int kk) {
  if constexpr (V < 0) {
    return kk;
  } else {
    return lowest_equal<V - 1>(eq, sel_mask_const<V>(kk, eq[V]));
  }
}

__device__ __forceinline__ void state_resolve(const BlockState& s, int h, float& M, int& J) {
  // every compare writes its own lane mask first, then the selects read
  // them: compares chained through one condition register would each wait
  // two cycles before their select
  uint64_t eq[15];
#pragma unroll
  for (int v = 0; v < 15; ++v) eq[v] = __builtin_amdgcn_ballot_w64(s.best_val[v] == s.run_max);
  const int kk = lowest_equal<14>(eq, 15);
  M = s.run_max;
  J = s.best_tile * kTile + acc_row(kk, h);
}

// Larger value wins; equal values keep the lower index.
__device__ __forceinline__ void merge_mj(float& M, int& J, float M2, int J2) {
  bool take = (M2 > M) || (M2 == M && J2 < J);
  M = take ? M2 : M;
  J = take ? J2 : J;
}

// The value of lane (l ^ 32), by one swap of the wave's halves (a VALU
// operation, no LDS round trip): the swap returns the upper half of its first
// operand's lanes moved down in its second result and the lower half moved up
// in its first.
__device__ __forceinline__ uint32_t xor32_u32(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane < 32 ? r[1] : r[0];
}
__device__ __forceinline__ float xor32_f32(float x, int lane) {
  return __uint_as_float(xor32_u32(__float_as_uint(x), lane));
}

// After the two row halves of a column are merged, lane L of the wave holds
// the result of slot L (NB == 2: block L/32, column L%32) or slot L%32
// (NB == 1, both halves hold it).
template <int NB>
__device__ __forceinline__ void combine_halves(const float (&M)[NB], const int (&J)[NB], int lane,
                                               float& Mout, int& Jout) {
  if constexpr (NB == 2) {
    bool lo = lane < 32;
    float own_m = lo ? M[0] : M[1];
    int own_j = lo ? J[0] : J[1];
    float give_m = lo ? M[1] : M[0];
    int give_j = lo ? J[1] : J[0];
    float oth_m = xor32_f32(give_m, lane);
    int oth_j = (int)xor32_u32((uint32_t)give_j, lane);
    merge_mj(own_m, own_j, oth_m, oth_j);
    Mout = own_m;
    Jout = own_j;
  } else {
    float own_m = M[0];
    int own_j = J[0];
    merge_mj(own_m, own_j, xor32_f32(own_m, lane), (int)xor32_u32((uint32_t)own_j, lane));
    Mout = own_m;
    Jout = own_j;
  }
}

// Inclusive sum of v over the lanes of a segment [seg_start, lane] (segments
// are contiguous lane ranges inside groups of `width` lanes).
template <int WIDTH>
__device__ __forceinline__ float segmented_scan(float v, int lane_in, int seg_start) {
#pragma unroll
  for (int k = 1; k < WIDTH; k <<= 1) {
    float t = __shfl_up(v, k, WIDTH);
    if (lane_in - k >= seg_start) v += t;
  }
  return v;
}

// Sum of v over lanes 0..31 (returned in lane 31) and over lanes 32..63
// (returned in lane 63), by DPP row shifts and a row broadcast: no LDS.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float half_sum32(float v) {
  v += dpp_f32<0x111, 0xf>(v);   // row_shr:1
  v += dpp_f32<0x112, 0xf>(v);   // row_shr:2
  v += dpp_f32<0x114, 0xf>(v);   // row_shr:4
  v += dpp_f32<0x118, 0xf>(v);   // row_shr:8  -> lane 15 of each row holds its row sum
  v += dpp_f32<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
  return v;
}

// Element conversion for the backward's float32 arithmetic.
template <Elem E> __device__ __forceinline__ void chunk_to_float(u32x4 c, float (&f)[ElemInfo<E>::kPerChunk]);
template <> __device__ __forceinline__ void chunk_to_float<Elem::BF16>(u32x4 c, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = c[k];
    f[2 * k] = __uint_as_float(w << 16);
    f[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void chunk_to_float<Elem::F16>(u32x4 c, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = c[k];
    const uint16_t lo = (uint16_t)(w & 0xffffu), hi = (uint16_t)(w >> 16);
    f[2 * k] = (float)__builtin_bit_cast(_Float16, lo);
    f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, hi);
  }
}
template <> __device__ __forceinline__ void chunk_to_float<Elem::F32>(u32x4 c, float (&f)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = c[k];
    f[k] = __uint_as_float(w);
  }
}

}  // namespace lik
