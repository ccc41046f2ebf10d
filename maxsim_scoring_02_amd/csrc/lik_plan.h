// Launch plans shared by the C ABI (host) and the kernels: how a MaxSim call
// is cut into work units and where its scratch lives in the workspace.
// Plans depend on shapes only, never on data, so the workspace size can be
// queried before any device memory exists.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lik {

enum Layout : int { kAllPairs = 0, kPairwise = 1, kKd = 2 };

struct FwdPlan {
  int layout = 0;
  int elem = 0;             // 0 f16, 1 bf16, 2 f32, 3 f32 through split bf16 rows
  int dim = 0;
  int NB = 2;               // 32-column MFMA blocks per wave
  int SPW = 64;             // query-token slots per wave (32 * NB)
  int64_t Nq = 0, Lq = 0;   // queries (B for pairwise/kd) and tokens per query
  int64_t n_docs = 0;       // documents (Nd; B; B*N)
  int64_t Ld = 0;
  int64_t K = 1;            // documents per query for pairwise (1) / kd (N)
  int64_t nwords = 0;       // 32-bit mask words per document
  int64_t ntiles_max = 0;   // ceil(Ld / 32)
  bool has_dmask = false;
  bool partial = false;     // per-slot partials + combine kernel
  // all-pairs with a query mask: only the valid query tokens get slots, packed
  // in (query, token) order from a device-side list (n_cg is then an upper
  // bound; workgroups past the last valid token leave at once)
  bool compact = false;
  // slot mapping (all-pairs): qpw > 0 packs qpw whole queries per wave,
  // qpw == 0 flattens (q, i) so a query may span waves.
  int64_t qpw = 0;
  int64_t n_cg = 0;         // column groups: waves (all-pairs) or slot groups per query (pairs)
  int NW = 8;               // waves per workgroup (all-pairs)
  int64_t n_sb = 0;         // slot blocks (all-pairs)
  int64_t nchunks = 1, tpc = 0;  // split of a document's tiles
  int64_t upw = 1;          // units per workgroup (all-pairs)
  int64_t n_groups = 0, gpx = 0;
  int64_t n_units = 0;      // pairs: waves launched
  // workspace layout (bytes)
  size_t off_bits = 0, off_tiles = 0, off_partM = 0, off_partJ = 0, off_tok = 0,
         off_cnt = 0, off_sq = 0, off_sd = 0, fwd_bytes = 0;
};

// Split float32 rows (elem 3) are made for the all-pairs forward at these
// dims; every other call with elem 3 computes exactly in float32 (elem 2).
inline bool split_supported(int layout, int64_t dim) {
  return layout == kAllPairs && (dim == 64 || dim == 128);
}
// the split copies of Q and D (as many bytes as the float32 inputs) stay
// within this part of the workspace
constexpr int64_t kSplitMaxBytes = int64_t(1) << 30;
inline int64_t split_bytes(int64_t q_rows, int64_t d_rows, int64_t dim) {
  return (q_rows + d_rows) * dim * 4;
}

// grad_D strategies
enum GdMode : int {
  kGdSort = 0,    // sort kernel + row kernel through the workspace (any shape)
  kGdSorted = 1,  // all-pairs: per document, one workgroup sorts its hits in LDS and sums them
  kGdPairs = 2    // pairwise / kd: waves per document stream contiguous row ranges
};
// pairwise / kd grad_D: at least this many waves per document, and enough
// over the batch to fill the chip (few long documents split finer)
constexpr int kGdPairsMinParts = 4;
constexpr int64_t kGdPairsWaves = 65536;
constexpr int64_t kGdPairsMinRows = 64;   // rows a wave streams, at least
constexpr size_t kSortWsMax = size_t(256) << 20;  // workspace-sort batches stay within this
constexpr int kGsThreads = 1024;       // threads of the sorted grad_D workgroup
constexpr int kGsLdsMax = 160 * 1024;  // LDS of one CU
constexpr int kPairsMaxLq = 256;   // longest query of the pairs grad_D kernel
constexpr int64_t kGqSliceMinDocs = 64;

struct BwdPlan {
  FwdPlan fwd;              // used when the argmax must be recomputed
  bool recompute = false;
  int64_t H = 0;            // hits per document (all-pairs Nq*Lq; pairs Lq)
  int key_bits = 1;
  int gd_mode = kGdSort;
  int gd_parts = kGdPairsMinParts;   // pairwise / kd grad_D: waves per document
  // sorted grad_D: sorting waves, workgroups per document, dynamic LDS layout
  // (sorted hits, row starts, the document's upstream grads, then a region
  // that holds the keys and row histograms while sorting and the partial rows
  // while summing)
  int gs_sw = 0, gs_split = 1;
  int gs_masks = 0;         // ranks from LDS match masks (else from ballots over the key bits)
  int gs_off_sorted = 0, gs_off_start = 0, gs_off_gl = 0, gs_off_keys = 0, gs_off_hist = 0,
      gs_off_masks = 0, gs_off_part = 0;
  size_t gs_lds = 0;
  int64_t sort_batch = 0;   // workspace sort: documents sorted per batch (bounded workspace)
  bool gq_ap = false;       // all-pairs grad_Q by document rounds (gradq_ap_kernel)
  int gq_slices = 1;        // >1: grad_Q gathered per document slice, then reduced
  size_t off_argmax = 0, off_scores = 0, off_sorted = 0, off_sorted_g = 0, off_roff = 0, off_fwd = 0,
         off_gq_part = 0, total = 0;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// all-pairs forward: a workgroup's units span at most kApMaxDocs documents
// and kApMaxWords tile words (their counts and words are kept in LDS)
constexpr int kApMaxDocs = 64;
constexpr int kApMaxWords = 1024;
// all-pairs schedule entries pack (document << 8 | chunk): documents below
// 2^23, chunks of 1024 rows below 256
constexpr int64_t kApMaxDocIndex = (int64_t(1) << 23) - 1;
constexpr int64_t kApMaxLd = 255 * 1024;
// all-pairs query-token slots are numbered in 32-bit arithmetic
constexpr int64_t kApMaxTokens = int64_t(1) << 30;
// schedule entries: a super-tile (2 tiles) each, or one per empty unit
constexpr int kApMaxST = kApMaxWords / 2 + 2 * kApMaxDocs;
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// Number of 32-column blocks per wave for an element type and dim.
inline int blocks_per_wave(int elem, int64_t dim) {
  if (elem == 2) return 1;
  return dim <= 128 ? 2 : 1;
}

// largest Nq * Lq whose valid tokens are compacted (one workgroup lists them)
constexpr int64_t kCompactMaxTokens = int64_t(1) << 22;

inline FwdPlan make_fwd_plan(int layout, int elem, int64_t nq_or_b, int64_t Lq,
                             int64_t nd_or_n, int64_t Ld, int64_t dim, bool has_dmask,
                             bool keep_argmax, bool has_qmask = false) {
  (void)keep_argmax;
  FwdPlan p;
  if (elem == 3 && !split_supported(layout, dim)) elem = 2;
  p.layout = layout;
  p.elem = elem;
  p.dim = (int)dim;
  // split rows are bfloat16 rows of twice the width
  p.NB = elem == 3 ? blocks_per_wave(1, 2 * dim) : blocks_per_wave(elem, dim);
  // a pair has one query: one 32-column block suffices when Lq <= 32
  if (layout != kAllPairs && Lq <= 32) p.NB = 1;
  p.SPW = 32 * p.NB;
  p.Nq = nq_or_b;
  p.Lq = Lq;
  p.Ld = Ld;
  p.has_dmask = has_dmask;
  if (layout == kAllPairs) {
    p.n_docs = nd_or_n;
    p.K = 0;
  } else if (layout == kPairwise) {
    p.n_docs = nq_or_b;
    p.K = 1;
  } else {
    p.n_docs = nq_or_b * nd_or_n;
    p.K = nd_or_n;
  }
  p.nwords = cdiv(Ld, 32);
  p.ntiles_max = p.nwords;
  if (p.Nq == 0 || p.n_docs == 0) return p;  // nothing to do

  size_t off = 0;
  if (has_dmask) {
    p.off_bits = off;
    off = align256(off + (size_t)p.n_docs * p.nwords * 4);
    p.off_tiles = off;
    off = align256(off + (size_t)p.n_docs * 4);
  }
  if (Lq == 0) {  // only the empty-document test is needed
    p.fwd_bytes = off;
    return p;
  }

  if (layout == kAllPairs) {
    p.compact = has_qmask && Lq > 1 && p.Nq * Lq <= kCompactMaxTokens;
    if (p.compact) {
      p.qpw = 0;
      p.n_cg = cdiv(p.Nq * Lq, p.SPW);
    } else if (Lq <= p.SPW) {
      p.qpw = p.SPW / Lq;
      p.n_cg = cdiv(p.Nq, p.qpw);
    } else {
      p.qpw = 0;
      p.n_cg = cdiv(p.Nq * Lq, p.SPW);
    }
    p.NW = 4;   // waves per workgroup of the all-pairs kernel
    p.n_sb = cdiv(p.n_cg, p.NW);
    // Long documents are cut into chunks of 32 tiles (1024 rows) so that
    // work units stay short and the chip fills; chunk maxima merge exactly.
    if (p.ntiles_max > 64) {
      p.tpc = 32;
      p.nchunks = cdiv(p.ntiles_max, p.tpc);
    } else {
      p.tpc = p.ntiles_max > 0 ? p.ntiles_max : 1;
      p.nchunks = 1;
    }
    p.partial = (p.nchunks > 1) || (p.qpw == 0);   // compact has qpw == 0
    int64_t units = p.n_docs * p.nchunks;
    // About 1024 workgroups; each keeps its query fragments for upw units.
    // Units of at most 16 tiles (short documents) take 512, so a workgroup
    // pays its set-up over twice as many units (in-batch text kernel
    // 105.3 -> 103.2 us; long documents, 32-tile units, lose 2% that way).
    // With compacted tokens the workgroups past the last valid token leave
    // at once, so twice as many smaller ones keep the last round short.
    int64_t target = p.compact ? 2048 : (p.tpc <= 16 ? 512 : 1024);
    int64_t per_sb = cdiv(target, p.n_sb);
    p.upw = per_sb >= units ? 1 : cdiv(units, per_sb);
    if (p.upw < 1) p.upw = 1;
    const int64_t cap_docs = (kApMaxDocs - 1) * p.nchunks;
    const int64_t cap_words = kApMaxWords / p.tpc;
    if (p.upw > cap_docs) p.upw = cap_docs;
    if (p.upw > cap_words) p.upw = cap_words;
    p.n_groups = cdiv(units, p.upw);
    p.gpx = cdiv(p.n_groups, 8);
  } else {
    p.n_cg = cdiv(Lq, p.SPW);
    int64_t pairs = p.n_docs * p.n_cg;
    // about 6 waves per SIMD: documents are split along Ld (the chunk maxima
    // merge exactly) until that many waves stream; measured on kd (4096
    // documents of 1030 rows, now 2 chunks each) and long rerank (64 of
    // 32768 rows): 4096 waves left both below 0.7 of HBM peak, 16384 made
    // the merge cost more than the split saved
    int64_t want = 6144;
    int64_t nch = pairs >= want ? 1 : cdiv(want, pairs);
    int64_t max_nch = p.ntiles_max >= 4 ? p.ntiles_max / 4 : 1;
    if (nch > max_nch) nch = max_nch;
    if (nch < 1) nch = 1;
    p.tpc = p.ntiles_max > 0 ? cdiv(p.ntiles_max, nch) : 1;
    p.nchunks = p.ntiles_max > 0 ? cdiv(p.ntiles_max, p.tpc) : 1;
    p.partial = (p.nchunks > 1) || (p.n_cg > 1);
    p.n_units = pairs * p.nchunks;
  }
  if (p.compact) {
    const size_t nt = (size_t)p.Nq * Lq;
    p.off_tok = off;
    off = align256(off + nt * 4);
    p.off_cnt = off;
    off = align256(off + 4);
  }
  if (p.partial) {
    size_t n = (size_t)p.nchunks * p.n_docs * p.n_cg * p.SPW;
    p.off_partM = off;
    off = align256(off + n * 4);
    p.off_partJ = off;
    off = align256(off + n * 4);
  }
  if (p.elem == 3) {
    p.off_sq = off;
    off = align256(off + (size_t)p.Nq * Lq * dim * 4);
    p.off_sd = off;
    off = align256(off + (size_t)p.n_docs * Ld * dim * 4);
  }
  p.fwd_bytes = off;
  return p;
}

inline BwdPlan make_bwd_plan(int layout, int elem, int64_t nq_or_b, int64_t Lq, int64_t nd_or_n,
                             int64_t Ld, int64_t dim, bool has_dmask, bool have_argmax,
                             bool has_qmask = false) {
  BwdPlan b;
  b.fwd = make_fwd_plan(layout, elem, nq_or_b, Lq, nd_or_n, Ld, dim, has_dmask, true, has_qmask);
  const FwdPlan& f = b.fwd;
  if (f.Nq == 0 || f.n_docs == 0) return b;
  b.recompute = !have_argmax;
  b.H = (layout == kAllPairs) ? f.Nq * Lq : Lq;
  int bits = 1;
  while (bits < 31 && (int64_t(1) << bits) < Ld) ++bits;
  b.key_bits = bits;
  // grad_D strategy
  const int esize = elem >= 2 ? 4 : 2;   // float32 inputs (exact or split)
  const int64_t q_bytes = f.Nq * Lq * dim * esize;
  if (layout == kAllPairs && b.H <= 65535 && Ld <= 65535 && Lq > 0 && Ld > 0 &&
      q_bytes < (int64_t(1) << 32)) {
    // one workgroup sorts a document's hits by row (stable, in LDS) and its
    // lane groups (one 16-byte chunk of a row per lane) sum them
    const size_t cpr = (size_t)dim * esize / 16;
    const size_t ng = kGsThreads / cpr;
    const size_t part = ng * 2 * (size_t)dim * 4;
    const size_t sorted = align16((size_t)b.H * 4);
    const size_t start = align16((size_t)(Ld + 1) * 4);
    const size_t gl = align16((size_t)f.Nq * 4);
    const size_t keys = align16((size_t)b.H * 4);   // key | rank << 16 | count << 22 per hit
    const int64_t chunks = cdiv(b.H, 64);
    // ranks from per-wave LDS match masks (one 64-bit word per row) when they
    // fit, else from ballots over the key bits (long documents)
    for (int use_masks = 1; use_masks >= 0 && b.gd_mode != kGdSorted; --use_masks) {
      for (int sw = kGsThreads / 64; sw >= 1; sw /= 2) {
        if (sw > 1 && sw > chunks) continue;        // no more sorting waves than 64-hit chunks
        const size_t hist = align16((size_t)sw * Ld * 4);
        const size_t masks = use_masks ? (size_t)sw * Ld * 8 : 0;
        const size_t uni = part > keys + hist + masks ? part : keys + hist + masks;
        const size_t tot = sorted + start + gl + uni;
        if (tot <= (size_t)kGsLdsMax) {
          b.gd_mode = kGdSorted;
          b.gs_sw = sw;
          b.gs_masks = use_masks;
          b.gs_off_sorted = 0;
          b.gs_off_start = (int)sorted;
          b.gs_off_gl = (int)(sorted + start);
          b.gs_off_keys = (int)(sorted + start + gl);
          b.gs_off_hist = (int)(sorted + start + gl + keys);
          b.gs_off_masks = (int)(sorted + start + gl + keys + hist);
          b.gs_off_part = (int)(sorted + start + gl);
          b.gs_lds = tot;
          break;
        }
      }
    }
    if (b.gd_mode == kGdSorted) {
      // every CU holds one such workgroup: split documents until about 256 run
      int64_t sp = cdiv(256, f.n_docs);
      b.gs_split = (int)(sp < 1 ? 1 : (sp > 8 ? 8 : sp));
    }
  } else if (layout != kAllPairs && Lq > 0 && Lq <= kPairsMaxLq && Ld > 0) {
    b.gd_mode = kGdPairs;
    int64_t parts = cdiv(kGdPairsWaves, f.n_docs);
    const int64_t by_rows = Ld / kGdPairsMinRows;
    if (parts > by_rows) parts = by_rows;
    if (parts < kGdPairsMinParts) parts = kGdPairsMinParts;
    b.gd_parts = (int)parts;
  }
  // grad_Q over many documents: the documents are cut into slices bound to
  // XCDs, each gathered by its own workgroups, then added in slice order.
  // When D takes at most half the last-level cache (128 of 256 MB), two slices (even and odd
  // XCDs) write the fewest partials; a larger D is read from HBM, and one
  // slice per XCD fetches each gathered row once.  Measured: in-batch text
  // (D 19.7 MB) 81 / 79 / 78 / 102 us of backward with 8 / 4 / 2 / 1 slices;
  // long documents (D 2.1 GB) 777 us with 8 slices, 825 with 2.  (Rows of one
  // slice are indexed with 32 bits.)
  const int64_t d_bytes = f.n_docs * Ld * dim * esize;
  const int slices = d_bytes <= (int64_t(128) << 20) ? 2 : 8;
  // a slice's rows are addressed with 32-bit byte offsets
  if (layout == kAllPairs && f.n_docs >= kGqSliceMinDocs && Lq > 0 && Ld > 0 &&
      cdiv(f.n_docs, slices) * Ld * dim * esize < (int64_t(1) << 32)) {
    b.gq_ap = true;
    b.gq_slices = slices;
  }

  size_t off = 0;
  if (b.recompute && Lq > 0) {
    int64_t pairs = (layout == kAllPairs) ? f.Nq * f.n_docs : f.n_docs;
    b.off_argmax = off;
    off = align256(off + (size_t)pairs * Lq * 4);
    b.off_scores = off;
    off = align256(off + (size_t)pairs * 4);
    b.off_fwd = off;
    off = align256(off + f.fwd_bytes);
  }
  if (Lq > 0 && Ld > 0 && b.gd_mode == kGdSort) {
    // sorted hit lists and row offsets for at most sort_batch documents at a
    // time, so that the workspace stays within kSortWsMax (one document may
    // exceed it on its own)
    const size_t per_doc = (size_t)b.H * 8 + (size_t)(Ld + 1) * 4;
    int64_t nbat = (int64_t)(kSortWsMax / per_doc);
    if (nbat < 1) nbat = 1;
    if (nbat > f.n_docs) nbat = f.n_docs;
    b.sort_batch = nbat;
    b.off_sorted = off;
    off = align256(off + (size_t)nbat * b.H * 4);
    b.off_sorted_g = off;
    off = align256(off + (size_t)nbat * b.H * 4);
    b.off_roff = off;
    off = align256(off + (size_t)nbat * (Ld + 1) * 4);
  }
  if (b.gq_slices > 1) {
    b.off_gq_part = off;
    off = align256(off + (size_t)b.gq_slices * f.Nq * Lq * dim * 4);
  }
  b.total = off;
  return b;
}

}  // namespace lik
