"""Host-side invariants of the launch plans (lik_plan.h), on the CPU.

A small C++ program includes the plan header, makes forward and backward
plans over a sweep of shapes and checks what the kernels rely on without
checking it themselves:

- all-pairs forward: units (document, chunk) dealt strided to workgroups
  (unit k of group g is g + k * n_groups) cover every unit exactly once; no
  workgroup holds more than 64 units (the wave-0 scan and the set-up loop) or
  more schedule entries than the LDS schedule holds; chunks cover the
  longest document; the grid covers every group and slot block;
- pairs forward: chunks cover the document and the unit count matches;
- workspace offsets are 256-byte aligned and inside the reported size;
- a query mask switches all-pairs to compacted token slots: split path,
  slots for every token, token tables inside the workspace;
- fused grad_D: its LDS layout fits the size the plan reports and each
  sorting wave ranks at most the hits it can hold;
- workspace-sort grad_D: documents in the largest batches whose sorted
  lists stay within the workspace cap, regions inside the workspace;
- pairwise / kd grad_D: waves per document at least the minimum, split
  finer only when the batch is too small to fill the chip, never below the
  minimum rows per wave, and the grid fits.

A second test pins the benchmark's work accounting (valid-token flops;
bytes with every input row counted once per step) to hand-written sums.

The numeric constants the kernels use (64 units, 32 entries per unit, 256
threads, 8 sort-wave slots) are restated here as the kernels' own limits.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "maxsim_scoring_02_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "lik_plan.h"
using namespace lik;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails < 20) { std::printf("FAIL %s: ", #c); \
  std::printf(__VA_ARGS__); std::printf("\n"); } ++fails; } } while (0)

static void fwd_case(int layout, int elem, long Nq, long Lq, long Nd, long Ld, long dim, bool mask,
                     bool qmask = false) {
  FwdPlan p = make_fwd_plan(layout, elem, Nq, Lq, Nd, Ld, dim, mask, true, qmask);
  if (p.Nq == 0 || p.n_docs == 0 || Lq == 0) return;
  CHECK(p.SPW == 32 * p.NB, "SPW");
  if (p.compact) {
    CHECK(layout == kAllPairs && qmask, "compact only for all-pairs with a query mask");
    CHECK(p.partial && p.qpw == 0, "compact uses the split path");
    CHECK(p.n_cg * p.SPW >= p.Nq * Lq, "compact slots cover every token");
    CHECK(p.off_tok % 256 == 0 && p.off_cnt >= p.off_tok + (size_t)p.Nq * Lq * 4 &&
              p.off_cnt + 4 <= p.fwd_bytes,
          "compact tables");
  } else if (layout == kAllPairs && qmask && Lq > 1) {
    CHECK(p.Nq * Lq > kCompactMaxTokens, "a query mask compacts unless the token list is too long");
  }
  if (layout == kAllPairs) {
    const long n_units = p.n_docs * p.nchunks;
    CHECK(p.nchunks * p.tpc >= p.ntiles_max, "chunks %ld x %ld < tiles %ld", p.nchunks, p.tpc, p.ntiles_max);
    CHECK(p.upw >= 1 && p.upw <= kApMaxDocs, "upw %ld", p.upw);
    CHECK(p.n_groups * p.upw >= n_units, "groups x upw < units");
    CHECK(p.n_groups <= n_units, "more groups than units");
    CHECK(p.n_sb * 4 >= p.n_cg, "slot blocks");
    CHECK(8 * p.gpx >= p.n_groups, "grid groups");
    // strided assignment: every unit exactly once, capacities respected
    std::vector<int> seen(n_units, 0);
    for (long g = 0; g < p.n_groups; ++g) {
      long n_my = (n_units - g + p.n_groups - 1) / p.n_groups;
      if (n_my > p.upw) n_my = p.upw;
      CHECK(n_my >= 1 && n_my <= kApMaxDocs, "n_my %ld", n_my);
      long entries = 0;
      for (long k = 0; k < n_my; ++k) {
        const long u = g + k * p.n_groups;
        CHECK(u < n_units, "unit %ld out of range", u);
        if (u < n_units) seen[u]++;
        const long c = u / p.n_docs;
        const long t0 = c * p.tpc;
        long t1 = t0 + p.tpc < p.ntiles_max ? t0 + p.tpc : p.ntiles_max;
        if (t1 < t0) t1 = t0;
        entries += t1 > t0 ? (t1 - t0 + 1) / 2 : 1;
        CHECK((t1 - t0 + 1) / 2 <= 32, "entries per unit");
      }
      CHECK(entries <= kApMaxST, "entries %ld > %d", entries, kApMaxST);
    }
    for (long u = 0; u < n_units; ++u) CHECK(seen[u] == 1, "unit %ld seen %d times", u, seen[u]);
    CHECK(p.n_docs <= kApMaxDocIndex || true, "docs");
  } else {
    CHECK(p.nchunks * p.tpc >= p.ntiles_max, "pairs chunks");
    CHECK(p.n_units == p.n_docs * p.n_cg * p.nchunks, "pairs units");
  }
  const size_t offs[] = {p.off_bits, p.off_tiles, p.off_partM, p.off_partJ, p.off_tok,
                         p.off_cnt, p.off_sq, p.off_sd};
  for (size_t o : offs) CHECK(o % 256 == 0 && o <= p.fwd_bytes, "fwd offset %zu / %zu", o, p.fwd_bytes);
  // float32 through split rows: only all-pairs at dim 64 / 128, bf16 rows of
  // twice the width (NB of bf16 at 2 * dim), the copies after every other
  // region and inside the workspace
  if (elem == 3) {
    const bool split = layout == kAllPairs && (dim == 64 || dim == 128);
    CHECK(p.elem == (split ? 3 : 2), "split elem %d", p.elem);
    if (split) {
      CHECK(p.NB == blocks_per_wave(1, 2 * dim), "split NB %d", p.NB);
      size_t other_end = 0;
      if (mask) other_end = p.off_tiles + (size_t)p.n_docs * 4;
      if (p.compact) other_end = p.off_cnt + 4;
      if (p.partial)
        other_end = p.off_partJ + (size_t)p.nchunks * p.n_docs * p.n_cg * p.SPW * 4;
      CHECK(p.off_sq >= other_end, "split copies after the other regions");
      CHECK(p.off_sd >= p.off_sq + (size_t)p.Nq * Lq * dim * 4 &&
                p.off_sd + (size_t)p.n_docs * Ld * dim * 4 <= p.fwd_bytes,
            "split copies inside the workspace");
    }
  }
}

static void bwd_case(int layout, int elem, long Nq, long Lq, long Nd, long Ld, long dim) {
  BwdPlan b = make_bwd_plan(layout, elem, Nq, Lq, Nd, Ld, dim, true, true);
  if (b.fwd.Nq == 0 || b.fwd.n_docs == 0) return;
  if (b.gd_mode == kGdSorted) {
    // the sorted grad_D kernel: at most one sorting wave per 64-hit chunk,
    // every LDS region inside the allocation and disjoint from the others,
    // the keys and histograms (sorting) and the partial rows (summing) in the
    // same region, and Q rows addressed with 32-bit offsets
    const long esize = elem >= 2 ? 4 : 2;
    const long cpr = dim * esize / 16;
    const size_t part = (size_t)(kGsThreads / cpr) * 2 * dim * 4;
    CHECK(layout == kAllPairs, "sorted grad_D only for all-pairs");
    CHECK(b.gs_sw >= 1 && b.gs_sw <= kGsThreads / 64, "sort waves %d", b.gs_sw);
    CHECK(b.gs_sw == 1 || (long)b.gs_sw * 64 <= b.H + 63, "more sort waves than chunks");
    CHECK(b.gs_split >= 1 && b.gs_split <= 8, "split");
    CHECK(b.H <= 65535 && Ld <= 65535, "16-bit keys and hit numbers");
    CHECK(Nq * Lq * dim * esize < (1L << 32), "Q offsets");
    CHECK(b.gs_off_sorted == 0 && b.gs_off_start >= (int)(b.H * 4), "sorted area");
    CHECK(b.gs_off_gl - b.gs_off_start >= (int)((Ld + 1) * 4), "start area");
    CHECK(b.gs_off_keys - b.gs_off_gl >= (int)(Nq * 4), "gl area");
    CHECK(b.gs_off_hist - b.gs_off_keys >= (int)(b.H * 4), "keys area");
    CHECK((size_t)b.gs_off_hist + (size_t)b.gs_sw * Ld * 4 <= (size_t)b.gs_off_masks,
          "histograms before the match words");
    CHECK(!b.gs_masks || (size_t)b.gs_off_masks + (size_t)b.gs_sw * Ld * 8 <= b.gs_lds,
          "match words inside LDS");
    CHECK(b.gs_off_masks % 8 == 0, "match words aligned");
    CHECK(b.gs_off_part == b.gs_off_keys && b.gs_off_part + part <= b.gs_lds, "partials inside LDS");
    CHECK(b.gs_lds <= (size_t)kGsLdsMax, "LDS %zu", b.gs_lds);
    CHECK(b.gs_off_hist % 16 == 0 && b.gs_off_part % 16 == 0, "alignment");
  }
  if (b.gd_mode == kGdSort && Lq > 0 && Ld > 0) {
    // workspace sort: documents in batches whose sorted lists and row
    // offsets stay within kSortWsMax (one document may exceed it), the
    // largest such batch, and the regions inside the workspace
    const size_t per_doc = (size_t)b.H * 8 + (size_t)(Ld + 1) * 4;
    const size_t ws = (size_t)b.sort_batch * per_doc;
    CHECK(b.sort_batch >= 1 && b.sort_batch <= b.fwd.n_docs, "sort batch %ld", (long)b.sort_batch);
    CHECK(b.sort_batch == 1 || ws <= kSortWsMax, "sort workspace %zu", ws);
    CHECK(b.sort_batch == b.fwd.n_docs || ws + per_doc > kSortWsMax, "sort batch not maximal");
    CHECK(b.off_sorted_g >= b.off_sorted + (size_t)b.sort_batch * b.H * 4 &&
              b.off_roff >= b.off_sorted_g + (size_t)b.sort_batch * b.H * 4 &&
              b.off_roff + (size_t)b.sort_batch * (Ld + 1) * 4 <= b.total,
          "sort regions");
  }
  if (b.gq_ap) {
    const long esize = elem >= 2 ? 4 : 2;
    CHECK(layout == kAllPairs && b.gq_slices >= 1, "grad_Q rounds");
    CHECK(((b.fwd.n_docs + b.gq_slices - 1) / b.gq_slices) * Ld * dim * esize < (1L << 32),
          "slice offsets");
  }
  if (b.gd_mode == kGdPairs) {
    // waves per document: at least the minimum, never more than the rows
    // allow beyond it, and the launch (4 waves per workgroup) fits the grid
    CHECK(layout != kAllPairs && Lq <= kPairsMaxLq, "pairs grad_D only for pairwise / kd");
    CHECK(b.gd_parts >= kGdPairsMinParts, "parts %d", b.gd_parts);
    CHECK(b.gd_parts == kGdPairsMinParts || (long)b.gd_parts * kGdPairsMinRows <= Ld,
          "parts %d for Ld %ld", b.gd_parts, Ld);
    CHECK(b.fwd.n_docs * b.gd_parts >= kGdPairsWaves || b.gd_parts == kGdPairsMinParts ||
              (long)b.gd_parts == Ld / kGdPairsMinRows,
          "parts %d do not fill the chip", b.gd_parts);
    CHECK((b.fwd.n_docs * b.gd_parts + 3) / 4 < (1L << 31), "grid");
  }
  CHECK(b.total >= b.fwd.fwd_bytes || !b.recompute, "bwd total");
}

int main() {
  const long dims[] = {64, 128, 256};
  const long Lqs[] = {1, 7, 20, 32, 33, 64, 100};
  const long Lds[] = {1, 31, 32, 33, 300, 1030, 2049, 2111, 8192, 32768};
  const long Nqs[] = {1, 2, 16, 128, 256};
  const long Nds[] = {1, 4, 75, 256, 1000};
  for (int elem = 0; elem < 4; ++elem)
    for (long dim : dims)
      for (long Lq : Lqs)
        for (long Ld : Lds)
          for (long Nq : Nqs)
            for (long Nd : Nds) {
              fwd_case(kAllPairs, elem, Nq, Lq, Nd, Ld, dim, true);
              fwd_case(kAllPairs, elem, Nq, Lq, Nd, Ld, dim, Nd % 2 == 0, true);
              fwd_case(kPairwise, elem, Nq, Lq, 1, Ld, dim, true);
              fwd_case(kKd, elem, Nq, Lq, 16, Ld, dim, false);
              bwd_case(kAllPairs, elem, Nq, Lq, Nd, Ld, dim);
              bwd_case(kPairwise, elem, Nq, Lq, 1, Ld, dim);
              bwd_case(kKd, elem, Nq, Lq, Nd % 32 + 1, Ld, dim);
            }
  // hit lists past the sorted kernel's 16-bit hit numbers: the workspace sort
  // in one batch, several batches, and one document per batch
  for (int elem = 0; elem < 4; ++elem) {
    bwd_case(kAllPairs, elem, 2100, 32, 150, 64, 128);
    bwd_case(kAllPairs, elem, 2100, 32, 600, 64, 128);
    bwd_case(kAllPairs, elem, 20000, 32, 1000, 300, 128);
    bwd_case(kAllPairs, elem, 4, 32, 3, 40000, 128);
    bwd_case(kPairwise, elem, 64, 100, 1, 32768, 128);
  }
  std::printf("fails %d\n", fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_launch_plan_invariants(tmp_path):
    src = tmp_path / "plan_check.cpp"
    exe = tmp_path / "plan_check"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert "fails 0" in r.stdout


def test_bench_work_accounting():
    """bench.work on a tiny all-pairs and a kd workload, against sums written
    out by hand: valid-token flops, and each input row counted once per step
    (in the forward's bytes)."""
    import sys

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import bench
    from maxsim_scoring_02_amd.workloads import Workload

    Q = torch.zeros((2, 3, 64), dtype=torch.bfloat16)
    D = torch.zeros((4, 5, 64), dtype=torch.bfloat16)
    qm = torch.tensor([[1, 1, 0], [1, 0, 0]], dtype=torch.bool)
    dm = torch.tensor([[1] * 5, [1, 1, 0, 0, 0], [0] * 5, [1, 0, 1, 0, 1]], dtype=torch.bool)
    w = Workload("t", "allpairs", "bf16", Q, D, qm, dm, None)
    f_fwd, f_bwd, b_fwd, b_bwd = bench.work(w)
    qv, dv = np.array([2, 1]), np.array([5, 2, 0, 3])
    assert f_fwd == 2 * 64 * qv.sum() * dv.sum()
    assert f_bwd == 4 * 64 * qv.sum() * 3                 # three non-empty documents
    pairs = 2 * 4
    assert b_fwd == (qv.sum() + dv.sum()) * 64 * 2 + qm.numel() + dm.numel() + pairs * 4 + pairs * 3 * 4
    assert b_bwd == pairs * 4 + pairs * 3 * 4 + 2 * 3 * 64 * 4 + 4 * 5 * 64 * 4
    # kd: B=2 queries with N=3 candidates of 7 tokens, no masks
    wk = Workload("k", "kd", "f16", torch.zeros((2, 4, 64), dtype=torch.float16),
                  torch.zeros((2, 3, 7, 64), dtype=torch.float16), None, None, None)
    f_fwd, f_bwd, b_fwd, b_bwd = bench.work(wk, keep_argmax=False)
    assert f_fwd == 2 * 64 * 4 * 7 * 6 and f_bwd == 4 * 64 * 4 * 6
    assert b_fwd == (2 * 4 + 6 * 7) * 64 * 2 + 6 * 4
