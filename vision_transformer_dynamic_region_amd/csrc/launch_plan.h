// Host-side launch arithmetic, plain C++ with no HIP types so that host-only
// tests can check it: how the persistent attention kernels deal units to
// XCDs and workgroups and how many images one launch may take (so that a
// workgroup's routing table of idx rows in LDS stays within a fixed size),
// and how the LePE backward splits rows into strips.
#pragma once

#include <cstddef>

namespace bra {

// LDS bytes a persistent attention workgroup may spend on its routing table.
// A batch whose table would be larger runs as several launches over image
// ranges; the table then never costs occupancy.
constexpr size_t kTableBytes = 8 * 1024;

// Units of a launch are split into `xcds` contiguous ranges of this many
// units (rounded up to a multiple of `align`, so that a workgroup's units
// share their channel block).
inline long long units_per_xcd(long long units, int xcds, int align) {
  const long long p = (units + xcds - 1) / xcds;
  return (p + align - 1) / align * align;
}

// Units one workgroup holds when a range of per_xcd units is dealt
// round-robin to bpx workgroups.
inline long long units_per_workgroup(long long per_xcd, long long bpx) {
  if (bpx > per_xcd) bpx = per_xcd;
  return bpx > 0 ? (per_xcd + bpx - 1) / bpx : 0;
}

// The largest image count b <= B for which a launch of b images
// (units_per_image units each) leaves every workgroup at most
// table_bytes / (4 * topk) units, given that the launcher deals each XCD's
// range to at least min_bpx workgroups.  Returns 0 when not even one image
// fits (the caller then takes a kernel without a table).
inline int images_per_launch(int B, long long units_per_image, int xcds, int align, int min_bpx,
                             int topk, size_t table_bytes) {
  if (B < 1 || units_per_image < 1 || topk < 1 || min_bpx < 1) return 0;
  const long long cap = (long long)(table_bytes / (4 * (size_t)topk));
  auto fits = [&](long long b) {
    return units_per_workgroup(units_per_xcd(b * units_per_image, xcds, align), min_bpx) <= cap;
  };
  if (!fits(1)) return 0;
  long long lo = 1, hi = B;          // fits(lo); the table grows with b
  while (lo < hi) {
    const long long mid = lo + (hi - lo + 1) / 2;
    if (fits(mid)) lo = mid;
    else hi = mid - 1;
  }
  return (int)lo;
}

// Thread counts of the kernels' workgroups (the device code asserts these).
constexpr int kPlanThreads = 256, kPlanWaves = 4;

// LePE backward (the dw / db partial sums and the LePE term of dV): a
// workgroup takes cpb channel pairs of xc thread columns, each thread NCOL
// adjacent pixel columns, over a strip of sr rows; every (image, strip,
// column block) writes one partial row of C x (ks*ks + 1) float32 sums.
struct DwPlan {
  int cpb, xc, nxb, ncb, sr, nstrips;   // pairs/workgroup, columns/workgroup, blocks, strip rows
  long long rows;                       // partial rows
};
constexpr int kMaxCols = 16;            // thread columns of a workgroup: 256 / (C / 2), C >= 32

// columns per thread of the LePE backward kernel: two up to 5 x 5 (the
// weights and dw sums of a channel pair are then shared by twice the
// pixels), else one
inline int lepe_cols(int ks) { return ks <= 5 ? 2 : 1; }

inline DwPlan dw_plan(int B, int H, int W, int C, int ks) {
  const int ncol = lepe_cols(ks);
  DwPlan p;
  const int CP = C / 2;
  p.cpb = CP < kPlanThreads ? CP : kPlanThreads;
  p.xc = kPlanThreads / p.cpb;
  if (p.xc > kMaxCols) p.xc = kMaxCols;
  p.nxb = (W + p.xc * ncol - 1) / (p.xc * ncol);
  p.ncb = (CP + p.cpb - 1) / p.cpb;
  // row strips for one generation of resident wavefronts: 1024 SIMDs (256
  // CUs x 4) times the wavefronts a SIMD holds at the kernel's register use
  // (4 up to 3 x 3, 2 at 5 x 5, 1 at 7 x 7).  A second generation would pay
  // the strip prologue and the batch waits again, and on MI355X ran 25-40%
  // slower; strips stay at least two batches long, so the KS - 1 halo rows
  // each strip reads stay a small share
  const long long waves = (long long)B * p.nxb * p.ncb * kPlanWaves;
  const long long target = 1024LL * (ks <= 3 ? 4 : ks == 5 ? 2 : 1);
  long long ns = (target + waves - 1) / waves;
  const long long nmax = H / (2 * ks) > 1 ? H / (2 * ks) : 1;
  if (ns > nmax) ns = nmax;
  if (ns < 1) ns = 1;
  p.sr = (int)((H + ns - 1) / ns);
  p.nstrips = (H + p.sr - 1) / p.sr;
  p.rows = (long long)B * p.nstrips * p.nxb;
  return p;
}

}  // namespace bra
