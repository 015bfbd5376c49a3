// Host check of the persistent attention launch arithmetic: a launch of
// images_per_launch(...) images keeps every workgroup's routing table within
// the byte limit, one more image would not (unless the whole batch fits),
// and the image ranges of a batch cover it exactly.
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "launch_plan.h"

using namespace bra;

static long long checked = 0;

static void fail(const char* what, int B, long long upi, int align, int min_bpx, int topk) {
  std::printf("FAIL %s B=%d upi=%lld align=%d min_bpx=%d topk=%d\n", what, B, upi, align, min_bpx,
              topk);
  std::exit(1);
}

static long long table_units(long long images, long long upi, int align, int min_bpx) {
  return units_per_workgroup(units_per_xcd(images * upi, 8, align), min_bpx);
}

static void check(int B, long long upi, int align, int min_bpx, int topk, size_t bytes) {
  ++checked;
  const int per = images_per_launch(B, upi, 8, align, min_bpx, topk, bytes);
  const long long cap = (long long)(bytes / (4 * (size_t)topk));
  if (per < 0 || per > B) fail("range", B, upi, align, min_bpx, topk);
  if (per == 0) {
    if (table_units(1, upi, align, min_bpx) <= cap) fail("one image fits", B, upi, align, min_bpx, topk);
    return;
  }
  if (table_units(per, upi, align, min_bpx) > cap) fail("table too big", B, upi, align, min_bpx, topk);
  if (per < B && table_units(per + 1, upi, align, min_bpx) <= cap)
    fail("not the largest", B, upi, align, min_bpx, topk);
  // the launches of a batch cover it exactly
  long long covered = 0;
  for (int b0 = 0; b0 < B; b0 += per) covered += (B - b0 < per ? B - b0 : per);
  if (covered != B) fail("cover", B, upi, align, min_bpx, topk);
}

int main() {
  // units_per_xcd: contiguous ranges of whole channel blocks
  for (long long u = 0; u < 5000; ++u)
    for (int align : {1, 2, 4}) {
      const long long p = units_per_xcd(u, 8, align);
      if (p % align || p * 8 < u || (p - align) * 8 >= u + 8 * align) {
        std::printf("FAIL units_per_xcd %lld %d -> %lld\n", u, align, p);
        return 1;
      }
    }
  // the workload shapes: one launch at their batch sizes
  //   st1 (R 49, 2 channel blocks, top-1), st2 (R 49, top-4), st3 (R 49, 2 blocks, top-16),
  //   dense (R 256, 2 blocks, top-4)
  struct { int B; long long upi; int align, topk; } wl[] = {
      {64, 98, 2, 1}, {64, 49, 1, 4}, {64, 98, 2, 16}, {8, 512, 2, 4}};
  for (auto& w : wl)
    if (images_per_launch(w.B, w.upi, 8, w.align, 32, w.topk, kTableBytes) != w.B) {
      std::printf("FAIL workload shape B=%d split\n", w.B);
      return 1;
    }
  // large batches split; the dense shape at B = 3520 used to need a 112 KB table
  if (images_per_launch(3520, 512, 8, 2, 32, 4, kTableBytes) >= 3520) {
    std::printf("FAIL dense B=3520 not split\n");
    return 1;
  }
  for (int B : {1, 2, 3, 7, 64, 100, 333, 334, 335, 1000, 4600, 4800, 100000})
    for (long long upi : {1LL, 4LL, 49LL, 98LL, 196LL, 512LL, 1024LL, 4096LL})
      for (int align : {1, 2, 4})
        for (int min_bpx : {1, 4, 28, 32, 64})
          for (int topk : {1, 2, 4, 16, 64, 256, 1024, 4096})
            check(B, upi * align, align, min_bpx, topk, kTableBytes);
  std::printf("ok %lld\n", checked);
  return 0;
}
