// Host-only helpers the C-ABI front end uses to validate and size calls:
// workspace bytes of the backward pass and the LayerNorm lane split.  Plain
// C++ (no device code), so the front end can be built and checked for the
// host alone.

#include <cstddef>

#include "bra_internal.h"
#include "launch_plan.h"

namespace bra {

size_t bwd_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk, int ks,
                           bool lepe) {
  (void)S; (void)topk;
  const size_t px = (size_t)B * H * W;
  size_t bytes = 2 * px * heads * sizeof(float);                   // lse, D
  bytes = (bytes + 255) / 256 * 256;
  if (lepe) {
    const DwPlan p = dw_plan(B, H, W, C, ks);
    bytes += px * C * sizeof(float);                               // dV_L
    bytes += (size_t)p.rows * C * (ks * ks + 1) * sizeof(float);   // dw / db partial rows
  }
  return (bytes + 255) / 256 * 256;
}

// L lanes per row (a power of two up to 64 dividing the row's 16-byte
// groups), each holding NG <= 4 groups.
bool layer_norm_shape(int C, bool bf16, int* L, int* NG) {
  const int vec = bf16 ? 8 : 4;
  if (C % vec) return false;
  const int G = C / vec;
  int l = 1;
  while (l * 2 <= 64 && G % (l * 2) == 0) l *= 2;
  if (G / l > 4) return false;
  *L = l;
  *NG = G / l;
  return true;
}

}  // namespace bra
