// Host check of the C-ABI front end under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with arguments it
// must reject, and each call must return the expected status, before any
// launch, with a non-empty error text.  The pointers are fake, 16-byte
// aligned addresses that are never dereferenced; no call here passes
// validation, so nothing reaches the GPU.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "../../include/bra.h"

namespace {

int failures = 0, checked = 0;

void* ptr(uintptr_t a) { return reinterpret_cast<void*>(a); }
const float* fp(uintptr_t a) { return reinterpret_cast<const float*>(a); }
int32_t* ip(uintptr_t a) { return reinterpret_cast<int32_t*>(a); }

const uintptr_t P = 0x10000, P2 = 0x20000000, P3 = 0x40000000, P4 = 0x60000000,
                PO = 0x70000000, PW = 0x7A000000, P5 = 0x50000000;

void expect(const char* what, bra_status got, bra_status want, const char* msg) {
  ++checked;
  const char* err = bra_last_error();
  if (got != want || std::strlen(err) == 0 || (msg && !std::strstr(err, msg))) {
    std::printf("FAIL %s: status %d (want %d), error \"%s\" (want \"%s\")\n", what, (int)got,
                (int)want, err, msg ? msg : "");
    ++failures;
  }
}

bra_status route(uintptr_t q = P, int H = 8, int S = 2, int topk = 2, int C = 64,
                 float scale = 0.125f, uintptr_t idx = P3, uintptr_t ws = P4,
                 size_t wsb = 1 << 20, int dt = BRA_BF16) {
  return bra_route(ptr(q), ptr(P2), 2, H, 8, C, S, topk, (bra_dtype)dt, scale, ip(idx), nullptr,
                   ptr(ws), wsb, nullptr);
}

bra_status attend(int heads = 2, int C = 64, float scale = 0.17f, uintptr_t w = 0, int ks = 5,
                  uintptr_t b = 0, uintptr_t out = PO, uintptr_t v = P3, int topk = 2) {
  return bra_attend(ptr(P), ptr(P2), ptr(v), ip(P4), 2, 8, 8, C, heads, 2, topk, BRA_BF16, scale,
                    fp(w), fp(b), ks, ptr(out), nullptr);
}

}  // namespace

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  // sizes
  if (bra_workspace_bytes(64, 7, 64) != 2ull * 64 * 49 * 64 * 8 || bra_workspace_bytes(0, 7, 64))
    ++failures;
  if (bra_video_workspace_bytes(2, 4, 2, 64) != 2ull * 2 * 4 * 4 * 64 * 8) ++failures;
  if (bra_module_workspace_bytes(0, 8, 8, 64, 2, BRA_BF16, 1) ||
      bra_block_workspace_bytes(2, 8, 8, 64, 0, BRA_BF16))
    ++failures;
  if (!(bra_backward_workspace_bytes(2, 8, 8, 64, 2, 2, 2, 5) >
        bra_backward_workspace_bytes(2, 8, 8, 64, 2, 2, 2, 0)))
    ++failures;
  if (std::strcmp(bra_strerror(0), "ok") || std::strcmp(bra_strerror(99), "unknown status")) ++failures;

  // bra_route
  expect("route H", route(P, 9), BRA_E_INVAL, "divide");
  expect("route topk 0", route(P, 8, 2, 0), BRA_E_INVAL, "topk");
  expect("route topk 5", route(P, 8, 2, 5), BRA_E_INVAL, "topk");
  expect("route q null", route(0), BRA_E_INVAL, "q is NULL");
  expect("route q align", route(P + 8), BRA_E_INVAL, "aligned");
  expect("route idx null", route(P, 8, 2, 2, 64, 0.125f, 0), BRA_E_INVAL, "idx");
  expect("route scale 0", route(P, 8, 2, 2, 64, 0.f), BRA_E_INVAL, "route_scale");
  expect("route scale nan", route(P, 8, 2, 2, 64, nan), BRA_E_INVAL, "route_scale");
  expect("route scale inf", route(P, 8, 2, 2, 64, inf), BRA_E_INVAL, "route_scale");
  expect("route ws null", route(P, 8, 2, 2, 64, 0.125f, P3, 0), BRA_E_WORKSPACE, "NULL");
  expect("route ws small", route(P, 8, 2, 2, 64, 0.125f, P3, P4, 100), BRA_E_WORKSPACE, "needed");
  expect("route dtype", route(P, 8, 2, 2, 64, 0.125f, P3, P4, 1 << 20, 7), BRA_E_INVAL, "dtype");
  expect("route C 60", route(P, 8, 2, 2, 60), BRA_E_UNSUPPORTED, "multiple of 8");
  expect("route C 2048", route(P, 8, 2, 2, 2048), BRA_E_UNSUPPORTED, "exceeds");

  // bra_attend
  expect("attend heads 3", attend(3), BRA_E_INVAL, "heads");
  expect("attend heads 0", attend(0), BRA_E_INVAL, "heads");
  expect("attend head width", attend(1), BRA_E_UNSUPPORTED, "head width");
  expect("attend v null", attend(2, 64, 0.17f, 0, 5, 0, PO, 0), BRA_E_INVAL, "v is NULL");
  expect("attend out null", attend(2, 64, 0.17f, 0, 5, 0, 0), BRA_E_INVAL, "out is NULL");
  expect("attend out overlaps", attend(2, 64, 0.17f, 0, 5, 0, P + 1024), BRA_E_INVAL, "overlaps");
  expect("attend scale inf", attend(2, 64, inf), BRA_E_INVAL, "attn_scale");
  expect("attend scale neg", attend(2, 64, -0.2f), BRA_E_INVAL, "attn_scale");
  expect("attend ks 4", attend(2, 64, 0.17f, P, 4), BRA_E_UNSUPPORTED, "lepe_ks");
  expect("attend ks 9", attend(2, 64, 0.17f, P, 9), BRA_E_UNSUPPORTED, "lepe_ks");
  expect("attend bias align", attend(2, 64, 0.17f, P, 5, P + 4), BRA_E_INVAL, "bias");
  expect("attend topk 9", attend(2, 64, 0.17f, 0, 5, 0, PO, P3, 9), BRA_E_INVAL, "topk");

  // bra_forward: both halves are checked before anything runs
  expect("forward ws", bra_forward(ptr(P), ptr(P2), ptr(P3), 2, 8, 8, 64, 2, 2, 2, BRA_BF16,
                                   0.125f, 0.17f, nullptr, nullptr, 5, ptr(PO), ip(P4), nullptr,
                                   nullptr, 0, nullptr),
         BRA_E_WORKSPACE, nullptr);
  expect("forward heads", bra_forward(ptr(P), ptr(P2), ptr(P3), 2, 8, 8, 64, 3, 2, 2, BRA_BF16,
                                      0.125f, 0.17f, nullptr, nullptr, 5, ptr(PO), ip(P4),
                                      nullptr, ptr(PW), 1 << 20, nullptr),
         BRA_E_INVAL, "heads");

  // bra_forward_noalloc: the means must fit the static scratch
  expect("noalloc too big", bra_forward_noalloc(ptr(P), ptr(P2), ptr(P3), 1024, 64, 64, 256, 8, 8, 4,
                                                BRA_BF16, 0.125f, 0.17f, nullptr, nullptr, 5,
                                                ptr(PO), ip(P4), nullptr, nullptr),
         BRA_E_UNSUPPORTED, "scratch");
  expect("noalloc heads", bra_forward_noalloc(ptr(P), ptr(P2), ptr(P3), 2, 8, 8, 64, 3, 2, 2,
                                              BRA_BF16, 0.125f, 0.17f, nullptr, nullptr, 5,
                                              ptr(PO), ip(P4), nullptr, nullptr),
         BRA_E_INVAL, "heads");
  expect("noalloc out overlaps", bra_forward_noalloc(ptr(P), ptr(P2), ptr(P3), 2, 8, 8, 64, 2, 2,
                                                     2, BRA_BF16, 0.125f, 0.17f, nullptr, nullptr,
                                                     5, ptr(P + 1024), ip(P4), nullptr, nullptr),
         BRA_E_INVAL, "overlaps");

  // bra_lepe
  expect("lepe C", bra_lepe(ptr(P), fp(P2), nullptr, 5, 2, 8, 8, 48, BRA_BF16, ptr(P3), nullptr),
         BRA_E_UNSUPPORTED, nullptr);
  expect("lepe w null", bra_lepe(ptr(P), nullptr, nullptr, 5, 2, 8, 8, 64, BRA_BF16, ptr(P3),
                                 nullptr), BRA_E_INVAL, nullptr);
  expect("lepe overlap", bra_lepe(ptr(P), fp(P2), nullptr, 5, 2, 8, 8, 64, BRA_BF16, ptr(P + 64),
                                  nullptr), BRA_E_INVAL, nullptr);

  // bra_linear
  expect("linear K", bra_linear(ptr(P), 100, 48, ptr(P2), nullptr, 64, 0, nullptr, BRA_BF16,
                                ptr(P4), nullptr), BRA_E_UNSUPPORTED, "multiple of 32");
  expect("linear rows", bra_linear(ptr(P), 0, 64, ptr(P2), nullptr, 64, 0, nullptr, BRA_BF16,
                                   ptr(P4), nullptr), BRA_E_INVAL, "positive");
  expect("linear act", bra_linear(ptr(P), 100, 64, ptr(P2), nullptr, 64, 2, nullptr, BRA_BF16,
                                  ptr(P4), nullptr), BRA_E_INVAL, "act");
  expect("linear big", bra_linear(ptr(P), 1 << 24, 64, ptr(P2), nullptr, 64, 0, nullptr,
                                  BRA_BF16, ptr(P4), nullptr), BRA_E_UNSUPPORTED, "2 GiB");

  // bra_mlp
  expect("mlp f32", bra_mlp(ptr(P), 100, 64, 192, ptr(P2), nullptr, ptr(P3), nullptr, ptr(P5),
                            BRA_F32, ptr(P4), nullptr), BRA_E_UNSUPPORTED, "bf16 only");
  expect("mlp C", bra_mlp(ptr(P), 100, 96, 288, ptr(P2), nullptr, ptr(P3), nullptr, ptr(P5),
                          BRA_BF16, ptr(P4), nullptr), BRA_E_UNSUPPORTED, "C in");
  expect("mlp Hd", bra_mlp(ptr(P), 100, 64, 100, ptr(P2), nullptr, ptr(P3), nullptr, ptr(P5),
                           BRA_BF16, ptr(P4), nullptr), BRA_E_UNSUPPORTED, "Hd");
  expect("mlp x null", bra_mlp(nullptr, 100, 64, 192, ptr(P2), nullptr, ptr(P3), nullptr, ptr(P5),
                               BRA_BF16, ptr(P4), nullptr), BRA_E_INVAL, "x is NULL");
  expect("mlp b1 align", bra_mlp(ptr(P), 100, 64, 192, ptr(P2), fp(P3 + 4), ptr(P3), nullptr,
                                 ptr(P5), BRA_BF16, ptr(P4), nullptr), BRA_E_INVAL, "aligned");
  expect("mlp overlap", bra_mlp(ptr(P), 100, 64, 192, ptr(P2), nullptr, ptr(P3), nullptr,
                                ptr(P5), BRA_BF16, ptr(P + 64), nullptr), BRA_E_INVAL, "overlaps x");
  expect("mlp big", bra_mlp(ptr(P), 1 << 24, 64, 192, ptr(P2), nullptr, ptr(P3), nullptr,
                            ptr(P5), BRA_BF16, ptr(P4), nullptr), BRA_E_UNSUPPORTED, "2 GiB");

  // bra_module_forward
  expect("module w_qkv", bra_module_forward(ptr(P), 2, 8, 8, 64, 2, 2, 2, BRA_BF16, nullptr,
                                            nullptr, 0.125f, 0.17f, nullptr, nullptr, 5, nullptr,
                                            nullptr, ptr(PO), ip(P4), ptr(PW), 1 << 24, nullptr),
         BRA_E_INVAL, "w_qkv is NULL");
  expect("module ws", bra_module_forward(ptr(P), 2, 8, 8, 64, 2, 2, 2, BRA_BF16, ptr(P2), nullptr,
                                         0.125f, 0.17f, nullptr, nullptr, 5, nullptr, nullptr,
                                         ptr(PO), ip(P4), ptr(PW), 1000, nullptr),
         BRA_E_WORKSPACE, "needed");
  expect("module b_out", bra_module_forward(ptr(P), 2, 8, 8, 64, 2, 2, 2, BRA_BF16, ptr(P2),
                                            nullptr, 0.125f, 0.17f, nullptr, nullptr, 5, nullptr,
                                            fp(P3), ptr(PO), ip(P4), ptr(PW), 1 << 24, nullptr),
         BRA_E_INVAL, "without w_out");

  // bra_layer_norm, bra_pos_conv
  expect("ln C", bra_layer_norm(ptr(P), 100, 60, fp(P2), fp(P3), 1e-5f, BRA_BF16, ptr(P4), nullptr),
         BRA_E_UNSUPPORTED, "multiple of 8");
  expect("ln eps", bra_layer_norm(ptr(P), 100, 64, fp(P2), fp(P3), 0.f, BRA_BF16, ptr(P4), nullptr),
         BRA_E_INVAL, "eps");
  expect("pos w", bra_pos_conv(ptr(P), nullptr, nullptr, 2, 8, 8, 64, BRA_BF16, ptr(P4), nullptr),
         BRA_E_INVAL, nullptr);
  expect("pos overlap", bra_pos_conv(ptr(P), fp(P2), nullptr, 2, 8, 8, 64, BRA_BF16, ptr(P + 64),
                                     nullptr), BRA_E_INVAL, nullptr);

  // bra_block_forward
  bra_block_params bp;
  std::memset(&bp, 0, sizeof(bp));
  expect("block params", bra_block_forward(ptr(P), 2, 8, 8, 64, 2, 2, 2, BRA_BF16, nullptr, 0.125f,
                                           0.17f, ptr(PO), ip(P4), ptr(PW), 1 << 26, nullptr),
         BRA_E_INVAL, "params is NULL");
  bp.pos_w = fp(0x1000000); bp.ln1_g = fp(0x1100000); bp.ln1_b = fp(0x1200000);
  bp.w_qkv = ptr(0x1300000); bp.w_out = ptr(0x1400000); bp.ln2_g = fp(0x1500000);
  bp.ln2_b = fp(0x1600000); bp.w_fc1 = ptr(0x1700000);
  expect("block fc2", bra_block_forward(ptr(P), 2, 8, 8, 64, 2, 2, 2, BRA_BF16, &bp, 0.125f, 0.17f,
                                        ptr(PO), ip(P4), ptr(PW), 1 << 26, nullptr),
         BRA_E_INVAL, "w_fc2");

  // bra_attend_backward
  expect("bwd f32", bra_attend_backward(ptr(P), ptr(P2), ptr(P3), ip(P4), ptr(0x50000000), 2, 8, 8,
                                        64, 2, 2, 2, BRA_F32, 0.17f, nullptr, 5, ptr(PO),
                                        ptr(0x74000000), ptr(0x78000000), nullptr, nullptr,
                                        ptr(0x7C000000), 1 << 26, nullptr),
         BRA_E_UNSUPPORTED, "bf16");
  expect("bwd overlap", bra_attend_backward(ptr(P), ptr(P2), ptr(P3), ip(P4), ptr(0x50000000), 2, 8,
                                            8, 64, 2, 2, 2, BRA_BF16, 0.17f, nullptr, 5, ptr(P2),
                                            ptr(0x74000000), ptr(0x78000000), nullptr, nullptr,
                                            ptr(0x7C000000), 1 << 26, nullptr),
         BRA_E_INVAL, "overlaps");
  expect("bwd ws", bra_attend_backward(ptr(P), ptr(P2), ptr(P3), ip(P4), ptr(0x50000000), 2, 8, 8,
                                       64, 2, 2, 2, BRA_BF16, 0.17f, nullptr, 5, ptr(PO),
                                       ptr(0x74000000), ptr(0x78000000), nullptr, nullptr,
                                       ptr(0x7C000000), 16, nullptr),
         BRA_E_WORKSPACE, nullptr);

  // video
  auto vf = [&](int T, int S, int topk, size_t wsb) {
    return bra_video_forward(ptr(P), ptr(P2), ptr(P3), 2, T, 16, 16, 64, 2, S, topk, BRA_BF16,
                             0.125f, 0.17f, nullptr, nullptr, 5, ptr(PO), ip(0x74000000), nullptr,
                             ptr(0x7C000000), wsb, nullptr);
  };
  expect("video T", vf(0, 2, 3, 1 << 26), BRA_E_INVAL, "T=0");
  expect("video S", vf(4, 3, 3, 1 << 26), BRA_E_INVAL, nullptr);
  expect("video topk", vf(4, 2, 17, 1 << 26), BRA_E_INVAL, "T*S*S=16");
  expect("video ws", vf(4, 2, 3, 16), BRA_E_WORKSPACE, nullptr);
  expect("video route ws", bra_video_route(ptr(P), ptr(P2), 2, 4, 16, 16, 64, 2, 3, BRA_BF16,
                                           0.125f, ip(0x74000000), nullptr, ptr(0x7C000000), 16,
                                           nullptr),
         BRA_E_WORKSPACE, nullptr);
  expect("video attend out", bra_video_attend(ptr(P), ptr(P2), ptr(P3), ip(P4), 2, 4, 16, 16, 64, 2,
                                              2, 3, BRA_BF16, 0.17f, nullptr, nullptr, 5, nullptr,
                                              nullptr),
         BRA_E_INVAL, "out is NULL");

  if (failures) {
    std::printf("%d of %d checks failed\n", failures, checked);
    return 1;
  }
  std::printf("ok %d\n", checked);
  return 0;
}
