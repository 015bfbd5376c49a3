// C-ABI front end of libbra: argument checks, workspace layout and the
// launch sequence of the BRA forward pass.  Every check runs on the host
// before anything is enqueued, so a rejected call leaves the stream untouched.
//
// Page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层路由注意力机制解析"
// (§3 step list), p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何革新
// 视觉Transformer的计算范式" (§4 TopkRouting and the LePE conv, §5 fixed index).

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bra.h"
#include "bra_internal.h"

namespace {

thread_local char g_last_error[512] = "";

bra_status fail(bra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

constexpr int kHeadDim = 32;
constexpr int kMaxRegions = 1024;
constexpr int kMaxLepeRowBlocks = 65535;   // grid y of the LePE launch

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_size(bra_dtype dt) { return dt == BRA_F32 ? 4 : 2; }

bool overlaps(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

// [a, a + an) and [b, b + bn) intersect
bool overlaps2(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

// Shape checks shared by every entry point.  heads <= 0 means "not used".
bra_status check_shape(int B, int H, int W, int C, int S, int heads, int topk, bra_dtype dt,
                       bra::Shape* out) {
  if (dt != BRA_F32 && dt != BRA_BF16) return fail(BRA_E_INVAL, "dtype %d is not BRA_F32 or BRA_BF16", (int)dt);
  if (B < 1 || H < 1 || W < 1 || C < 1 || S < 1)
    return fail(BRA_E_INVAL, "B=%d H=%d W=%d C=%d S=%d must all be positive", B, H, W, C, S);
  if (H % S || W % S) return fail(BRA_E_INVAL, "S=%d must divide H=%d and W=%d", S, H, W);
  if (S > 32 || S * S > kMaxRegions)
    return fail(BRA_E_UNSUPPORTED, "S*S=%lld regions exceed the supported %d", (long long)S * S, kMaxRegions);
  if (topk < 1 || topk > S * S) return fail(BRA_E_INVAL, "topk=%d must be in [1, S*S=%d]", topk, S * S);
  if (heads != 0) {
    if (heads < 1 || C % heads) return fail(BRA_E_INVAL, "heads=%d must divide C=%d", heads, C);
    if (C / heads != kHeadDim)
      return fail(BRA_E_UNSUPPORTED, "head width C/heads=%d; only %d is supported", C / heads, kHeadDim);
  }
  if (C % 8) return fail(BRA_E_UNSUPPORTED, "C=%d must be a multiple of 8", C);
  const int cmax = dt == BRA_BF16 ? 1024 : 512;
  if (C > cmax) return fail(BRA_E_UNSUPPORTED, "C=%d exceeds %d for this dtype", C, cmax);
  const long long pixels = (long long)B * H * W;
  if (pixels > (1LL << 31) / 8 || (long long)B * S * S > (1LL << 24))
    return fail(BRA_E_UNSUPPORTED, "problem too large (B*H*W=%lld)", pixels);
  if ((long long)H * W * C >= (1LL << 31))
    return fail(BRA_E_UNSUPPORTED, "one image of H*W*C=%lld elements exceeds 2^31", (long long)H * W * C);
  const long long n = (long long)(H / S) * (W / S);
  if (n * topk > (1LL << 30)) return fail(BRA_E_UNSUPPORTED, "topk*n=%lld keys per query is too many", n * topk);
  bra::Shape s;
  s.B = B; s.H = H; s.W = W; s.C = C; s.S = S; s.heads = heads; s.topk = topk;
  s.hs = H / S; s.ws = W / S; s.n = (int)n; s.R = S * S; s.Hf = H;
  *out = s;
  return BRA_OK;
}

bra_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(BRA_E_INVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(BRA_E_INVAL, "%s is not 16-byte aligned", name);
  return BRA_OK;
}

bra_status check_route_args(const void* q, const void* k, const bra::Shape& s, bra_dtype dt,
                            float route_scale, const int32_t* idx, const float* logits,
                            const void* ws, size_t ws_bytes) {
  bra_status st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k"))) return st;
  if (!idx) return fail(BRA_E_INVAL, "idx is NULL");
  if ((uintptr_t)idx & 3u) return fail(BRA_E_INVAL, "idx is not 4-byte aligned");
  if (logits && ((uintptr_t)logits & 3u)) return fail(BRA_E_INVAL, "topk_logits is not 4-byte aligned");
  if (!(route_scale > 0.f) || !std::isfinite(route_scale))
    return fail(BRA_E_INVAL, "route_scale=%g must be positive and finite", (double)route_scale);
  const size_t need = (size_t)2 * s.B * s.R * s.C * sizeof(double);   // means of q, then k
  if (!ws) return fail(BRA_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(BRA_E_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(BRA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  (void)dt;
  return BRA_OK;
}

bra_status check_lepe_args(const float* w, const float* b, int ks, const bra::Shape& s) {
  if (!w) return fail(BRA_E_INVAL, "lepe weight is NULL");
  if ((uintptr_t)w & 3u) return fail(BRA_E_INVAL, "lepe weight is not 4-byte aligned");
  if (b && !aligned16(b)) return fail(BRA_E_INVAL, "lepe bias is not 16-byte aligned");
  if (ks < 1 || ks > 7 || ks % 2 == 0) return fail(BRA_E_UNSUPPORTED, "lepe_ks=%d must be odd in 1..7", ks);
  if (s.C % 32) return fail(BRA_E_UNSUPPORTED, "LePE needs C=%d to be a multiple of 32", s.C);
  const long long strips = (s.H + 7) / 8;
  if ((long long)s.B * strips > kMaxLepeRowBlocks)
    return fail(BRA_E_UNSUPPORTED, "B*ceil(H/8)=%lld too large for the LePE grid", (long long)s.B * strips);
  return BRA_OK;
}

bra_status check_attend_args(const void* q, const void* k, const void* v, const int32_t* idx,
                             const bra::Shape& s, bra_dtype dt, float attn_scale,
                             const float* w, const float* b, int ks, const void* out) {
  bra_status st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(out, "out")))
    return st;
  if (!idx) return fail(BRA_E_INVAL, "idx is NULL");
  if ((uintptr_t)idx & 3u) return fail(BRA_E_INVAL, "idx is not 4-byte aligned");
  if (!(attn_scale > 0.f) || !std::isfinite(attn_scale))
    return fail(BRA_E_INVAL, "attn_scale=%g must be positive and finite", (double)attn_scale);
  const size_t bytes = (size_t)s.B * s.H * s.W * s.C * elem_size(dt);
  if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
    return fail(BRA_E_INVAL, "out overlaps q, k or v");
  if (w && (st = check_lepe_args(w, b, ks, s))) return st;
  return BRA_OK;
}

constexpr long long kMaxOperandBytes = 1LL << 31;   // 32-bit buffer offsets

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the module workspace parts (see bra_module_workspace_bytes).
struct ModuleLayout {
  size_t xm, qm, km, q, k, v, y, total;
};

ModuleLayout module_layout(int B, int H, int W, int C, int S, bra_dtype dt, bool with_out) {
  ModuleLayout l;
  const size_t means = align256((size_t)B * S * S * C * sizeof(double));
  const size_t tensor = align256((size_t)B * H * W * C * elem_size(dt));
  l.xm = 0;
  l.qm = l.xm + means;
  l.km = l.qm + means;
  l.q = l.km + means;
  l.k = l.q + tensor;
  l.v = l.k + tensor;
  l.y = l.v + tensor;
  l.total = l.y + (with_out ? tensor : 0);
  return l;
}

bra_status check_bias(const float* b, const char* name) {
  if (b && !aligned16(b)) return fail(BRA_E_INVAL, "%s is not 16-byte aligned", name);
  return BRA_OK;
}

bra_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BRA_OK;
  return fail(BRA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLayerNormEps = 1e-5f;

// The module's launch sequence on validated arguments; ws holds the module
// workspace laid out as l.  With w_out, y goes to the workspace and out =
// y w_out^T + b_out (+ resid when resid is not null); without, out = y.
bra_status module_launches(const void* x, const bra::Shape& s, bra_dtype dtype, const void* w_qkv,
                           const float* b_qkv, float route_scale, float attn_scale,
                           const float* lepe_w, const float* lepe_b, int lepe_ks,
                           const void* w_out, const float* b_out, const void* resid, void* out,
                           int32_t* idx, unsigned char* w8, const ModuleLayout& l, hipStream_t hs) {
  bra_status st;
  const bool bf16 = dtype == BRA_BF16;
  const int C = s.C;
  double* xm = (double*)(w8 + l.xm);
  double* qm = (double*)(w8 + l.qm);
  double* km = (double*)(w8 + l.km);
  void* qkv[3] = {w8 + l.q, w8 + l.k, w8 + l.v};
  void* y = w_out ? (void*)(w8 + l.y) : out;
  const int T = s.B * s.H * s.W;
  // routing: region means of x, projected in float64 (mean commutes with
  // the per-token map), scaled affinity and top-k
  if ((st = hip_status(bra::launch_pool(x, nullptr, xm, nullptr, s, bf16, hs), "pool launch")))
    return st;
  if ((st = hip_status(bra::launch_means_proj(xm, s.B * s.R, C, w_qkv, b_qkv, bf16, qm, km, hs),
                       "means projection launch")))
    return st;
  if ((st = hip_status(bra::launch_route(qm, km, s, (double)route_scale, idx, nullptr, hs),
                       "route launch")))
    return st;
  const size_t xbytes = (size_t)T * C * elem_size(dtype);
  if (bf16 && bra::attend_xproj_ok(s, lepe_w, lepe_ks) && !overlaps(y, x, xbytes)) {
    // fused form: Q, K and V projected inside the attention kernel (the
    // workspace's Q, K and V parts stay unwritten); not when y is x's
    // memory, which that kernel still reads while it writes
    if ((st = hip_status(bra::launch_attend_xproj(x, w_qkv, b_qkv, idx, s, attn_scale, lepe_w,
                                                  lepe_b, lepe_ks, y, hs),
                         "fused attend launch")))
      return st;
  } else {
    // Q, K, V
    if ((st = hip_status(bra::launch_linear(x, T, C, w_qkv, b_qkv, 3 * C, qkv, 3, bf16, hs),
                         "qkv projection launch")))
      return st;
    // attention + LePE on the projected V
    if ((st = hip_status(bra::launch_attend(qkv[0], qkv[1], qkv[2], idx, s, bf16, attn_scale,
                                            lepe_w, lepe_b, lepe_ks, y, hs),
                         "attend launch")))
      return st;
  }
  if (!w_out) return BRA_OK;
  void* outs[1] = {out};
  return hip_status(bra::launch_linear(y, T, C, w_out, b_out, C, outs, 1, bf16, hs,
                                       resid ? 2 : 0, resid),
                    "output projection launch");
}

// Byte offsets of the block workspace: x1, n1, x2, n2 ([B,H,W,C] each), then
// a module workspace with its output projection (whose Q/K/V space later
// holds the [B,H,W,3C] hidden tensor of the MLP).
struct BlockLayout {
  size_t x1, n1, x2, n2, mod, total;
  ModuleLayout ml;
};

BlockLayout block_layout(int B, int H, int W, int C, int S, bra_dtype dt) {
  BlockLayout b;
  const size_t tensor = align256((size_t)B * H * W * C * elem_size(dt));
  b.x1 = 0;
  b.n1 = b.x1 + tensor;
  b.x2 = b.n1 + tensor;
  b.n2 = b.x2 + tensor;
  b.mod = b.n2 + tensor;
  b.ml = module_layout(B, H, W, C, S, dt, true);
  b.total = b.mod + b.ml.total;
  return b;
}

// region means and routing: one fused launch where it applies (up to 64
// regions), else pooling then routing.  keep_means: the means must be in
// qm, km afterwards (the fused launch otherwise keeps them on chip)
bra_status route_launches(const void* q, const void* k, const bra::Shape& s, bool bf16,
                          float route_scale, int32_t* idx, float* topk_logits, double* qm,
                          double* km, bool keep_means, hipStream_t hs) {
  bra_status st;
  const hipError_t e = bra::launch_pool_route(q, k, keep_means ? qm : nullptr,
                                              keep_means ? km : nullptr, s, bf16,
                                              (double)route_scale, idx, topk_logits, hs);
  if (e != hipErrorNotSupported) return hip_status(e, "pool-route launch");
  if ((st = hip_status(bra::launch_pool(q, k, qm, km, s, bf16, hs), "pool launch"))) return st;
  return hip_status(bra::launch_route(qm, km, s, (double)route_scale, idx, topk_logits, hs),
                    "route launch");
}

// pool, route, attend on validated arguments (an image batch or a clip batch)
bra_status forward_launches(const void* q, const void* k, const void* v, const bra::Shape& s,
                            bra_dtype dtype, float route_scale, float attn_scale,
                            const float* lepe_w, const float* lepe_b, int lepe_ks, void* out,
                            int32_t* idx, float* topk_logits, void* ws, void* stream) {
  bra_status st;
  hipStream_t hs = (hipStream_t)stream;
  const bool bf16 = dtype == BRA_BF16;
  double* qm = (double*)ws;
  double* km = qm + (size_t)s.B * s.R * s.C;
  if ((st = route_launches(q, k, s, bf16, route_scale, idx, topk_logits, qm, km, false, hs)))
    return st;
  return hip_status(bra::launch_attend(q, k, v, idx, s, bf16, attn_scale, lepe_w, lepe_b, lepe_ks,
                                       out, hs),
                    "attend launch");
}

// A clip batch [B, T, H, W, C] as the frame-stacked image batch [B, T*H, W, C]
// with a (T*S) x S region grid: region r = t*S*S + ry*S + rx, one frame each.
bra_status check_video_shape(int B, int T, int H, int W, int C, int S, int heads, int topk,
                             bra_dtype dt, bra::Shape* out) {
  bra_status st;
  if (T < 1) return fail(BRA_E_INVAL, "T=%d frames must be positive", T);
  if (heads < 0) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);   // 0: unused
  if ((long long)B * T > (1 << 30)) return fail(BRA_E_UNSUPPORTED, "B*T=%lld clips x frames", (long long)B * T);
  // one frame as an image of the batch of B*T frames
  if ((st = check_shape(B * T, H, W, C, S, heads, 1, dt, out))) return st;
  const long long R = (long long)T * S * S;
  if (R > kMaxRegions)
    return fail(BRA_E_UNSUPPORTED, "T*S*S=%lld regions per clip exceed the supported %d", R, kMaxRegions);
  if (topk < 1 || topk > R) return fail(BRA_E_INVAL, "topk=%d must be in [1, T*S*S=%lld]", topk, R);
  if ((long long)T * H * W * C >= (1LL << 31))
    return fail(BRA_E_UNSUPPORTED, "one clip of T*H*W*C=%lld elements exceeds 2^31", (long long)T * H * W * C);
  if ((long long)B * R > (1LL << 24)) return fail(BRA_E_UNSUPPORTED, "B*T*S*S=%lld regions", (long long)B * R);
  if ((long long)out->n * topk > (1LL << 30)) return fail(BRA_E_UNSUPPORTED, "topk*n too large");
  out->B = B;
  out->H = T * H;
  out->Hf = H;
  out->R = (int)R;
  out->topk = topk;
  return BRA_OK;
}

}  // namespace

extern "C" {

size_t bra_workspace_bytes(int B, int S, int C) {
  if (B < 1 || S < 1 || C < 1) return 0;
  return (size_t)2 * B * S * S * C * sizeof(double);
}

bra_status bra_route(const void* q, const void* k, int B, int H, int W, int C, int S, int topk,
                     bra_dtype dtype, float route_scale, int32_t* idx, float* topk_logits,
                     void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if ((st = check_shape(B, H, W, C, S, 0, topk, dtype, &s))) return st;
  if ((st = check_route_args(q, k, s, dtype, route_scale, idx, topk_logits, ws, ws_bytes))) return st;
  hipStream_t hs = (hipStream_t)stream;
  double* qm = (double*)ws;
  double* km = qm + (size_t)B * s.R * C;
  return route_launches(q, k, s, dtype == BRA_BF16, route_scale, idx, topk_logits, qm, km, true,
                        hs);
}

bra_status bra_attend(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                      int H, int W, int C, int heads, int S, int topk, bra_dtype dtype,
                      float attn_scale, const float* lepe_w, const float* lepe_b, int lepe_ks,
                      void* out, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_attend_args(q, k, v, idx, s, dtype, attn_scale, lepe_w, lepe_b, lepe_ks, out)))
    return st;
  hipStream_t hs = (hipStream_t)stream;
  const bool bf16 = dtype == BRA_BF16;
  return hip_status(bra::launch_attend(q, k, v, idx, s, bf16, attn_scale, lepe_w, lepe_b, lepe_ks,
                                       out, hs),
                    "attend launch");
}

bra_status bra_forward(const void* q, const void* k, const void* v, int B, int H, int W, int C,
                       int heads, int S, int topk, bra_dtype dtype, float route_scale,
                       float attn_scale, const float* lepe_w, const float* lepe_b, int lepe_ks,
                       void* out, int32_t* idx, float* topk_logits, void* ws, size_t ws_bytes,
                       void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_route_args(q, k, s, dtype, route_scale, idx, topk_logits, ws, ws_bytes))) return st;
  if ((st = check_attend_args(q, k, v, idx, s, dtype, attn_scale, lepe_w, lepe_b, lepe_ks, out)))
    return st;
  return forward_launches(q, k, v, s, dtype, route_scale, attn_scale, lepe_w, lepe_b, lepe_ks, out,
                          idx, topk_logits, ws, stream);
}

bra_status bra_forward_noalloc(const void* q, const void* k, const void* v, int B, int H, int W,
                               int C, int heads, int S, int topk, bra_dtype dtype,
                               float route_scale, float attn_scale, const float* lepe_w,
                               const float* lepe_b, int lepe_ks, void* out, int32_t* idx,
                               float* topk_logits, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  const size_t need = bra_workspace_bytes(B, S, C);
  if (need > bra::kScratchBytes)
    return fail(BRA_E_UNSUPPORTED,
                "needs %zu bytes of scratch (2*B*S*S*C*8); the static scratch holds %zu", need,
                bra::kScratchBytes);
  // the workspace checks below see the static scratch's size; its address
  // is looked up only once the arguments are valid
  const void* probe = reinterpret_cast<const void*>((uintptr_t)256);
  if ((st = check_route_args(q, k, s, dtype, route_scale, idx, topk_logits, probe,
                             bra::kScratchBytes)))
    return st;
  if ((st = check_attend_args(q, k, v, idx, s, dtype, attn_scale, lepe_w, lepe_b, lepe_ks, out)))
    return st;
  void* ws = nullptr;
  if ((st = hip_status(bra::scratch_buffer(&ws), "scratch lookup"))) return st;
  return forward_launches(q, k, v, s, dtype, route_scale, attn_scale, lepe_w, lepe_b, lepe_ks, out,
                          idx, topk_logits, ws, stream);
}

bra_status bra_video_route(const void* q, const void* k, int B, int T, int H, int W, int C, int S,
                           int topk, bra_dtype dtype, float route_scale, int32_t* idx,
                           float* topk_logits, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if ((st = check_video_shape(B, T, H, W, C, S, 0, topk, dtype, &s))) return st;
  if ((st = check_route_args(q, k, s, dtype, route_scale, idx, topk_logits, ws, ws_bytes))) return st;
  hipStream_t hs = (hipStream_t)stream;
  double* qm = (double*)ws;
  double* km = qm + (size_t)B * s.R * C;
  return route_launches(q, k, s, dtype == BRA_BF16, route_scale, idx, topk_logits, qm, km, true,
                        hs);
}

bra_status bra_video_attend(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                            int T, int H, int W, int C, int heads, int S, int topk,
                            bra_dtype dtype, float attn_scale, const float* lepe_w,
                            const float* lepe_b, int lepe_ks, void* out, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_video_shape(B, T, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_attend_args(q, k, v, idx, s, dtype, attn_scale, lepe_w, lepe_b, lepe_ks, out)))
    return st;
  if (lepe_w) {
    bra::Shape f = s;
    f.B = B * T;
    f.H = H;
    if ((st = check_lepe_args(lepe_w, lepe_b, lepe_ks, f))) return st;
  }
  return hip_status(bra::launch_attend(q, k, v, idx, s, dtype == BRA_BF16, attn_scale, lepe_w,
                                       lepe_b, lepe_ks, out, (hipStream_t)stream),
                    "attend launch");
}

size_t bra_video_workspace_bytes(int B, int T, int S, int C) {
  if (B < 1 || T < 1 || S < 1 || C < 1) return 0;
  return (size_t)2 * B * T * S * S * C * sizeof(double);
}

bra_status bra_video_forward(const void* q, const void* k, const void* v, int B, int T, int H,
                             int W, int C, int heads, int S, int topk, bra_dtype dtype,
                             float route_scale, float attn_scale, const float* lepe_w,
                             const float* lepe_b, int lepe_ks, void* out, int32_t* idx,
                             float* topk_logits, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_video_shape(B, T, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_route_args(q, k, s, dtype, route_scale, idx, topk_logits, ws, ws_bytes))) return st;
  if ((st = check_attend_args(q, k, v, idx, s, dtype, attn_scale, lepe_w, lepe_b, lepe_ks, out)))
    return st;
  if (lepe_w) {
    // the LePE grid runs over the batch of B*T frames
    bra::Shape f = s;
    f.B = B * T;
    f.H = H;
    if ((st = check_lepe_args(lepe_w, lepe_b, lepe_ks, f))) return st;
  }
  return forward_launches(q, k, v, s, dtype, route_scale, attn_scale, lepe_w, lepe_b, lepe_ks, out,
                          idx, topk_logits, ws, stream);
}


bra_status bra_lepe(const void* v, const float* w, const float* b, int ks, int B, int H, int W,
                    int C, bra_dtype dtype, void* out, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  // LePE has no regions: validate as a single region holding the whole map.
  if ((st = check_shape(B, H, W, C, 1, 0, 1, dtype, &s))) return st;
  if ((st = check_tensor(v, "v")) || (st = check_tensor(out, "out"))) return st;
  if (overlaps(out, v, (size_t)B * H * W * C * elem_size(dtype))) return fail(BRA_E_INVAL, "out overlaps v");
  if ((st = check_lepe_args(w, b, ks, s))) return st;
  return hip_status(bra::launch_lepe(v, w, b, ks, s, dtype == BRA_BF16, out, (hipStream_t)stream),
                    "lepe launch");
}

bra_status bra_linear(const void* x, int rows, int K, const void* w, const float* b, int N,
                      int act, const void* r, bra_dtype dtype, void* y, void* stream) {
  g_last_error[0] = 0;
  bra_status st;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return fail(BRA_E_INVAL, "dtype %d is not BRA_F32 or BRA_BF16", (int)dtype);
  if (rows < 1 || K < 1 || N < 1) return fail(BRA_E_INVAL, "rows=%d K=%d N=%d must be positive", rows, K, N);
  if ((st = check_tensor(x, "x")) || (st = check_tensor(w, "w")) || (st = check_tensor(y, "y")) ||
      (st = check_bias(b, "b")))
    return st;
  if (act != 0 && act != 1) return fail(BRA_E_INVAL, "act=%d must be 0 (none) or 1 (GELU)", act);
  if (r && act) return fail(BRA_E_UNSUPPORTED, "a residual with an activation is not supported");
  if (r && (st = check_tensor(r, "r"))) return st;
  if (K % 32) return fail(BRA_E_UNSUPPORTED, "K=%d must be a multiple of 32", K);
  if (N % 4) return fail(BRA_E_UNSUPPORTED, "N=%d must be a multiple of 4", N);
  const size_t es = elem_size(dtype);
  if ((long long)rows * K * (long long)es >= kMaxOperandBytes ||
      (long long)rows * N * (long long)es >= kMaxOperandBytes)
    return fail(BRA_E_UNSUPPORTED, "operands of %d rows exceed 2 GiB", rows);
  const size_t ybytes = (size_t)rows * N * es;
  if (overlaps2(y, ybytes, x, (size_t)rows * K * es) || overlaps2(y, ybytes, w, (size_t)N * K * es))
    return fail(BRA_E_INVAL, "y overlaps x or w");
  if (r && r != y && overlaps2(y, ybytes, r, ybytes)) return fail(BRA_E_INVAL, "y overlaps r (other than in place)");
  void* ys[1] = {y};
  return hip_status(bra::launch_linear(x, rows, K, w, b, N, ys, 1, dtype == BRA_BF16,
                                       (hipStream_t)stream, r ? 2 : act, r),
                    "linear launch");
}

bra_status bra_pos_conv(const void* x, const float* w, const float* b, int B, int H, int W, int C,
                        bra_dtype dtype, void* out, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if ((st = check_shape(B, H, W, C, 1, 0, 1, dtype, &s))) return st;
  if ((st = check_tensor(x, "x")) || (st = check_tensor(out, "out")) || (st = check_bias(b, "b")))
    return st;
  if ((st = check_tensor(w, "w"))) return st;
  if (dtype == BRA_F32 ? C % 4 : C % 8) return fail(BRA_E_UNSUPPORTED, "C=%d must be a multiple of %d", C, dtype == BRA_F32 ? 4 : 8);
  const size_t bytes = (size_t)B * H * W * C * elem_size(dtype);
  if (overlaps2(x, bytes, out, bytes)) return fail(BRA_E_INVAL, "out overlaps x");
  return hip_status(bra::launch_pos_conv(x, w, b, s, dtype == BRA_BF16, out, (hipStream_t)stream),
                    "position conv launch");
}

size_t bra_module_workspace_bytes(int B, int H, int W, int C, int S, bra_dtype dtype,
                                  int with_out_proj) {
  if (B < 1 || H < 1 || W < 1 || C < 1 || S < 1) return 0;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return 0;
  return module_layout(B, H, W, C, S, dtype, with_out_proj != 0).total;
}

bra_status bra_module_forward(const void* x, int B, int H, int W, int C, int heads, int S,
                              int topk, bra_dtype dtype, const void* w_qkv, const float* b_qkv,
                              float route_scale, float attn_scale, const float* lepe_w,
                              const float* lepe_b, int lepe_ks, const void* w_out,
                              const float* b_out, void* out, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_tensor(x, "x")) || (st = check_tensor(w_qkv, "w_qkv")) ||
      (st = check_tensor(out, "out")) || (st = check_bias(b_qkv, "b_qkv")) ||
      (st = check_bias(b_out, "b_out")))
    return st;
  if (w_out && (st = check_tensor(w_out, "w_out"))) return st;
  if (b_out && !w_out) return fail(BRA_E_INVAL, "b_out given without w_out");
  if (!idx) return fail(BRA_E_INVAL, "idx is NULL");
  if ((uintptr_t)idx & 3u) return fail(BRA_E_INVAL, "idx is not 4-byte aligned");
  if (!(route_scale > 0.f) || !std::isfinite(route_scale))
    return fail(BRA_E_INVAL, "route_scale=%g must be positive and finite", (double)route_scale);
  if (!(attn_scale > 0.f) || !std::isfinite(attn_scale))
    return fail(BRA_E_INVAL, "attn_scale=%g must be positive and finite", (double)attn_scale);
  if (lepe_w && (st = check_lepe_args(lepe_w, lepe_b, lepe_ks, s))) return st;
  const size_t es = elem_size(dtype);
  const size_t tbytes = (size_t)B * H * W * C * es;
  if ((long long)tbytes >= kMaxOperandBytes)
    return fail(BRA_E_UNSUPPORTED, "a [B,H,W,C] tensor of %zu bytes exceeds 2 GiB", tbytes);
  const ModuleLayout l = module_layout(B, H, W, C, S, dtype, w_out != nullptr);
  if (!ws) return fail(BRA_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", l.total);
  if (!aligned16(ws)) return fail(BRA_E_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < l.total) return fail(BRA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, l.total);
  const size_t ibytes = (size_t)B * s.R * topk * sizeof(int32_t);
  if (overlaps2(ws, l.total, x, tbytes)) return fail(BRA_E_INVAL, "workspace overlaps x");
  if (overlaps2(ws, l.total, out, tbytes)) return fail(BRA_E_INVAL, "workspace overlaps out");
  if (overlaps2(ws, l.total, idx, ibytes)) return fail(BRA_E_INVAL, "workspace overlaps idx");
  if (overlaps2(out, tbytes, idx, ibytes) || overlaps2(x, tbytes, idx, ibytes))
    return fail(BRA_E_INVAL, "idx overlaps x or out");
  if (overlaps2(out, tbytes, w_qkv, (size_t)3 * C * C * es) ||
      (w_out && overlaps2(out, tbytes, w_out, (size_t)C * C * es)))
    return fail(BRA_E_INVAL, "out overlaps a weight");
  return module_launches(x, s, dtype, w_qkv, b_qkv, route_scale, attn_scale, lepe_w, lepe_b,
                         lepe_ks, w_out, b_out, nullptr, out, idx, (unsigned char*)ws, l,
                         (hipStream_t)stream);
}

bra_status bra_layer_norm(const void* x, int rows, int C, const float* gamma, const float* beta,
                          float eps, bra_dtype dtype, void* y, void* stream) {
  g_last_error[0] = 0;
  bra_status st;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return fail(BRA_E_INVAL, "dtype %d is not BRA_F32 or BRA_BF16", (int)dtype);
  if (rows < 1 || C < 1) return fail(BRA_E_INVAL, "rows=%d C=%d must be positive", rows, C);
  if ((st = check_tensor(x, "x")) || (st = check_tensor(y, "y")) || (st = check_tensor(gamma, "gamma")) ||
      (st = check_tensor(beta, "beta")))
    return st;
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(BRA_E_INVAL, "eps=%g must be positive and finite", (double)eps);
  int L, NG;
  if (!bra::layer_norm_shape(C, dtype == BRA_BF16, &L, &NG))
    return fail(BRA_E_UNSUPPORTED, "C=%d: LayerNorm needs C a multiple of %d with at most 4 groups per lane",
                C, dtype == BRA_BF16 ? 8 : 4);
  const size_t bytes = (size_t)rows * C * elem_size(dtype);
  if (overlaps2(x, bytes, y, bytes) && x != y) return fail(BRA_E_INVAL, "y overlaps x (other than in place)");
  return hip_status(bra::launch_layer_norm(x, rows, C, gamma, beta, eps, dtype == BRA_BF16, y,
                                           (hipStream_t)stream),
                    "layer norm launch");
}

bra_status bra_mlp(const void* x, int rows, int C, int Hd, const void* w1, const float* b1,
                   const void* w2, const float* b2, const void* r, bra_dtype dtype, void* out,
                   void* stream) {
  g_last_error[0] = 0;
  bra_status st;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return fail(BRA_E_INVAL, "dtype %d is not BRA_F32 or BRA_BF16", (int)dtype);
  if (rows < 1 || C < 1 || Hd < 1) return fail(BRA_E_INVAL, "rows=%d C=%d Hd=%d must be positive", rows, C, Hd);
  if ((st = check_tensor(x, "x")) || (st = check_tensor(w1, "w1")) || (st = check_tensor(w2, "w2")) ||
      (st = check_tensor(r, "r")) || (st = check_tensor(out, "out")))
    return st;
  if ((b1 && !aligned16(b1)) || (b2 && !aligned16(b2))) return fail(BRA_E_INVAL, "b1 / b2 must be 16-byte aligned");
  if (dtype != BRA_BF16) return fail(BRA_E_UNSUPPORTED, "the fused MLP is bf16 only (bra_linear covers float32)");
  if ((C != 64 && C != 128 && C != 256) || Hd % 32)
    return fail(BRA_E_UNSUPPORTED, "C=%d Hd=%d: the fused MLP needs C in {64, 128, 256} and Hd %% 32 == 0", C, Hd);
  const size_t bytes = (size_t)rows * C * 2;
  if (bytes >= ((size_t)1 << 31) || (size_t)Hd * C * 2 >= ((size_t)1 << 31))
    return fail(BRA_E_UNSUPPORTED, "rows=%d C=%d Hd=%d: a tensor of 2 GiB or more", rows, C, Hd);
  if (overlaps2(out, bytes, x, bytes)) return fail(BRA_E_INVAL, "out overlaps x");
  if (overlaps2(out, bytes, r, bytes) && out != r) return fail(BRA_E_INVAL, "out overlaps r (other than in place)");
  return hip_status(bra::launch_mlp(x, rows, C, Hd, w1, b1, w2, b2, r, out, (hipStream_t)stream),
                    "mlp launch");
}

size_t bra_block_workspace_bytes(int B, int H, int W, int C, int S, bra_dtype dtype) {
  if (B < 1 || H < 1 || W < 1 || C < 1 || S < 1) return 0;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return 0;
  return block_layout(B, H, W, C, S, dtype).total;
}

bra_status bra_block_forward(const void* x, int B, int H, int W, int C, int heads, int S, int topk,
                             bra_dtype dtype, const bra_block_params* p, float route_scale,
                             float attn_scale, void* out, int32_t* idx, void* ws, size_t ws_bytes,
                             void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (!p) return fail(BRA_E_INVAL, "params is NULL");
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  if ((st = check_tensor(x, "x")) || (st = check_tensor(out, "out"))) return st;
  if ((st = check_tensor(p->pos_w, "pos_w")) || (st = check_bias(p->pos_b, "pos_b")) ||
      (st = check_tensor(p->ln1_g, "ln1_g")) || (st = check_tensor(p->ln1_b, "ln1_b")) ||
      (st = check_tensor(p->w_qkv, "w_qkv")) || (st = check_bias(p->b_qkv, "b_qkv")) ||
      (st = check_tensor(p->w_out, "w_out")) || (st = check_bias(p->b_out, "b_out")) ||
      (st = check_tensor(p->ln2_g, "ln2_g")) || (st = check_tensor(p->ln2_b, "ln2_b")) ||
      (st = check_tensor(p->w_fc1, "w_fc1")) || (st = check_bias(p->b_fc1, "b_fc1")) ||
      (st = check_tensor(p->w_fc2, "w_fc2")) || (st = check_bias(p->b_fc2, "b_fc2")))
    return st;
  if (!idx) return fail(BRA_E_INVAL, "idx is NULL");
  if ((uintptr_t)idx & 3u) return fail(BRA_E_INVAL, "idx is not 4-byte aligned");
  if (!(route_scale > 0.f) || !std::isfinite(route_scale))
    return fail(BRA_E_INVAL, "route_scale=%g must be positive and finite", (double)route_scale);
  if (!(attn_scale > 0.f) || !std::isfinite(attn_scale))
    return fail(BRA_E_INVAL, "attn_scale=%g must be positive and finite", (double)attn_scale);
  if (p->lepe_w && (st = check_lepe_args(p->lepe_w, p->lepe_b, p->lepe_ks, s))) return st;
  int L, NG;
  if (!bra::layer_norm_shape(C, dtype == BRA_BF16, &L, &NG))
    return fail(BRA_E_UNSUPPORTED, "C=%d: LayerNorm needs at most 4 channel groups per lane", C);
  const size_t es = elem_size(dtype);
  const size_t tbytes = (size_t)B * H * W * C * es;
  if ((long long)tbytes * 3 >= kMaxOperandBytes)
    return fail(BRA_E_UNSUPPORTED, "the [B,H,W,3C] hidden tensor of %zu bytes exceeds 2 GiB", tbytes * 3);
  const BlockLayout bl = block_layout(B, H, W, C, S, dtype);
  if (!ws) return fail(BRA_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", bl.total);
  if (!aligned16(ws)) return fail(BRA_E_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < bl.total) return fail(BRA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, bl.total);
  const size_t ibytes = (size_t)B * s.R * topk * sizeof(int32_t);
  if (overlaps2(ws, bl.total, x, tbytes)) return fail(BRA_E_INVAL, "workspace overlaps x");
  if (overlaps2(ws, bl.total, out, tbytes)) return fail(BRA_E_INVAL, "workspace overlaps out");
  if (overlaps2(ws, bl.total, idx, ibytes)) return fail(BRA_E_INVAL, "workspace overlaps idx");
  if (overlaps2(out, tbytes, idx, ibytes) || overlaps2(x, tbytes, idx, ibytes))
    return fail(BRA_E_INVAL, "idx overlaps x or out");
  hipStream_t hs = (hipStream_t)stream;
  const bool bf16 = dtype == BRA_BF16;
  unsigned char* w8 = (unsigned char*)ws;
  void* x1 = w8 + bl.x1;
  void* n1 = w8 + bl.n1;
  void* x2 = w8 + bl.x2;
  void* n2 = w8 + bl.n2;
  unsigned char* mws = w8 + bl.mod;
  const int T = B * H * W;
  // x1 = x + pos conv;  x2 = x1 + module(LN1(x1))
  // x1 and LN1(x1) in one launch where the pixel's channel groups fit a
  // wavefront, else two
  const hipError_t pe = bra::launch_pos_conv(x, p->pos_w, p->pos_b, s, bf16, x1, hs, p->ln1_g,
                                             p->ln1_b, kLayerNormEps, n1);
  if (pe != hipErrorNotSupported) {
    if ((st = hip_status(pe, "position conv launch"))) return st;
  } else {
    if ((st = hip_status(bra::launch_pos_conv(x, p->pos_w, p->pos_b, s, bf16, x1, hs),
                         "position conv launch")))
      return st;
    if ((st = hip_status(bra::launch_layer_norm(x1, T, C, p->ln1_g, p->ln1_b, kLayerNormEps, bf16,
                                                n1, hs),
                         "layer norm launch")))
      return st;
  }
  // bf16 at C <= 128: the module without its output projection (y, the
  // attention output, into the module workspace), then the output
  // projection, LN2 and the MLP in one launch (x2 and n2 still stored)
  if (bf16 && (C == 64 || C == 128)) {
    void* y = mws + bl.ml.y;
    if ((st = module_launches(n1, s, dtype, p->w_qkv, p->b_qkv, route_scale, attn_scale,
                              p->lepe_w, p->lepe_b, p->lepe_ks, nullptr, nullptr, nullptr, y, idx,
                              mws, bl.ml, hs)))
      return st;
    const hipError_t e = bra::launch_block_tail(y, x1, T, C, 3 * C, p->w_out, p->b_out, p->ln2_g,
                                                p->ln2_b, kLayerNormEps, p->w_fc1, p->b_fc1,
                                                p->w_fc2, p->b_fc2, x2, n2, out, hs);
    return hip_status(e, "block tail launch");
  }
  if ((st = module_launches(n1, s, dtype, p->w_qkv, p->b_qkv, route_scale, attn_scale, p->lepe_w,
                            p->lepe_b, p->lepe_ks, p->w_out, p->b_out, x1, x2, idx, mws, bl.ml, hs)))
    return st;
  // out = x2 + fc2(GELU(fc1(LN2(x2)))); the hidden tensor reuses the module's Q/K/V space
  if ((st = hip_status(bra::launch_layer_norm(x2, T, C, p->ln2_g, p->ln2_b, kLayerNormEps, bf16, n2, hs),
                       "layer norm launch")))
    return st;
  // the MLP in one launch where the fused kernel covers the shape (bf16)
  if (bf16) {
    const hipError_t e = bra::launch_mlp(n2, T, C, 3 * C, p->w_fc1, p->b_fc1, p->w_fc2, p->b_fc2,
                                         x2, out, hs);
    if (e != hipErrorNotSupported) return hip_status(e, "mlp launch");
  }
  void* h = mws + bl.ml.q;
  void* hv[1] = {h};
  if ((st = hip_status(bra::launch_linear(n2, T, C, p->w_fc1, p->b_fc1, 3 * C, hv, 1, bf16, hs, 1),
                       "fc1 launch")))
    return st;
  void* ov[1] = {out};
  return hip_status(bra::launch_linear(h, T, 3 * C, p->w_fc2, p->b_fc2, C, ov, 1, bf16, hs, 2, x2),
                    "fc2 launch");
}

size_t bra_backward_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk,
                                    int lepe_ks) {
  if (B < 1 || H < 1 || W < 1 || C < 1 || heads < 1 || S < 1 || topk < 1 || lepe_ks < 0) return 0;
  return bra::bwd_workspace_bytes(B, H, W, C, heads, S, topk, lepe_ks, lepe_ks > 0);
}

bra_status bra_attend_backward(const void* q, const void* k, const void* v, const int32_t* idx,
                               const void* dout, int B, int H, int W, int C, int heads, int S,
                               int topk, bra_dtype dtype, float attn_scale, const float* lepe_w,
                               int lepe_ks, void* dq, void* dk, void* dv, float* dlepe_w,
                               float* dlepe_b, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  bra::Shape s;
  bra_status st;
  if (heads < 1) return fail(BRA_E_INVAL, "heads=%d must be positive", heads);
  if ((st = check_shape(B, H, W, C, S, heads, topk, dtype, &s))) return st;
  if (dtype != BRA_BF16) return fail(BRA_E_UNSUPPORTED, "the backward pass runs in bf16 only");
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(dout, "dout")) || (st = check_tensor(dq, "dq")) ||
      (st = check_tensor(dk, "dk")) || (st = check_tensor(dv, "dv")))
    return st;
  if (!idx) return fail(BRA_E_INVAL, "idx is NULL");
  if ((uintptr_t)idx & 3u) return fail(BRA_E_INVAL, "idx is not 4-byte aligned");
  if (!(attn_scale > 0.f) || !std::isfinite(attn_scale))
    return fail(BRA_E_INVAL, "attn_scale=%g must be positive and finite", (double)attn_scale);
  if (s.topk * s.n > 256)
    return fail(BRA_E_UNSUPPORTED, "topk*n=%d routed keys per query; the backward pass takes up to 256",
                s.topk * s.n);
  if (lepe_w) {
    if ((st = check_lepe_args(lepe_w, nullptr, lepe_ks, s))) return st;
    if (!dlepe_w) return fail(BRA_E_INVAL, "dlepe_w is NULL while lepe_w is given");
    if ((uintptr_t)dlepe_w & 3u) return fail(BRA_E_INVAL, "dlepe_w is not 4-byte aligned");
  }
  if (dlepe_b && ((uintptr_t)dlepe_b & 3u)) return fail(BRA_E_INVAL, "dlepe_b is not 4-byte aligned");
  const size_t tb = (size_t)B * H * W * C * 2;
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps2(outs[i], tb, ins[j], tb)) return fail(BRA_E_INVAL, "a gradient overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps2(outs[i], tb, outs[j], tb)) return fail(BRA_E_INVAL, "two gradients overlap");
  }
  const size_t need = bra::bwd_workspace_bytes(B, H, W, C, heads, S, topk, lepe_ks, lepe_w != nullptr);
  if (!ws) return fail(BRA_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(BRA_E_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(BRA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return hip_status(bra::launch_backward(q, k, v, idx, dout, s, attn_scale, lepe_w, lepe_ks, dq, dk,
                                         dv, lepe_w ? dlepe_w : nullptr, lepe_w ? dlepe_b : nullptr,
                                         ws, (hipStream_t)stream),
                    "backward launch");
}

const char* bra_strerror(int status) {
  switch (status) {
    case BRA_OK: return "ok";
    case BRA_E_INVAL: return "invalid argument";
    case BRA_E_UNSUPPORTED: return "unsupported problem";
    case BRA_E_WORKSPACE: return "workspace missing or too small";
    case BRA_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* bra_last_error(void) { return g_last_error; }

}  // extern "C"
