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
  s.hs = H / S; s.ws = W / S; s.n = (int)n; s.R = S * S;
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
  const size_t need = bra_workspace_bytes(s.B, s.S, s.C);
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

bra_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BRA_OK;
  return fail(BRA_E_HIP, "%s: %s", what, hipGetErrorString(e));
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
  if ((st = hip_status(bra::launch_pool(q, k, qm, km, s, dtype == BRA_BF16, hs), "pool launch")))
    return st;
  return hip_status(bra::launch_route(qm, km, s, (double)route_scale, idx, topk_logits, hs),
                    "route launch");
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
  hipStream_t hs = (hipStream_t)stream;
  const bool bf16 = dtype == BRA_BF16;
  double* qm = (double*)ws;
  double* km = qm + (size_t)B * s.R * C;
  if ((st = hip_status(bra::launch_pool(q, k, qm, km, s, bf16, hs), "pool launch"))) return st;
  if ((st = hip_status(bra::launch_route(qm, km, s, (double)route_scale, idx, topk_logits, hs),
                       "route launch")))
    return st;
  return hip_status(bra::launch_attend(q, k, v, idx, s, bf16, attn_scale, lepe_w, lepe_b, lepe_ks,
                                       out, hs),
                    "attend launch");
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
