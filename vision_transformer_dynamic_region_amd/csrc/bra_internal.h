// Internal interface between the C-ABI front end (bra_api.cpp) and the HIP
// kernels (bra_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bra {

// Bytes of the device scratch array of the allocation-free entry points.
constexpr size_t kScratchBytes = (size_t)16 << 20;

// Device address of this device's scratch array (kScratchBytes, 256-byte
// aligned), looked up once per device.
hipError_t scratch_buffer(void** out);

// Problem shape after validation.  All sizes are positive, S divides H and
// W, heads * 32 == C.
struct Shape {
  int B, H, W, C, S, heads, topk;
  int hs, ws;     // region height / width in pixels
  int n;          // pixels per region = hs * ws
  int R;          // regions per image: S * S, or T * S * S for a clip of T frames
  int Hf;         // rows of one frame (H for an image); a clip of T frames is
                  // stacked as H = T * Hf rows, and LePE stays inside a frame
};

// Region means of q and k into qm, km (float64 [B, R, C] each); with k (and
// km) null, the means of q alone.
hipError_t launch_pool(const void* q, const void* k, double* qm, double* km,
                       const Shape& s, bool bf16, hipStream_t st);

// y[g] = columns [g*N/groups, (g+1)*N/groups) of x w^T + b, for x [T, K],
// w [N, K], b [N] or null (groups <= 3).  K % 32 == 0, N % 4 == 0 and, with
// several groups, N / groups % 8 == 0.  epi 1 applies GELU (exact form)
// after the bias; epi 2 adds resid [T, N] (one group) before the rounding.
hipError_t launch_linear(const void* x, int T, int K, const void* w, const float* b, int N,
                         void* const* y, int groups, bool bf16, hipStream_t st, int epi = 0,
                         const void* resid = nullptr);

// out = resid + fc2(GELU(fc1(x))) in bf16 in one launch (the hidden layer
// [T, Hd] rounded once to bf16, never written): x, resid, out [T, C], w1
// [Hd, C], w2 [C, Hd], b1 [Hd] / b2 [C] float32 or null.  C in {64, 128,
// 256}, Hd % 32 == 0; hipErrorNotSupported otherwise, before anything is
// enqueued.
hipError_t launch_mlp(const void* x, long long T, int C, int Hd, const void* w1, const float* b1,
                      const void* w2, const float* b2, const void* resid, void* out,
                      hipStream_t st);

// The block's last three layers in one launch (bf16): x2 = x1 + y w_out^T
// + b_out and n2 = LN2(x2) (eps; gamma ln_g, beta ln_b), each rounded once
// to bf16 and written to x2 / n2 when those are not null, then out = x2 +
// fc2(GELU(fc1(n2))) as launch_mlp.  C in {64, 128}, Hd % 32 == 0;
// hipErrorNotSupported otherwise, before anything is enqueued.
hipError_t launch_block_tail(const void* y, const void* x1, long long T, int C, int Hd,
                             const void* w_out, const float* b_out, const float* ln_g,
                             const float* ln_b, float eps, const void* w1, const float* b1,
                             const void* w2, const float* b2, void* x2, void* n2, void* out,
                             hipStream_t st);

// out = x + b + depthwise 3x3 cross-correlation of x (w [C, 3, 3], zero
// padding 1), [B, H, W, C].
// With nout, also nout = LayerNorm(out) (gamma ln_g, beta ln_b, eps; out
// rounded first, one rounding) where a pixel's 16-byte groups are a power
// of two up to 64; hipErrorNotSupported (nothing enqueued) otherwise.
hipError_t launch_pos_conv(const void* x, const float* w, const float* b, const Shape& s,
                           bool bf16, void* out, hipStream_t st, const float* ln_g = nullptr,
                           const float* ln_b = nullptr, float eps = 0.f, void* nout = nullptr);

// Backward pass with a fixed routing index (bf16, head width 32, topk * n
// <= 256): dq, dk, dv (bf16, dV with the LePE term when w is not null) and
// dw, db (float32; db may be null).  ws holds bwd_workspace_bytes.
size_t bwd_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk, int ks,
                           bool lepe);
hipError_t launch_backward(const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* dout, const Shape& s, float attn_scale, const float* w,
                           int ks, void* dq, void* dk, void* dv, float* dw, float* db, void* ws,
                           hipStream_t st);

// LayerNorm of each of `rows` rows of C channels (biased variance, eps).
// layer_norm_shape says whether C is supported and how rows are split.
bool layer_norm_shape(int C, bool bf16, int* lanes_per_row, int* groups_per_lane);
hipError_t launch_layer_norm(const void* x, long long rows, int C, const float* g,
                             const float* b, float eps, bool bf16, void* y, hipStream_t st);

// qm = xm Wq^T + bq, km = xm Wk^T + bk in float64, with Wq, Wk the first two
// C-row blocks of w_qkv [3C, C] and bq, bk those of b_qkv (or null).
hipError_t launch_means_proj(const double* xm, int rows, int C, const void* w_qkv,
                             const float* b_qkv, bool bf16, double* qm, double* km,
                             hipStream_t st);

// Region means of q and k (float64; written to qm and km as launch_pool
// does unless qm is null) and the scaled affinity's per-row top-k in one
// launch, for up to 64 regions per image; hipErrorNotSupported for other
// shapes, before anything is enqueued.
hipError_t launch_pool_route(const void* q, const void* k, double* qm, double* km,
                             const Shape& s, bool bf16, double route_scale, int32_t* idx,
                             float* logits, hipStream_t st);

// Scaled affinity of the region means and per-row top-k.
hipError_t launch_route(const double* qm, const double* km, const Shape& s,
                        double route_scale, int32_t* idx, float* logits,
                        hipStream_t st);

// Gather-attention over the routed regions, plus the LePE term when w is
// not null (fused into the attention epilogue when the region's halo tile
// fits in LDS, otherwise written first by the standalone kernel).
hipError_t launch_attend(const void* q, const void* k, const void* v,
                         const int32_t* idx, const Shape& s, bool bf16,
                         float attn_scale, const float* w, const float* bias,
                         int ks, void* out, hipStream_t st);

// The same for bf16 inputs of a region shape with a dedicated kernel (LePE
// fused); hipErrorNotSupported for any other shape, before anything is
// enqueued.
hipError_t launch_attend_region(const void* q, const void* k, const void* v,
                                const int32_t* idx, const Shape& s,
                                float attn_scale, const float* w,
                                const float* bias, int ks, void* out,
                                hipStream_t st);

// The module's fused form of launch_attend_region for bf16 x with C = 64,
// 8x8-pixel regions, top-1 and a 5x5 LePE (attend_xproj_ok): Q, K and V are
// projected from x inside the attention kernel with w_qkv ([3C, C] bf16)
// and b_qkv (float32 [3C] or null), bias added and rounded to bf16 as
// launch_linear does, so they are never written.  hipErrorNotSupported for
// other shapes, before anything is enqueued.
bool attend_xproj_ok(const Shape& s, const float* w, int ks);
hipError_t launch_attend_xproj(const void* x, const void* w_qkv, const float* b_qkv,
                               const int32_t* idx, const Shape& s, float attn_scale,
                               const float* w, const float* bias, int ks, void* out,
                               hipStream_t st);

// The same with the whole image's K and V for one head resident in LDS
// (bf16, 5x5 LePE fused, the 4x4 / top-4 and 2x2 / top-16 region shapes on
// maps whose padded image fits LDS); hipErrorNotSupported for any other
// shape, before anything is enqueued.
hipError_t launch_attend_image(const void* q, const void* k, const void* v,
                               const int32_t* idx, const Shape& s,
                               float attn_scale, const float* w,
                               const float* bias, int ks, void* out,
                               hipStream_t st);

// out += bias + depthwise ks x ks cross-correlation of v.
hipError_t launch_lepe(const void* v, const float* w, const float* b, int ks,
                       const Shape& s, bool bf16, void* out, hipStream_t st);

}  // namespace bra
