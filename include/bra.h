/*
 * bra.h -- C ABI of libbra: the Bi-Level Routing Attention (BRA) forward pass
 * of BiFormer on AMD Instinct MI355X (gfx950).
 *
 * What is computed (page keys: p1 = cybasar.com "CVPR2023: BiFormer中的双层
 * 路由注意力机制解析", p2 = snabindia.com "从静态到动态：BRA双层路由注意力如何
 * 革新视觉Transformer的计算范式", p5 = hyper.ai abstract of arXiv 2303.08810):
 *
 *   1. partition (p1 §3): an H x W map is split into S x S regions of
 *      hs = H/S by ws = W/S pixels; regions are numbered row-major over the
 *      grid, pixels row-major inside a region;
 *   2. region means (p1 §3, p2 §2): q_r, k_r = mean of Q, K over each region;
 *   3. affinity (p1 §3, p2 §4): A[r][s] = route_scale * <q_r[r], k_r[s]>;
 *   4. routing (p1 §3, p2 §4): idx[r] = the topk columns of row r of A,
 *      largest first, equal values by lower region index;
 *   5. attention (p1 §3, p5): every query pixel of region r attends, per head
 *      (d = C / heads contiguous channels), over all tokens of the regions
 *      idx[r][0..topk-1] with softmax(attn_scale * q.k) weights;
 *   6. LePE (p2 §4, p1 §3): out = attention + bias + depthwise ks x ks
 *      cross-correlation of V over the whole image, zero padded.
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V and out are [B, H, W, C] channels-last, contiguous,
 *     in the element type `dtype` (BRA_F32 or BRA_BF16), 16-byte aligned.
 *   - idx is int32 [B, S*S, topk], contiguous.
 *   - LePE weights are float32 [C, ks, ks] (PyTorch depthwise Conv2d weight
 *     without its singleton axis); bias is float32 [C] or NULL.  In bf16
 *     with ks = 5 and d = 32, the attention kernels of 8x8-pixel regions
 *     (C of 32, 64, 96, 128, 192 or 256, top-1, 2 or 4), 4x4 (top-2, 4
 *     or 8) and 2x2 (top-16) fuse the LePE on v_dot2_f32_bf16: the
 *     weights are rounded once to bf16 (relative error at most 2^-9
 *     each), the products
 *     with the bf16 pixels are exact and the sums float32.  Every other path
 *     (float32 data, other ks, other shapes, bra_lepe) uses the float32
 *     weights as given.
 *   - All pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; it enqueues kernels on
 *     `stream` (a hipStream_t; NULL means the default stream) and returns.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     rejected call enqueues nothing.  A failed launch returns BRA_E_HIP.
 *     bra_last_error() gives a thread-local message for the last failure.
 *   - Supported: head width d = C / heads == 32, odd ks in 1..7, S*S <= 1024,
 *     C <= 1024.  Other valid shapes return BRA_E_UNSUPPORTED.
 *   - Calls on one stream are ordered; calls that share a workspace or
 *     output on different streams race.
 */
#ifndef BRA_H_
#define BRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BRA_F32 = 0, BRA_BF16 = 1 } bra_dtype;

typedef enum {
  BRA_OK = 0,
  BRA_E_INVAL = 1,        /* bad shape, pointer, alignment or value     */
  BRA_E_UNSUPPORTED = 2,  /* valid BRA problem this build does not run  */
  BRA_E_WORKSPACE = 3,    /* workspace missing or too small             */
  BRA_E_HIP = 4           /* a HIP launch or runtime call failed        */
} bra_status;

/* Bytes of workspace bra_route / bra_forward need: two float64 tensors
 * [B, S*S, C] holding the region means of Q (first) and K (second).  After a
 * successful call the workspace holds exactly those means (p1 §3 region-mean
 * step), which callers may read.  Returns 0 for non-positive sizes. */
size_t bra_workspace_bytes(int B, int S, int C);

/* Steps 1-4: region means of Q and K, scaled region affinity and per-row
 * top-k (p1 §3; p2 §2 and §4 TopkRouting).
 *   q, k        [B,H,W,C] dtype, device.
 *   route_scale positive scale of the affinity (p2 §4); any positive value
 *               gives the same idx.  Non-positive or non-finite: BRA_E_INVAL.
 *   idx         out: int32 [B, S*S, topk], device.
 *   topk_logits out: float32 [B, S*S, topk] affinities of the chosen regions
 *               (same order as idx), device; may be NULL.
 *   ws          device workspace of at least bra_workspace_bytes(B, S, C). */
bra_status bra_route(const void* q, const void* k, int B, int H, int W, int C,
                     int S, int topk, bra_dtype dtype, float route_scale,
                     int32_t* idx, float* topk_logits, void* ws,
                     size_t ws_bytes, void* stream);

/* Steps 5-6 with a caller-supplied routing index: gather-attention over the
 * routed regions (p1 §3; p5) plus, when lepe_w is not NULL, the LePE term
 * (p2 §4).  This is also the fixed-routing use: an index held constant
 * across calls (p2 §5).
 *   idx         int32 [B, S*S, topk], device; entries must lie in
 *               [0, S*S) (entries outside are clamped, not trusted).
 *   attn_scale  positive, finite scale of q.k inside the softmax
 *               (1/sqrt(d) usual); anything else: BRA_E_INVAL.
 *   lepe_w      float32 [C, ks, ks] or NULL (no LePE); lepe_b float32 [C]
 *               or NULL; lepe_ks odd in 1..7 (ignored when lepe_w is NULL).
 *   out         [B,H,W,C] dtype, device; must not overlap q, k or v. */
bra_status bra_attend(const void* q, const void* k, const void* v,
                      const int32_t* idx, int B, int H, int W, int C,
                      int heads, int S, int topk, bra_dtype dtype,
                      float attn_scale, const float* lepe_w,
                      const float* lepe_b, int lepe_ks, void* out,
                      void* stream);

/* The whole forward pass, steps 1-6 (p1 §3): bra_route then bra_attend on
 * the same stream.  Arguments as above, except that ws is scratch: its
 * contents afterwards are unspecified (where routing runs as one launch the
 * region means never leave the chip). */
bra_status bra_forward(const void* q, const void* k, const void* v, int B,
                       int H, int W, int C, int heads, int S, int topk,
                       bra_dtype dtype, float route_scale, float attn_scale,
                       const float* lepe_w, const float* lepe_b, int lepe_ks,
                       void* out, int32_t* idx, float* topk_logits, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): bra_forward without a
 * workspace argument.  The workspace bra_forward would take (the float64
 * region means, where they pass through memory) is a device array inside
 * the library (BRA_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until
 * the process ends); the call allocates nothing.  Sizes whose means exceed
 * that array, 2*B*S*S*C*8 bytes > BRA_NOALLOC_SCRATCH_BYTES, return
 * BRA_E_UNSUPPORTED before anything is enqueued.  Every call on a GPU
 * shares its array: calls that overlap on one GPU (different streams,
 * different threads) race; calls on one stream are ordered.  Arguments,
 * results and the other errors as bra_forward.
 * ------------------------------------------------------------------------ */
#define BRA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

bra_status bra_forward_noalloc(const void* q, const void* k, const void* v,
                               int B, int H, int W, int C, int heads, int S,
                               int topk, bra_dtype dtype, float route_scale,
                               float attn_scale, const float* lepe_w,
                               const float* lepe_b, int lepe_ks, void* out,
                               int32_t* idx, float* topk_logits, void* stream);

/* Step 6 alone, in place: out += bias + depthwise ks x ks cross-correlation
 * of v (p2 §4 depthwise Conv2d; p1 §3 adds it to the attention output).
 *   v, out [B,H,W,C] dtype, device, not overlapping; w float32 [C,ks,ks];
 *   b float32 [C] or NULL. */
bra_status bra_lepe(const void* v, const float* w, const float* b, int ks,
                    int B, int H, int W, int C, bra_dtype dtype, void* out,
                    void* stream);

/* ------------------------------------------------------------------------
 * The module around the method (p1 §3: q_proj / k_proj / v_proj of x before
 * the routing; the pages show no output projection, so it is optional).
 * Weights follow the PyTorch Linear convention y = x W^T + b: a weight is
 * [out_features, in_features] row-major in `dtype`, 16-byte aligned; biases
 * are float32, 16-byte aligned, or NULL.
 * ------------------------------------------------------------------------ */

/* Per-token linear map y = act(x w^T + b) + r on the matrix cores (float32
 * accumulation, one rounding to dtype).
 *   x   [rows, K] dtype, device;  w [N, K] dtype, device;  b float32 [N] or
 *       NULL;  y out: [rows, N] dtype, device, not overlapping x or w.
 *   act 0: none, 1: GELU in its exact (erf) form (the block's MLP).
 *   r   [rows, N] dtype, device, or NULL: a residual added after act (the
 *       block's residual connections); may be y itself; not with act 1.
 *   K must be a multiple of 32 and N of 4; every operand must stay below
 *   2 GiB (BRA_E_UNSUPPORTED otherwise). */
bra_status bra_linear(const void* x, int rows, int K, const void* w,
                      const float* b, int N, int act, const void* r,
                      bra_dtype dtype, void* y, void* stream);

/* Bytes of workspace bra_module_forward needs for these sizes; with_out_proj
 * non-zero when an output projection will be passed.  Layout, each part
 * starting on a 256-byte boundary: float64 [B, S*S, C] region means of x,
 * float64 [B, S*S, C] region means of Q, the same of K, then Q, K, V as
 * [B, H, W, C] dtype each, then (with_out_proj) y = attention + LePE as
 * [B, H, W, C] dtype.  After a successful call the workspace holds exactly
 * those values, which callers may read, except that the Q, K and V parts
 * are left unwritten where Q, K and V are projected inside the attention
 * kernel (bf16, C = 64, 8x8-pixel regions, top-1, 5x5 LePE, and y not x's
 * memory).
 * 0 for invalid sizes. */
size_t bra_module_workspace_bytes(int B, int H, int W, int C, int S,
                                  bra_dtype dtype, int with_out_proj);

/* The BRA module forward pass:
 *   Q, K, V = x w_qkv^T + b_qkv (w_qkv [3C, C]: rows 0..C-1 give Q, then K,
 *             then V; b_qkv float32 [3C] or NULL);
 *   steps 1-6 above on Q, K, V (LePE on the projected V);
 *   out = y w_out^T + b_out when w_out ([C, C]) is not NULL, else out = y.
 * Routing uses the region means of x projected in float64 (a region mean
 * commutes with a per-token linear map), so idx matches a float64
 * evaluation of the definition up to exact ties.
 *   x    [B,H,W,C] dtype, device (may be the same memory as out).
 *   out  [B,H,W,C] dtype, device; idx out: int32 [B, S*S, topk], device.
 *   ws   device workspace of >= bra_module_workspace_bytes(...) bytes, not
 *        overlapping x, out or idx.
 * Other arguments and limits as in bra_forward. */
bra_status bra_module_forward(const void* x, int B, int H, int W, int C,
                              int heads, int S, int topk, bra_dtype dtype,
                              const void* w_qkv, const float* b_qkv,
                              float route_scale, float attn_scale,
                              const float* lepe_w, const float* lepe_b,
                              int lepe_ks, const void* w_out,
                              const float* b_out, void* out, int32_t* idx,
                              void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The BiFormer block around the module (p3 §3.1: pre-norm residual blocks,
 * x + bra(norm1(x)), x + ffn(norm2(x)); p1 §4: a 3x3 convolution as the
 * position encoding and a two-layer MLP of ratio 3):
 *   x1  = x + dwconv3x3(x) + pos_b        (depthwise, zero padding 1)
 *   x2  = x1 + module(LN1(x1))             (bra_module_forward, with w_out)
 *   out = x2 + fc2(GELU(fc1(LN2(x2))))     (fc1 [3C, C], fc2 [C, 3C])
 * LayerNorm: over C, biased variance, eps 1e-5, per-channel scale/shift.
 * GELU: exact (erf) form.  Every layer output above is stored in dtype.
 * ------------------------------------------------------------------------ */

/* out = x + b + depthwise 3x3 cross-correlation of x over each image (zero
 * padding 1): the block's position encoding (p1 §4).
 *   x, out [B,H,W,C] dtype, device, not overlapping; w float32 [C, 3, 3];
 *   b float32 [C] or NULL (all 16-byte aligned); C a multiple of 8 (bf16)
 *   or 4 (f32). */
bra_status bra_pos_conv(const void* x, const float* w, const float* b, int B,
                        int H, int W, int C, bra_dtype dtype, void* out,
                        void* stream);

/* LayerNorm of `rows` rows of C channels: (x - mean) / sqrt(var + eps) *
 * gamma + beta, float32 statistics, one rounding to dtype.
 *   x, y [rows, C] dtype, device (y may be x); gamma, beta float32 [C].
 *   C must be a multiple of 8 (bf16) or 4 (f32) whose 16-byte groups split
 *   into at most 4 per lane (every multiple of 32 up to 512 does). */
bra_status bra_layer_norm(const void* x, int rows, int C, const float* gamma,
                          const float* beta, float eps, bra_dtype dtype,
                          void* y, void* stream);

/* The block's MLP with its residual, one launch (p1 §2: a block is the BRA
 * attention then a 2-layer MLP, each with a residual connection):
 *   out = r + fc2(GELU(fc1(x))),  fc1 = x w1^T + b1,  fc2 = h w2^T + b2,
 * with the hidden layer h = GELU(fc1(x)) rounded once to bf16, as the
 * block stores it, but kept on chip; fc2, b2 and r are summed in float32
 * and rounded once.
 *   x, r, out [rows, C] bf16, device (out may be r, not x); w1 [Hd, C],
 *   w2 [C, Hd] bf16; b1 [Hd], b2 [C] float32 or NULL; all 16-byte aligned.
 *   Supported: dtype BRA_BF16, C in {64, 128, 256}, Hd a multiple of 32;
 *   other valid sizes return BRA_E_UNSUPPORTED (bra_linear covers them in
 *   two calls). */
bra_status bra_mlp(const void* x, int rows, int C, int Hd, const void* w1,
                   const float* b1, const void* w2, const float* b2,
                   const void* r, bra_dtype dtype, void* out, void* stream);

/* Parameters of one block: device pointers, float32 unless noted; weights
 * in the PyTorch Linear / depthwise Conv2d layouts, 16-byte aligned. */
typedef struct {
  const float* pos_w;   /* [C, 3, 3] position conv                         */
  const float* pos_b;   /* [C] or NULL                                      */
  const float* ln1_g;   /* [C]                                              */
  const float* ln1_b;   /* [C]                                              */
  const void* w_qkv;    /* [3C, C] dtype                                    */
  const float* b_qkv;   /* [3C] or NULL                                     */
  const float* lepe_w;  /* [C, ks, ks] or NULL                              */
  const float* lepe_b;  /* [C] or NULL                                      */
  int lepe_ks;          /* odd, 1..7                                        */
  const void* w_out;    /* [C, C] dtype (required)                          */
  const float* b_out;   /* [C] or NULL                                      */
  const float* ln2_g;   /* [C]                                              */
  const float* ln2_b;   /* [C]                                              */
  const void* w_fc1;    /* [3C, C] dtype                                    */
  const float* b_fc1;   /* [3C] or NULL                                     */
  const void* w_fc2;    /* [C, 3C] dtype                                    */
  const float* b_fc2;   /* [C] or NULL                                      */
} bra_block_params;

/* Bytes of workspace bra_block_forward needs: x1, LN1(x1), x2, LN2(x2) as
 * [B,H,W,C] dtype each (256-byte aligned), then a module workspace with
 * output projection (bra_module_workspace_bytes(..., 1)), whose Q/K/V space
 * later holds the MLP's [B,H,W,3C] hidden tensor where the MLP runs as two
 * linear calls (where bra_mlp's one launch covers the shape, the hidden
 * tensor is not written).  0 for invalid sizes. */
size_t bra_block_workspace_bytes(int B, int H, int W, int C, int S,
                                 bra_dtype dtype);

/* One BiFormer block.  x, out [B,H,W,C] dtype, device (out may be x);
 * idx out: int32 [B, S*S, topk]; ws as above, not overlapping x, out, idx.
 * Other arguments and limits as in bra_module_forward. */
bra_status bra_block_forward(const void* x, int B, int H, int W, int C,
                             int heads, int S, int topk, bra_dtype dtype,
                             const bra_block_params* params, float route_scale,
                             float attn_scale, void* out, int32_t* idx,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward pass with the routing index held fixed (training with frozen
 * routing: p2 §4 detaches the routing inputs unless diff_routing is set;
 * p1 §5 and p2 §5 keep the index constant).  The index gets no gradient.
 * For out = attention(Q, K, V; idx) + LePE(V):
 *   dV includes the LePE term (the transposed depthwise conv of dout);
 *   dK, dV collect the terms of every query region that routes to a key;
 *   dw = sum over pixels of dout * shifted V, db = sum of dout.
 * bf16 only (BRA_E_UNSUPPORTED for f32), topk * n <= 256 keys per query.
 * Deterministic: every sum has a fixed order, no atomics.
 * ------------------------------------------------------------------------ */

/* Bytes of workspace bra_attend_backward needs (lepe_ks 0 without LePE):
 * per-pixel softmax statistics and, with LePE, the float32 LePE term of dV
 * and float32 partial sums of dw and db. */
size_t bra_backward_workspace_bytes(int B, int H, int W, int C, int heads,
                                    int S, int topk, int lepe_ks);

/* Gradients of bra_attend's output (with LePE when lepe_w is not NULL).
 *   q, k, v, dout [B,H,W,C] bf16, device; idx int32 [B, S*S, topk] (entries
 *   clamped into [0, S*S) as in bra_attend); attn_scale as in bra_attend.
 *   dq, dk, dv out: [B,H,W,C] bf16, device, overlapping no input or each
 *   other.  dlepe_w out: float32 [C, ks, ks] (required with lepe_w);
 *   dlepe_b out: float32 [C] or NULL.  ws: device workspace of at least
 *   bra_backward_workspace_bytes(...) bytes. */
bra_status bra_attend_backward(const void* q, const void* k, const void* v,
                               const int32_t* idx, const void* dout, int B,
                               int H, int W, int C, int heads, int S, int topk,
                               bra_dtype dtype, float attn_scale,
                               const float* lepe_w, int lepe_ks, void* dq,
                               void* dk, void* dv, float* dlepe_w,
                               float* dlepe_b, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Video clips (p3 §6.1: the spatio-temporal cube cut into T x K x K
 * regions).  A region is one frame's S x S block (K = S), numbered
 * r = t*S*S + ry*S + rx; routing runs over all T*S*S regions of a clip, so
 * a region may attend to regions of other frames; LePE is the 2-D
 * depthwise conv of each frame, zero padded at the frame's borders.
 * ------------------------------------------------------------------------ */

/* Workspace bytes of bra_video_forward: 2*B*T*S*S*C*8 (float64 region means
 * of q, then of k). */
size_t bra_video_workspace_bytes(int B, int T, int S, int C);

/* Region means, affinity and top-k over each clip's T*S*S regions
 * (bra_route for clips): q, k [B, T, H, W, C]; idx [B, T*S*S, topk];
 * ws of bra_video_workspace_bytes(B, T, S, C). */
bra_status bra_video_route(const void* q, const void* k, int B, int T, int H,
                           int W, int C, int S, int topk, bra_dtype dtype,
                           float route_scale, int32_t* idx,
                           float* topk_logits, void* ws, size_t ws_bytes,
                           void* stream);

/* Gather-attention over the routed regions of a clip plus per-frame LePE,
 * with a caller-supplied index (bra_attend for clips; the fixed-routing use
 * of p2 §5): idx [B, T*S*S, topk], entries clamped into [0, T*S*S). */
bra_status bra_video_attend(const void* q, const void* k, const void* v,
                            const int32_t* idx, int B, int T, int H, int W,
                            int C, int heads, int S, int topk,
                            bra_dtype dtype, float attn_scale,
                            const float* lepe_w, const float* lepe_b,
                            int lepe_ks, void* out, void* stream);

/* The forward pass on clips: bra_video_route then bra_video_attend.
 *   q, k, v, out  [B, T, H, W, C] dtype, device (frames contiguous; as for
 *                 bra_forward, out must not overlap q, k or v).
 *   idx           out: int32 [B, T*S*S, topk], device; topk_logits
 *                 float32 of the same shape or NULL.
 *   T*S*S <= 1024 regions per clip and T*H*W*C < 2^31 (BRA_E_UNSUPPORTED
 *   otherwise); the remaining arguments and errors as bra_forward, with
 *   topk in [1, T*S*S]. */
bra_status bra_video_forward(const void* q, const void* k, const void* v,
                             int B, int T, int H, int W, int C, int heads,
                             int S, int topk, bra_dtype dtype,
                             float route_scale, float attn_scale,
                             const float* lepe_w, const float* lepe_b,
                             int lepe_ks, void* out, int32_t* idx,
                             float* topk_logits, void* ws, size_t ws_bytes,
                             void* stream);

/* Static text for a status code. */
const char* bra_strerror(int status);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char* bra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BRA_H_ */
