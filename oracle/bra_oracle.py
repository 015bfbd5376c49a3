"""fp64 CPU oracle for the Bi-Level Routing Attention (BRA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, helper,
constant or table with the HIP library; the only thing both sides share is the
seeded input generator (``vision_transformer_dynamic_region_amd.workloads``),
which holds none of the method's arithmetic.

Everything here is plain NumPy in float64, written as the definitions the
pages give, step by step, with no blocking, fusion or reordering.

Sources (the pages, cited by key, page title and section):

  p1  "CVPR2023: BiFormer中的双层路由注意力机制解析" (cybasar.com news 187266)
      §2 (the core design: region-level routing, then token-level attention),
      §3 (the implementation walk-through with a PyTorch-style sketch),
      §4 (architecture: per-stage top-k), §5 (tuning: S per task).
  p2  "从静态到动态：BRA双层路由注意力如何革新视觉Transformer的计算范式"
      (snabindia.com news 101103)
      §2 (region mean pooling over the region-internal axes),
      §4 (TopkRouting: scaled region affinity, top-k; the LePE depthwise conv),
      §5 (routing index held fixed at deployment).
  p4  "Biformer注意力机制的原理及数学公式推导" (un.csdn.net) -- a different
      method; only its local-window softmax(QK^T/sqrt(d_k))V formula is used,
      as a special case in the tests.
  p5  "BiFormer: Vision Transformer mit Bi-Level-Routing-Attention"
      (hyper.ai, arXiv 2303.08810 abstract): filter irrelevant key/value pairs
      at region level, then token-to-token attention over the union of the
      routed regions.

Readings taken where the pages are silent or garbled (each one is listed with
its reason in the design notes of the repository):

  R1  The sketch in p1 §3 lost its '=', '@' and '+=' operators in extraction;
      it is read with them restored.
  R2  Regions are row-major over the S x S grid; tokens are row-major inside a
      region (p1 §3: reshape to (S, H/S, S, W/S, C), swap axes 1 and 2).
  R3  H and W must be divisible by S; nothing is padded.
  R4  Routing is per image over all C channels and is shared by every head
      (the region affinity in p1 §3 has no head axis).
  R5  Routing scale: p1 §3 has none, p2 §4 multiplies by a scale; it is a
      caller-chosen positive number (default C**-0.5).  A positive scale never
      changes the order of the affinities.
  R6  Top-k order: descending affinity, ties go to the lower region index.
      A region's own index is not forced into its route.
  R7  Region descriptor is the mean (both sketches use a mean).
  R8  Heads are contiguous d-channel slices, d = C / heads; attention scale is
      a caller-chosen number (default d**-0.5).
  R9  LePE is a depthwise ks x ks cross-correlation (PyTorch Conv2d
      convention) of V over the whole image, zero padding ks // 2, stride 1,
      optional per-channel bias, added to the attention output (p2 §4, p1 §3).
  R10 Softmax is max-subtracted, with no dropout and no mask other than the
      routing.
  R11 Output of the method is (out, idx); no Q/K/V or output projection.

Readings for the module around the method (``module_forward``):

  M1  Q, K and V are per-token linear maps of the input x (p1 §3 q_proj,
      k_proj, v_proj) in the PyTorch Linear convention y = x W^T + b.  The
      three weights are stacked into one [3C, C] matrix (rows 0..C-1 give Q,
      then K, then V) with an optional [3C] bias; p2 §2 slices its keys out
      of one projected tensor, which is the same thing.  A per-token map
      commutes with the partition, so it is applied before it.
  M2  The pages show no output projection.  The module takes an optional
      [C, C] output Linear (with optional bias) applied to out = O + L;
      without it the module returns O + L.
  M3  LePE is taken on the projected V (p1 §3 adds lce(v) to the output).
  M4  The pages fix no precision.  A model that runs in a narrower format
      stores each layer's output in that format: Q, K and V as the
      projection's output, y = O + L as the attention layer's output
      (``storage``: None keeps float64, "f32" / "bf16" round to nearest
      even).  The region means that decide the routing are those of the
      projections as computed, before they are stored (equivalently the
      projection of x's region means, since a region mean commutes with a
      per-token linear map).

Readings for the BiFormer block around the module (``block_forward``):

  B1  Structure (p3 §3.1 BiFormerBlock, pre-norm residuals; p1 §4 3x3 conv
      position encoding and a two-layer MLP of ratio 3):
        x1 = x + dwconv3x3(x) + b_pos
        x2 = x1 + module(LN1(x1))
        x3 = x2 + fc2(GELU(fc1(LN2(x2))))
      p3's ConvFFN is not used: p1 (the more detailed page on the block's
      parts) gives a plain two-layer MLP, and the 3x3 conv is the position
      encoding before the attention.
  B2  The position encoding is a depthwise 3x3 cross-correlation (groups = C,
      zero padding 1) with bias, like the LePE term.
  B3  LayerNorm over the C channels of each token, biased variance, eps 1e-5
      (PyTorch nn.LayerNorm, as p3's block uses), with per-channel scale and
      shift.
  B4  The MLP's activation is GELU in its exact (erf) form; the pages name no
      activation, and GELU is the usual one of a transformer MLP.
  B5  Storage (as M4): x1, LN1(x1), the module's stored values, x2,
      LN2(x2), the hidden GELU output and x3 are layer outputs, stored per
      ``storage``.

The backward pass with a fixed routing index (``bra_backward``): the pages
train with the routing held fixed for a while (p2 §5 and p1 §5 keep the
index constant; p2 §4 detaches the routing inputs unless diff_routing is
set), so the index receives no gradient and the gradients of
out = O(Q, K, V; idx) + LePE(V) are those of the attention and of the
depthwise conv:

  G1  Per query region and head, with p = softmax(s), s = scale q k^T over
      the routed keys: dv = p^T do, dp = do v^T, ds = p * (dp - rowsum(p *
      dp)), dq = scale ds k, dk = scale ds^T q; dk and dv are added into the
      key tokens' rows (a key region routed from several query regions
      collects all their terms).
  G2  LePE: db = the sum of dout over the pixels, dw[c, i, j] = the sum of
      dout * V shifted by (i - P, j - P) (zero outside), and dV gains the
      transposed conv of dout with w.

Readings for video (``video_forward``), from the one line p3 gives under
§6.1 (video adaptation: the spatio-temporal cube is cut into T x K x K
regions):

  V1  T is the clip's frame count, so a region is one frame's K x K block
      (K = S, the image model's grid); regions are numbered frame-major, then
      row-major over the frame's grid: r = t * S*S + ry * S + rx, tokens
      row-major inside the region (as R2).
  V2  Routing runs over all T*S*S regions of a clip: one affinity matrix per
      clip and a top-k per row, as in the image case (R4-R6), so a region
      may route to regions of other frames.
  V3  LePE is the image model's 2-D depthwise conv applied to each frame
      (zero padding at the frame's borders); the pages give no temporal
      kernel.
  V4  p3 §6.1's optical-flow modulation of the temporal routing weights and
      its cross-frame token sharing are not modelled: no flow input is given
      and the sharing is not specified.

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "region_shape",
    "region_token_maps",
    "region_mean",
    "region_affinity",
    "topk_route",
    "region_tokens",
    "routed_attention",
    "lepe",
    "bra_forward",
    "linear",
    "round_storage",
    "module_forward",
    "layer_norm",
    "gelu",
    "block_forward",
    "bra_backward",
    "video_regions",
    "video_forward",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def region_shape(H: int, W: int, S: int) -> tuple[int, int]:
    """Region height and width for an S x S grid (p1 §2, §3; reading R3)."""
    if S < 1 or H % S or W % S:
        raise ValueError(f"S={S} must divide H={H} and W={W}")
    return H // S, W // S


def region_token_maps(H: int, W: int, S: int) -> tuple[np.ndarray, np.ndarray]:
    """Partition step (p1 §3, reading R2).

    Returns two int arrays of shape [H, W]: the region index of each pixel
    (row-major over the S x S grid) and its token index inside its region
    (row-major over the hs x ws region).
    """
    hs, ws = region_shape(H, W, S)
    y = np.arange(H)[:, None]
    x = np.arange(W)[None, :]
    region = (y // hs) * S + (x // ws)
    token = (y % hs) * ws + (x % ws)
    return region.astype(np.int64), token.astype(np.int64)


def region_tokens(H: int, W: int, S: int, r: int) -> tuple[np.ndarray, np.ndarray]:
    """(ys, xs) pixel coordinates of region r's tokens in token order (R2)."""
    hs, ws = region_shape(H, W, S)
    ry, rx = divmod(int(r), S)
    t = np.arange(hs * ws)
    return ry * hs + t // ws, rx * ws + t % ws


def region_mean(X, S: int) -> np.ndarray:
    """Region pooling (p1 §3 region-mean step; p2 §2 mean over the region axes).

    X: [B, H, W, C].  Returns [B, S*S, C]: the mean of each region's tokens,
    regions row-major (R2, R7).
    """
    X = _f64(X)
    B, H, W, C = X.shape
    hs, ws = region_shape(H, W, S)
    out = np.empty((B, S * S, C), dtype=np.float64)
    for i in range(S):
        for j in range(S):
            block = X[:, i * hs:(i + 1) * hs, j * ws:(j + 1) * ws, :]
            out[:, i * S + j, :] = block.reshape(B, hs * ws, C).mean(axis=1)
    return out


def region_affinity(q_r, k_r, route_scale: float) -> np.ndarray:
    """Region-to-region affinity (p1 §3; p2 §4 with its scale; R4, R5).

    q_r, k_r: [B, S*S, C] region means.  Returns [B, S*S, S*S] with entry
    [b, r, s] = route_scale * <q_r[b, r], k_r[b, s]>.
    """
    q_r = _f64(q_r)
    k_r = _f64(k_r)
    return float(route_scale) * np.matmul(q_r, np.swapaxes(k_r, -1, -2))


def topk_route(A, topk: int) -> np.ndarray:
    """Top-k routing index (p1 §3 top-k over the affinity rows; p2 §4; R6).

    A: [B, R, R].  Returns int32 [B, R, topk]: per row, the column indices of
    the topk largest entries, largest first, equal values by lower index.
    """
    A = _f64(A)
    R = A.shape[-1]
    if not 1 <= topk <= R:
        raise ValueError(f"topk={topk} must be in [1, {R}]")
    # A stable sort of the negated values keeps equal values in index order.
    order = np.argsort(-A, axis=-1, kind="stable")
    return order[..., :topk].astype(np.int32)


def routed_attention(Q, K, V, idx, heads: int, S: int, attn_scale: float) -> np.ndarray:
    """Token-to-token attention over the routed regions (p1 §3 gather and
    attention; p5: attention over the union of the routed regions; R8, R10).

    Q, K, V: [B, H, W, C]; idx: [B, S*S, topk] region indices.
    For query pixel p in region r, the keys are all tokens of the regions
    idx[b, r, 0..topk-1] (region order, then token order; the order does not
    change the result).  Per head m (channels m*d .. m*d+d-1):
        O_p = sum_t softmax_t(attn_scale * <Q_p, K_t>) V_t.
    Returns O: [B, H, W, C] float64.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    idx = np.asarray(idx)
    B, H, W, C = Q.shape
    if C % heads:
        raise ValueError("heads must divide C")
    d = C // heads
    n_reg = S * S
    coords = [region_tokens(H, W, S, r) for r in range(n_reg)]
    O = np.zeros_like(Q)
    for b in range(B):
        for r in range(n_reg):
            ys, xs = coords[r]
            q = Q[b, ys, xs, :].reshape(-1, heads, d)            # [n, h, d]
            key_y = np.concatenate([coords[s][0] for s in idx[b, r]])
            key_x = np.concatenate([coords[s][1] for s in idx[b, r]])
            k = K[b, key_y, key_x, :].reshape(-1, heads, d)      # [m, h, d]
            v = V[b, key_y, key_x, :].reshape(-1, heads, d)
            logits = attn_scale * np.einsum("nhd,mhd->hnm", q, k)
            logits = logits - logits.max(axis=-1, keepdims=True)
            p = np.exp(logits)
            p = p / p.sum(axis=-1, keepdims=True)
            o = np.einsum("hnm,mhd->nhd", p, v)
            O[b, ys, xs, :] = o.reshape(-1, C)
    return O


def lepe(V, w, bias=None) -> np.ndarray:
    """Local enhancement term (p2 §4 depthwise Conv2d on V; p1 §3 adds it to the
    attention output; R9).

    V: [B, H, W, C]; w: [C, ks, ks]; bias: [C] or None.
    L[b, y, x, c] = bias[c] + sum_{i,j} w[c, i, j] * V[b, y+i-ks//2, x+j-ks//2, c],
    with V taken as zero outside the image.
    """
    V = _f64(V)
    w = _f64(w)
    B, H, W, C = V.shape
    ks = w.shape[-1]
    if w.shape != (C, ks, ks) or ks % 2 == 0:
        raise ValueError("w must be [C, ks, ks] with odd ks")
    p = ks // 2
    Vp = np.zeros((B, H + 2 * p, W + 2 * p, C), dtype=np.float64)
    Vp[:, p:p + H, p:p + W, :] = V
    L = np.zeros_like(V)
    for i in range(ks):
        for j in range(ks):
            L += w[:, i, j] * Vp[:, i:i + H, j:j + W, :]
    if bias is not None:
        L += _f64(bias)
    return L


def bra_forward(Q, K, V, heads: int, S: int, topk: int, w=None, bias=None,
                route_scale: float | None = None, attn_scale: float | None = None,
                return_parts: bool = False):
    """The whole BRA forward pass in the pages' order (p1 §3; p2 §2, §4).

    partition -> region means -> scaled affinity -> top-k index ->
    attention over the routed regions -> + LePE(V).
    Returns (out, idx) or, with return_parts, a dict with every intermediate.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    B, H, W, C = Q.shape
    region_shape(H, W, S)
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    q_r = region_mean(Q, S)
    k_r = region_mean(K, S)
    A = region_affinity(q_r, k_r, route_scale)
    idx = topk_route(A, topk)
    O = routed_attention(Q, K, V, idx, heads, S, attn_scale)
    L = lepe(V, w, bias) if w is not None else np.zeros_like(O)
    out = O + L
    if return_parts:
        return {"out": out, "idx": idx, "q_r": q_r, "k_r": k_r, "A": A,
                "O": O, "L": L}
    return out, idx


def video_regions(T: int, H: int, W: int, S: int) -> list:
    """3-D partition of a clip (p3 §6.1; readings V1, V2).

    Returns, for r = t * S*S + ry * S + rx, the (ts, ys, xs) coordinates of
    region r's tokens in token order: frame t, rows ry*hs .. ry*hs+hs-1,
    columns rx*ws .. rx*ws+ws-1, row-major.
    """
    hs, ws = region_shape(H, W, S)
    regs = []
    for t in range(T):
        for ry in range(S):
            for rx in range(S):
                tok = np.arange(hs * ws)
                regs.append((np.full(hs * ws, t), ry * hs + tok // ws, rx * ws + tok % ws))
    return regs


def video_forward(Q, K, V, heads: int, S: int, topk: int, w=None, bias=None,
                  route_scale: float | None = None, attn_scale: float | None = None,
                  return_parts: bool = False, idx=None):
    """BRA on a clip (p3 §6.1 T x K x K regions; readings V1-V4).

    Q, K, V: [B, T, H, W, C].  Per clip: the means of the T*S*S regions, the
    scaled affinity between them, the top-k index per region (over the whole
    clip), attention of each query token over the tokens of its routed
    regions, plus the per-frame LePE of V.  Returns (out [B, T, H, W, C],
    idx [B, T*S*S, topk]) or, with return_parts, a dict of intermediates.
    With idx given, that index is used for the attention (the fixed-routing
    use) and the routing only fills the returned parts.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    B, T, H, W, C = Q.shape
    if C % heads:
        raise ValueError("heads must divide C")
    d = C // heads
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = d ** -0.5
    regs = video_regions(T, H, W, S)
    R = len(regs)
    q_r = np.empty((B, R, C))
    k_r = np.empty((B, R, C))
    for r, (ts, ys, xs) in enumerate(regs):
        q_r[:, r] = Q[:, ts, ys, xs].mean(axis=1)
        k_r[:, r] = K[:, ts, ys, xs].mean(axis=1)
    A = region_affinity(q_r, k_r, route_scale)
    idx = topk_route(A, topk) if idx is None else np.asarray(idx)
    O = np.zeros_like(Q)
    for b in range(B):
        for r, (ts, ys, xs) in enumerate(regs):
            q = Q[b, ts, ys, xs].reshape(-1, heads, d)
            kt = np.concatenate([regs[s][0] for s in idx[b, r]])
            ky = np.concatenate([regs[s][1] for s in idx[b, r]])
            kx = np.concatenate([regs[s][2] for s in idx[b, r]])
            k = K[b, kt, ky, kx].reshape(-1, heads, d)
            v = V[b, kt, ky, kx].reshape(-1, heads, d)
            logits = attn_scale * np.einsum("nhd,mhd->hnm", q, k)
            logits = logits - logits.max(axis=-1, keepdims=True)
            p = np.exp(logits)
            p = p / p.sum(axis=-1, keepdims=True)
            O[b, ts, ys, xs] = np.einsum("hnm,mhd->nhd", p, v).reshape(-1, C)
    if w is not None:
        L = lepe(V.reshape(B * T, H, W, C), w, bias).reshape(B, T, H, W, C)
    else:
        L = np.zeros_like(O)
    out = O + L
    if return_parts:
        return {"out": out, "idx": idx, "q_r": q_r, "k_r": k_r, "A": A, "O": O, "L": L}
    return out, idx


def linear(X, w, b=None) -> np.ndarray:
    """Per-token linear map in the PyTorch Linear convention (p1 §3 q_proj /
    k_proj / v_proj; readings M1, M2).

    X: [..., K]; w: [N, K]; b: [N] or None.  Returns X w^T + b, [..., N].
    """
    X = _f64(X)
    w = _f64(w)
    if w.ndim != 2 or w.shape[1] != X.shape[-1]:
        raise ValueError("w must be [N, K] with K the last axis of X")
    Y = np.matmul(X, w.T)
    if b is not None:
        Y = Y + _f64(b)
    return Y


def round_storage(X, storage):
    """Round to a layer output's storage format (reading M4): None keeps
    float64, "f32" rounds to float32 (NumPy's cast rounds to nearest even),
    "bf16" to bfloat16 with round-to-nearest-even on the float64 value
    (8 significant bits; below 2**-126 a fixed spacing of 2**-133, as in
    float32; finite values only)."""
    X = _f64(X)
    if storage is None:
        return X
    if storage == "f32":
        return X.astype(np.float32).astype(np.float64)
    if storage != "bf16":
        raise ValueError(f"storage {storage!r} is not None, 'f32' or 'bf16'")
    _, e = np.frexp(X)                    # X = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)               # spacing 2**(e - 8), at least 2**-133
    return np.ldexp(np.round(np.ldexp(X, 8 - e)), e - 8)


def module_forward(x, w_qkv, b_qkv, heads: int, S: int, topk: int, lepe_w=None,
                   lepe_b=None, w_out=None, b_out=None, route_scale: float | None = None,
                   attn_scale: float | None = None, storage: str | None = None,
                   return_parts: bool = False, idx=None):
    """BRA as a module (p1 §3): Q, K, V = projections of x (M1); routing on
    their region means; attention over the routed regions and LePE on the
    projected V (M3), with Q, K, V and y = O + L stored per ``storage`` (M4);
    then the optional output projection (M2).

    x: [B, H, W, C]; w_qkv: [3C, C]; b_qkv: [3C] or None; w_out: [C, C] or
    None; b_out: [C] or None.  idx: [B, S*S, topk] to attend over a given
    route instead of the top-k of the affinities (the fixed-index use of
    p2 §5; the affinities are still returned).  Returns (out, idx) or, with
    return_parts, a dict with every intermediate: q, k, v (as stored), q_r,
    k_r, A, idx, O, L, y (as stored) and out.
    """
    x = _f64(x)
    B, H, W, C = x.shape
    region_shape(H, W, S)
    if np.shape(w_qkv) != (3 * C, C):
        raise ValueError("w_qkv must be [3C, C]")
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    qkv = linear(x, w_qkv, b_qkv)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    q_r = region_mean(q, S)
    k_r = region_mean(k, S)
    A = region_affinity(q_r, k_r, route_scale)
    if idx is None:
        idx = topk_route(A, topk)
    else:
        idx = np.asarray(idx, dtype=np.int64)
        if idx.shape != (B, S * S, topk) or idx.min() < 0 or idx.max() >= S * S:
            raise ValueError("idx must be [B, S*S, topk] with entries in [0, S*S)")
    q, k, v = (round_storage(t, storage) for t in (q, k, v))
    O = routed_attention(q, k, v, idx, heads, S, attn_scale)
    L = lepe(v, lepe_w, lepe_b) if lepe_w is not None else np.zeros_like(O)
    y = round_storage(O + L, storage)
    out = linear(y, w_out, b_out) if w_out is not None else y
    if return_parts:
        return {"q": q, "k": k, "v": v, "q_r": q_r, "k_r": k_r, "A": A, "idx": idx, "O": O,
                "L": L, "y": y, "out": out}
    return out, idx


def layer_norm(X, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis (reading B3): (X - mean) / sqrt(var + eps)
    * gamma + beta, with the biased variance of the channels."""
    X = _f64(X)
    mu = X.mean(axis=-1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=-1, keepdims=True)
    return (X - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def gelu(X) -> np.ndarray:
    """GELU, exact form (reading B4): x * Phi(x) = x / 2 * (1 + erf(x / sqrt 2))."""
    from scipy.special import erf          # the error function, as a library step
    X = _f64(X)
    return 0.5 * X * (1.0 + erf(X / math.sqrt(2.0)))


def block_forward(x, p: dict, heads: int, S: int, topk: int, route_scale: float | None = None,
                  attn_scale: float | None = None, storage: str | None = None,
                  return_parts: bool = False, idx=None):
    """One BiFormer block (readings B1-B5) around the BRA module.

    p holds the parameters: pos_w [C, 3, 3], pos_b [C]; ln1_g, ln1_b [C];
    w_qkv [3C, C], b_qkv [3C]; lepe_w [C, ks, ks], lepe_b [C] or None; w_out
    [C, C], b_out [C]; ln2_g, ln2_b [C]; w_fc1 [3C, C], b_fc1 [3C]; w_fc2
    [C, 3C], b_fc2 [C].  idx, if given, is the module's route (see
    module_forward).  Returns (out, idx) or, with return_parts, every stored
    intermediate (x1, n1, the module's parts under "mod", x2, n2, h, out).
    """
    st = lambda t: round_storage(t, storage)
    x = _f64(x)
    x1 = st(x + lepe(x, p["pos_w"], p["pos_b"]))
    n1 = st(layer_norm(x1, p["ln1_g"], p["ln1_b"]))
    mod = module_forward(n1, p["w_qkv"], p["b_qkv"], heads, S, topk, p["lepe_w"], p["lepe_b"],
                         p["w_out"], p["b_out"], route_scale, attn_scale, storage,
                         return_parts=True, idx=idx)
    x2 = st(x1 + mod["out"])
    n2 = st(layer_norm(x2, p["ln2_g"], p["ln2_b"]))
    h = st(gelu(linear(n2, p["w_fc1"], p["b_fc1"])))
    out = st(x2 + linear(h, p["w_fc2"], p["b_fc2"]))
    if return_parts:
        return {"x1": x1, "n1": n1, "mod": mod, "x2": x2, "n2": n2, "h": h, "out": out,
                "idx": mod["idx"]}
    return out, mod["idx"]


def bra_backward(Q, K, V, idx, heads: int, S: int, dout, w=None, bias=None,
                 attn_scale: float | None = None) -> dict:
    """Gradients of out = routed attention(Q, K, V; idx) + LePE(V) with the
    routing index held fixed (readings G1, G2).

    dout: [B, H, W, C], the gradient of the output.  Returns a dict with dQ,
    dK, dV ([B, H, W, C]) and, when w is given, dw [C, ks, ks] and db [C]
    (db is returned whether or not the forward pass had a bias).
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    G = _f64(dout)
    idx = np.asarray(idx)
    B, H, W, C = Q.shape
    if C % heads:
        raise ValueError("heads must divide C")
    d = C // heads
    if attn_scale is None:
        attn_scale = d ** -0.5
    coords = [region_tokens(H, W, S, r) for r in range(S * S)]
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for r in range(S * S):
            ys, xs = coords[r]
            ky = np.concatenate([coords[s][0] for s in idx[b, r]])
            kx = np.concatenate([coords[s][1] for s in idx[b, r]])
            q = Q[b, ys, xs].reshape(-1, heads, d)
            k = K[b, ky, kx].reshape(-1, heads, d)
            v = V[b, ky, kx].reshape(-1, heads, d)
            do = G[b, ys, xs].reshape(-1, heads, d)
            s_ = attn_scale * np.einsum("nhd,mhd->hnm", q, k)
            p = np.exp(s_ - s_.max(axis=-1, keepdims=True))
            p = p / p.sum(axis=-1, keepdims=True)                   # [h, n, m]
            dv = np.einsum("hnm,nhd->mhd", p, do)
            dp = np.einsum("nhd,mhd->hnm", do, v)
            ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
            dq = attn_scale * np.einsum("hnm,mhd->nhd", ds, k)
            dk = attn_scale * np.einsum("hnm,nhd->mhd", ds, q)
            dQ[b, ys, xs] += dq.reshape(-1, C)
            # keys may repeat across (and, for a caller's index, within) rows
            np.add.at(dK[b], (ky, kx), dk.reshape(-1, C))
            np.add.at(dV[b], (ky, kx), dv.reshape(-1, C))
    out = {"dQ": dQ, "dK": dK, "dV": dV}
    if w is not None:
        w = _f64(w)
        ks = w.shape[-1]
        P = ks // 2
        Vp = np.zeros((B, H + 2 * P, W + 2 * P, C))
        Vp[:, P:P + H, P:P + W] = V
        Gp = np.zeros((B, H + 2 * P, W + 2 * P, C))
        Gp[:, P:P + H, P:P + W] = G
        dw = np.zeros((C, ks, ks))
        for i in range(ks):
            for j in range(ks):
                dw[:, i, j] = np.sum(G * Vp[:, i:i + H, j:j + W], axis=(0, 1, 2))
                # L[y, x] += w[i, j] V[y + i - P, x + j - P], so V[y', x'] feeds
                # L[y' - i + P, x' - j + P]
                dV += w[:, i, j] * Gp[:, 2 * P - i:2 * P - i + H, 2 * P - j:2 * P - j + W]
        out["dw"] = dw
        out["db"] = G.sum(axis=(0, 1, 2))
    return out
