"""Bi-Level Routing Attention (BiFormer) forward pass on AMD MI355X.

A thin ctypes binding over ``libbra.so`` (declared in ``include/bra.h``).
It only marshals arguments: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.

    out, idx = forward(q, k, v, heads, S, topk, lepe_w)

q, k, v: CUDA tensors [B, H, W, C] (float32 or bfloat16), contiguous;
lepe_w: float32 [C, ks, ks] (depthwise conv weight), optional.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["BraError", "lib_path", "load", "workspace_bytes", "route", "attend",
           "forward", "forward_noalloc", "lepe", "linear", "module_workspace_bytes", "module_forward",
           "layer_norm", "pos_conv", "block_workspace_bytes", "block_forward", "BLOCK_PARAMS",
           "attend_backward", "video_workspace_bytes", "video_forward", "video_route",
           "video_attend", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS = {0: "BRA_OK", 1: "BRA_E_INVAL", 2: "BRA_E_UNSUPPORTED", 3: "BRA_E_WORKSPACE",
          4: "BRA_E_HIP"}
_F32, _BF16 = 0, 1

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "bra_workspace_bytes": (_sz, [_i, _i, _i]),
    "bra_route": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "bra_attend": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i,
                        _vp, _vp]),
    "bra_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _f, _vp, _vp, _i,
                         _vp, _vp, _vp, _vp, _sz, _vp]),
    "bra_forward_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _f, _vp, _vp,
                                 _i, _vp, _vp, _vp, _vp]),
    "bra_lepe": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_linear": (_i, [_vp, _i, _i, _vp, _vp, _i, _i, _vp, _i, _vp, _vp]),
    "bra_pos_conv": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_module_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "bra_module_forward": (_i, [_vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _f, _f, _vp, _vp,
                                _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bra_layer_norm": (_i, [_vp, _i, _i, _vp, _vp, _f, _i, _vp, _vp]),
    "bra_mlp": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp]),
    "bra_block_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "bra_block_forward": (_i, [_vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _f, _f, _vp, _vp, _vp,
                               _sz, _vp]),
    "bra_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "bra_attend_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                                 _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bra_video_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "bra_video_route": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz,
                             _vp]),
    "bra_video_attend": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                              _vp, _i, _vp, _vp]),
    "bra_video_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _f, _vp,
                               _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bra_strerror": (ctypes.c_char_p, [_i]),
    "bra_last_error": (ctypes.c_char_p, []),
}


class BraError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def lib_path() -> str:
    return os.path.join(_HERE, "libbra.so")


def load(require_torch: bool = True):
    """Load libbra.so once.  With require_torch, torch is imported first so
    that the library binds to the HIP runtime torch already loaded."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if require_torch:
        import torch  # noqa: F401
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m vision_transformer_dynamic_region_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int):
    if status != 0:
        raise BraError(status, load().bra_last_error().decode())


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return _F32
    if t.dtype == torch.bfloat16:
        return _BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _on_device(t) -> bool:
    return t.device.type == "cuda"


def _dev(t, name, dtype=None, shape=None):
    """data_ptr() of a contiguous CUDA tensor, after checking its dtype and
    (when given) its exact shape.  Every pointer the binding hands to the
    library passes through here, so a host tensor or a short buffer is
    rejected before anything is launched."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(t):
        raise ValueError(f"{name} must be a CUDA (HIP) tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    return t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def workspace_bytes(B: int, S: int, C: int) -> int:
    return int(load().bra_workspace_bytes(B, S, C))


def _bhwc(q):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, W, C]")
    return tuple(int(x) for x in q.shape)


def _workspace(ws, need: int, device):
    """(pointer, bytes) of the caller's workspace, or of a new one of
    max(need, 16) bytes; a given workspace must hold at least need bytes."""
    import torch
    if ws is None:
        ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device=device)
    ptr = _dev(ws, "workspace")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace has {nbytes} bytes, {need} needed")
    return ptr, nbytes


def _lepe_args(lepe_w, lepe_b, C):
    import torch
    if lepe_w is None:
        return None, None, 0
    _dev(lepe_w, "lepe_w", torch.float32)
    if lepe_w.dim() != 3 or lepe_w.shape[0] != C or lepe_w.shape[1] != lepe_w.shape[2]:
        raise ValueError("lepe_w must be [C, ks, ks]")
    bptr = None
    if lepe_b is not None:
        _dev(lepe_b, "lepe_b", torch.float32)
        if tuple(lepe_b.shape) != (C,):
            raise ValueError("lepe_b must be [C]")
        bptr = lepe_b.data_ptr()
    return lepe_w.data_ptr(), bptr, int(lepe_w.shape[-1])


def route(q, k, S: int, topk: int, route_scale: float | None = None, workspace=None,
          return_logits: bool = False):
    """Region means, scaled region affinity and per-row top-k (bra_route).

    Returns idx int32 [B, S*S, topk] (and float32 logits with return_logits).
    workspace, if given, is a CUDA uint8 tensor of >= workspace_bytes(B, S, C)
    bytes; after the call it holds the float64 region means of q then k.
    """
    import torch
    B, H, W, C = _bhwc(q)
    dt = _dtype_code(q)
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    if tuple(k.shape) != (B, H, W, C):
        raise ValueError("q and k must have the same shape")
    if route_scale is None:
        route_scale = C ** -0.5
    idx = torch.empty((B, S * S, topk), dtype=torch.int32, device=q.device)
    logits = torch.empty((B, S * S, topk), dtype=torch.float32, device=q.device) if return_logits else None
    wsp, wsb = _workspace(workspace, workspace_bytes(B, S, C), q.device)
    _check(load().bra_route(q.data_ptr(), k.data_ptr(), B, H, W, C, S, topk, dt, float(route_scale),
                            idx.data_ptr(), logits.data_ptr() if logits is not None else None,
                            wsp, wsb, _stream(q)))
    return (idx, logits) if return_logits else idx


def attend(q, k, v, idx, heads: int, S: int, attn_scale: float | None = None, lepe_w=None,
           lepe_b=None, out=None):
    """Gather-attention over the routed regions plus optional LePE (bra_attend)."""
    import torch
    B, H, W, C = _bhwc(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype)
        if tuple(t.shape) != (B, H, W, C):
            raise ValueError("q, k, v must have the same shape")
    _dev(idx, "idx", torch.int32)
    if idx.dim() != 3 or idx.shape[0] != B or idx.shape[1] != S * S:
        raise ValueError("idx must be [B, S*S, topk]")
    topk = int(idx.shape[2])
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, (B, H, W, C))
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), B, H, W, C,
                             heads, S, topk, dt, float(attn_scale), wp, bp, ks, out.data_ptr(),
                             _stream(q)))
    return out


def forward(q, k, v, heads: int, S: int, topk: int, lepe_w=None, lepe_b=None,
            route_scale: float | None = None, attn_scale: float | None = None, out=None,
            idx=None, workspace=None, return_logits: bool = False):
    """The whole BRA forward pass (bra_forward).  Returns (out, idx) or
    (out, idx, logits) with return_logits.  workspace, if given, is scratch
    (its contents afterwards are unspecified)."""
    import torch
    B, H, W, C = _bhwc(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype)
        if tuple(t.shape) != (B, H, W, C):
            raise ValueError("q, k, v must have the same shape")
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, (B, H, W, C))
    if idx is None:
        idx = torch.empty((B, S * S, topk), dtype=torch.int32, device=q.device)
    _dev(idx, "idx", torch.int32, (B, S * S, topk))
    logits = torch.empty((B, S * S, topk), dtype=torch.float32, device=q.device) if return_logits else None
    wsp, wsb = _workspace(workspace, workspace_bytes(B, S, C), q.device)
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, W, C, heads, S, topk,
                              dt, float(route_scale), float(attn_scale), wp, bp, ks, out.data_ptr(),
                              idx.data_ptr(), logits.data_ptr() if logits is not None else None,
                              wsp, wsb, _stream(q)))
    return (out, idx, logits) if return_logits else (out, idx)


def forward_noalloc(q, k, v, heads: int, S: int, topk: int, out, idx, lepe_w=None, lepe_b=None,
                    route_scale: float | None = None, attn_scale: float | None = None,
                    logits=None):
    """bra_forward_noalloc: the forward pass for callers that cannot allocate.
    Nothing is allocated here or in the library: out ([B, H, W, C], q's
    dtype) and idx (int32 [B, S*S, topk]) are the caller's, as is logits
    (float32 [B, S*S, topk]) if given; the region means go to the library's
    static device scratch.  Returns (out, idx)."""
    import torch
    B, H, W, C = _bhwc(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype, (B, H, W, C))
    _dev(out, "out", q.dtype, (B, H, W, C))
    _dev(idx, "idx", torch.int32, (B, S * S, topk))
    lp = _dev(logits, "logits", torch.float32, (B, S * S, topk)) if logits is not None else None
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, W, C, heads,
                                      S, topk, dt, float(route_scale), float(attn_scale), wp, bp,
                                      ks, out.data_ptr(), idx.data_ptr(), lp, _stream(q)))
    return out, idx


def lepe(v, w, b, out):
    """out += b + depthwise conv(v, w) in place (bra_lepe).  Returns out."""
    B, H, W, C = _bhwc(v)
    dt = _dtype_code(v)
    _dev(v, "v")
    _dev(out, "out", v.dtype)
    if tuple(out.shape) != (B, H, W, C):
        raise ValueError("v and out must have the same shape")
    wp, bp, ks = _lepe_args(w, b, C)
    if wp is None:
        raise ValueError("w is required")
    _check(load().bra_lepe(v.data_ptr(), wp, bp, ks, B, H, W, C, dt, out.data_ptr(), _stream(v)))
    return out


def _opt(t, name, dtype, shape):
    """Pointer of an optional device tensor of the given dtype and shape."""
    if t is None:
        return None
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}")
    return t.data_ptr()


def linear(x, w, b=None, out=None, act: str | None = None, residual=None):
    """y = act(x w^T + b) + residual over the last axis (bra_linear): x [..., K],
    w [N, K] in x's dtype, b float32 [N] or None, act None or "gelu",
    residual [..., N] in x's dtype or None.  Returns y [..., N]."""
    import torch
    dt = _dtype_code(x)
    _dev(x, "x")
    _dev(w, "w", x.dtype)
    if w.dim() != 2 or w.shape[1] != x.shape[-1]:
        raise ValueError("w must be [N, K] with K = x.shape[-1]")
    N, K = int(w.shape[0]), int(w.shape[1])
    rows = x.numel() // K
    bp = _opt(b, "b", torch.float32, (N,))
    if act not in (None, "gelu"):
        raise ValueError("act must be None or 'gelu'")
    if out is None:
        out = torch.empty((*x.shape[:-1], N), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    if out.numel() != rows * N:
        raise ValueError("out must hold rows * N elements")
    rp = None
    if residual is not None:
        _dev(residual, "residual", x.dtype)
        if residual.numel() != rows * N:
            raise ValueError("residual must hold rows * N elements")
        rp = residual.data_ptr()
    _check(load().bra_linear(x.data_ptr(), rows, K, w.data_ptr(), bp, N, 1 if act else 0, rp, dt,
                             out.data_ptr(), _stream(x)))
    return out


def pos_conv(x, w, b=None, out=None):
    """out = x + b + depthwise 3x3 conv of x (bra_pos_conv); w float32 [C, 3, 3]."""
    import torch
    B, H, W, C = _bhwc(x)
    dt = _dtype_code(x)
    _dev(x, "x")
    _opt(w, "w", torch.float32, (C, 3, 3))
    bp = _opt(b, "b", torch.float32, (C,))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (B, H, W, C))
    _check(load().bra_pos_conv(x.data_ptr(), w.data_ptr(), bp, B, H, W, C, dt, out.data_ptr(),
                               _stream(x)))
    return out


def module_workspace_bytes(B: int, H: int, W: int, C: int, S: int, dtype_code: int,
                           with_out_proj: bool) -> int:
    return int(load().bra_module_workspace_bytes(B, H, W, C, S, dtype_code, int(bool(with_out_proj))))


def module_forward(x, w_qkv, b_qkv, heads: int, S: int, topk: int, lepe_w=None, lepe_b=None,
                   w_out=None, b_out=None, route_scale: float | None = None,
                   attn_scale: float | None = None, out=None, idx=None, workspace=None):
    """The BRA module (bra_module_forward): Q, K, V = x w_qkv^T + b_qkv, the
    BRA forward pass with LePE on V, then the optional output projection.
    Returns (out, idx).  workspace, if given, is a CUDA uint8 tensor of at
    least module_workspace_bytes(...) bytes; afterwards it holds the region
    means of x, Q and K and the tensors Q, K, V (and y when w_out is given),
    except Q, K and V where they are projected inside the attention kernel
    (bf16, C = 64, 8x8-pixel regions, top-1, 5x5 LePE, y not in x's memory)."""
    import torch
    B, H, W, C = _bhwc(x)
    dt = _dtype_code(x)
    _dev(x, "x")
    _dev(w_qkv, "w_qkv", x.dtype)
    if tuple(w_qkv.shape) != (3 * C, C):
        raise ValueError("w_qkv must be [3C, C]")
    bq = _opt(b_qkv, "b_qkv", torch.float32, (3 * C,))
    wo = _opt(w_out, "w_out", x.dtype, (C, C))
    bo = _opt(b_out, "b_out", torch.float32, (C,))
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (B, H, W, C))
    if idx is None:
        idx = torch.empty((B, S * S, topk), dtype=torch.int32, device=x.device)
    _dev(idx, "idx", torch.int32, (B, S * S, topk))
    wsp, wsb = _workspace(workspace, module_workspace_bytes(B, H, W, C, S, dt, w_out is not None),
                          x.device)
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_module_forward(x.data_ptr(), B, H, W, C, heads, S, topk, dt,
                                     w_qkv.data_ptr(), bq, float(route_scale), float(attn_scale),
                                     wp, bp, ks, wo, bo, out.data_ptr(), idx.data_ptr(),
                                     wsp, wsb, _stream(x)))
    return out, idx


def mlp(x, w1, b1, w2, b2, residual, out=None):
    """out = residual + fc2(GELU(fc1(x))) over the last axis in one launch
    (bra_mlp, bf16): x, residual [..., C]; w1 [Hd, C] and w2 [C, Hd] in x's
    dtype; b1 float32 [Hd] or None, b2 float32 [C] or None.  The hidden layer
    is rounded to bf16 and never written.  Returns out [..., C]."""
    import torch
    dt = _dtype_code(x)
    _dev(x, "x")
    C = int(x.shape[-1])
    _dev(w1, "w1", x.dtype)
    if w1.dim() != 2 or w1.shape[1] != C:
        raise ValueError("w1 must be [Hd, C] with C = x.shape[-1]")
    Hd = int(w1.shape[0])
    _dev(w2, "w2", x.dtype, (C, Hd))
    _dev(residual, "residual", x.dtype, tuple(x.shape))
    b1p = _opt(b1, "b1", torch.float32, (Hd,))
    b2p = _opt(b2, "b2", torch.float32, (C,))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, tuple(x.shape))
    _check(load().bra_mlp(x.data_ptr(), x.numel() // C, C, Hd, w1.data_ptr(), b1p,
                          w2.data_ptr(), b2p, residual.data_ptr(), dt, out.data_ptr(),
                          _stream(x)))
    return out


def layer_norm(x, gamma, beta, eps: float = 1e-5, out=None):
    """LayerNorm over the last axis (bra_layer_norm); gamma, beta float32 [C]."""
    import torch
    dt = _dtype_code(x)
    _dev(x, "x")
    C = int(x.shape[-1])
    _opt(gamma, "gamma", torch.float32, (C,))
    _opt(beta, "beta", torch.float32, (C,))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, tuple(x.shape))
    _check(load().bra_layer_norm(x.data_ptr(), x.numel() // C, C, gamma.data_ptr(),
                                 beta.data_ptr(), float(eps), dt, out.data_ptr(), _stream(x)))
    return out


# field order of bra_block_params (include/bra.h)
BLOCK_PARAMS = ("pos_w", "pos_b", "ln1_g", "ln1_b", "w_qkv", "b_qkv", "lepe_w", "lepe_b",
                "lepe_ks", "w_out", "b_out", "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2",
                "b_fc2")


class _BlockParams(ctypes.Structure):
    _fields_ = [(n, _i if n == "lepe_ks" else _vp) for n in BLOCK_PARAMS]


def block_workspace_bytes(B: int, H: int, W: int, C: int, S: int, dtype_code: int) -> int:
    return int(load().bra_block_workspace_bytes(B, H, W, C, S, dtype_code))


def block_forward(x, params: dict, heads: int, S: int, topk: int,
                  route_scale: float | None = None, attn_scale: float | None = None, out=None,
                  idx=None, workspace=None):
    """One BiFormer block (bra_block_forward).  params maps the names of
    BLOCK_PARAMS to CUDA tensors (weights w_qkv, w_out, w_fc1, w_fc2 in x's
    dtype, the rest float32; biases and lepe_w may be None; lepe_ks is taken
    from lepe_w).  Returns (out, idx)."""
    import torch
    B, H, W, C = _bhwc(x)
    dt = _dtype_code(x)
    _dev(x, "x")
    shapes = {"pos_w": (C, 3, 3), "pos_b": (C,), "ln1_g": (C,), "ln1_b": (C,),
              "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "lepe_b": (C,), "w_out": (C, C),
              "b_out": (C,), "ln2_g": (C,), "ln2_b": (C,), "w_fc1": (3 * C, C),
              "b_fc1": (3 * C,), "w_fc2": (C, 3 * C), "b_fc2": (C,)}
    wdt = {"w_qkv", "w_out", "w_fc1", "w_fc2"}
    p = _BlockParams()
    for n, shp in shapes.items():
        setattr(p, n, _opt(params.get(n), n, x.dtype if n in wdt else torch.float32, shp))
    wp, _, ks = _lepe_args(params.get("lepe_w"), None, C)
    p.lepe_w, p.lepe_ks = wp, ks
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (B, H, W, C))
    if idx is None:
        idx = torch.empty((B, S * S, topk), dtype=torch.int32, device=x.device)
    _dev(idx, "idx", torch.int32, (B, S * S, topk))
    wsp, wsb = _workspace(workspace, block_workspace_bytes(B, H, W, C, S, dt), x.device)
    _check(load().bra_block_forward(x.data_ptr(), B, H, W, C, heads, S, topk, dt, ctypes.byref(p),
                                    float(route_scale), float(attn_scale), out.data_ptr(),
                                    idx.data_ptr(), wsp, wsb, _stream(x)))
    return out, idx


def attend_backward(q, k, v, idx, dout, heads: int, S: int, attn_scale: float | None = None,
                    lepe_w=None, workspace=None):
    """Gradients of attend(q, k, v, idx, heads, S, lepe_w=lepe_w) with the
    routing index held fixed (bra_attend_backward, bf16).  Returns (dq, dk,
    dv) or, with lepe_w, (dq, dk, dv, dw, db)."""
    import torch
    B, H, W, C = _bhwc(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _dev(t, n, q.dtype)
        if tuple(t.shape) != (B, H, W, C):
            raise ValueError("q, k, v, dout must have the same shape")
    _dev(idx, "idx", torch.int32)
    if idx.dim() != 3 or idx.shape[0] != B or idx.shape[1] != S * S:
        raise ValueError("idx must be [B, S*S, topk]")
    topk = int(idx.shape[2])
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    wp, _, ks = _lepe_args(lepe_w, None, C)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dw = torch.empty_like(lepe_w) if lepe_w is not None else None
    db = torch.empty(C, dtype=torch.float32, device=q.device) if lepe_w is not None else None
    need = int(load().bra_backward_workspace_bytes(B, H, W, C, heads, S, topk, ks))
    wsp, wsb = _workspace(workspace, need, q.device)
    _check(load().bra_attend_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                      dout.data_ptr(), B, H, W, C, heads, S, topk, dt,
                                      float(attn_scale), wp, ks, dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), dw.data_ptr() if dw is not None else None,
                                      db.data_ptr() if db is not None else None,
                                      wsp, wsb, _stream(q)))
    return (dq, dk, dv, dw, db) if lepe_w is not None else (dq, dk, dv)


def video_workspace_bytes(B: int, T: int, S: int, C: int) -> int:
    return int(load().bra_video_workspace_bytes(B, T, S, C))


def _clip_shape(q):
    if q.dim() != 5:
        raise ValueError("clips must be [B, T, H, W, C]")
    return tuple(int(x) for x in q.shape)


def video_forward(q, k, v, heads: int, S: int, topk: int, lepe_w=None, lepe_b=None,
                  route_scale: float | None = None, attn_scale: float | None = None, out=None,
                  idx=None, workspace=None, return_logits: bool = False):
    """BRA on clips [B, T, H, W, C] (bra_video_forward): T*S*S regions of one
    frame each, routing over the whole clip, per-frame LePE.  Returns
    (out, idx) or (out, idx, logits)."""
    import torch
    B, T, H, W, C = _clip_shape(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype, (B, T, H, W, C))
    if route_scale is None:
        route_scale = C ** -0.5
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    R = T * S * S
    out = torch.empty_like(q) if out is None else out
    _dev(out, "out", q.dtype, (B, T, H, W, C))
    idx = torch.empty((B, R, topk), dtype=torch.int32, device=q.device) if idx is None else idx
    _dev(idx, "idx", torch.int32, (B, R, topk))
    logits = torch.empty((B, R, topk), dtype=torch.float32, device=q.device) if return_logits else None
    wsp, wsb = _workspace(workspace, video_workspace_bytes(B, T, S, C), q.device)
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_video_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, W, C, heads,
                                    S, topk, dt, float(route_scale), float(attn_scale), wp, bp, ks,
                                    out.data_ptr(), idx.data_ptr(),
                                    logits.data_ptr() if logits is not None else None,
                                    wsp, wsb, _stream(q)))
    return (out, idx, logits) if return_logits else (out, idx)


def video_route(q, k, S: int, topk: int, route_scale: float | None = None, workspace=None):
    """Routing of clips (bra_video_route): idx int32 [B, T*S*S, topk]."""
    import torch
    B, T, H, W, C = _clip_shape(q)
    dt = _dtype_code(q)
    _dev(q, "q")
    _dev(k, "k", q.dtype, (B, T, H, W, C))
    if route_scale is None:
        route_scale = C ** -0.5
    idx = torch.empty((B, T * S * S, topk), dtype=torch.int32, device=q.device)
    wsp, wsb = _workspace(workspace, video_workspace_bytes(B, T, S, C), q.device)
    _check(load().bra_video_route(q.data_ptr(), k.data_ptr(), B, T, H, W, C, S, topk, dt,
                                  float(route_scale), idx.data_ptr(), None, wsp, wsb, _stream(q)))
    return idx


def video_attend(q, k, v, idx, heads: int, S: int, attn_scale: float | None = None, lepe_w=None,
                 lepe_b=None, out=None):
    """Attention of clips over a given index plus per-frame LePE (bra_video_attend)."""
    import torch
    B, T, H, W, C = _clip_shape(q)
    dt = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype, (B, T, H, W, C))
    if not (isinstance(idx, torch.Tensor) and idx.dim() == 3):
        raise ValueError("idx must be [B, T*S*S, topk]")
    topk = int(idx.shape[-1])
    _dev(idx, "idx", torch.int32, (B, T * S * S, topk))
    if attn_scale is None:
        attn_scale = (C // heads) ** -0.5
    out = torch.empty_like(q) if out is None else out
    _dev(out, "out", q.dtype, (B, T, H, W, C))
    wp, bp, ks = _lepe_args(lepe_w, lepe_b, C)
    _check(load().bra_video_attend(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), B, T,
                                   H, W, C, heads, S, topk, dt, float(attn_scale), wp, bp, ks,
                                   out.data_ptr(), _stream(q)))
    return out
