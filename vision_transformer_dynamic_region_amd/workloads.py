"""Seeded synthetic inputs for the BRA forward pass.

This module only draws numbers: it holds none of the method's arithmetic.
Both the HIP path's callers (tests, bench) and the fp64 oracle take their
inputs from here, so that they see the same bits.

Recipe (stands in for the BiFormer stage shapes of 224x224 ImageNet
classification and the stride-4 map of 512x512 segmentation):

* NumPy ``default_rng(seed)`` (PCG64), float64 draws, cast to float32.
* seed = 1000 * config_index + {Q: 0, K: 1, V: 2, w: 3, mu_Q: 4, mu_K: 5, mu_V: 6}.
* Q, K, V ~ N(0, 1) i.i.d.; the dense-prediction shape also adds a per-region
  offset mu[b, region, c] ~ N(0, 0.5), drawn separately for Q, K and V and
  broadcast over the region's pixels, so that routing is non-uniform.
* LePE weights w ~ N(0, 0.02), shape [C, 5, 5], float32; no bias.
* For bf16 workloads the float32 values are rounded to bfloat16 with
  round-to-nearest-even; the rounded values (exact in float32 and float64)
  are what both sides receive.

The module around the method (projections of an input x) draws, with the
same seed base: x ~ N(0, 1) (seed + 7; the dense shape adds its per-region
offset, seed + 12), w_qkv ~ N(0, C**-0.5) [3C, C] (seed + 8), b_qkv ~ N(0, 0.1)
[3C] (seed + 9), w_out ~ N(0, C**-0.5) [C, C] (seed + 10), b_out ~ N(0, 0.1)
[C] (seed + 11) and the LePE weights as above.  x and the two weights are
rounded to bf16 for bf16 workloads; biases stay float32.

The BiFormer block adds (same seed base): the 3x3 position-encoding conv
pos_w ~ N(0, 0.1) [C, 3, 3] (seed + 13) and pos_b ~ N(0, 0.02) (seed + 14),
LayerNorm scales 1 + N(0, 0.1) and shifts N(0, 0.1) (seeds + 15 .. + 18), the
MLP's fc1 ~ N(0, C**-0.5) [3C, C] (seed + 19) with bias N(0, 0.1) (seed + 20)
and fc2 ~ N(0, (3C)**-0.5) [C, 3C] (seed + 21) with bias N(0, 0.1) (seed + 22);
conv and LayerNorm parameters and biases are float32, fc weights follow the
workload dtype.

Video clips (``VIDEO_WORKLOADS``, ``make_video_inputs``) draw Q, K, V ~ N(0, 1)
as [B, T, H, W, C] (seeds + 0, 1, 2) plus, when region_offset_std > 0, one
offset per clip, region position and channel ~ N(0, region_offset_std)
(seeds + 4, 5, 6), the same in every frame, so that a region position looks
alike across frames and routing across frames is not uniform; the LePE
weights as above.  The stage-1 clip: 8 clips of 8 frames of 56x56, C = 64,
S = 7 (392 regions a clip), top-4.

The backward pass (bf16 only) takes Q, K, V and w as above, all rounded to
bf16 whatever the workload's dtype, an output gradient dout ~ N(0, 1)
rounded to bf16 (seed + 23), and a routing index drawn uniformly: for each
image and query region, topk distinct regions in random order (one
permutation per row, generator seed + 24).  The index is an input of the
backward pass, so any valid index tests it; a routing computed by the
forward pass is used where the timing should see its skew.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "bf16_round", "bf16_bits", "make_inputs",
           "make_module_inputs", "make_block_inputs", "make_backward_inputs", "workload",
           "VIDEO_WORKLOADS", "make_video_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed base = 1000 * index
    dtype: str          # "f32" or "bf16"
    B: int
    H: int
    W: int
    C: int
    heads: int
    S: int
    topk: int
    lepe_ks: int = 5
    region_offset_std: float = 0.0   # std of the per-region mean offset (0: none)
    T: int = 1                       # frames of a clip (video workloads)

    @property
    def tokens(self) -> int:
        return self.B * self.T * self.H * self.W

    @property
    def n(self) -> int:
        """Tokens per region."""
        return (self.H // self.S) * (self.W // self.S)

    @property
    def keys(self) -> int:
        """Keys seen by each query: topk routed regions of n tokens."""
        return self.topk * self.n

    @property
    def d(self) -> int:
        return self.C // self.heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def tensor_bytes(self) -> int:
        return self.tokens * self.C * self.elem_bytes

    @property
    def attn_flops(self) -> int:
        """Routed attention work: 2 GEMMs of 2*keys*C flops per token."""
        return 4 * self.tokens * self.keys * self.C

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, "f32", 1, 28, 28, 64, 2, 7, 4),
    "st1": Workload("st1", 1, "bf16", 64, 56, 56, 64, 2, 7, 1),
    "st2": Workload("st2", 2, "bf16", 64, 28, 28, 128, 4, 7, 4),
    "st3": Workload("st3", 3, "bf16", 64, 14, 14, 256, 8, 7, 16),
    "dense": Workload("dense", 4, "bf16", 8, 128, 128, 64, 2, 16, 4,
                      region_offset_std=0.5),
}


VIDEO_WORKLOADS = {
    # 8 clips of 8 frames at the stage-1 map (56x56, C = 64), 7x7 regions of
    # 8x8 pixels per frame (392 regions a clip), top-4 routed regions
    "video": Workload("video", 5, "bf16", 8, 56, 56, 64, 2, 7, 4, region_offset_std=0.5, T=8),
    "video_tiny": Workload("video_tiny", 6, "f32", 1, 16, 16, 64, 2, 2, 3, T=4),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Finite inputs only (the generators never produce inf or nan).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    bits = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def _normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, size=shape)


def make_inputs(wl: Workload, seed_base: int | None = None, with_weights: bool = True):
    """Draw (Q, K, V, w) for a workload.

    Returns a dict with float32 arrays ``q``, ``k``, ``v`` [B, H, W, C]
    (already rounded to bf16 values for bf16 workloads), ``w`` [C, ks, ks]
    float32 (or None) and ``bias`` (always None: the workloads carry none).
    """
    base = 1000 * wl.index if seed_base is None else seed_base
    shape = (wl.B, wl.H, wl.W, wl.C)
    out = {}
    for name, off, mu_off in (("q", 0, 4), ("k", 1, 5), ("v", 2, 6)):
        x = _normal(base + off, shape)
        if wl.region_offset_std > 0.0:
            hs, ws = wl.H // wl.S, wl.W // wl.S
            mu = _normal(base + mu_off, (wl.B, wl.S, wl.S, wl.C), wl.region_offset_std)
            # broadcast the per-region offset over the region's pixels
            x = x + np.repeat(np.repeat(mu, hs, axis=1), ws, axis=2)
        x = x.astype(np.float32)
        if wl.dtype == "bf16":
            x = bf16_round(x)
        out[name] = x
    if with_weights and wl.lepe_ks > 0:
        out["w"] = _normal(base + 3, (wl.C, wl.lepe_ks, wl.lepe_ks), 0.02).astype(np.float32)
    else:
        out["w"] = None
    out["bias"] = None
    return out


def make_module_inputs(wl: Workload, seed_base: int | None = None):
    """Draw the module's input x and its weights for a workload.

    Returns a dict: ``x`` [B, H, W, C], ``w_qkv`` [3C, C], ``w_out`` [C, C]
    (bf16-rounded for bf16 workloads), ``b_qkv`` [3C], ``b_out`` [C] float32,
    ``w`` [C, ks, ks] float32 LePE weights and ``bias`` (None).
    """
    base = 1000 * wl.index if seed_base is None else seed_base
    C = wl.C
    x = _normal(base + 7, (wl.B, wl.H, wl.W, C))
    if wl.region_offset_std > 0.0:
        hs, ws = wl.H // wl.S, wl.W // wl.S
        mu = _normal(base + 12, (wl.B, wl.S, wl.S, C), wl.region_offset_std)
        x = x + np.repeat(np.repeat(mu, hs, axis=1), ws, axis=2)
    rnd = (lambda a: bf16_round(a.astype(np.float32))) if wl.dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    out = {
        "x": rnd(x),
        "w_qkv": rnd(_normal(base + 8, (3 * C, C), C ** -0.5)),
        "b_qkv": _normal(base + 9, (3 * C,), 0.1).astype(np.float32),
        "w_out": rnd(_normal(base + 10, (C, C), C ** -0.5)),
        "b_out": _normal(base + 11, (C,), 0.1).astype(np.float32),
        "w": _normal(base + 3, (C, wl.lepe_ks, wl.lepe_ks), 0.02).astype(np.float32),
        "bias": None,
    }
    return out


def make_block_inputs(wl: Workload, seed_base: int | None = None):
    """Draw the BiFormer block's input and parameters for a workload: the
    module's (x, w_qkv, b_qkv, w_out, b_out, LePE w as ``lepe_w``) plus
    pos_w, pos_b, ln1_g, ln1_b, ln2_g, ln2_b, w_fc1, b_fc1, w_fc2, b_fc2."""
    base = 1000 * wl.index if seed_base is None else seed_base
    C = wl.C
    m = make_module_inputs(wl, seed_base)
    rnd = (lambda a: bf16_round(a.astype(np.float32))) if wl.dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    f32 = lambda a: a.astype(np.float32)
    out = {"x": m["x"], "w_qkv": m["w_qkv"], "b_qkv": m["b_qkv"], "w_out": m["w_out"],
           "b_out": m["b_out"], "lepe_w": m["w"], "lepe_b": None,
           "pos_w": f32(_normal(base + 13, (C, 3, 3), 0.1)),
           "pos_b": f32(_normal(base + 14, (C,), 0.02)),
           "ln1_g": f32(1.0 + _normal(base + 15, (C,), 0.1)),
           "ln1_b": f32(_normal(base + 16, (C,), 0.1)),
           "ln2_g": f32(1.0 + _normal(base + 17, (C,), 0.1)),
           "ln2_b": f32(_normal(base + 18, (C,), 0.1)),
           "w_fc1": rnd(_normal(base + 19, (3 * C, C), C ** -0.5)),
           "b_fc1": f32(_normal(base + 20, (3 * C,), 0.1)),
           "w_fc2": rnd(_normal(base + 21, (C, 3 * C), (3 * C) ** -0.5)),
           "b_fc2": f32(_normal(base + 22, (C,), 0.1))}
    return out


def make_backward_inputs(wl: Workload, seed_base: int | None = None):
    """Draw the backward pass's inputs for a workload: ``q``, ``k``, ``v``
    [B, H, W, C] and ``dout`` (bf16-rounded float32), ``w`` [C, ks, ks]
    float32 (None when the workload has no LePE) and ``idx`` int32
    [B, S*S, topk] with distinct regions in each row."""
    base = 1000 * wl.index if seed_base is None else seed_base
    x = make_inputs(wl, seed_base)
    out = {n: bf16_round(x[n]) for n in ("q", "k", "v")}
    out["w"] = x["w"]
    out["dout"] = bf16_round(_normal(base + 23, (wl.B, wl.H, wl.W, wl.C)).astype(np.float32))
    rng = np.random.default_rng(base + 24)
    R = wl.S * wl.S
    idx = np.empty((wl.B, R, wl.topk), dtype=np.int32)
    for b in range(wl.B):
        for r in range(R):
            idx[b, r] = rng.permutation(R)[:wl.topk]
    out["idx"] = idx
    return out


def make_video_inputs(wl: Workload, seed_base: int | None = None, with_weights: bool = True):
    """Draw (Q, K, V, w) for a clip workload: ``q``, ``k``, ``v`` [B, T, H, W,
    C] float32 (bf16-rounded for bf16 workloads), ``w`` [C, ks, ks] float32
    (or None) and ``bias`` (None)."""
    base = 1000 * wl.index if seed_base is None else seed_base
    shape = (wl.B, wl.T, wl.H, wl.W, wl.C)
    out = {}
    for name, off, mu_off in (("q", 0, 4), ("k", 1, 5), ("v", 2, 6)):
        x = _normal(base + off, shape)
        if wl.region_offset_std > 0.0:
            hs, ws = wl.H // wl.S, wl.W // wl.S
            mu = _normal(base + mu_off, (wl.B, 1, wl.S, wl.S, wl.C), wl.region_offset_std)
            x = x + np.repeat(np.repeat(mu, hs, axis=2), ws, axis=3)
        x = x.astype(np.float32)
        if wl.dtype == "bf16":
            x = bf16_round(x)
        out[name] = x
    if with_weights and wl.lepe_ks > 0:
        out["w"] = _normal(base + 3, (wl.C, wl.lepe_ks, wl.lepe_ks), 0.02).astype(np.float32)
    else:
        out["w"] = None
    out["bias"] = None
    return out
