"""The backward pass with a fixed routing index (bra_attend_backward) against
the fp64 oracle's bra_backward, through the C ABI.

Inputs are bf16 values (the oracle sees the same values exactly); the
gradients dQ, dK, dV are bf16 outputs and are held to the bf16 contract:
max |err| <= 2e-2 * RMS after granting each element the half ulp its own
rounding costs.  dw and db are float32 sums over every pixel and are held
to the float32 contract, 1e-4 * RMS.  The index is fixed input: uniform
random rows of distinct regions, plus cases with skewed, repeated and
out-of-range entries (clamped into [0, S*S) as the forward pass does)."""

from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, to_dev, to_host
from vision_transformer_dynamic_region_amd.workloads import (WORKLOADS, Workload,
                                                              make_backward_inputs)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, index variant, with LePE)
    "tiny": (WORKLOADS["tiny"], "uniform", True),
    "st1": (WORKLOADS["st1"], "uniform", True),
    "st2": (WORKLOADS["st2"], "uniform", True),
    "st3": (WORKLOADS["st3"], "uniform", True),
    "dense": (WORKLOADS["dense"], "uniform", True),
    # n = 15 tokens a region (ragged 16-row blocks), 60 routed keys
    "ragged": (Workload("ragged", 50, "bf16", 2, 12, 20, 96, 3, 4, 4), "uniform", True),
    # n = 36, 180 routed keys (six 32-key steps), 7x7 LePE
    "n36_k5_ks7": (Workload("n36", 51, "bf16", 2, 24, 24, 64, 2, 4, 5, lepe_ks=7), "uniform",
                   True),
    # every query region routes to region 0 first, then a repeat of region 0
    # and an out-of-range entry; 3x3 LePE
    "skewed_repeats": (Workload("skew", 52, "bf16", 2, 16, 16, 64, 2, 4, 3, lepe_ks=3),
                       "skewed", True),
    "no_lepe": (Workload("nolepe", 53, "bf16", 2, 16, 24, 128, 4, 4, 2, lepe_ks=0), "uniform",
                False),
    # a 4 x 64 region with 7x7 LePE: its dout halo does not fit the dK/dV
    # kernel's LDS, so the LePE term of dV takes the float32 path
    "wide_ks7_float32_term": (Workload("wide", 55, "bf16", 1, 4, 64, 64, 2, 1, 1, lepe_ks=7),
                              "uniform", True),
    # 1x1 LePE, a single region (global attention)
    "global_ks1": (Workload("glob", 54, "bf16", 1, 8, 16, 64, 2, 1, 1, lepe_ks=1), "uniform",
                   True),
}


@functools.lru_cache(maxsize=None)
def case(name):
    wl, variant, lepe = CASES[name]
    x = make_backward_inputs(wl)
    idx = x["idx"]
    R = wl.S * wl.S
    if variant == "skewed":
        idx = idx.copy()
        idx[:, :, 0] = 0
        idx[:, :, 1] = 0
        idx[:, ::2, 2] = R + 5          # clamped to R - 1
        idx[:, 1::2, 2] = -3            # clamped to 0
    idx_c = np.clip(idx, 0, R - 1)
    w = x["w"] if lepe else None
    ref = oracle.bra_backward(x["q"], x["k"], x["v"], idx_c, wl.heads, wl.S, x["dout"], w)
    return wl, x, idx, w, ref


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(cuda, name):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, idx, w, ref = case(name)
    print(f"[backward] {name} {wl}", flush=True)
    q, k, v, g = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    ti = torch.from_numpy(np.ascontiguousarray(idx)).to(cuda)
    tw = torch.from_numpy(w).to(cuda) if w is not None else None
    res = bra.attend_backward(q, k, v, ti, g, wl.heads, wl.S, lepe_w=tw)
    torch.cuda.synchronize()
    errs = {}
    for got, nm in zip(res[:3], ("dQ", "dK", "dV")):
        errs[nm] = assert_close(to_host(got), ref[nm], "bf16", f"{name} {nm}")
    if w is not None:
        errs["dw"] = assert_close(to_host(res[3]), ref["dw"], "f32", f"{name} dw")
        errs["db"] = assert_close(to_host(res[4]), ref["db"], "f32", f"{name} db")
    print(f"[backward] {name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


def test_backward_deterministic_and_workspace_reuse(cuda):
    """Two calls with one workspace give the same bits (no atomics)."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, idx, w, _ = case("ragged")
    q, k, v, g = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    ti = torch.from_numpy(idx).to(cuda)
    tw = torch.from_numpy(w).to(cuda)
    need = bra.load().bra_backward_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.S,
                                                   wl.topk, wl.lepe_ks)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=cuda)
    a = bra.attend_backward(q, k, v, ti, g, wl.heads, wl.S, lepe_w=tw, workspace=ws)
    b = bra.attend_backward(q, k, v, ti, g, wl.heads, wl.S, lepe_w=tw, workspace=ws)
    torch.cuda.synchronize()
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def test_backward_rejects_f32(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    q = torch.zeros(1, 8, 8, 64, device=cuda)
    idx = torch.zeros(1, 1, 1, dtype=torch.int32, device=cuda)
    with pytest.raises(bra.BraError, match="bf16"):
        bra.attend_backward(q, q.clone(), q.clone(), idx, q.clone(), 2, 1)
