"""HIP path vs the fp64 oracle on the five workloads at full size, through
the C ABI (bra_forward, bra_route, bra_attend, bra_lepe)."""

from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
from gpu_util import (TOL, assert_close, check_idx, oracle_parts, rel_err, to_dev,
                      to_host)
from vision_transformer_dynamic_region_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "st1", "st2", "st3", "dense"]


@functools.lru_cache(maxsize=None)
def case(name):
    wl = WORKLOADS[name]
    x = make_inputs(wl)
    parts = oracle_parts(x, wl.heads, wl.S, wl.topk, x["w"])
    return wl, x, parts


@pytest.mark.parametrize("name", NAMES)
def test_forward_parity(cuda, name):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, ref = case(name)
    print(f"[parity] forward {name} {wl}", flush=True)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    ws = torch.empty(bra.workspace_bytes(wl.B, wl.S, wl.C), dtype=torch.uint8, device=cuda)
    out, idx, logits = bra.forward(q, k, v, wl.heads, wl.S, wl.topk, w, workspace=ws,
                                   return_logits=True)
    # the forward pass's workspace is scratch; bra_route's holds the float64
    # means of Q then K, and its index is the forward pass's
    ws2 = torch.empty_like(ws)
    idx_r = bra.route(q, k, wl.S, wl.topk, workspace=ws2)
    torch.cuda.synchronize()
    means = ws2.view(torch.float64).cpu().numpy().reshape(2, wl.B, wl.S * wl.S, wl.C)
    scale = max(1.0, float(np.abs(ref["q_r"]).max()))
    assert np.max(np.abs(means[0] - ref["q_r"])) <= 1e-12 * scale
    assert np.max(np.abs(means[1] - ref["k_r"])) <= 1e-12 * scale
    assert torch.equal(idx_r, idx)
    # routing index: exact modulo near-ties
    idx_g = idx.cpu().numpy()
    ties = check_idx(idx_g, ref["idx"], ref["A"])
    # chosen affinities (float32 copies of the fp64 values)
    lg = logits.cpu().numpy().astype(np.float64)
    want = np.take_along_axis(ref["A"], idx_g.astype(np.int64), -1)
    assert np.allclose(lg, want, rtol=1e-5, atol=1e-7 * np.abs(ref["A"]).max())
    # output
    if ties:
        print(f"[parity] {name}: {len(ties)} near-tie rows; comparing with the GPU index",
              flush=True)
        O = oracle.routed_attention(x["q"], x["k"], x["v"], idx_g, wl.heads, wl.S, wl.d ** -0.5)
        out_ref = O + ref["L"]
    else:
        out_ref = ref["out"]
    e = assert_close(to_host(out), out_ref, wl.dtype, f"{name} out")
    print(f"[parity] {name}: idx exact ({len(ties)} tie rows), out err/RMS {e:.2e}", flush=True)


@pytest.mark.parametrize("name", NAMES)
def test_attend_and_lepe_alone(cuda, name):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, ref = case(name)
    print(f"[parity] attend/lepe {name}", flush=True)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    idx = torch.from_numpy(ref["idx"]).to(cuda)
    O = bra.attend(q, k, v, idx, wl.heads, wl.S)
    w = torch.from_numpy(x["w"]).to(cuda)
    L = torch.zeros_like(v)
    bra.lepe(v, w, None, L)
    torch.cuda.synchronize()
    assert_close(to_host(O), ref["O"], wl.dtype, f"{name} attention only")
    assert_close(to_host(L), ref["L"], wl.dtype, f"{name} LePE only")


@pytest.mark.parametrize("name", NAMES)
def test_route_alone(cuda, name):
    import vision_transformer_dynamic_region_amd as bra
    wl, x, ref = case(name)
    print(f"[parity] route {name}", flush=True)
    q, k = (to_dev(x[n], wl.dtype) for n in ("q", "k"))
    idx = bra.route(q, k, wl.S, wl.topk).cpu().numpy()
    check_idx(idx, ref["idx"], ref["A"])


@pytest.mark.parametrize("name", ["st1", "st2", "st3", "dense"])
def test_repeated_launches(cuda, name):
    """Many launches in a row of the persistent attention kernel on the same
    inputs: every launch writes every output element, bit for bit as the
    first, which matches the oracle."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, ref = case(name)
    print(f"[parity] repeated launches {name}", flush=True)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    idx = torch.from_numpy(ref["idx"]).to(cuda)
    w = torch.from_numpy(x["w"]).to(cuda)
    first = bra.attend(q, k, v, idx, wl.heads, wl.S, lepe_w=w)
    outs = [torch.full_like(first, float("nan")) for _ in range(40)]
    for o in outs:
        bra.attend(q, k, v, idx, wl.heads, wl.S, lepe_w=w, out=o)
    torch.cuda.synchronize()
    assert_close(to_host(first), ref["out"], wl.dtype, f"{name} first launch")
    for i, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), first.view(torch.int16)), f"launch {i + 1}"
