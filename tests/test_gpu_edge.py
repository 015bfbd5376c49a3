"""Edge cases of the HIP path vs the fp64 oracle, through the C ABI:
ragged regions and key tails, non-square regions, topk = 1 and S*S, S = 1,
one pixel per region, many tasks per region, the largest region grid, wide
channels, float32, LePE kernel sizes and bias, the shapes with a dedicated
kernel at small batch, the 8x8-region family (C 32..256, top-1/2/4) on the
per-region kernel, exact ties, identity routing, out-of-range indices,
determinism and a non-default stream."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, check_idx, oracle_parts, to_dev, to_host
from vision_transformer_dynamic_region_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

EDGE = {
    # name: (B, H, W, C, heads, S, topk, dtype, ks)
    "ragged_n36": (2, 12, 12, 64, 2, 2, 3, "bf16", 5),
    "nonsquare_3x5": (1, 12, 20, 64, 2, 4, 5, "bf16", 5),
    "topk1": (2, 16, 16, 64, 2, 4, 1, "bf16", 5),
    "topk_all": (2, 16, 16, 64, 2, 4, 16, "bf16", 5),
    "S1_plain": (2, 8, 8, 64, 2, 1, 1, "bf16", 5),
    "one_pixel_regions": (1, 4, 4, 32, 1, 4, 3, "bf16", 3),
    "many_tasks": (1, 16, 16, 256, 8, 2, 2, "bf16", 5),
    "S32_R1024": (1, 64, 64, 32, 1, 32, 8, "bf16", 5),
    "S10_R100": (2, 40, 40, 64, 2, 10, 7, "bf16", 5),      # 16 lanes x 8 slots a row
    "S12_R144_ragged_slots": (1, 48, 36, 64, 2, 12, 9, "bf16", 3),   # 16 x 9 candidates
    "S20_R400": (1, 40, 40, 32, 1, 20, 5, "f32", 3),        # 32 lanes a row
    # more than 64 regions with the query rows staged in several 64-channel
    # chunks (and a half-filled last chunk)
    "S9_R81_C256": (1, 18, 18, 256, 8, 9, 4, "bf16", 3),
    "S9_R81_f32_C96": (2, 18, 18, 96, 3, 9, 5, "f32", 3),
    "wide_C1024": (1, 8, 8, 1024, 32, 2, 2, "bf16", 3),
    "f32_ragged": (1, 12, 12, 64, 2, 2, 3, "f32", 5),
    "f32_all": (2, 16, 16, 128, 4, 4, 16, "f32", 7),
    "f32_wide_C512": (1, 8, 8, 512, 16, 2, 2, "f32", 1),
    "ks7_tall": (2, 24, 8, 96, 3, 4, 6, "bf16", 7),
    # the shapes with a dedicated kernel, at small batch (workgroups left
    # without units) and with a LePE bias
    "st1_shape_B2": (2, 56, 56, 64, 2, 7, 1, "bf16", 5),
    "st2_shape_B1": (1, 28, 28, 128, 4, 7, 4, "bf16", 5),
    "st3_shape_B1": (1, 14, 14, 256, 8, 7, 16, "bf16", 5),
    "dense_shape_B1": (1, 128, 128, 64, 2, 16, 4, "bf16", 5),
    # the rest of the 8x8-region family on the per-region kernel: C of 32 to
    # 256 in heads of 32, top-1, 2 or 4 (BiFormer-B's stage-1 width is 96)
    "rc8_C96_top1": (2, 56, 56, 96, 3, 7, 1, "bf16", 5),
    "rc8_C64_top2": (2, 56, 56, 64, 2, 7, 2, "bf16", 5),
    "rc8_C128_top4": (1, 64, 64, 128, 4, 8, 4, "bf16", 5),
    "rc8_C96_top4": (1, 48, 48, 96, 3, 6, 4, "bf16", 5),
    "rc8_C32_top2_S2": (3, 16, 16, 32, 1, 2, 2, "bf16", 5),
    "rc8_C256_top1": (2, 56, 56, 256, 8, 7, 1, "bf16", 5),
    "rc8_C192_top2": (1, 32, 32, 192, 6, 4, 2, "bf16", 5),
    "rc8_C256_top4": (1, 32, 32, 256, 8, 4, 4, "bf16", 5),
    # pixels of 24 and 48 16-byte groups (BiFormer-B's stage-2 and stage-3
    # widths): the fused pooling and routing on 32 and 64 lanes a pixel
    "groups24_C192": (2, 28, 28, 192, 6, 7, 4, "bf16", 5),
    "groups48_C384": (2, 14, 14, 384, 12, 7, 16, "bf16", 5),
    # 32 lanes a pixel at 8x8 regions, in bf16 and f32 (64 passes a region)
    "lanes32_C256_8x8": (1, 32, 32, 256, 8, 4, 3, "bf16", 5),
    "lanes32_f32_C96_8x8": (1, 24, 24, 96, 3, 3, 2, "f32", 3),
}


def run(cuda, name, B, H, W, C, heads, S, topk, dtype, ks, bias=True, seed=None):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl = Workload(name, 100 + (seed or 0), dtype, B, H, W, C, heads, S, topk, lepe_ks=ks)
    x = make_inputs(wl)
    b = np.random.default_rng(7).normal(0, 0.1, size=C).astype(np.float32) if bias else None
    ref = oracle_parts(x, heads, S, topk, x["w"], b)
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    bt = torch.from_numpy(b).to(cuda) if b is not None else None
    out, idx = bra.forward(q, k, v, heads, S, topk, w, bt)
    torch.cuda.synchronize()
    return wl, x, ref, out, idx, (q, k, v, w, bt)


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_forward(cuda, name):
    print(f"[edge] {name} {EDGE[name]}", flush=True)
    wl, x, ref, out, idx, _ = run(cuda, name, *EDGE[name])
    idx_g = idx.cpu().numpy()
    ties = check_idx(idx_g, ref["idx"], ref["A"])
    out_ref = ref["out"]
    if ties:
        O = oracle.routed_attention(x["q"], x["k"], x["v"], idx_g, wl.heads, wl.S, wl.d ** -0.5)
        out_ref = O + ref["L"]
    assert_close(to_host(out), out_ref, wl.dtype, name)


def test_exact_ties_go_to_lower_index(cuda):
    """Q = 0 makes every affinity 0: the route must be 0, 1, ..., topk-1."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S, topk = 2, 16, 16, 64, 2, 4, 5
    wl = Workload("ties", 200, "bf16", B, H, W, C, heads, S, topk)
    x = make_inputs(wl)
    x["q"] = np.zeros_like(x["q"])
    ref = oracle_parts(x, heads, S, topk, x["w"])
    assert np.array_equal(ref["idx"][0, 0], np.arange(topk))
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    out, idx = bra.forward(q, k, v, heads, S, topk, w)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    assert_close(to_host(out), ref["out"], "bf16", "ties")


def test_identity_route_is_window_attention(cuda):
    """bra_attend with idx[r] = [r] (topk 1) is window attention inside each
    region; the oracle's routed attention with that index is pinned to the
    window formula on the CPU."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S = 2, 16, 16, 64, 2, 4
    wl = Workload("window", 300, "bf16", B, H, W, C, heads, S, 1)
    x = make_inputs(wl)
    ident = np.tile(np.arange(S * S, dtype=np.int32)[None, :, None], (B, 1, 1))
    ref = oracle.routed_attention(x["q"], x["k"], x["v"], ident, heads, S, wl.d ** -0.5)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    out = bra.attend(q, k, v, torch.from_numpy(ident).to(cuda), heads, S)
    assert_close(to_host(out), ref, "bf16", "window")


def test_out_of_range_index_is_clamped(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S, topk = 1, 8, 8, 64, 2, 2, 2
    wl = Workload("clamp", 400, "f32", B, H, W, C, heads, S, topk)
    x = make_inputs(wl)
    bad = np.array([[[9, -3], [1, 0], [2, 77], [-1, 3]]], dtype=np.int32)
    ref = oracle.routed_attention(x["q"], x["k"], x["v"], np.clip(bad, 0, S * S - 1), heads, S,
                                  wl.d ** -0.5)
    q, k, v = (to_dev(x[n], "f32") for n in ("q", "k", "v"))
    out = bra.attend(q, k, v, torch.from_numpy(bad).to(cuda), heads, S)
    assert_close(to_host(out), ref, "f32", "clamped index")


@pytest.mark.parametrize("name", ["topk_all", "st1_shape_B2"])
def test_deterministic_and_stream(cuda, name):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl, x, ref, out, idx, (q, k, v, w, bt) = run(cuda, name, *EDGE[name])
    B, H, W, C, heads, S, topk, dtype, ks = EDGE[name]
    for _ in range(3):
        out2, idx2 = bra.forward(q, k, v, heads, S, topk, w, bt)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)
        assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out3, idx3 = bra.forward(q, k, v, heads, S, topk, w, bt)
    s.synchronize()
    assert torch.equal(idx3, idx)
    assert torch.equal(out3.view(torch.int16), out.view(torch.int16))


POOL = {
    # name: (B, H, W, C, S, dtype): the float64 region means of every pooling
    # kernel and lane layout
    "two_regions_per_wave_odd_count": (43, 28, 28, 64, 7, "bf16"),     # 2107 regions
    "two_regions_per_wave_full_batch": (43, 56, 56, 64, 7, "bf16"),    # 8 passes a region
    "ragged_passes": (2, 12, 12, 64, 2, "bf16"),        # 36 pixels: 5 of 8 passes hold tokens
    "f32_G16": (3, 16, 16, 64, 4, "f32"),
    "f32_G32": (2, 8, 8, 128, 2, "f32"),
    "G64_no_scatter": (3, 4, 4, 512, 2, "bf16"),        # a lane's values span q and k
    "G4_wave_kernel": (2, 16, 16, 32, 4, "bf16"),
    "G12_lane_kernel": (2, 24, 8, 96, 4, "bf16"),
    "G64_many_passes": (1, 8, 8, 512, 2, "bf16"),       # 16 pixels: more than one batch
}


@pytest.mark.parametrize("name", list(POOL))
def test_region_means(cuda, name):
    """bra_route's workspace holds the float64 means of Q then K; summing bf16
    or f32 values in float64 is exact or within a rounding of the oracle's."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, S, dtype = POOL[name]
    print(f"[edge] pool {name} {POOL[name]}", flush=True)
    wl = Workload(name, 500, dtype, B, H, W, C, max(1, C // 32), S, 1)
    x = make_inputs(wl)
    q, k = to_dev(x["q"], dtype), to_dev(x["k"], dtype)
    ws = torch.full((bra.workspace_bytes(B, S, C),), 0xFF, dtype=torch.uint8, device=cuda)
    bra.route(q, k, S, 1, workspace=ws)
    torch.cuda.synchronize()
    means = ws.view(torch.float64).cpu().numpy().reshape(2, B, S * S, C)
    for got, t in ((means[0], x["q"]), (means[1], x["k"])):
        want = oracle.region_mean(t, S)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, float(np.abs(want).max())), name


# The fused pooling and routing with each region in 2 or 4 runs of 8 passes
# (more than 8 passes a region): taken only when the launch has a workgroup
# for every CU, so these run at that size.  (B, H, W, C, S, topk, dtype)
RUNS = {
    "runs2_C96_st1": (64, 56, 56, 96, 7, 1, "bf16"),      # BiFormer-B stage 1
    "runs4_C256_S2": (256, 16, 16, 256, 2, 2, "bf16"),
    "runs4_f32_C96_S2": (256, 16, 16, 96, 2, 3, "f32"),
}


@pytest.mark.parametrize("name", list(RUNS))
def test_route_in_runs(cuda, name):
    """Region means (bra_route's workspace) and indices against the oracle;
    the forward pass (which keeps the means on chip) gives the same indices."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, S, topk, dtype = RUNS[name]
    print(f"[edge] runs {name} {RUNS[name]}", flush=True)
    heads = C // 32
    wl = Workload(name, 600, dtype, B, H, W, C, heads, S, topk)
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    ws = torch.full((bra.workspace_bytes(B, S, C),), 0xFF, dtype=torch.uint8, device=cuda)
    idx = bra.route(q, k, S, topk, workspace=ws)
    torch.cuda.synchronize()
    means = ws.view(torch.float64).cpu().numpy().reshape(2, B, S * S, C)
    q_r, k_r = oracle.region_mean(x["q"], S), oracle.region_mean(x["k"], S)
    for got, want in ((means[0], q_r), (means[1], k_r)):
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, float(np.abs(want).max())), name
    A = oracle.region_affinity(q_r, k_r, C ** -0.5)
    check_idx(idx.cpu().numpy(), oracle.topk_route(A, topk), A)
    w = torch.from_numpy(x["w"]).to(cuda)
    _, idx_f = bra.forward(q, k, v, heads, S, topk, w)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx), name
