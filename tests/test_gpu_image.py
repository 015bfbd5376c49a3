"""The whole-image attention kernels (one head of one image's K and V resident
in LDS; the 4x4-pixel / top-4 and 2x2-pixel / top-16 region shapes, the
latter in its grouped form up to 64 regions, its masked form where the image
has no more keys than the routed ones, and its gather form above) against
the fp64 oracle, through the C ABI: batches that leave XCD slots empty,
region grids other than 7x7, other head counts, a LePE bias, caller indices
with repeated and out-of-range entries (a repeated region counts twice, as
in a gather), and a map too large for LDS (which runs on the per-region
kernel instead)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, check_idx, oracle_parts, to_dev, to_host
from vision_transformer_dynamic_region_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, H, W, C, heads, S, topk)
    "st2_B3": (3, 28, 28, 128, 4, 7, 4),
    # 4x4 regions routed to 8 or to 2 (128 or 32 keys a query)
    "st2_top8_B3": (3, 28, 28, 128, 4, 7, 8),
    "img4_top2_C64": (2, 16, 16, 64, 2, 4, 2),
    "st3_B9": (9, 14, 14, 256, 8, 7, 16),
    # 16 regions of 2x2 routed to all 16: no more keys than the routed ones,
    # so the masked form runs (the grouped form takes the larger grids)
    "st3_masked_S4_C64": (2, 8, 8, 64, 2, 4, 16),
    "st3_region_S8_C64": (2, 16, 16, 64, 2, 8, 16),
    "st3_region_S5_C32": (3, 10, 10, 32, 1, 5, 16),
    "st2_region_S8_C32": (2, 32, 32, 32, 1, 8, 4),
    "st2_region_S3_C192": (2, 12, 12, 192, 6, 3, 4),
    "st2_region_too_big_for_lds": (1, 48, 48, 128, 4, 12, 4),
    # 81 regions of 2x2: past the masked form's 64, so the gather form runs
    "st3_gather_S9_C64": (3, 18, 18, 64, 2, 9, 16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_image_kernel_forward(cuda, name):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S, topk = CASES[name]
    print(f"[image] {name} {CASES[name]}", flush=True)
    wl = Workload(name, 700, "bf16", B, H, W, C, heads, S, topk)
    x = make_inputs(wl)
    b = np.random.default_rng(11).normal(0, 0.1, size=C).astype(np.float32)
    ref = oracle_parts(x, heads, S, topk, x["w"], b)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    out, idx = bra.forward(q, k, v, heads, S, topk, w, torch.from_numpy(b).to(cuda))
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()
    ties = check_idx(idx_g, ref["idx"], ref["A"])
    out_ref = ref["out"]
    if ties:
        O = oracle.routed_attention(x["q"], x["k"], x["v"], idx_g, heads, S, wl.d ** -0.5)
        out_ref = O + ref["L"]
    assert_close(to_host(out), out_ref, "bf16", name)


@pytest.mark.parametrize("shape", [(2, 14, 14, 256, 8, 7, 16), (2, 28, 28, 128, 4, 7, 4)])
def test_image_kernel_repeated_and_clamped_index(cuda, shape):
    """A caller index may repeat a region (its keys then enter the softmax
    twice) or hold entries outside [0, R) (clamped)."""
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S, topk = shape
    R = S * S
    wl = Workload("image_idx", 710, "bf16", B, H, W, C, heads, S, topk)
    x = make_inputs(wl)
    rng = np.random.default_rng(5)
    idx = rng.integers(-3, R + 3, size=(B, R, topk)).astype(np.int32)
    idx[:, ::3, 1] = idx[:, ::3, 0]                  # repeats within a row
    idx[0, 0, :] = 0                                 # one row routed to region 0 only
    ref = oracle.routed_attention(x["q"], x["k"], x["v"], np.clip(idx, 0, R - 1), heads, S,
                                  wl.d ** -0.5) + oracle.lepe(x["v"], x["w"])
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    out = bra.attend(q, k, v, torch.from_numpy(idx).to(cuda), heads, S,
                     lepe_w=torch.from_numpy(x["w"]).to(cuda))
    torch.cuda.synchronize()
    assert_close(to_host(out), ref, "bf16", "repeated/clamped index")
