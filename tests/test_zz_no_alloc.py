"""bra_forward_noalloc (the forward pass that allocates nothing: its region
means go to the library's static device scratch) against bra_forward,
through the C ABI: the same output bits and routing index on two calls in a
row, the second with a smaller input, so the scratch holds the first call's
means when the second runs."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import to_dev
from vision_transformer_dynamic_region_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _call(cuda, wl, bias):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    b = torch.from_numpy(np.random.default_rng(3).normal(0, 0.1, size=wl.C).astype(np.float32)
                         ).to(cuda) if bias else None
    want_out, want_idx, want_lg = bra.forward(q, k, v, wl.heads, wl.S, wl.topk, w, b,
                                              return_logits=True)
    out = torch.full_like(q, float("nan"))
    idx = torch.full((wl.B, wl.S * wl.S, wl.topk), -7, dtype=torch.int32, device=cuda)
    lg = torch.full((wl.B, wl.S * wl.S, wl.topk), float("nan"), dtype=torch.float32, device=cuda)
    bra.forward_noalloc(q, k, v, wl.heads, wl.S, wl.topk, out, idx, w, b, logits=lg)
    torch.cuda.synchronize()
    return (out, idx, lg), (want_out, want_idx, want_lg)


@pytest.mark.parametrize("first,second", [("st3", "st3:B=5"), ("st2", "tiny"), ("dense", "st1:B=3")])
def test_noalloc_matches_forward(cuda, first, second):
    import torch
    for spec, bias in ((first, False), (second, True)):
        name, _, b = spec.partition(":B=")
        wl = WORKLOADS[name].scaled(B=int(b)) if b else WORKLOADS[name]
        print(f"[noalloc] {spec}", flush=True)
        (out, idx, lg), (wo, wi, wlg) = _call(cuda, wl, bias)
        assert torch.equal(idx, wi), spec
        assert torch.equal(lg, wlg), spec
        if out.dtype == torch.bfloat16:
            assert torch.equal(out.view(torch.int16), wo.view(torch.int16)), spec
        else:
            assert torch.equal(out, wo), spec


def test_noalloc_rejects_oversized_means(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    B, H, W, C, heads, S, topk = 64, 64, 64, 512, 16, 8, 4    # means of 2*B*S*S*C*8 = 32 MiB
    q = torch.zeros((B, H, W, C), dtype=torch.bfloat16, device=cuda)
    out = torch.empty_like(q)
    idx = torch.empty((B, S * S, topk), dtype=torch.int32, device=cuda)
    with pytest.raises(bra.BraError, match="scratch"):
        bra.forward_noalloc(q, q, q, heads, S, topk, out, idx)
