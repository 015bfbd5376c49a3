"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph on
the ROCm build): the forward pass, the backward pass and the video forward
pass are captured once with preallocated outputs and workspaces, replayed
several times with eager work in between, and every replay is compared bit
for bit with the eager result.  None of these launches records a memset."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import to_dev
from vision_transformer_dynamic_region_amd.workloads import (VIDEO_WORKLOADS, WORKLOADS,
                                                              make_backward_inputs, make_inputs,
                                                              make_video_inputs)

pytestmark = pytest.mark.gpu


def _replays(cuda, run, outs, eager):
    """Capture run() in a graph, replay it 5 times with an eager torch op in
    between, and compare outs with eager after every replay."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(5):
        for o in outs:
            o.fill_(0) if o.dtype != torch.int32 else o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=cuda).sum()      # eager work between replays
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"
        del junk


def test_forward_graph(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl = WORKLOADS["st2"].scaled(B=4)
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    ws = torch.empty(bra.workspace_bytes(wl.B, wl.S, wl.C), dtype=torch.uint8, device=cuda)
    out = torch.empty_like(q)
    idx = torch.empty((wl.B, wl.S * wl.S, wl.topk), dtype=torch.int32, device=cuda)
    e_out, e_idx = bra.forward(q, k, v, wl.heads, wl.S, wl.topk, w)
    torch.cuda.synchronize()

    def run():
        bra.forward(q, k, v, wl.heads, wl.S, wl.topk, w, out=out, idx=idx, workspace=ws)
    _replays(cuda, run, [out, idx], [e_out, e_idx])


def test_backward_graph(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl = WORKLOADS["st2"].scaled(B=4)
    x = make_backward_inputs(wl)
    q, k, v, g = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    w = torch.from_numpy(x["w"]).to(cuda)
    idx = torch.from_numpy(x["idx"]).to(cuda)
    need = bra.load().bra_backward_workspace_bytes(wl.B, wl.H, wl.W, wl.C, wl.heads, wl.S,
                                                   wl.topk, wl.lepe_ks)
    ws = torch.empty(need, dtype=torch.uint8, device=cuda)
    eager = bra.attend_backward(q, k, v, idx, g, wl.heads, wl.S, lepe_w=w)
    torch.cuda.synchronize()
    outs = [torch.empty_like(t) for t in eager]
    L = bra.load()

    def run():
        st = L.bra_attend_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                   g.data_ptr(), wl.B, wl.H, wl.W, wl.C, wl.heads, wl.S, wl.topk,
                                   1, wl.d ** -0.5, w.data_ptr(), wl.lepe_ks, outs[0].data_ptr(),
                                   outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
                                   outs[4].data_ptr(), ws.data_ptr(), need,
                                   torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.bra_last_error()
    _replays(cuda, run, outs, list(eager))


def test_video_graph(cuda):
    import torch
    import vision_transformer_dynamic_region_amd as bra
    wl = VIDEO_WORKLOADS["video"].scaled(B=2, T=2)
    x = make_video_inputs(wl)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    w = torch.from_numpy(x["w"]).to(cuda)
    ws = torch.empty(bra.video_workspace_bytes(wl.B, wl.T, wl.S, wl.C), dtype=torch.uint8,
                     device=cuda)
    out = torch.empty_like(q)
    idx = torch.empty((wl.B, wl.T * wl.S * wl.S, wl.topk), dtype=torch.int32, device=cuda)
    e_out, e_idx = bra.video_forward(q, k, v, wl.heads, wl.S, wl.topk, w)
    torch.cuda.synchronize()

    def run():
        bra.video_forward(q, k, v, wl.heads, wl.S, wl.topk, w, out=out, idx=idx, workspace=ws)
    _replays(cuda, run, [out, idx], [e_out, e_idx])
