"""The Python binding's argument checks, on the host.

The binding hands raw pointers to the C ABI, which cannot see a tensor's
shape or device.  So every tensor must be checked in the binding: a host
tensor, a wrong dtype or a short buffer has to raise before anything is
launched.  Here the device test is made to accept host tensors and the
library's launching entry points are replaced by recorders, so each case
shows whether the call got as far as a launch.  The *_workspace_bytes
queries go to the real library (they touch no GPU).
"""

import os

import pytest
import torch

import vision_transformer_dynamic_region_amd as bra


class _Recorder:
    """Stands in for libbra.so: launch entry points record their name and
    succeed; size queries and error texts come from the real library."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name.endswith("_workspace_bytes") or name in ("bra_last_error", "bra_strerror"):
            return getattr(self.real, name)

        def launch(*args):
            self.calls.append(name)
            return 0
        return launch


@pytest.fixture
def rec(monkeypatch):
    if not os.path.exists(bra.lib_path()):
        pytest.skip("libbra.so not built")
    r = _Recorder(bra.load(require_torch=False))
    monkeypatch.setattr(bra, "load", lambda require_torch=True: r)
    monkeypatch.setattr(bra, "_on_device", lambda t: True)
    monkeypatch.setattr(bra, "_stream", lambda t: None)
    return r


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


B, H, W, C, S, K, HEADS = 2, 8, 8, 64, 2, 2, 2


def test_host_tensor_is_rejected(monkeypatch):
    # without the stand-in, a host tensor never reaches the library
    with pytest.raises(ValueError, match="CUDA"):
        bra._dev(bf(4), "q")


def test_forward_checks(rec):
    q = bf(B, H, W, C)
    bra.forward(q, bf(B, H, W, C), bf(B, H, W, C), HEADS, S, K)
    assert rec.calls == ["bra_forward"]
    bad = [
        dict(k=bf(B, H, W, C - 8)),
        dict(v=bf(1, H, W, C)),
        dict(out=bf(B, H, W, C - 8)),
        dict(out=bf(B, H, W + 1, C)),
        dict(idx=i32(B, S * S, K + 1)),
        dict(idx=i32(B * S * S * K)),                       # right count, wrong shape
        dict(workspace=torch.zeros(16, dtype=torch.uint8)),  # short
        dict(lepe_w=f32(C, 5, 4)),
        dict(lepe_w=f32(C, 5, 5), lepe_b=f32(C + 1)),
    ]
    for kw in bad:
        args = dict(k=bf(B, H, W, C), v=bf(B, H, W, C))
        args.update(kw)
        k, v = args.pop("k"), args.pop("v")
        with pytest.raises(ValueError):
            bra.forward(q, k, v, HEADS, S, K, **args)
    with pytest.raises(TypeError):
        bra.forward(q, bf(B, H, W, C), bf(B, H, W, C), HEADS, S, K, out=f32(B, H, W, C))
    assert rec.calls == ["bra_forward"]


def test_route_and_attend_checks(rec):
    q = bf(B, H, W, C)
    bra.route(q, bf(B, H, W, C), S, K)
    bra.attend(q, bf(B, H, W, C), bf(B, H, W, C), i32(B, S * S, K), HEADS, S)
    assert rec.calls == ["bra_route", "bra_attend"]
    with pytest.raises(ValueError):
        bra.route(q, bf(B, H, W - 1, C), S, K)
    with pytest.raises(ValueError):
        bra.route(q, bf(B, H, W, C), S, K, workspace=torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(ValueError):
        bra.attend(q, bf(B, H, W, C), bf(B, H, W, C), i32(B, S * S + 1, K), HEADS, S)
    with pytest.raises(ValueError):
        bra.attend(q, bf(B, H, W, C), bf(B, H, W, C), i32(B, S * S, K), HEADS, S,
                   out=bf(B, H, W, C // 2))
    assert rec.calls == ["bra_route", "bra_attend"]


def test_layer_checks(rec):
    x = bf(B, H, W, C)
    with pytest.raises(ValueError):
        bra.pos_conv(x, f32(C, 3, 3), out=bf(B, H, W, C + 8))
    with pytest.raises(ValueError):
        bra.layer_norm(x, f32(C), f32(C), out=bf(B, H, W, 2 * C))
    with pytest.raises(ValueError):
        bra.module_forward(x, bf(3 * C, C), None, HEADS, S, K, out=bf(B, H, W, 2 * C))
    with pytest.raises(ValueError):
        bra.module_forward(x, bf(3 * C, C), None, HEADS, S, K, idx=i32(B, S * S, K + 1))
    with pytest.raises(ValueError):
        bra.module_forward(x, bf(3 * C, C), None, HEADS, S, K,
                           workspace=torch.zeros(1024, dtype=torch.uint8))
    params = {"pos_w": f32(C, 3, 3), "ln1_g": f32(C), "ln1_b": f32(C), "w_qkv": bf(3 * C, C),
              "ln2_g": f32(C), "ln2_b": f32(C), "w_fc1": bf(3 * C, C), "w_fc2": bf(C, 3 * C)}
    with pytest.raises(ValueError):
        bra.block_forward(x, params, HEADS, S, K, out=bf(B, H, W - 1, C))
    with pytest.raises(ValueError):
        bra.block_forward(x, params, HEADS, S, K, workspace=torch.zeros(64, dtype=torch.uint8))
    assert rec.calls == []
    bra.block_forward(x, params, HEADS, S, K)
    assert rec.calls == ["bra_block_forward"]


def test_backward_checks(rec):
    q = bf(B, H, W, C)
    t = lambda: bf(B, H, W, C)
    idx = i32(B, S * S, K)
    with pytest.raises(ValueError):
        bra.attend_backward(q, t(), t(), idx, bf(B, H, W, C + 8), HEADS, S)
    with pytest.raises(ValueError):
        bra.attend_backward(q, t(), t(), idx, t(), HEADS, S,
                            workspace=torch.zeros(16, dtype=torch.uint8))
    assert rec.calls == []
    bra.attend_backward(q, t(), t(), idx, t(), HEADS, S)
    assert rec.calls == ["bra_attend_backward"]


T = 3


def clip(c=C):
    return bf(B, T, H, W, c)


def test_video_forward_checks(rec):
    R = T * S * S
    bra.video_forward(clip(), clip(), clip(), HEADS, S, K)
    assert rec.calls == ["bra_video_forward"]
    bad = [
        dict(k=bf(B, T + 1, H, W, C)),
        dict(v=clip(C - 8)),
        dict(out=clip(C // 2)),
        dict(idx=i32(B, R, K + 1)),
        dict(idx=i32(B * R * K)),
        dict(workspace=torch.zeros(32, dtype=torch.uint8)),
    ]
    for kw in bad:
        args = dict(k=clip(), v=clip())
        args.update(kw)
        k, v = args.pop("k"), args.pop("v")
        with pytest.raises(ValueError):
            bra.video_forward(clip(), k, v, HEADS, S, K, **args)
    with pytest.raises(ValueError):
        bra.video_forward(bf(B, H, W, C), bf(B, H, W, C), bf(B, H, W, C), HEADS, S, K)
    assert rec.calls == ["bra_video_forward"]


def test_video_route_checks(rec):
    bra.video_route(clip(), clip(), S, K)
    assert rec.calls == ["bra_video_route"]
    with pytest.raises(ValueError):
        bra.video_route(clip(), clip(C - 8), S, K)
    with pytest.raises(ValueError):
        bra.video_route(clip(), bf(B, T, H, W), S, K)
    with pytest.raises(ValueError):
        bra.video_route(clip(), clip(), S, K, workspace=torch.zeros(32, dtype=torch.uint8))
    with pytest.raises(ValueError):
        bra.video_route(bf(B, H, W, C), bf(B, H, W, C), S, K)
    assert rec.calls == ["bra_video_route"]


def test_video_attend_checks(rec):
    R = T * S * S
    bra.video_attend(clip(), clip(), clip(), i32(B, R, K), HEADS, S)
    assert rec.calls == ["bra_video_attend"]
    bad = [
        dict(k=clip(C - 8)),
        dict(v=bf(B, T, H - 1, W, C)),
        dict(idx=i32(B, R + 1, K)),
        dict(idx=i32(B * R * K)),
        dict(idx=i32(B, R, K, 1)),
        dict(out=clip(C // 2)),
    ]
    for kw in bad:
        args = dict(k=clip(), v=clip(), idx=i32(B, R, K))
        args.update(kw)
        k, v, idx = args.pop("k"), args.pop("v"), args.pop("idx")
        with pytest.raises(ValueError):
            bra.video_attend(clip(), k, v, idx, HEADS, S, **args)
    assert rec.calls == ["bra_video_attend"]
