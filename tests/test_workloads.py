"""Seeded input generators (CPU only)."""

import numpy as np
import torch

from vision_transformer_dynamic_region_amd.workloads import (WORKLOADS, bf16_bits,
                                                              bf16_round, make_inputs,
                                                              make_backward_inputs,
                                                              make_video_inputs, VIDEO_WORKLOADS,
                                                              make_block_inputs,
                                                              make_module_inputs)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.normal(size=100000), r.normal(size=1000) * 1e-30,
                        r.normal(size=1000) * 1e30]).astype(np.float32)
    # include exact halfway cases (ties to even)
    u = (r.integers(0, 1 << 15, size=1000, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    x = x[np.isfinite(x)]            # the generators never produce inf or nan
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bf16_bits(x), ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(bf16_round(x), ref.float().numpy())


def test_workload_shapes():
    for wl in WORKLOADS.values():
        assert wl.H % wl.S == 0 and wl.W % wl.S == 0
        assert wl.C % wl.heads == 0 and wl.d == 32
        assert 1 <= wl.topk <= wl.S * wl.S
    assert WORKLOADS["st1"].keys == 64 and WORKLOADS["dense"].keys == 256
    assert WORKLOADS["st1"].attn_flops == 4 * 64 * 56 * 56 * 64 * 64


def test_inputs_seeded_and_rounded():
    wl = WORKLOADS["tiny"]
    a, b = make_inputs(wl), make_inputs(wl)
    for n in ("q", "k", "v", "w"):
        assert np.array_equal(a[n], b[n])
    assert a["q"].dtype == np.float32 and a["q"].shape == (1, 28, 28, 64)
    assert a["w"].shape == (64, 5, 5)
    assert abs(float(a["w"].std()) - 0.02) < 0.003
    small = WORKLOADS["st2"].scaled(B=2)
    x = make_inputs(small)
    assert np.array_equal(x["q"], bf16_round(x["q"]))


def test_dense_has_region_offsets():
    wl = WORKLOADS["dense"].scaled(B=1)
    x = make_inputs(wl)
    hs = wl.H // wl.S
    means = x["k"].reshape(1, wl.S, hs, wl.S, hs, wl.C).mean(axis=(2, 4))
    # region means carry the N(0, 0.5) offset on top of N(0, 1/64) noise
    assert 0.4 < float(means.std()) < 0.6


def test_module_inputs_seeded_and_rounded():
    wl = WORKLOADS["st2"].scaled(B=2)
    a, b = make_module_inputs(wl), make_module_inputs(wl)
    for n in ("x", "w_qkv", "b_qkv", "w_out", "b_out", "w"):
        assert np.array_equal(a[n], b[n]) and a[n].dtype == np.float32
    C = wl.C
    assert a["x"].shape == (2, 28, 28, C)
    assert a["w_qkv"].shape == (3 * C, C) and a["w_out"].shape == (C, C)
    assert a["b_qkv"].shape == (3 * C,) and a["b_out"].shape == (C,)
    for n in ("x", "w_qkv", "w_out"):
        assert np.array_equal(a[n], bf16_round(a[n]))
    # projections keep unit scale: w ~ N(0, C^-1/2)
    assert abs(float(a["w_qkv"].std()) * C ** 0.5 - 1.0) < 0.05


def test_block_inputs_seeded_and_shaped():
    wl = WORKLOADS["st1"].scaled(B=1)
    a, b = make_block_inputs(wl), make_block_inputs(wl)
    C = wl.C
    shapes = {"pos_w": (C, 3, 3), "pos_b": (C,), "ln1_g": (C,), "ln2_b": (C,),
              "w_fc1": (3 * C, C), "b_fc1": (3 * C,), "w_fc2": (C, 3 * C), "b_fc2": (C,)}
    for n, shp in shapes.items():
        assert a[n].shape == shp and a[n].dtype == np.float32
        assert np.array_equal(a[n], b[n])
    for n in ("w_fc1", "w_fc2"):
        assert np.array_equal(a[n], bf16_round(a[n]))
    assert np.array_equal(a["x"], make_module_inputs(wl)["x"])


def test_backward_inputs_seeded_and_valid():
    wl = WORKLOADS["tiny"]
    a, b = make_backward_inputs(wl), make_backward_inputs(wl)
    for n in ("q", "k", "v", "dout"):
        assert a[n].shape == (1, 28, 28, 64) and a[n].dtype == np.float32
        assert np.array_equal(a[n], b[n]) and np.array_equal(a[n], bf16_round(a[n]))
    assert np.array_equal(a["q"], bf16_round(make_inputs(wl)["q"]))
    idx = a["idx"]
    assert idx.shape == (1, 49, 4) and idx.dtype == np.int32 and np.array_equal(idx, b["idx"])
    assert idx.min() >= 0 and idx.max() < 49
    assert all(len(set(row)) == 4 for row in idx[0])


def test_video_inputs_seeded_and_shaped():
    wl = VIDEO_WORKLOADS["video"].scaled(B=1, T=2)
    a, b = make_video_inputs(wl), make_video_inputs(wl)
    for n in ("q", "k", "v"):
        assert a[n].shape == (1, 2, 56, 56, 64) and a[n].dtype == np.float32
        assert np.array_equal(a[n], b[n]) and np.array_equal(a[n], bf16_round(a[n]))
    # the per-position offset is shared by the frames: frame means of a region agree closely
    m = a["q"].reshape(1, 2, 7, 8, 7, 8, 64).mean(axis=(3, 5))
    assert np.corrcoef(m[0, 0].ravel(), m[0, 1].ravel())[0, 1] > 0.8
    assert VIDEO_WORKLOADS["video"].tokens == 8 * 8 * 56 * 56
