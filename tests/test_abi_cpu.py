"""The C ABI on the host: the library loads, exports what include/bra.h
declares, and rejects bad arguments before touching the GPU (CPU only; no
call here gets past argument checking)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import vision_transformer_dynamic_region_amd as bra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bra.h")

OK, INVAL, UNSUP, WSERR = 0, 1, 2, 3
F32, BF16 = 0, 1
P = 0x10000          # a fake, 16-byte aligned device address; never dereferenced
P2 = 0x20000000
P3 = 0x40000000
P4 = 0x60000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(bra_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bra.lib_path()):
        pytest.skip("libbra.so not built")
    return bra.load(require_torch=False)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("bra_route", "bra_attend", "bra_forward", "bra_lepe", "bra_workspace_bytes",
              "bra_strerror", "bra_last_error", "bra_linear", "bra_module_workspace_bytes",
              "bra_module_forward", "bra_layer_norm", "bra_block_workspace_bytes",
              "bra_block_forward", "bra_pos_conv", "bra_backward_workspace_bytes",
              "bra_attend_backward", "bra_video_workspace_bytes", "bra_video_forward",
              "bra_video_route", "bra_video_attend"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bra.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(bra_\w+)$", out, re.M))
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_workspace_bytes(lib):
    assert lib.bra_workspace_bytes(64, 7, 64) == 2 * 64 * 49 * 64 * 8
    assert lib.bra_workspace_bytes(0, 7, 64) == 0


def test_strerror(lib):
    assert lib.bra_strerror(0) == b"ok"
    assert b"workspace" in lib.bra_strerror(3)
    assert lib.bra_strerror(99) == b"unknown status"


def route(lib, q=P, k=P2, B=2, H=8, W=8, C=64, S=2, topk=2, dt=BF16, scale=0.125, idx=P3,
          logits=None, ws=P4, wsb=1 << 20):
    return lib.bra_route(q, k, B, H, W, C, S, topk, dt, scale, idx, logits, ws, wsb, None)


def attend(lib, q=P, k=P2, v=P3, idx=P4, B=2, H=8, W=8, C=64, heads=2, S=2, topk=2, dt=BF16,
           scale=0.17, w=None, b=None, ks=5, out=0x70000000):
    return lib.bra_attend(q, k, v, idx, B, H, W, C, heads, S, topk, dt, scale, w, b, ks, out, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=9), INVAL, "divide"),
    (dict(S=3), INVAL, "divide"),
    (dict(topk=0), INVAL, "topk"),
    (dict(topk=5), INVAL, "topk"),
    (dict(B=0), INVAL, "positive"),
    (dict(q=None), INVAL, "q is NULL"),
    (dict(q=P + 8), INVAL, "aligned"),
    (dict(idx=None), INVAL, "idx"),
    (dict(scale=0.0), INVAL, "route_scale"),
    (dict(scale=-1.0), INVAL, "route_scale"),
    (dict(scale=math.nan), INVAL, "route_scale"),
    (dict(scale=math.inf), INVAL, "route_scale"),
    (dict(ws=None), WSERR, "NULL"),
    (dict(wsb=100), WSERR, "needed"),
    (dict(ws=P4 + 8), WSERR, "aligned"),
    (dict(dt=7), INVAL, "dtype"),
    (dict(C=60), UNSUP, "multiple of 8"),
    (dict(C=2048), UNSUP, "exceeds"),
    (dict(H=66, W=66, S=33), UNSUP, "regions"),
])
def test_route_rejects(lib, kw, status, msg):
    assert route(lib, **kw) == status
    assert msg in lib.bra_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(heads=3), INVAL, "heads"),
    (dict(heads=0), INVAL, "heads"),
    (dict(heads=1), UNSUP, "head width"),
    (dict(C=128, heads=2), UNSUP, "head width"),
    (dict(v=None), INVAL, "v is NULL"),
    (dict(out=None), INVAL, "out is NULL"),
    (dict(out=P + 1024), INVAL, "overlaps"),
    (dict(out=P3), INVAL, "overlaps"),
    (dict(scale=math.inf), INVAL, "attn_scale"),
    (dict(scale=0.0), INVAL, "attn_scale"),
    (dict(scale=-0.2), INVAL, "attn_scale"),
    (dict(w=P, ks=4), UNSUP, "lepe_ks"),
    (dict(w=P, ks=9), UNSUP, "lepe_ks"),
    (dict(w=P, ks=5, b=P + 4), INVAL, "bias"),
    (dict(dt=F32, C=1024, heads=32), UNSUP, "exceeds"),
    (dict(topk=9), INVAL, "topk"),
])
def test_attend_rejects(lib, kw, status, msg):
    assert attend(lib, **kw) == status
    assert msg in lib.bra_last_error().decode()


def test_forward_checks_both_halves(lib):
    st = lib.bra_forward(P, P2, P3, 2, 8, 8, 64, 2, 2, 2, BF16, 0.125, 0.17, None, None, 5,
                         0x70000000, P4, None, None, 0, None)
    assert st == WSERR
    st = lib.bra_forward(P, P2, P3, 2, 8, 8, 64, 3, 2, 2, BF16, 0.125, 0.17, None, None, 5,
                         0x70000000, P4, None, 0x7A000000, 1 << 20, None)
    assert st == INVAL


def test_lepe_rejects(lib):
    assert lib.bra_lepe(P, P2, None, 5, 2, 8, 8, 48, BF16, P3, None) == UNSUP
    assert lib.bra_lepe(P, None, None, 5, 2, 8, 8, 64, BF16, P3, None) == INVAL
    assert lib.bra_lepe(P, P2, None, 6, 2, 8, 8, 64, BF16, P3, None) == UNSUP
    assert lib.bra_lepe(P, P2, None, 5, 2, 8, 8, 64, BF16, P + 64, None) == INVAL


def test_error_is_thread_local_and_cleared(lib):
    assert route(lib, topk=0) == INVAL
    assert lib.bra_last_error() != b""
    # a later rejected call overwrites the message
    assert route(lib, q=None) == INVAL
    assert b"q is NULL" in lib.bra_last_error()


def test_module_workspace_layout(lib):
    # means: 3 x B*S*S*C float64; tensors: Q, K, V (+ y) of B*H*W*C elements;
    # each part rounded up to 256 bytes
    B, H, W, C, S = 2, 14, 14, 64, 7
    means = 2 * 49 * 64 * 8
    tensor = 2 * 14 * 14 * 64 * 2
    up = lambda x: (x + 255) // 256 * 256
    assert lib.bra_module_workspace_bytes(B, H, W, C, S, BF16, 0) == 3 * up(means) + 3 * up(tensor)
    assert lib.bra_module_workspace_bytes(B, H, W, C, S, BF16, 1) == 3 * up(means) + 4 * up(tensor)
    assert lib.bra_module_workspace_bytes(B, H, W, C, S, F32, 1) == 3 * up(means) + 4 * up(2 * tensor)
    assert lib.bra_module_workspace_bytes(0, H, W, C, S, BF16, 1) == 0
    assert lib.bra_module_workspace_bytes(B, H, W, C, S, 5, 1) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=48), UNSUP, "multiple of 32"),
    (dict(N=6), UNSUP, "multiple of 4"),
    (dict(rows=0), INVAL, "positive"),
    (dict(x=None), INVAL, "x is NULL"),
    (dict(w=P2 + 8), INVAL, "aligned"),
    (dict(b=P3 + 4), INVAL, "aligned"),
    (dict(y=P + 64), INVAL, "overlaps"),
    (dict(dt=3), INVAL, "dtype"),
    (dict(rows=1 << 24, K=64), UNSUP, "2 GiB"),
    (dict(act=2), INVAL, "act"),
    (dict(act=1, r=P3), UNSUP, "residual with an activation"),
    (dict(r=P4 + 64), INVAL, "overlaps r"),
])
def test_linear_rejects(lib, kw, status, msg):
    a = dict(x=P, rows=100, K=64, w=P2, b=None, N=64, act=0, r=None, dt=BF16, y=P4)
    a.update(kw)
    assert lib.bra_linear(a["x"], a["rows"], a["K"], a["w"], a["b"], a["N"], a["act"], a["r"],
                          a["dt"], a["y"], None) == status
    assert msg in lib.bra_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(heads=3), INVAL, "heads"),
    (dict(heads=1), UNSUP, "head width"),
    (dict(w_qkv=None), INVAL, "w_qkv is NULL"),
    (dict(b_qkv=P3 + 4), INVAL, "b_qkv"),
    (dict(b_out=P3), INVAL, "without w_out"),
    (dict(idx=None), INVAL, "idx is NULL"),
    (dict(rs=0.0), INVAL, "route_scale"),
    (dict(ascale=math.nan), INVAL, "attn_scale"),
    (dict(ws=None), WSERR, "NULL"),
    (dict(wsb=1000), WSERR, "needed"),
    (dict(ws=P + 256), INVAL, "workspace overlaps x"),
    (dict(lw=P2, ks=4), UNSUP, "lepe_ks"),
])
def test_module_rejects(lib, kw, status, msg):
    a = dict(x=P, B=2, H=8, W=8, C=64, heads=2, S=2, topk=2, dt=BF16, w_qkv=P2, b_qkv=None,
             rs=0.125, ascale=0.17, lw=None, lb=None, ks=5, w_out=None, b_out=None,
             out=0x70000000, idx=P4, ws=0x7A000000, wsb=1 << 24)
    a.update(kw)
    st = lib.bra_module_forward(a["x"], a["B"], a["H"], a["W"], a["C"], a["heads"], a["S"],
                                a["topk"], a["dt"], a["w_qkv"], a["b_qkv"], a["rs"], a["ascale"],
                                a["lw"], a["lb"], a["ks"], a["w_out"], a["b_out"], a["out"],
                                a["idx"], a["ws"], a["wsb"], None)
    assert st == status
    assert msg in lib.bra_last_error().decode()


def test_block_workspace_layout(lib):
    B, H, W, C, S = 2, 14, 14, 64, 7
    up = lambda x: (x + 255) // 256 * 256
    tensor = up(2 * 14 * 14 * 64 * 2)
    assert lib.bra_block_workspace_bytes(B, H, W, C, S, BF16) == \
        4 * tensor + lib.bra_module_workspace_bytes(B, H, W, C, S, BF16, 1)
    assert lib.bra_block_workspace_bytes(B, H, W, C, 0, BF16) == 0


@pytest.mark.parametrize("kw,status,msg", [
    (dict(C=60), UNSUP, "multiple of 8"),
    (dict(C=64, dt=F32, rows=0), INVAL, "positive"),
    (dict(eps=0.0), INVAL, "eps"),
    (dict(gamma=None), INVAL, "gamma is NULL"),
    (dict(y=P + 64), INVAL, "overlaps"),
])
def test_layer_norm_rejects(lib, kw, status, msg):
    a = dict(x=P, rows=100, C=64, gamma=P2, beta=P3, eps=1e-5, dt=BF16, y=P4)
    a.update(kw)
    assert lib.bra_layer_norm(a["x"], a["rows"], a["C"], a["gamma"], a["beta"], a["eps"], a["dt"],
                              a["y"], None) == status
    assert msg in lib.bra_last_error().decode()


def test_block_rejects(lib):
    import ctypes
    P_ = bra._BlockParams()
    for i, n in enumerate(bra.BLOCK_PARAMS):
        if n != "lepe_ks":
            setattr(P_, n, 0x1000000 + i * 0x100000)
    P_.lepe_w = None
    call = lambda p, **kw: lib.bra_block_forward(
        P, 2, 8, 8, 64, 2, 2, 2, BF16, p, 0.125, 0.17, 0x70000000, P4, kw.get("ws", 0x7A000000),
        kw.get("wsb", 1 << 26), None)
    assert call(None) == INVAL and "params is NULL" in lib.bra_last_error().decode()
    q = bra._BlockParams.from_buffer_copy(P_)
    q.w_fc2 = None
    assert call(ctypes.byref(q)) == INVAL and "w_fc2" in lib.bra_last_error().decode()
    q = bra._BlockParams.from_buffer_copy(P_)
    q.ln1_g = 0x1000004
    assert call(ctypes.byref(q)) == INVAL and "ln1_g" in lib.bra_last_error().decode()
    assert call(ctypes.byref(P_), wsb=100) == WSERR


def test_pos_conv_rejects(lib):
    assert lib.bra_pos_conv(P, None, None, 2, 8, 8, 64, BF16, P4, None) == INVAL
    assert lib.bra_pos_conv(P, P2, None, 2, 8, 8, 60, BF16, P4, None) == UNSUP
    assert lib.bra_pos_conv(P, P2, None, 2, 8, 8, 64, BF16, P + 64, None) == INVAL
    assert lib.bra_pos_conv(P, P2, P3 + 4, 2, 8, 8, 64, BF16, P4, None) == INVAL


def test_backward_rejects(lib):
    def call(**kw):
        a = dict(q=P, k=P2, v=P3, idx=P4, dout=0x50000000, dt=BF16, scale=0.17, w=None, ks=5,
                 dq=0x70000000, dk=0x74000000, dv=0x78000000, dw=None, db=None, ws=0x7C000000,
                 wsb=1 << 26, C=64, heads=2, topk=2)
        a.update(kw)
        return lib.bra_attend_backward(a["q"], a["k"], a["v"], a["idx"], a["dout"], 2, 8, 8, a["C"],
                                       a["heads"], 2, a["topk"], a["dt"], a["scale"], a["w"], a["ks"],
                                       a["dq"], a["dk"], a["dv"], a["dw"], a["db"], a["ws"],
                                       a["wsb"], None)
    assert call(dt=F32) == UNSUP and "bf16" in lib.bra_last_error().decode()
    assert call(dq=P2) == INVAL and "overlaps" in lib.bra_last_error().decode()
    assert call(dk=0x70000000) == INVAL
    assert call(w=P, dw=None) == INVAL and "dlepe_w" in lib.bra_last_error().decode()
    assert call(wsb=16) == WSERR
    assert call(scale=0.0) == INVAL
    assert lib.bra_backward_workspace_bytes(2, 8, 8, 64, 2, 2, 2, 5) > \
        lib.bra_backward_workspace_bytes(2, 8, 8, 64, 2, 2, 2, 0) > 0


def test_video_rejects(lib):
    def call(**kw):
        a = dict(B=2, T=4, H=16, W=16, C=64, heads=2, S=2, topk=3, dt=BF16, ws=0x7C000000,
                 wsb=1 << 26, w=None, out=0x70000000, idx=0x74000000)
        a.update(kw)
        return lib.bra_video_forward(P, P2, P3, a["B"], a["T"], a["H"], a["W"], a["C"], a["heads"],
                                     a["S"], a["topk"], a["dt"], 0.125, 0.17, a["w"], None, 5,
                                     a["out"], a["idx"], None, a["ws"], a["wsb"], None)
    assert call(T=0) == INVAL and "T=0" in lib.bra_last_error().decode()
    assert call(S=3) == INVAL                                   # S must divide H, W
    assert call(topk=17) == INVAL and "T*S*S=16" in lib.bra_last_error().decode()
    assert call(T=65, S=4, H=16) == UNSUP                       # 1040 regions a clip
    assert call(wsb=16) == WSERR
    assert lib.bra_video_workspace_bytes(2, 4, 2, 64) == 2 * 2 * 4 * 4 * 64 * 8
    assert lib.bra_video_workspace_bytes(0, 4, 2, 64) == 0
