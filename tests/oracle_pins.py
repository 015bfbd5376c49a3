"""Pins for the fp64 oracle: checks against facts the oracle does not produce.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, a hand-worked value, a brute-force definition written here
independently, or a library routine (PyTorch CPU, float64).  The same
functions run against deliberately broken copies of the oracle in
``test_oracle_mutations.py`` to show that each plausible mistake is caught.

Page keys (p1 cybasar.com BiFormer BRA explainer, p2 snabindia.com BRA
article, p4 un.csdn.net window-attention write-up, p5 the arXiv 2303.08810
abstract) are described in the oracle's header.
"""

from __future__ import annotations

import glob
import json
import os

import numpy as np

import oracle.bra_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol * scale:.3e}"


# --------------------------------------------------------------------------
# independent brute-force definitions (written here, not taken from the oracle)

def _pixel_region(H, W, S):
    """Region id per flattened pixel, computed by scanning the grid cells."""
    hs, ws = H // S, W // S
    reg = np.empty(H * W, dtype=np.int64)
    for y in range(H):
        for x in range(W):
            reg[y * W + x] = (y // hs) * S + (x // ws)
    return reg


def brute_masked_attention(Q, K, V, idx, heads, S, scale):
    """Dense HW x HW attention with every key outside the routed regions
    masked out (p5: attention over the union of the routed regions)."""
    B, H, W, C = Q.shape
    d = C // heads
    reg = _pixel_region(H, W, S)
    out = np.zeros((B, H * W, C))
    for b in range(B):
        q = Q[b].reshape(H * W, C)
        k = K[b].reshape(H * W, C)
        v = V[b].reshape(H * W, C)
        allowed = np.zeros((H * W, H * W), dtype=bool)
        for p in range(H * W):
            allowed[p] = np.isin(reg, idx[b, reg[p]])
        for m in range(heads):
            sl = slice(m * d, (m + 1) * d)
            logits = scale * (q[:, sl] @ k[:, sl].T)
            logits = np.where(allowed, logits, -np.inf)
            logits -= logits.max(axis=1, keepdims=True)
            e = np.exp(logits)
            out[b, :, sl] = (e / e.sum(axis=1, keepdims=True)) @ v[:, sl]
    return out.reshape(B, H, W, C)


def global_attention(Q, K, V, heads, scale):
    """Textbook multi-head softmax(scale Q K^T) V over all H*W keys."""
    B, H, W, C = Q.shape
    d = C // heads
    q = Q.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    k = K.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    v = V.reshape(B, H * W, heads, d).transpose(0, 2, 1, 3)
    s = scale * q @ k.transpose(0, 1, 3, 2)
    s -= s.max(-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(-1, keepdims=True)
    return (p @ v).transpose(0, 2, 1, 3).reshape(B, H, W, C)


def window_attention(Q, K, V, heads, S, scale):
    """p4's local window attention: split into non-overlapping windows,
    softmax(Q K^T / sqrt(d_k)) V inside each, merge back."""
    B, H, W, C = Q.shape
    hs, ws = H // S, W // S

    def split(X):  # [B, S, hs, S, ws, C] -> [B*S*S, hs*ws, C]
        return X.reshape(B, S, hs, S, ws, C).transpose(0, 1, 3, 2, 4, 5).reshape(-1, hs * ws, C)

    o = global_attention(split(Q)[:, :, None, :], split(K)[:, :, None, :],
                         split(V)[:, :, None, :], heads, scale)
    o = o.reshape(B, S, S, hs, ws, C).transpose(0, 1, 3, 2, 4, 5)
    return o.reshape(B, H, W, C)


def _rand(seed, B, H, W, C):
    r = _rng(seed)
    return r.normal(size=(B, H, W, C)), r.normal(size=(B, H, W, C)), r.normal(size=(B, H, W, C))


# --------------------------------------------------------------------------
# pins

def pin_golden():
    """Hand-worked fixtures under tests/golden/."""
    files = sorted(glob.glob(os.path.join(GOLDEN, "hand_*.json")))
    assert files, "no golden fixtures"
    for f in files:
        g = json.load(open(f))
        q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
        C, ks = g["C"], g["lepe_ks"]
        w = np.zeros((C, ks, ks))
        for c, i, j, val in g["lepe_taps"]:
            w[c, i, j] = val
        bias = None if g["bias"] is None else np.array(g["bias"], dtype=np.float64)
        parts = O.bra_forward(q, k, v, g["heads"], g["S"], g["topk"], w, bias,
                              return_parts=True)
        name = os.path.basename(f)
        assert np.array_equal(parts["idx"], np.array(g["expect_idx"])), f"{name}: idx"
        _close(parts["O"], g["expect_O"], 1e-14, f"{name}: O")
        if "expect_L" in g:
            _close(parts["L"], g["expect_L"], 1e-14, f"{name}: L")
        _close(parts["out"], g["expect_out"], 1e-14, f"{name}: out")


def pin_partition_layout():
    """Region/token order equals p1 §3's reshape (S, H/S, S, W/S, C) with
    axes 1 and 2 swapped, flattened to [S*S, n, C] (reading R2)."""
    for (B, H, W, S) in ((1, 4, 6, 2), (2, 6, 6, 3), (1, 8, 4, 4)):
        C = 3
        X = _rng(1).normal(size=(B, H, W, C))
        hs, ws = H // S, W // S
        view = X.reshape(B, S, hs, S, ws, C).transpose(0, 1, 3, 2, 4, 5).reshape(B, S * S, hs * ws, C)
        region, token = O.region_token_maps(H, W, S)
        for r in range(S * S):
            ys, xs = O.region_tokens(H, W, S, r)
            assert np.array_equal(X[:, ys, xs, :], view[:, r]), "region_tokens order"
            assert np.all(region[ys, xs] == r)
            assert np.array_equal(token[ys, xs], np.arange(hs * ws))


def pin_pool_avgpool():
    """Region mean equals torch avg_pool2d with kernel = stride = region size."""
    import torch
    import torch.nn.functional as F
    for (B, H, W, C, S) in ((2, 8, 8, 5, 2), (1, 12, 6, 4, 3), (1, 7, 7, 2, 7), (2, 4, 4, 3, 1)):
        X = _rng(2).normal(size=(B, H, W, C))
        ref = F.avg_pool2d(torch.from_numpy(X).permute(0, 3, 1, 2), (H // S, W // S))
        ref = ref.permute(0, 2, 3, 1).reshape(B, S * S, C).numpy()
        _close(O.region_mean(X, S), ref, 1e-13, "region_mean vs avg_pool2d")


def pin_affinity_orientation():
    """Constructed means: q_r = e0 for every region, k_r[s] = (s+1) e0, so
    A[r, s] = scale (s+1) and every row routes to the last regions first."""
    R, C = 9, 4
    q = np.zeros((1, R, C))
    q[..., 0] = 1.0
    k = np.zeros((1, R, C))
    k[0, :, 0] = np.arange(1, R + 1)
    A = O.region_affinity(q, k, 0.5)
    _close(A[0], np.tile(0.5 * np.arange(1, R + 1), (R, 1)), 1e-15, "affinity")
    idx = O.topk_route(A, 3)
    assert np.array_equal(idx[0], np.tile([8, 7, 6], (R, 1))), idx[0]
    # orientation: a row-specific query picks a row-specific key region
    q2 = np.eye(R)[None]
    k2 = np.eye(R)[None][:, ::-1]          # key region s is e_{R-1-s}
    idx2 = O.topk_route(O.region_affinity(q2, k2, 1.0), 1)[0, :, 0]
    assert np.array_equal(idx2, np.arange(R)[::-1]), idx2


def pin_topk_bruteforce():
    """Top-k equals a plain-Python selection (largest first, ties to the lower
    index) on small matrices with many exact ties, and torch.topk's values."""
    import torch
    r = _rng(3)
    for trial in range(20):
        R = int(r.integers(1, 12))
        A = r.integers(-3, 4, size=(2, R, R)).astype(np.float64)   # many ties
        for k in range(1, R + 1):
            idx = O.topk_route(A, k)
            for b in range(2):
                for row in range(R):
                    vals = list(A[b, row])
                    chosen = []
                    for _ in range(k):
                        best = None
                        for s in range(R):
                            if s in chosen:
                                continue
                            if best is None or vals[s] > vals[best]:
                                best = s
                        chosen.append(best)
                    assert list(idx[b, row]) == chosen, (A[b, row], idx[b, row], chosen)
            tv = torch.topk(torch.from_numpy(A), k, dim=-1).values.numpy()
            assert np.array_equal(np.take_along_axis(A, idx.astype(np.int64), -1), tv)


def pin_scale_invariance():
    """idx does not change under any positive routing scale (reading R5)."""
    Q, K, _ = _rand(4, 2, 8, 8, 6)
    qr, kr = O.region_mean(Q, 4), O.region_mean(K, 4)
    base = O.topk_route(O.region_affinity(qr, kr, 1.0), 5)
    for s in (1e-3, 0.37, 7.0):
        assert np.array_equal(O.topk_route(O.region_affinity(qr, kr, s), 5), base)


def pin_masked_dense():
    """BRA attention equals dense attention masked to the routed regions, for
    the oracle's own routes and for arbitrary routes (p5)."""
    r = _rng(5)
    for (B, H, W, C, heads, S) in ((2, 8, 8, 8, 2, 2), (1, 8, 8, 4, 1, 4), (1, 6, 9, 6, 3, 3)):
        Q, K, V = _rand(int(r.integers(1 << 30)), B, H, W, C)
        scale = (C // heads) ** -0.5
        for topk in range(1, S * S + 1):
            _, idx = O.bra_forward(Q, K, V, heads, S, topk)
            got = O.routed_attention(Q, K, V, idx, heads, S, scale)
            _close(got, brute_masked_attention(Q, K, V, idx, heads, S, scale), TIGHT,
                   f"masked dense S={S} topk={topk}")
            ridx = np.stack([np.stack([r.permutation(S * S)[:topk] for _ in range(S * S)])
                             for _ in range(B)]).astype(np.int32)
            got = O.routed_attention(Q, K, V, ridx, heads, S, scale)
            _close(got, brute_masked_attention(Q, K, V, ridx, heads, S, scale), TIGHT,
                   f"masked dense, random idx S={S} topk={topk}")


def pin_global_when_all_routed():
    """topk = S*S routes every region, so BRA is global attention + LePE."""
    for (B, H, W, C, heads, S) in ((1, 6, 6, 4, 2, 3), (2, 8, 4, 6, 3, 2)):
        Q, K, V = _rand(6, B, H, W, C)
        w = _rng(7).normal(size=(C, 3, 3))
        out, _ = O.bra_forward(Q, K, V, heads, S, S * S, w)
        ref = global_attention(Q, K, V, heads, (C // heads) ** -0.5) + O.lepe(V, w)
        _close(out, ref, TIGHT, "topk=S^2 vs global attention")


def pin_plain_when_one_region():
    """S = 1: one region holding every token, so BRA is plain attention."""
    Q, K, V = _rand(8, 2, 5, 7, 4)
    out, idx = O.bra_forward(Q, K, V, 2, 1, 1)
    assert np.array_equal(idx, np.zeros((2, 1, 1), dtype=np.int32))
    _close(out, global_attention(Q, K, V, 2, 2 ** -0.5), TIGHT, "S=1 vs plain attention")


def pin_window_when_identity():
    """idx[r] = [r] with topk = 1 is p4's non-overlapping window attention."""
    for (B, H, W, C, heads, S) in ((2, 8, 8, 4, 2, 2), (1, 9, 6, 6, 1, 3)):
        Q, K, V = _rand(9, B, H, W, C)
        idx = np.tile(np.arange(S * S, dtype=np.int32)[None, :, None], (B, 1, 1))
        scale = (C // heads) ** -0.5
        _close(O.routed_attention(Q, K, V, idx, heads, S, scale),
               window_attention(Q, K, V, heads, S, scale), TIGHT, "identity idx vs window")


def pin_sdpa_masked():
    """Attention equals torch scaled_dot_product_attention (fp64 CPU) with a
    boolean mask built from the routing index."""
    import torch
    import torch.nn.functional as F
    B, H, W, C, heads, S, topk = 2, 8, 8, 8, 2, 4, 3
    Q, K, V = _rand(10, B, H, W, C)
    _, idx = O.bra_forward(Q, K, V, heads, S, topk)
    d = C // heads
    reg = _pixel_region(H, W, S)
    mask = np.stack([np.stack([np.isin(reg, idx[b, reg[p]]) for p in range(H * W)])
                     for b in range(B)])                      # [B, HW, HW]
    t = lambda X: torch.from_numpy(X.reshape(B, H * W, heads, d)).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(t(Q), t(K), t(V),
                                         attn_mask=torch.from_numpy(mask)[:, None],
                                         scale=d ** -0.5)
    ref = ref.permute(0, 2, 1, 3).reshape(B, H, W, C).numpy()
    _close(O.routed_attention(Q, K, V, idx, heads, S, d ** -0.5), ref, 1e-12, "sdpa")


def pin_lepe_conv2d():
    """LePE equals torch conv2d(groups=C, padding=ks//2) -- p2 §4's depthwise
    Conv2d -- with an asymmetric kernel and a bias, for ks = 1, 3, 5, 7."""
    import torch
    import torch.nn.functional as F
    for ks in (1, 3, 5, 7):
        B, H, W, C = 2, 9, 6, 5
        V = _rng(11).normal(size=(B, H, W, C))
        w = _rng(12 + ks).normal(size=(C, ks, ks))
        b = _rng(13).normal(size=C)
        ref = F.conv2d(torch.from_numpy(V).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None],
                       torch.from_numpy(b), padding=ks // 2, groups=C)
        _close(O.lepe(V, w, b), ref.permute(0, 2, 3, 1).numpy(), 1e-13, f"lepe ks={ks}")


def pin_invariants():
    """Closed-form special cases of the attention and LePE steps."""
    B, H, W, C, heads, S, topk = 2, 8, 8, 6, 3, 4, 3
    Q, K, V = _rand(14, B, H, W, C)
    scale = (C // heads) ** -0.5
    _, idx = O.bra_forward(Q, K, V, heads, S, topk)
    base = O.routed_attention(Q, K, V, idx, heads, S, scale)
    # permuting the routed regions inside a row changes nothing
    perm = idx[..., ::-1].copy()
    _close(O.routed_attention(Q, K, V, perm, heads, S, scale), base, TIGHT, "idx permutation")
    # constant V: every output equals that vector
    cv = np.broadcast_to(np.arange(1.0, C + 1), V.shape).copy()
    _close(O.routed_attention(Q, K, cv, idx, heads, S, scale), cv, TIGHT, "constant V")
    # Q = 0: uniform weights, output = mean of the gathered V
    Z = np.zeros_like(Q)
    got = O.routed_attention(Z, K, V, idx, heads, S, scale)
    for b in range(B):
        for r in range(S * S):
            ys = np.concatenate([O.region_tokens(H, W, S, s)[0] for s in idx[b, r]])
            xs = np.concatenate([O.region_tokens(H, W, S, s)[1] for s in idx[b, r]])
            mean_v = V[b, ys, xs, :].mean(axis=0)
            qy, qx = O.region_tokens(H, W, S, r)
            _close(got[b, qy, qx, :], np.broadcast_to(mean_v, (len(qy), C)), TIGHT, "Q=0")
    # zero LePE weights: out = O; centre-tap delta: L = V
    ks = 5
    out0, _ = O.bra_forward(Q, K, V, heads, S, topk, np.zeros((C, ks, ks)))
    _close(out0, base, TIGHT, "w = 0")
    delta = np.zeros((C, ks, ks))
    delta[:, ks // 2, ks // 2] = 1.0
    _close(O.lepe(V, delta), V, TIGHT, "delta kernel")
    # one off-centre tap shifts V by one pixel with a zero border
    shift = np.zeros((C, ks, ks))
    shift[:, ks // 2, ks // 2 + 1] = 1.0
    ref = np.zeros_like(V)
    ref[:, :, :-1, :] = V[:, :, 1:, :]
    _close(O.lepe(V, shift), ref, TIGHT, "shift kernel")


def pin_route_ties():
    """Exactly equal affinities go to the lower region index (reading R6)."""
    R = 6
    A = np.zeros((1, R, R))
    A[0, 0] = [1, 3, 3, 2, 3, 0]
    idx = O.topk_route(A, 4)
    assert list(idx[0, 0]) == [1, 2, 4, 3]
    assert list(idx[0, 1]) == [0, 1, 2, 3]


# --------------------------------------------------------------------------
# the module around the method (readings M1-M3)

def _module_golden_args(g):
    C, ks = g["C"], g["lepe_ks"]
    w = np.zeros((C, ks, ks))
    for c, i, j, val in g["lepe_taps"]:
        w[c, i, j] = val
    a = lambda n: None if g[n] is None else np.array(g[n], dtype=np.float64)
    return (a("x"), a("w_qkv"), a("b_qkv"), g["heads"], g["S"], g["topk"], w, a("lepe_bias"),
            a("w_out"), a("b_out"))


def pin_module_golden():
    """Hand-worked module fixtures (tests/golden/module_*.json)."""
    files = sorted(glob.glob(os.path.join(GOLDEN, "module_*.json")))
    assert files, "no module fixtures"
    for f in files:
        g = json.load(open(f))
        parts = O.module_forward(*_module_golden_args(g), return_parts=True)
        name = os.path.basename(f)
        assert np.array_equal(parts["idx"], np.array(g["expect_idx"])), f"{name}: idx"
        _close(parts["y"], g["expect_y"], 1e-14, f"{name}: y")
        _close(parts["out"], g["expect_out"], 1e-14, f"{name}: out")


def pin_linear_torch():
    """The projection equals torch.nn.functional.linear in float64 (the
    PyTorch Linear of p1 §3's q_proj / k_proj / v_proj), with and without
    bias, on non-square and square weights."""
    import torch
    import torch.nn.functional as F
    X = _rng(21).normal(size=(2, 3, 5, 7))
    for N in (7, 12):
        w = _rng(22 + N).normal(size=(N, 7))
        b = _rng(23).normal(size=N)
        for bias in (None, b):
            ref = F.linear(torch.from_numpy(X), torch.from_numpy(w),
                           None if bias is None else torch.from_numpy(bias)).numpy()
            _close(O.linear(X, w, bias), ref, 1e-13, f"linear N={N} bias={bias is not None}")


def pin_module_reduces_to_bra():
    """With w_qkv = [I; I; I], no biases and no output projection the module
    is bra_forward(x, x, x); with w_out = I and no output bias it returns
    y = O + L unchanged (readings M1, M2)."""
    B, H, W, C, heads, S, topk = 1, 8, 8, 6, 2, 4, 3
    x = _rng(24).normal(size=(B, H, W, C))
    lw = _rng(25).normal(size=(C, 3, 3))
    eye3 = np.concatenate([np.eye(C)] * 3)
    out, idx = O.module_forward(x, eye3, None, heads, S, topk, lw)
    ref, ref_idx = O.bra_forward(x, x, x, heads, S, topk, lw)
    assert np.array_equal(idx, ref_idx)
    _close(out, ref, TIGHT, "identity projections")
    w = _rng(26).normal(size=(3 * C, C))
    b = _rng(27).normal(size=3 * C)
    p = O.module_forward(x, w, b, heads, S, topk, lw, w_out=np.eye(C), return_parts=True)
    _close(p["out"], p["y"], TIGHT, "identity output projection")


def pin_pool_commutes_with_projection():
    """Region means of a projection are the projection of the region means
    (the map is linear and the mean weights sum to one), so routing can be
    taken from the projected means of x: the two orders agree in float64."""
    B, H, W, C, S = 2, 12, 8, 5, 4
    x = _rng(28).normal(size=(B, H, W, C))
    w = _rng(29).normal(size=(3, C))
    b = _rng(30).normal(size=3)
    _close(O.region_mean(O.linear(x, w, b), S), O.linear(O.region_mean(x, S), w, b), 1e-13,
           "mean/projection order")


def pin_round_storage_torch():
    """bf16 storage rounding equals torch's float32 -> bfloat16 conversion
    (round to nearest even), on random values over a wide range and on exact
    halfway cases; f32 storage equals the float32 cast (reading M4)."""
    import torch
    r = _rng(31)
    x = np.concatenate([r.normal(size=20000), r.normal(size=2000) * 1e-20,
                        r.normal(size=2000) * 1e20]).astype(np.float32)
    u = (r.integers(0, 1 << 15, size=2000, dtype=np.uint32) << 16) | 0x8000   # ties
    u = u[(u >> 23) & 0xFF != 0xFF]
    x = np.concatenate([x, u.view(np.float32), np.float32([0.0, -0.0, 1.0, -3.5])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_storage(x.astype(np.float64), "bf16")
    assert np.array_equal(got, ref), "bf16 rounding"
    y = r.normal(size=1000)
    assert np.array_equal(O.round_storage(y, "f32"), y.astype(np.float32).astype(np.float64))
    assert np.array_equal(O.round_storage(y, None), y)


def pin_module_storage():
    """Reading M4: routing is decided on the projections as computed (the
    region means are those of the unrounded projections, and idx does not
    depend on the storage format); with projections that are exactly
    representable in bf16, storage changes only y, by rounding it."""
    B, H, W, C, heads, S, topk = 1, 8, 8, 6, 2, 4, 3
    x = _rng(32).normal(size=(B, H, W, C))
    w = _rng(33).normal(size=(3 * C, C))
    b = _rng(34).normal(size=3 * C)
    lw = _rng(35).normal(size=(C, 3, 3))
    p64 = O.module_forward(x, w, b, heads, S, topk, lw, return_parts=True)
    p16 = O.module_forward(x, w, b, heads, S, topk, lw, storage="bf16", return_parts=True)
    qkv = O.linear(x, w, b)
    _close(p16["q_r"], O.region_mean(qkv[..., :C], S), 1e-14, "means of unrounded q")
    _close(p16["k_r"], O.region_mean(qkv[..., C:2 * C], S), 1e-14, "means of unrounded k")
    assert np.array_equal(p16["idx"], p64["idx"])
    assert not np.array_equal(p16["q"], p64["q"])
    # bf16-exact projections: identity weights on bf16-representable x
    xb = O.round_storage(x, "bf16")
    eye3 = np.concatenate([np.eye(C)] * 3)
    a = O.module_forward(xb, eye3, None, heads, S, topk, lw, return_parts=True)
    c = O.module_forward(xb, eye3, None, heads, S, topk, lw, storage="bf16", return_parts=True)
    _close(c["O"], a["O"], 0.0, "O unchanged")
    assert np.array_equal(c["y"], O.round_storage(a["y"], "bf16"))


# --------------------------------------------------------------------------
# the BiFormer block (readings B1-B5)

def block_params(C, ks=5, seed=40):
    """Random block parameters (float64) for the pins."""
    r = _rng(seed)
    n = lambda *shape, s=1.0: r.normal(0.0, s, size=shape)
    return {"pos_w": n(C, 3, 3, s=0.3), "pos_b": n(C, s=0.1),
            "ln1_g": 1.0 + n(C, s=0.2), "ln1_b": n(C, s=0.2),
            "w_qkv": n(3 * C, C, s=C ** -0.5), "b_qkv": n(3 * C, s=0.1),
            "lepe_w": n(C, ks, ks, s=0.1), "lepe_b": n(C, s=0.1),
            "w_out": n(C, C, s=C ** -0.5), "b_out": n(C, s=0.1),
            "ln2_g": 1.0 + n(C, s=0.2), "ln2_b": n(C, s=0.2),
            "w_fc1": n(3 * C, C, s=C ** -0.5), "b_fc1": n(3 * C, s=0.1),
            "w_fc2": n(C, 3 * C, s=(3 * C) ** -0.5), "b_fc2": n(C, s=0.1)}


def pin_layer_norm_torch():
    """LayerNorm equals torch.nn.functional.layer_norm (eps 1e-5, affine) in
    float64 (reading B3)."""
    import torch
    import torch.nn.functional as F
    X = _rng(41).normal(size=(3, 5, 4, 12)) * 3.0 + 1.5
    g, b = _rng(42).normal(size=12), _rng(43).normal(size=12)
    ref = F.layer_norm(torch.from_numpy(X), (12,), torch.from_numpy(g), torch.from_numpy(b),
                       eps=1e-5).numpy()
    _close(O.layer_norm(X, g, b), ref, 1e-13, "layer_norm")


def pin_gelu_torch():
    """GELU equals torch's exact (erf) GELU in float64 (reading B4)."""
    import torch
    import torch.nn.functional as F
    X = np.concatenate([_rng(44).normal(size=5000) * 3, np.array([0.0, -0.0, 8.0, -8.0, 1e-8])])
    ref = F.gelu(torch.from_numpy(X), approximate="none").numpy()
    _close(O.gelu(X), ref, 1e-15, "gelu")


def pin_block_torch():
    """The block around the module equals the composition of torch's conv2d
    (groups = C, padding 1), layer_norm, linear and gelu with the pinned
    module (reading B1), in float64."""
    import torch
    import torch.nn.functional as F
    B, H, W, C, heads, S, topk = 1, 8, 8, 8, 2, 4, 3
    C = 8
    x = _rng(45).normal(size=(B, H, W, C))
    p = block_params(C, ks=3)
    out, idx = O.block_forward(x, p, 2, S, topk)
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    xt = T(x).permute(0, 3, 1, 2)
    x1 = (xt + F.conv2d(xt, T(p["pos_w"])[:, None], T(p["pos_b"]), padding=1, groups=C))
    x1 = x1.permute(0, 2, 3, 1)
    n1 = F.layer_norm(x1, (C,), T(p["ln1_g"]), T(p["ln1_b"]), eps=1e-5)
    mod, midx = O.module_forward(n1.numpy(), p["w_qkv"], p["b_qkv"], 2, S, topk, p["lepe_w"],
                                 p["lepe_b"], p["w_out"], p["b_out"])
    x2 = x1 + T(mod)
    n2 = F.layer_norm(x2, (C,), T(p["ln2_g"]), T(p["ln2_b"]), eps=1e-5)
    h = F.gelu(F.linear(n2, T(p["w_fc1"]), T(p["b_fc1"])), approximate="none")
    ref = x2 + F.linear(h, T(p["w_fc2"]), T(p["b_fc2"]))
    assert np.array_equal(idx, midx)
    _close(out, ref.numpy(), 1e-12, "block")


def pin_block_storage():
    """Reading B5: with bf16 storage every layer output the block keeps (x1,
    LN1(x1), x2, LN2(x2), the hidden tensor h and out) is a bf16 number, and
    each equals torch's float64 layer (conv2d with groups = C, layer_norm,
    linear, gelu) applied to the previous stored value and rounded to bf16,
    to within one bf16 ulp (two float64 evaluations may straddle a rounding
    boundary).  A storage point left out leaves a value that is not a bf16
    number; one moved to another place changes a value by up to an ulp."""
    import torch
    import torch.nn.functional as F
    B, H, W, C, heads, S, topk = 1, 8, 8, 16, 2, 4, 3
    x = O.round_storage(_rng(46).normal(size=(B, H, W, C)), "bf16")
    p = block_params(C, ks=3, seed=47)
    r = O.block_forward(x, p, heads, S, topk, storage="bf16", return_parts=True)
    for name in ("x1", "n1", "x2", "n2", "h", "out"):
        v = np.asarray(r[name])
        assert np.array_equal(O.round_storage(v, "bf16"), v), f"{name} is not stored in bf16"
    assert np.array_equal(O.round_storage(r["mod"]["y"], "bf16"), r["mod"]["y"])
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    rs = lambda t: O.round_storage(t.numpy(), "bf16")

    def ulp_close(got, want, what):
        a = np.maximum(np.abs(want), 2.0 ** -126)
        ulp = np.exp2(np.floor(np.log2(a)) - 7)
        assert np.all(np.abs(np.asarray(got) - want) <= ulp * (1 + 1e-12)), what

    xt = T(x).permute(0, 3, 1, 2)
    x1 = (xt + F.conv2d(xt, T(p["pos_w"])[:, None], T(p["pos_b"]), padding=1, groups=C))
    ulp_close(r["x1"], rs(x1.permute(0, 2, 3, 1)), "x1")
    ulp_close(r["n1"], rs(F.layer_norm(T(r["x1"]), (C,), T(p["ln1_g"]), T(p["ln1_b"]), eps=1e-5)),
              "n1")
    ulp_close(r["x2"], rs(T(r["x1"]) + T(r["mod"]["out"])), "x2")
    ulp_close(r["n2"], rs(F.layer_norm(T(r["x2"]), (C,), T(p["ln2_g"]), T(p["ln2_b"]), eps=1e-5)),
              "n2")
    ulp_close(r["h"], rs(F.gelu(F.linear(T(r["n2"]), T(p["w_fc1"]), T(p["b_fc1"])),
                                approximate="none")), "h")
    ulp_close(r["out"], rs(T(r["x2"]) + F.linear(T(r["h"]), T(p["w_fc2"]), T(p["b_fc2"]))), "out")
    # the module inside the block is the module of the stored LN1(x1)
    m = O.module_forward(r["n1"], p["w_qkv"], p["b_qkv"], heads, S, topk, p["lepe_w"],
                         p["lepe_b"], p["w_out"], p["b_out"], storage="bf16", return_parts=True)
    assert np.array_equal(m["out"], r["mod"]["out"])


def pin_block_given_route():
    """With idx given, the block attends over that route: the route the
    block computes itself gives back the same block, and any other route
    gives the module's output on that route (the fixed-index use)."""
    B, H, W, C, heads, S, topk = 1, 8, 8, 8, 2, 4, 2
    x = _rng(48).normal(size=(B, H, W, C))
    p = block_params(C, ks=3, seed=49)
    r = O.block_forward(x, p, heads, S, topk, return_parts=True)
    r2 = O.block_forward(x, p, heads, S, topk, return_parts=True, idx=r["idx"])
    assert np.array_equal(r2["out"], r["out"])
    other = (np.asarray(r["idx"]) + 1) % (S * S)
    r3 = O.block_forward(x, p, heads, S, topk, return_parts=True, idx=other)
    m = O.module_forward(r3["n1"], p["w_qkv"], p["b_qkv"], heads, S, topk, p["lepe_w"],
                         p["lepe_b"], p["w_out"], p["b_out"], return_parts=True, idx=other)
    assert np.array_equal(r3["idx"], other)
    _close(r3["out"], r3["x2"] + O.linear(r3["h"], p["w_fc2"], p["b_fc2"]), 1e-13, "block out")
    _close(r3["mod"]["out"], m["out"], 0.0, "module on the given route")
    assert not np.allclose(r3["out"], r["out"])


# --------------------------------------------------------------------------
# the backward pass with a fixed index (readings G1, G2)

def _torch_bra_loss(Qt, Kt, Vt, wt, bt, idx, heads, S, scale, Gt):
    """sum(out * dout) of the BRA forward written with torch ops: masked
    dense attention over the routed regions (the mask of pin P1) plus
    conv2d(groups = C) for LePE."""
    import torch
    import torch.nn.functional as F
    B, H, W, C = Qt.shape
    d = C // heads
    reg = torch.from_numpy(_pixel_region(H, W, S))
    out = torch.zeros_like(Qt)
    for b in range(B):
        allowed = torch.zeros(S * S, S * S, dtype=torch.bool)
        for r in range(S * S):
            allowed[r, torch.from_numpy(np.asarray(idx[b, r], dtype=np.int64))] = True
        mask = allowed[reg][:, reg]                                  # [HW, HW]
        q = Qt[b].reshape(H * W, heads, d).transpose(0, 1)
        k = Kt[b].reshape(H * W, heads, d).transpose(0, 1)
        v = Vt[b].reshape(H * W, heads, d).transpose(0, 1)
        logits = scale * q @ k.transpose(1, 2)
        logits = logits.masked_fill(~mask, float("-inf"))
        o = torch.softmax(logits, dim=-1) @ v
        out[b] = o.transpose(0, 1).reshape(H, W, C)
    if wt is not None:
        ks = wt.shape[-1]
        lep = F.conv2d(Vt.permute(0, 3, 1, 2), wt[:, None], bt, padding=ks // 2, groups=C)
        out = out + lep.permute(0, 2, 3, 1)
    return (out * Gt).sum()


def pin_backward_autograd():
    """The fixed-index gradients equal torch autograd of the same forward
    (masked dense attention + conv2d) in float64, with distinct routes per
    row and a key region that no row routes to."""
    import torch
    B, H, W, C, heads, S, topk, ks = 2, 8, 8, 8, 2, 4, 3, 5
    r = _rng(50)
    Q, K, V, G = (r.normal(size=(B, H, W, C)) for _ in range(4))
    w, b = r.normal(size=(C, ks, ks)) * 0.3, r.normal(size=C)
    others = np.array([s for s in range(S * S) if s != 5])   # region 5: routed from nowhere
    idx = np.stack([np.stack([r.permutation(others)[:topk] for _ in range(S * S)])
                    for _ in range(B)]).astype(np.int32)
    scale = (C // heads) ** -0.5
    got = O.bra_backward(Q, K, V, idx, heads, S, G, w, b)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    Qt, Kt, Vt, wt, bt = T(Q), T(K), T(V), T(w), T(b)
    _torch_bra_loss(Qt, Kt, Vt, wt, bt, idx, heads, S, scale, torch.from_numpy(G)).backward()
    for name, t in (("dQ", Qt), ("dK", Kt), ("dV", Vt), ("dw", wt), ("db", bt)):
        _close(got[name], t.grad.numpy(), 1e-11, f"backward {name}")
    ys, xs = O.region_tokens(H, W, S, 5)
    assert np.all(got["dK"][:, ys, xs] == 0.0), "a key region routed from nowhere gets no dK"


def pin_backward_finite_differences():
    """Central differences of sum(out * dout) in float64 match the analytic
    gradients at sampled coordinates of Q, K, V, w and b."""
    B, H, W, C, heads, S, topk, ks = 1, 4, 4, 4, 2, 2, 2, 3
    r = _rng(51)
    Q, K, V, G = (r.normal(size=(B, H, W, C)) for _ in range(4))
    w, b = r.normal(size=(C, ks, ks)) * 0.5, r.normal(size=C)
    idx = np.array([[[0, 2], [1, 3], [3, 0], [2, 1]]], dtype=np.int32)
    got = O.bra_backward(Q, K, V, idx, heads, S, G, w, b)

    def loss(Q_, K_, V_, w_, b_):
        out = O.routed_attention(Q_, K_, V_, idx, heads, S, (C // heads) ** -0.5) + O.lepe(V_, w_, b_)
        return float(np.sum(out * G))

    h = 1e-6
    args = {"dQ": Q, "dK": K, "dV": V, "dw": w, "db": b}
    order = ["dQ", "dK", "dV", "dw", "db"]
    for name in order:
        arr = args[name]
        for flat in r.choice(arr.size, size=min(6, arr.size), replace=False):
            pos = np.unravel_index(flat, arr.shape)
            plus = [a.copy() for a in (Q, K, V, w, b)]
            minus = [a.copy() for a in (Q, K, V, w, b)]
            plus[order.index(name)][pos] += h
            minus[order.index(name)][pos] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - got[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd,
                                                                         got[name][pos])


# --------------------------------------------------------------------------
# video: T x S x S regions, one frame each (readings V1-V4)

def pin_video_single_frame():
    """A one-frame clip is an image: video_forward equals bra_forward."""
    r = _rng(60)
    B, H, W, C, heads, S, topk, ks = 2, 8, 8, 8, 2, 2, 3, 3
    Q, K, V = (r.normal(size=(B, 1, H, W, C)) for _ in range(3))
    w, b = r.normal(size=(C, ks, ks)) * 0.3, r.normal(size=C)
    got, gi = O.video_forward(Q, K, V, heads, S, topk, w, b)
    want, wi = O.bra_forward(Q[:, 0], K[:, 0], V[:, 0], heads, S, topk, w, b)
    assert np.array_equal(gi, wi)
    _close(got[:, 0], want, 1e-12, "video T=1 vs image")


def _torch_video(Q, K, V, w, b, heads, S, topk):
    """BRA on a clip written with torch ops: region means by a reshape, the
    affinity by a matmul, torch.topk, masked dense attention over all the
    clip's tokens, and conv2d(groups = C) on the frames."""
    import torch
    import torch.nn.functional as F
    Qt, Kt, Vt = (torch.from_numpy(x) for x in (Q, K, V))
    B, T, H, W, C = Qt.shape
    hs, ws, d = H // S, W // S, C // heads
    mean = lambda X: X.reshape(B, T, S, hs, S, ws, C).mean(dim=(3, 5)).reshape(B, T * S * S, C)
    A = C ** -0.5 * mean(Qt) @ mean(Kt).transpose(1, 2)
    idx = torch.topk(A, topk, dim=-1).indices
    t = torch.arange(T)[:, None, None]
    y = torch.arange(H)[None, :, None]
    x = torch.arange(W)[None, None, :]
    reg = (t * S * S + (y // hs) * S + x // ws).reshape(-1)            # [T*H*W]
    out = torch.empty_like(Qt)
    for bb in range(B):
        allowed = torch.zeros(T * S * S, T * S * S, dtype=torch.bool)
        allowed.scatter_(1, idx[bb], True)
        mask = allowed[reg][:, reg]
        q = Qt[bb].reshape(-1, heads, d).transpose(0, 1)
        k = Kt[bb].reshape(-1, heads, d).transpose(0, 1)
        v = Vt[bb].reshape(-1, heads, d).transpose(0, 1)
        lg = (d ** -0.5) * q @ k.transpose(1, 2)
        o = torch.softmax(lg.masked_fill(~mask, float("-inf")), dim=-1) @ v
        out[bb] = o.transpose(0, 1).reshape(T, H, W, C)
    ksz = w.shape[-1]
    lep = F.conv2d(Vt.reshape(B * T, H, W, C).permute(0, 3, 1, 2), torch.from_numpy(w)[:, None],
                   torch.from_numpy(b), padding=ksz // 2, groups=C)
    out = out + lep.permute(0, 2, 3, 1).reshape(B, T, H, W, C)
    return out.numpy(), idx.numpy()


def pin_video_masked_dense_torch():
    """video_forward equals a torch formulation of the same definition
    (region means by reshape, topk, masked dense attention over the whole
    clip, per-frame conv2d), index included; V gets a value only in the
    first frame's last row so that LePE leaking across frames would show."""
    r = _rng(61)
    B, T, H, W, C, heads, S, topk, ks = 2, 3, 4, 4, 8, 2, 2, 3, 3
    Q, K, V = (r.normal(size=(B, T, H, W, C)) for _ in range(3))
    V[:, 1, 0] += 5.0                                   # next to frame 0's last row
    w, b = r.normal(size=(C, ks, ks)), r.normal(size=C)
    got, gi = O.video_forward(Q, K, V, heads, S, topk, w, b)
    want, wi = _torch_video(Q, K, V, w, b, heads, S, topk)
    assert np.array_equal(gi, wi), "video routing index"
    _close(got, want, 1e-12, "video vs torch")


def pin_video_frame_permutation():
    """Reordering the frames reorders the output and relabels the routing
    (region (t, j) of the new clip is region (perm[t], j) of the old)."""
    r = _rng(62)
    B, T, H, W, C, heads, S, topk, ks = 1, 4, 4, 4, 8, 2, 2, 5, 3
    Q, K, V = (r.normal(size=(B, T, H, W, C)) for _ in range(3))
    w = r.normal(size=(C, ks, ks)) * 0.3
    perm = np.array([2, 0, 3, 1])
    inv = np.argsort(perm)
    out, idx = O.video_forward(Q, K, V, heads, S, topk, w)
    out2, idx2 = O.video_forward(Q[:, perm], K[:, perm], V[:, perm], heads, S, topk, w)
    _close(out2, out[:, perm], 1e-12, "video frame permutation")
    SS = S * S
    rows = (perm[:, None] * SS + np.arange(SS)[None, :]).reshape(-1)   # new row -> old row
    mapped = idx[:, rows]                                              # old labels
    relabel = inv[mapped // SS] * SS + mapped % SS
    assert np.array_equal(idx2, relabel), "video routing relabelled"


ALL_PINS = [
    pin_golden, pin_partition_layout, pin_pool_avgpool, pin_affinity_orientation,
    pin_topk_bruteforce, pin_scale_invariance, pin_masked_dense,
    pin_global_when_all_routed, pin_plain_when_one_region, pin_window_when_identity,
    pin_sdpa_masked, pin_lepe_conv2d, pin_invariants, pin_route_ties,
    pin_module_golden, pin_linear_torch, pin_module_reduces_to_bra,
    pin_pool_commutes_with_projection, pin_round_storage_torch, pin_module_storage,
    pin_layer_norm_torch, pin_gelu_torch, pin_block_torch, pin_block_storage,
    pin_block_given_route,
    pin_backward_autograd, pin_backward_finite_differences,
    pin_video_single_frame, pin_video_masked_dense_torch, pin_video_frame_permutation,
]
