"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one of them.  Each mutant replaces one oracle function for the
duration of a test; at least one pin must then fail."""

import numpy as np
import pytest

import oracle.bra_oracle as O
from oracle_pins import ALL_PINS

_orig = {name: getattr(O, name) for name in
         ("region_mean", "region_affinity", "topk_route", "routed_attention", "lepe",
          "region_tokens", "linear", "module_forward", "round_storage", "layer_norm", "gelu",
          "block_forward", "bra_backward", "video_forward")}


def _mean_as_sum(X, S):
    B, H, W, C = np.shape(X)
    return _orig["region_mean"](X, S) * ((H // S) * (W // S))


def _mean_column_major(X, S):
    m = _orig["region_mean"](X, S)
    B, R, C = m.shape
    return m.reshape(B, S, S, C).transpose(0, 2, 1, 3).reshape(B, R, C)


def _affinity_transposed(q_r, k_r, s):
    return _orig["region_affinity"](k_r, q_r, s)


def _topk_smallest(A, k):
    return np.argsort(np.asarray(A), axis=-1, kind="stable")[..., :k].astype(np.int32)


def _topk_ties_high(A, k):
    A = np.asarray(A)
    R = A.shape[-1]
    order = np.argsort(-A[..., ::-1], axis=-1, kind="stable")
    return (R - 1 - order[..., :k]).astype(np.int32)


def _attn_unscaled(Q, K, V, idx, heads, S, scale):
    return _orig["routed_attention"](Q, K, V, idx, heads, S, 1.0)


def _attn_first_region_only(Q, K, V, idx, heads, S, scale):
    idx = np.asarray(idx)
    return _orig["routed_attention"](Q, K, V, np.repeat(idx[..., :1], idx.shape[-1], -1),
                                     heads, S, scale)


def _attn_heads_interleaved(Q, K, V, idx, heads, S, scale):
    C = np.shape(Q)[-1]
    d = C // heads
    perm = np.arange(C).reshape(d, heads).T.reshape(-1)      # channel c*heads+m -> head m
    inv = np.argsort(perm)
    P = lambda X: np.asarray(X, dtype=np.float64)[..., perm]
    return _orig["routed_attention"](P(Q), P(K), P(V), idx, heads, S, scale)[..., inv]


def _attn_softmax_over_queries(Q, K, V, idx, heads, S, scale):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, W, C = Q.shape
    d = C // heads
    out = np.zeros_like(Q)
    for b in range(B):
        for r in range(S * S):
            ys, xs = O.region_tokens(H, W, S, r)
            ky = np.concatenate([O.region_tokens(H, W, S, s)[0] for s in idx[b, r]])
            kx = np.concatenate([O.region_tokens(H, W, S, s)[1] for s in idx[b, r]])
            q = Q[b, ys, xs].reshape(-1, heads, d)
            k = K[b, ky, kx].reshape(-1, heads, d)
            v = V[b, ky, kx].reshape(-1, heads, d)
            lg = scale * np.einsum("nhd,mhd->hnm", q, k)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            out[b, ys, xs] = np.einsum("hnm,mhd->nhd", p, v).reshape(-1, C)
    return out


def _lepe_flipped(V, w, bias=None):
    return _orig["lepe"](V, np.asarray(w)[:, ::-1, ::-1], bias)


def _lepe_transposed(V, w, bias=None):
    return _orig["lepe"](V, np.swapaxes(np.asarray(w), 1, 2), bias)


def _lepe_no_bias(V, w, bias=None):
    return _orig["lepe"](V, w, None)


def _lepe_circular(V, w, bias=None):
    V = np.asarray(V, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ks = w.shape[-1]
    p = ks // 2
    L = np.zeros_like(V)
    for i in range(ks):
        for j in range(ks):
            L += w[:, i, j] * np.roll(V, shift=(p - i, p - j), axis=(1, 2))
    return L + (0 if bias is None else np.asarray(bias))


def _tokens_column_major(H, W, S, r):
    hs, ws = H // S, W // S
    ry, rx = divmod(int(r), S)
    t = np.arange(hs * ws)
    return ry * hs + t % hs, rx * ws + t // hs


def _linear_transposed(X, w, b=None):
    w = np.asarray(w)
    return _orig["linear"](X, w.T if w.shape[0] == w.shape[1] else w, b)


def _linear_no_bias(X, w, b=None):
    return _orig["linear"](X, w, None)


def _linear_bias_subtracted(X, w, b=None):
    return _orig["linear"](X, w, None if b is None else -np.asarray(b))


def _module_qk_swapped(x, w_qkv, b_qkv, *a, **k):
    C = np.shape(x)[-1]
    w = np.asarray(w_qkv)
    w = np.concatenate([w[C:2 * C], w[:C], w[2 * C:]])
    b = None if b_qkv is None else np.concatenate(
        [np.asarray(b_qkv)[C:2 * C], np.asarray(b_qkv)[:C], np.asarray(b_qkv)[2 * C:]])
    return _orig["module_forward"](x, w, b, *a, **k)


def _module_lepe_on_x(x, w_qkv, b_qkv, heads, S, topk, lepe_w=None, lepe_b=None, w_out=None,
                      b_out=None, route_scale=None, attn_scale=None, storage=None,
                      return_parts=False):
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[-1]
    qkv = O.linear(x, w_qkv, b_qkv)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    p = O.bra_forward(q, k, v, heads, S, topk, None, None, route_scale, attn_scale,
                      return_parts=True)
    y = p["O"] + (O.lepe(x, lepe_w, lepe_b) if lepe_w is not None else 0.0)
    out = O.linear(y, w_out, b_out) if w_out is not None else y
    if return_parts:
        return dict(p, q=q, k=k, v=v, y=y, out=out)
    return out, p["idx"]


def _module_out_before_lepe(x, w_qkv, b_qkv, heads, S, topk, lepe_w=None, lepe_b=None,
                            w_out=None, b_out=None, route_scale=None, attn_scale=None,
                            storage=None, return_parts=False):
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[-1]
    qkv = O.linear(x, w_qkv, b_qkv)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    p = O.bra_forward(q, k, v, heads, S, topk, None, None, route_scale, attn_scale,
                      return_parts=True)
    o = O.linear(p["O"], w_out, b_out) if w_out is not None else p["O"]
    L = O.lepe(v, lepe_w, lepe_b) if lepe_w is not None else 0.0
    y = p["O"] + L
    out = o + L
    if return_parts:
        return dict(p, q=q, k=k, v=v, y=y, out=out)
    return out, p["idx"]


def _round_truncating(X, storage):
    X = np.asarray(X, dtype=np.float64)
    if storage != "bf16":
        return _orig["round_storage"](X, storage)
    _, e = np.frexp(X)
    e = np.maximum(e, -125)
    return np.ldexp(np.trunc(np.ldexp(X, 8 - e)), e - 8)


def _round_ties_away(X, storage):
    X = np.asarray(X, dtype=np.float64)
    if storage != "bf16":
        return _orig["round_storage"](X, storage)
    _, e = np.frexp(X)
    e = np.maximum(e, -125)
    t = np.ldexp(X, 8 - e)
    return np.ldexp(np.sign(t) * np.floor(np.abs(t) + 0.5), e - 8)


def _module_round_before_routing(x, w_qkv, b_qkv, heads, S, topk, lepe_w=None, lepe_b=None,
                                 w_out=None, b_out=None, route_scale=None, attn_scale=None,
                                 storage=None, return_parts=False):
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[-1]
    qkv = O.round_storage(O.linear(x, w_qkv, b_qkv), storage)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    p = O.bra_forward(q, k, v, heads, S, topk, lepe_w, lepe_b, route_scale, attn_scale,
                      return_parts=True)
    y = O.round_storage(p["out"], storage)
    out = O.linear(y, w_out, b_out) if w_out is not None else y
    if return_parts:
        return dict(p, q=q, k=k, v=v, y=y, out=out)
    return out, p["idx"]


def _ln_unbiased(X, gamma, beta, eps=1e-5):
    X = np.asarray(X, dtype=np.float64)
    mu = X.mean(axis=-1, keepdims=True)
    var = ((X - mu) ** 2).sum(axis=-1, keepdims=True) / (X.shape[-1] - 1)
    return (X - mu) / np.sqrt(var + eps) * gamma + beta


def _ln_no_shift(X, gamma, beta, eps=1e-5):
    return _orig["layer_norm"](X, gamma, np.zeros_like(np.asarray(beta)), eps)


def _gelu_tanh(X):
    X = np.asarray(X, dtype=np.float64)
    return 0.5 * X * (1 + np.tanh(np.sqrt(2 / np.pi) * (X + 0.044715 * X ** 3)))


def _block_no_pos_residual(x, p, heads, S, topk, route_scale=None, attn_scale=None,
                           storage=None, return_parts=False, idx=None):
    x = np.asarray(x, dtype=np.float64)
    q = dict(p)
    # x1 = conv(x) + b only: subtract x again through a centre tap of -1
    w = np.array(p["pos_w"], dtype=np.float64)
    w[:, 1, 1] -= 1.0
    q["pos_w"] = w
    return _orig["block_forward"](x, q, heads, S, topk, route_scale, attn_scale, storage,
                                  return_parts, idx=idx)


def _block_storage_skipping(skip):
    """The block with the storage rounding of one layer output left out."""
    def block(x, p, heads, S, topk, route_scale=None, attn_scale=None, storage=None,
              return_parts=False, idx=None):
        st = lambda name, t: t if name == skip else O.round_storage(t, storage)
        x = np.asarray(x, dtype=np.float64)
        x1 = st("x1", x + O.lepe(x, p["pos_w"], p["pos_b"]))
        n1 = st("n1", O.layer_norm(x1, p["ln1_g"], p["ln1_b"]))
        mod = O.module_forward(n1, p["w_qkv"], p["b_qkv"], heads, S, topk, p["lepe_w"],
                               p["lepe_b"], p["w_out"], p["b_out"], route_scale, attn_scale,
                               storage, return_parts=True, idx=idx)
        x2 = st("x2", x1 + mod["out"])
        n2 = st("n2", O.layer_norm(x2, p["ln2_g"], p["ln2_b"]))
        h = st("h", O.gelu(O.linear(n2, p["w_fc1"], p["b_fc1"])))
        out = st("out", x2 + O.linear(h, p["w_fc2"], p["b_fc2"]))
        if return_parts:
            return {"x1": x1, "n1": n1, "mod": mod, "x2": x2, "n2": n2, "h": h, "out": out,
                    "idx": mod["idx"]}
        return out, mod["idx"]
    block.__name__ = f"_block_{skip}_unrounded"
    return block


def _block_ignores_given_route(x, p, heads, S, topk, route_scale=None, attn_scale=None,
                               storage=None, return_parts=False, idx=None):
    return _orig["block_forward"](x, p, heads, S, topk, route_scale, attn_scale, storage,
                                  return_parts)


def _block_post_norm(x, p, heads, S, topk, route_scale=None, attn_scale=None, storage=None,
                     return_parts=False, idx=None):
    x = np.asarray(x, dtype=np.float64)
    x1 = x + O.lepe(x, p["pos_w"], p["pos_b"])
    mod, idx = O.module_forward(x1, p["w_qkv"], p["b_qkv"], heads, S, topk, p["lepe_w"],
                                p["lepe_b"], p["w_out"], p["b_out"], route_scale, attn_scale)
    x2 = O.layer_norm(x1 + mod, p["ln1_g"], p["ln1_b"])
    out = O.layer_norm(x2 + O.linear(O.gelu(O.linear(x2, p["w_fc1"], p["b_fc1"])), p["w_fc2"],
                                     p["b_fc2"]), p["ln2_g"], p["ln2_b"])
    return (dict(out=out, idx=idx) if return_parts else (out, idx))


def _bw_scale_dk_twice(Q, K, V, idx, heads, S, dout, w=None, bias=None, attn_scale=None):
    g = _orig["bra_backward"](Q, K, V, idx, heads, S, dout, w, bias, attn_scale)
    g["dK"] = g["dK"] * 2.0
    return g


def _bw_no_softmax_term(Q, K, V, idx, heads, S, dout, w=None, bias=None, attn_scale=None):
    """ds = p * dp (the rowsum term dropped): recompute dQ/dK that way."""
    g = _orig["bra_backward"](Q, K, V, idx, heads, S, dout, w, bias, attn_scale)
    Q_, K_, V_, G = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, dout))
    B, H, W, C = Q_.shape
    d = C // heads
    sc = d ** -0.5 if attn_scale is None else attn_scale
    dQ = np.zeros_like(Q_)
    for b in range(B):
        for r in range(S * S):
            ys, xs = O.region_tokens(H, W, S, r)
            ky = np.concatenate([O.region_tokens(H, W, S, s)[0] for s in idx[b, r]])
            kx = np.concatenate([O.region_tokens(H, W, S, s)[1] for s in idx[b, r]])
            q = Q_[b, ys, xs].reshape(-1, heads, d)
            k = K_[b, ky, kx].reshape(-1, heads, d)
            v = V_[b, ky, kx].reshape(-1, heads, d)
            do = G[b, ys, xs].reshape(-1, heads, d)
            lg = sc * np.einsum("nhd,mhd->hnm", q, k)
            p = np.exp(lg - lg.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            ds = p * np.einsum("nhd,mhd->hnm", do, v)
            dQ[b, ys, xs] = (sc * np.einsum("hnm,mhd->nhd", ds, k)).reshape(-1, C)
    g["dQ"] = dQ
    return g


def _bw_lepe_not_transposed(Q, K, V, idx, heads, S, dout, w=None, bias=None, attn_scale=None):
    g = _orig["bra_backward"](Q, K, V, idx, heads, S, dout, None, None, attn_scale)
    if w is not None:
        g["dV"] = g["dV"] + O.lepe(dout, w)              # correlation instead of its transpose
        full = _orig["bra_backward"](Q, K, V, idx, heads, S, dout, w, bias, attn_scale)
        g["dw"], g["db"] = full["dw"], full["db"]
    return g


def _bw_dw_unshifted(Q, K, V, idx, heads, S, dout, w=None, bias=None, attn_scale=None):
    g = _orig["bra_backward"](Q, K, V, idx, heads, S, dout, w, bias, attn_scale)
    if w is not None:
        g["dw"] = g["dw"][:, ::-1, ::-1].copy()
    return g


def _video_lepe_stacked(Q, K, V, heads, S, topk, w=None, bias=None, route_scale=None,
                        attn_scale=None, return_parts=False):
    """LePE over the frame-stacked image: it leaks across frame borders."""
    out, idx = _orig["video_forward"](Q, K, V, heads, S, topk, None, None, route_scale, attn_scale)
    if w is not None:
        B, T, H, W, C = np.shape(V)
        out = out + O.lepe(np.reshape(V, (B, T * H, W, C)), w, bias).reshape(B, T, H, W, C)
    return out, idx


def _video_route_within_frame(Q, K, V, heads, S, topk, w=None, bias=None, route_scale=None,
                              attn_scale=None, return_parts=False):
    """Each frame routed on its own (no cross-frame routing)."""
    T = np.shape(Q)[1]
    C = np.shape(Q)[-1]
    rs = C ** -0.5 if route_scale is None else route_scale
    outs, idxs = [], []
    for t in range(T):
        o, i = _orig["video_forward"](Q[:, t:t + 1], K[:, t:t + 1], V[:, t:t + 1], heads, S,
                                      min(topk, S * S), w, bias, rs, attn_scale)
        outs.append(o)
        idxs.append(i + t * S * S)
    out = np.concatenate(outs, axis=1)
    idx = np.concatenate(idxs, axis=1)
    if idx.shape[-1] < topk:
        idx = np.concatenate([idx, np.repeat(idx[..., -1:], topk - idx.shape[-1], -1)], -1)
    return out, idx


def _video_time_minor_labels(Q, K, V, heads, S, topk, w=None, bias=None, route_scale=None,
                             attn_scale=None, return_parts=False):
    """Regions numbered with time as the fastest axis."""
    out, idx = _orig["video_forward"](Q, K, V, heads, S, topk, w, bias, route_scale, attn_scale)
    T, SS = np.shape(Q)[1], S * S
    lab = lambda r: (r % SS) * T + r // SS
    rows = np.argsort(lab(np.arange(T * SS)))
    return out, lab(idx)[:, rows]


def _video_rows_cols_swapped(Q, K, V, heads, S, topk, w=None, bias=None, route_scale=None,
                             attn_scale=None, return_parts=False):
    """Regions column-major inside a frame (rows and columns swapped)."""
    tr = lambda X: None if X is None else np.swapaxes(np.asarray(X, dtype=np.float64), 2, 3)
    out, idx = _orig["video_forward"](tr(Q), tr(K), tr(V), heads, S, topk,
                                      None if w is None else np.swapaxes(w, 1, 2), bias,
                                      route_scale, attn_scale)
    return tr(out), idx


MUTANTS = {
    "region_mean": [_mean_as_sum, _mean_column_major],
    "region_affinity": [_affinity_transposed],
    "topk_route": [_topk_smallest, _topk_ties_high],
    "routed_attention": [_attn_unscaled, _attn_first_region_only, _attn_heads_interleaved,
                         _attn_softmax_over_queries],
    "lepe": [_lepe_flipped, _lepe_transposed, _lepe_no_bias, _lepe_circular],
    "region_tokens": [_tokens_column_major],
    "linear": [_linear_transposed, _linear_no_bias, _linear_bias_subtracted],
    "module_forward": [_module_qk_swapped, _module_lepe_on_x, _module_out_before_lepe,
                       _module_round_before_routing],
    "round_storage": [_round_truncating, _round_ties_away],
    "layer_norm": [_ln_unbiased, _ln_no_shift],
    "gelu": [_gelu_tanh],
    "block_forward": [_block_no_pos_residual, _block_post_norm, _block_storage_skipping("h"),
                      _block_storage_skipping("n2"), _block_storage_skipping("x1"),
                      _block_ignores_given_route],
    "bra_backward": [_bw_scale_dk_twice, _bw_no_softmax_term, _bw_lepe_not_transposed,
                     _bw_dw_unshifted],
    "video_forward": [_video_lepe_stacked, _video_route_within_frame, _video_time_minor_labels,
                      _video_rows_cols_swapped],
}
CASES = [(name, m) for name, ms in MUTANTS.items() for m in ms]


@pytest.mark.parametrize("name,mutant", CASES, ids=[m.__name__.strip("_") for _, m in CASES])
def test_mutant_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # AssertionError, or a shape error from the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {mutant.__name__} of {name}"
