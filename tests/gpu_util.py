"""Helpers for the GPU parity tests: upload seeded inputs, run the oracle,
compare at the accuracy contract of the path.

Tolerances (floating point): max |gpu - ref| <= tol * RMS(ref) over the whole
tensor, tol = 1e-4 for float32 and 2e-2 for bfloat16; a bfloat16 output is
also granted half an ulp of its own format at each element, which rounding
the exact result alone can spend (see test_tolerance_reading.py).  Routing indices must
match the oracle exactly, except rows where the oracle's fp64 affinities of
the two choices at every differing position agree within 1e-6 relative
(near-ties); for such rows the output is compared with the oracle run on the
GPU's (validated) indices.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from vision_transformer_dynamic_region_amd.workloads import bf16_bits

TOL = {"f32": 1e-4, "bf16": 2e-2}
TIE_RTOL = 1e-6


def to_dev(x: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300) if ref.size else 0.0


def bf16_half_ulp(ref) -> np.ndarray:
    """Half the spacing of bfloat16 numbers at |ref| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def excess_err(got, ref, dtype: str, stored: bool = False) -> float:
    """max |got - ref| / RMS(ref), after granting bf16 outputs the half-ulp
    their own format costs at each element (zero for float32).  With stored,
    the reference is itself a rounded (stored) value, and a full ulp is
    granted: two roundings of nearly equal values can land on neighbours."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-300)
    d = np.abs(got - ref)
    if dtype == "bf16":
        d = np.maximum(d - (2.0 if stored else 1.0) * bf16_half_ulp(ref), 0.0)
    return float(np.max(d)) / rms


def assert_close(got, ref, dtype: str, what: str, stored: bool = False, tol: float | None = None):
    """Tolerance of the contract: max-abs error <= tol * RMS(ref), tol 1e-4
    (f32) or 2e-2 (bf16).  For bf16 the output's own rounding (half an ulp of
    the exact value, up to 3.8e-2 * RMS on the stage-1 workload even for a
    perfectly computed result) is granted on top; a full ulp when the
    reference is a stored (rounded) value."""
    tol = TOL[dtype] if tol is None else tol
    e = excess_err(got, ref, dtype, stored)
    raw = rel_err(got, ref)
    assert e <= tol, (f"{what}: max(|err| - bf16 {'ulp' if stored else 'half-ulp'})/RMS = "
                      f"{e:.3e} > {tol:.1e} (raw max|err|/RMS {raw:.3e})")
    return e


def check_idx(idx_gpu: np.ndarray, idx_ref: np.ndarray, A: np.ndarray):
    """Return the (b, r) rows where the GPU index differs from the oracle's;
    assert that every such difference is a near-tie of the fp64 affinities."""
    idx_gpu = np.asarray(idx_gpu)
    assert idx_gpu.shape == idx_ref.shape, (idx_gpu.shape, idx_ref.shape)
    R = A.shape[-1]
    assert idx_gpu.min() >= 0 and idx_gpu.max() < R, "index out of range"
    bad = np.argwhere(np.any(idx_gpu != idx_ref, axis=-1))
    for b, r in bad:
        g, o = idx_gpu[b, r], idx_ref[b, r]
        assert len(set(g.tolist())) == len(g), f"row ({b},{r}) repeats a region: {g}"
        ag, ao = A[b, r, g], A[b, r, o]
        lim = TIE_RTOL * np.maximum(np.abs(ag), np.abs(ao))
        assert np.all(np.abs(ag - ao) <= lim), (
            f"row ({b},{r}): gpu {g} vs oracle {o}, affinities {ag} vs {ao}")
    return [tuple(x) for x in bad]


def oracle_parts(x, wl_heads, S, topk, w=None, bias=None):
    return oracle.bra_forward(x["q"], x["k"], x["v"], wl_heads, S, topk, w, bias,
                              return_parts=True)
