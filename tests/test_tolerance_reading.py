"""Why the bf16 parity check grants half an ulp of the output format (CPU).

The contract asks for max-abs error <= 2e-2 * RMS(out) on bf16 workloads.
On the stage-1 workload, rounding the oracle's own exact fp64 output to
bfloat16 -- the best answer any bf16 output can hold -- already exceeds that,
because a few outputs are more than 10x the RMS and bf16 keeps 8 bits.  The
GPU tests therefore measure the error beyond that unavoidable rounding."""

import numpy as np

import oracle
from gpu_util import bf16_half_ulp, excess_err, rel_err
from vision_transformer_dynamic_region_amd.workloads import WORKLOADS, bf16_round, make_inputs


def test_rounding_the_exact_answer_breaks_the_raw_bound():
    wl = WORKLOADS["st1"]
    x = make_inputs(wl)
    O = oracle.bra_forward(x["q"], x["k"], x["v"], wl.heads, wl.S, wl.topk,
                           return_parts=True)["O"]
    best = bf16_round(O.astype(np.float32)).astype(np.float64)
    assert rel_err(best, O) > 2e-2            # the raw bound fails for a perfect result
    # and is met once the half-ulp is granted (the float32 step on the way to
    # bf16 can add a few 1e-8 of rounding)
    assert excess_err(best, O, "bf16") < 1e-6
    assert np.all(np.abs(best - O) <= bf16_half_ulp(O) * (1 + 1e-4))


def test_excess_error_still_catches_real_errors():
    r = np.random.default_rng(0)
    ref = r.normal(size=10000)
    got = bf16_round(ref.astype(np.float32)).astype(np.float64)
    assert excess_err(got, ref, "bf16") == 0.0
    got[17] += 0.05 * np.sqrt(np.mean(ref ** 2))   # one element off by 5% of RMS
    assert excess_err(got, ref, "bf16") > 2e-2
    assert excess_err(ref * (1 + 1e-3), ref, "f32") > 1e-4
