"""fp64 CPU oracle for the BRA forward pass -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import it.  It shares no code with the HIP library.
"""

from .bra_oracle import (  # noqa: F401
    block_forward,
    bra_backward,
    bra_forward,
    gelu,
    layer_norm,
    lepe,
    linear,
    module_forward,
    round_storage,
    region_affinity,
    region_mean,
    region_shape,
    region_token_maps,
    region_tokens,
    routed_attention,
    topk_route,
    video_forward,
    video_regions,
)
