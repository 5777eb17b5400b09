"""CPU oracle for the W4A16 MoE layer -- test infrastructure, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""

from .moe import (  # noqa: F401
    GROUP,
    ZERO_POINT,
    bf16_to_f64,
    f64_to_bf16,
    f32_to_bf16,
    unpack_codes,
    pack_codes,
    dequant,
    dequant_f64,
    silu,
    expert_mlp,
    routed_y,
    combine,
    moe_layer,
    moe_align,
    layer_from_alignment,
    grouped_contiguous,
    grouped_masked,
    combine_rows,
    dispatch_contiguous,
    dispatch_masked,
)
