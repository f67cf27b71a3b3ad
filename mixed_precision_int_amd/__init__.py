"""Tile-aligned W4/W8 x A8 mixed-precision linear layer for MI355X (gfx950).

The compute path is the HIP library libaq.so behind the C ABI of
include/aq.h; this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    AQ_PHASE_DECODE,
    AQ_PHASE_PREFILL,
    EXPORTS,
    LIB_PATH,
    AqError,
    AqPacked,
    AqPlan,
    PackedWeights,
    aq_abi_version,
    aq_alloc_packed,
    aq_decode_split,
    aq_labels_from_map,
    aq_act_group_shape,
    aq_linear_decode,
    aq_linear_decode_noalloc,
    AQ_DECODE_SCRATCH_BYTES,
    aq_linear_decode_grouped,
    aq_linear_prefill_grouped,
    aq_linear_tile_partials_grouped,
    aq_quant_act_grouped,
    aq_linear_prefill,
    aq_linear_prefill_prepared,
    aq_linear_prefill_transformed,
    aq_prefill_prepare,
    aq_linear_tile_partials,
    aq_pack_weights,
    aq_plan_pack,
    aq_quant_act,
    aq_quant_act_transformed,
    aq_transform_out,
    aq_transform_rows,
    aq_transform_weights,
    aq_workspace_bytes,
    AqTransformTables,
    lib,
    transform_tables,
)
