"""CPU oracle for MoE top-k routing, dispatch and combine.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  It shares no code with the HIP path
(``combine_topk_route_amd``) and imports nothing from it.

See ``oracle.moe`` for the definitions and the passages each one follows.
"""
from .moe import (  # noqa: F401
    bf16_to_f32,
    f32_to_bf16_rne,
    fmaf,
    route_topk,
    route_topk_grouped,
    route_topk_bruteforce,
    expert_counts,
    expert_offsets,
    rank_offsets,
    dispatch_slots,
    dispatch_slots_sequential,
    dispatch_rows,
    combine,
    combine_tokens,
    combine_exact,
    fmaf_exact,
)
from .quant import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize_rows,
    dequantize_rows,
    dispatch_rows_fp8,
)
