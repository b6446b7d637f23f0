"""W4A16 INT4 mixture-of-experts expert GEMM for AMD Instinct MI355X (gfx950).

BF16 activations x INT4 weights with BF16 group-32 scales, routed through
sorted_ids / expert_ids / num_tokens_padded (indexed) or the grouped
contiguous / masked layouts.  The computation lives in the HIP library built
from csrc/ (C ABI: include/w4a16_moe.h); this package is its binding.
"""
from .api import (Config, PackedW4, Routing, W4A16Error, align_capacity, config,  # noqa: F401
                  grouped_contiguous, grouped_masked, indexed_config, moe_align, moe_gate_up_silu,
                  moe_w4a16_gemm, pack_w4, select, weight_desc, workspace_bytes)
from ._lib import lib_path, load  # noqa: F401
