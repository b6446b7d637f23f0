"""W4A16 INT4 mixture-of-experts expert GEMM for AMD Instinct MI355X (gfx950).

BF16 activations x INT4 weights with BF16 group-32 scales, routed through
sorted_ids / expert_ids / num_tokens_padded (indexed) or the grouped
contiguous / masked layouts; and the A4W4 variant (MXFP4 activations x
MXFP4 weights) on the same indexed routing.  The computation lives in the HIP library built
from csrc/ (C ABI: include/w4a16_moe.h); this package is its binding.
"""
from .api import (Config, MXRows, PackedW4, Routing, W4A16Error, align_capacity, config,  # noqa: F401
                  grouped_contiguous, grouped_masked, grouped_workspace_bytes, indexed_config, moe_align, moe_gate_up_silu,
                  moe_mxfp4_gate_up_silu, moe_mxfp4_gemm, moe_w4a16_gemm, mxfp4_config, mxfp4_quant,
                  mxfp4_quant_local_slots, mxfp4_select, mxfp4_weight_desc, mxfp4_workspace_bytes, pack_mxfp4, pack_w4, select,
                  weight_desc, workspace_bytes)
from ._lib import lib_path, load  # noqa: F401
