"""MI355X (gfx950) mixture-of-experts layer: forward and backward in HIP.

The compute lives in the HIP library libmoe_mi355x.so (C ABI: include/moe.h);
this package is its thin Python binding.  Importing the package does not load
the library; the first call does, and fails loudly if it is not built."""
from .api import (  # noqa: F401
    MoeError, make_desc, desc_from_config, route_hist_elems, workspace_bytes, grouped_gemm_workspace_bytes,
    moe_route, moe_permute, moe_grouped_gemm, moe_combine, moe_forward, moe_forward_no_workspace, moe_backward, moe_bias_update,
    moe_quantize_fp8, moe_quantize_fp8_tensorwise, moe_quantize_fp8_transposed, moe_grouped_gemm_fp8,
    moe_grouped_gemm_gather, moe_grouped_gemm_fp8_gather, moe_fp8_weights_quantize, moe_forward_fp8,
    moe_backward_fp8, alloc_fp8_weights, mfma_ceiling, hbm_ceiling, moe_quantize_fp8_colwise, quantize_fp8_colwise_bytes,
    moe_grouped_gemm_fp8_wgrad,
    alloc_saved, alloc_saved_one_buffer, alloc_grads, alloc_workspace, stage_timing, stage_times,
)
