"""MI355X-native (gfx950) multi-scale deformable attention core.

The compute is the HIP library ``libmsda.so`` (C ABI in include/msda.h); this
package is its Python binding. Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from ._binding import (MSDA_DTYPE_BF16, MSDA_DTYPE_F16, MSDA_DTYPE_F32, MsdaError, MSDeformAttnFunction,
                       MSDeformAttnFusedFunction, dcn_output_size, library, ms_deform_attn,
                       ms_deform_attn_fused, msda_dcn_backward, msda_dcn_backward_workspace_size,
                       msda_dcn_forward,
                       msda_backward, msda_backward_fused, msda_backward_noalloc, msda_backward_fused_workspace_size,
                       msda_backward_workspace_size, msda_backward_workspace_min_size,
                       msda_check_tables, msda_forward,
                       msda_forward_fused, msda_layer_backward, msda_layer_forward,
                       msda_layer_sizes, msda_linear_backward,
                       msda_linear_backward_workspace_size, msda_linear_forward, msda_version)

__all__ = ["msda_forward", "msda_backward", "msda_backward_workspace_size", "msda_backward_noalloc", "msda_backward_workspace_min_size",
           "msda_forward_fused", "msda_backward_fused", "msda_backward_fused_workspace_size",
           "msda_linear_forward", "msda_linear_backward", "msda_linear_backward_workspace_size",
           "msda_layer_forward", "msda_layer_backward", "msda_layer_sizes",
           "msda_dcn_forward", "msda_dcn_backward", "msda_dcn_backward_workspace_size",
           "dcn_output_size", "msda_check_tables", "msda_version", "library", "ms_deform_attn",
           "MSDeformAttnFunction", "ms_deform_attn_fused", "MSDeformAttnFusedFunction",
           "MsdaError", "MSDA_DTYPE_F32", "MSDA_DTYPE_BF16", "MSDA_DTYPE_F16"]
