"""Sparse-BitLinear (W1.58A8, N:M) for AMD MI355X.

The compute path lives in libsbl.so (HIP kernels for gfx950 behind the C ABI
declared in include/sbl.h); `sbl` is its thin Python binding.  Importing the
package does not load the library: `sbl.load()` (or the first call) does.
"""

from .sbl import (SBL_FMT_DENSE2, SBL_FMT_NM, SblError, linear, load, new_backward_workspace, new_workspace,
                  quant_acts, sbl_backward_workspace_bytes,
                  quant_weights, sbl_abi_version, sbl_linear, sbl_linear_acts_batch, sbl_linear_backward,
                  sbl_linear_batch, sbl_linear_grouped, sbl_linear_kgrouped, sbl_meta_bytes,
                  sbl_linear_blocked, sbl_quant_acts_kgrouped, sbl_quant_weights_blocked,
                  sbl_quant_weights_grouped, sbl_workspace_bytes_blocked, sbl_workspace_bytes_grouped,
                  sbl_pack,
                  sbl_packed_bytes, sbl_quant_acts, sbl_quant_weights, sbl_quant_weights_batch,
                  sbl_quant_weights_batch_noalloc,
                  sbl_workspace_bytes,
                  sbl_workspace_init)

__all__ = [
    "SBL_FMT_DENSE2", "SBL_FMT_NM", "SblError", "linear", "load", "new_backward_workspace", "new_workspace",
    "quant_acts", "sbl_backward_workspace_bytes",
    "quant_weights", "sbl_abi_version", "sbl_linear", "sbl_linear_acts_batch", "sbl_linear_backward",
    "sbl_linear_batch", "sbl_linear_grouped", "sbl_linear_kgrouped", "sbl_meta_bytes",
    "sbl_linear_blocked", "sbl_quant_acts_kgrouped", "sbl_quant_weights_blocked",
    "sbl_quant_weights_grouped", "sbl_workspace_bytes_blocked", "sbl_workspace_bytes_grouped",
    "sbl_pack",
    "sbl_packed_bytes", "sbl_quant_acts", "sbl_quant_weights", "sbl_quant_weights_batch",
    "sbl_quant_weights_batch_noalloc",
    "sbl_workspace_bytes",
    "sbl_workspace_init",
]
