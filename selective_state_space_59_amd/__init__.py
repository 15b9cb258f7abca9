"""MI355X-native selective-scan (Mamba-1 S6) library.

The compute path is the C-ABI HIP library libssm_hip.so (include/ssm.h); the
`ssm` module is its thin Python binding.  The library is loaded on first use
and its absence raises an error; nothing here computes on the CPU.
"""
from .ssm import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    BlockPlan,
    SSMError,
    abi_version,
    causal_conv1d_silu,
    checkpoint_shape,
    lib,
    mamba_block_fwd,
    selective_scan,
    selective_scan_bwd,
    selective_scan_args,
    selective_scan_fwd,
    selective_scan_fwd_noalloc,
    selective_scan_workspace_size,
    ssd_fwd,
    ssd_step,
    ssd_step_args,
    state_update,
    state_update_args,
    status_string,
)

__all__ = ["NOALLOC_SCRATCH_BYTES", "BlockPlan", "SSMError", "abi_version", "causal_conv1d_silu", "checkpoint_shape", "lib", "mamba_block_fwd",
           "selective_scan", "selective_scan_args", "selective_scan_bwd", "selective_scan_fwd",
           "selective_scan_fwd_noalloc", "selective_scan_workspace_size", "ssd_fwd",
           "ssd_step", "ssd_step_args", "state_update", "state_update_args", "status_string"]
