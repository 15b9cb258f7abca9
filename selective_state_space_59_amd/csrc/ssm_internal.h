// ssm_internal.h -- host-side interface between the argument-checking C ABI
// (ssm_api.cpp) and the kernel launchers (*.hip).  Launchers assume their
// arguments were validated: sizes in range, required pointers non-NULL,
// outputs not aliasing inputs, workspace large enough.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ssm.h"

namespace ssm {

// Scan: bytes of workspace the chosen launch plan needs (0 if none).
size_t scan_workspace_bytes(const ssm_scan_args_t &a);
// Scan: enqueue the kernels.  a.batch, a.seqlen > 0.
hipError_t launch_scan_fwd(const ssm_scan_args_t &a, hipStream_t stream);
// Scan checkpoints for the backward: the state entering every 16-step block,
// [ceil(L / 16)][B][D][16] fp32 at `ckpt` (a.dstate == 16), from a.x, a.delta,
// a.A, a.Bm, a.h0, the delta bias/softplus and the conv prologue; no outputs
// (a.y, a.z, a.Dskip, a.h_final and a.workspace are not used).  a.batch, a.seqlen > 0.
hipError_t launch_scan_ckpt(const ssm_scan_args_t &a, float *ckpt, hipStream_t stream);

// Device address of the no-allocation scan's scratch array
// (SSM_NOALLOC_SCRATCH_BYTES, 256-aligned) on the device of `stream`.
hipError_t noalloc_scratch(hipStream_t stream, void **out);

// Standalone conv1d + SiLU.  B, L > 0.
hipError_t launch_conv1d_silu(int64_t B, int64_t L, int64_t D, int K, int io_dtype,
                              const void *x, const float *w, const float *bias, void *u,
                              hipStream_t stream);

// Decode step.  a.batch > 0.
hipError_t launch_state_update(const ssm_state_update_args_t &a, hipStream_t stream);

// Scan backward: workspace bytes and launch (a.batch > 0; a.seqlen may be 0).
size_t scan_bwd_workspace_bytes(const ssm_scan_bwd_args_t &a);
hipError_t launch_scan_bwd(const ssm_scan_bwd_args_t &a, hipStream_t stream);

// Mamba block (block.hip).
ssm_status_t block_plan_create(const ssm_block_dims_t &d, ssm_block_plan **out);
void block_plan_destroy(ssm_block_plan *p);
size_t block_workspace_bytes(const ssm_block_plan &p);
const ssm_block_dims_t &block_dims(const ssm_block_plan &p);
hipError_t launch_block_fwd(const ssm_block_plan &p, const ssm_block_weights_t &w, const void *h_in, void *h_out,
                            void *workspace, hipStream_t stream);

// SSD (Mamba-2) layer (ssd.hip).  a.batch > 0; sizes checked by ssd_supported.
bool ssd_supported(int64_t headdim, int64_t dstate);
size_t ssd_workspace_bytes(const ssm_ssd_args_t &a);
bool ssd_step_supported(int64_t dstate);
hipError_t launch_ssd_step(const ssm_ssd_step_args_t &a, hipStream_t stream);
hipError_t launch_ssd_fwd(const ssm_ssd_args_t &a, hipStream_t stream);

// Copy or zero-fill the final state for an empty (L == 0) scan.
hipError_t launch_empty_scan_state(const ssm_scan_args_t &a, hipStream_t stream);

}  // namespace ssm
