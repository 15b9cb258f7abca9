// conv1d.hip -- depthwise causal conv1d (width K <= 4) + SiLU on gfx950.
//
// The prologue of the Mamba block (paper summary page "Mamba: Linear-Time
// Sequence Modeling with Selective State Spaces", sec. 4a: Conv1d then SiLU
// ahead of the SSM; width 4 from "2. Mamba 상세", d_conv: 4):
//   u[b,t,d] = silu(sum_k w[d,k] x[b,t-(K-1)+k,d] + bias[d]),  x[t<0] = 0.
//
// HBM-bound (one read of x, one write of u).  Each lane owns one channel over
// a run of TCHUNK time steps, so a wave reads and writes 64 consecutive
// channels per step (coalesced) and keeps the 3-step history in registers;
// only the 3 steps before each run are re-read.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kConvTChunk = 64;

template <typename IO>
__global__ __launch_bounds__(256) void conv1d_silu_kernel(int64_t L, int64_t D, int K,
                                                          const void *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ bias,
                                                          void *__restrict__ u) {
    const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * kConvTChunk;
    const int64_t b = blockIdx.z;
    if (d >= D) return;
    float wp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < K; ++k) wp[4 - K + k] = w[d * K + k];
    const float cb = bias ? bias[d] : 0.0f;
    const int64_t base = b * L * D + d;
    float xm3 = 0.0f, xm2 = 0.0f, xm1 = 0.0f;
    if (t0 >= 3) xm3 = load_io<IO>(x, base + (t0 - 3) * D);
    if (t0 >= 2) xm2 = load_io<IO>(x, base + (t0 - 2) * D);
    if (t0 >= 1) xm1 = load_io<IO>(x, base + (t0 - 1) * D);
    const int64_t t1 = (t0 + kConvTChunk < L) ? t0 + kConvTChunk : L;
    for (int64_t t = t0; t < t1; ++t) {
        const float xv = load_io<IO>(x, base + t * D);
        const float v = cb + wp[0] * xm3 + wp[1] * xm2 + wp[2] * xm1 + wp[3] * xv;
        store_io<IO>(u, base + t * D, silu(v));
        xm3 = xm2;
        xm2 = xm1;
        xm1 = xv;
    }
}

}  // namespace

hipError_t launch_conv1d_silu(int64_t B, int64_t L, int64_t D, int K, int io_dtype,
                              const void *x, const float *w, const float *bias, void *u,
                              hipStream_t stream) {
    dim3 grid((unsigned)((D + 255) / 256), (unsigned)((L + kConvTChunk - 1) / kConvTChunk),
              (unsigned)B);
    if (io_dtype == SSM_BF16)
        conv1d_silu_kernel<io_bf16><<<grid, 256, 0, stream>>>(L, D, K, x, w, bias, u);
    else
        conv1d_silu_kernel<io_f32><<<grid, 256, 0, stream>>>(L, D, K, x, w, bias, u);
    return hipGetLastError();
}

}  // namespace ssm
