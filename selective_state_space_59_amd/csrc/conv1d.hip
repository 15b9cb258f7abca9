// conv1d.hip -- depthwise causal conv1d (width K <= 4) + SiLU on gfx950.
//
// The prologue of the Mamba block (paper summary page "Mamba: Linear-Time
// Sequence Modeling with Selective State Spaces", sec. 4a: Conv1d then SiLU
// ahead of the SSM; width 4 from "2. Mamba 상세", d_conv: 4):
//   u[b,t,d] = silu(sum_k w[d,k] x[b,t-(K-1)+k,d] + bias[d]),  x[t<0] = 0.
//
// HBM-bound (one read of x, one write of u).  Each lane owns one channel (or,
// in the wide form, one 16-byte group of channels) over a run of time steps,
// so a wave reads and writes consecutive channels per step (coalesced) and
// keeps the 3-step history in registers; only the 3 steps before each run are
// re-read.
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

// Wide form: each lane owns V = 16 / sizeof(element) consecutive channels
// (one 16-byte load and store per time step) over a run of kConvVecT steps.
// It issues the loads of all kConvVecT + 3 rows it needs at once (a single
// memory round trip), then runs the steps as straight-line code; the taps are
// a template argument, so nothing in the loop branches.  Lanes are numbered
// channel-group fastest, so a wave's loads cover 1 KiB of one row.
constexpr int kConvVecT = 16;

template <typename IO>
__device__ __forceinline__ void unpack16(const uint4 &q, float (&v)[16 / IO::bytes]) {
    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
    if constexpr (IO::bytes == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(wv[i] << 16);
            v[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(wv[i]);
    }
}

template <typename IO>
__device__ __forceinline__ uint4 pack16(const float (&v)[16 / IO::bytes]) {
    uint32_t wv[4];
    if constexpr (IO::bytes == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[i] = __float_as_uint(v[i]);
    }
    return make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

template <typename IO, int K>
__global__ __launch_bounds__(256) void conv1d_silu_vec_kernel(int64_t L, int64_t D, int64_t nchunks,
                                                              int64_t total, const void *__restrict__ x,
                                                              const float *__restrict__ w,
                                                              const float *__restrict__ bias,
                                                              void *__restrict__ u) {
    constexpr int V = 16 / IO::bytes;
    constexpr int R = kConvVecT + 3;  // rows t0-3 .. t0+kConvVecT-1
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int64_t DV = D / V;
    const int64_t dv = gid % DV;
    const int64_t rest = gid / DV;
    const int64_t t0 = (rest % nchunks) * kConvVecT;
    const int64_t b = rest / nchunks;
    const int64_t d0 = dv * V;
    const char *xb = static_cast<const char *>(x) + ((b * L) * D + d0) * IO::bytes;
    char *ub = static_cast<char *>(u) + ((b * L) * D + d0) * IO::bytes;
    const int64_t row = D * IO::bytes;
    uint4 q[R];
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int64_t t = t0 - 3 + s;
        q[s] = (t >= 0 && t < L) ? *reinterpret_cast<const uint4 *>(xb + t * row) : make_uint4(0, 0, 0, 0);
    }
    float wk[K][V], cb[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) wk[k][i] = w[(d0 + i) * K + k];
        cb[i] = bias ? bias[d0 + i] : 0.0f;
    }
    // win[j] holds x at time t-(K-1)+j for the current step t
    float win[K][V];
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) unpack16<IO>(q[3 - (K - 1) + j], win[j + 1]);
#pragma unroll
    for (int s = 0; s < kConvVecT; ++s) {
#pragma unroll
        for (int j = 0; j + 1 < K; ++j)
#pragma unroll
            for (int i = 0; i < V; ++i) win[j][i] = win[j + 1][i];
        unpack16<IO>(q[3 + s], win[K - 1]);
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float v = cb[i];
#pragma unroll
            for (int k = 0; k < K; ++k) v = __builtin_fmaf(wk[k][i], win[k][i], v);
            o[i] = silu(v);
        }
        if (t0 + s < L) *reinterpret_cast<uint4 *>(ub + (t0 + s) * row) = pack16<IO>(o);
    }
}

template <typename IO>
void launch_conv_vec(int64_t B, int64_t L, int64_t D, int K, const void *x, const float *w, const float *bias,
                     void *u, hipStream_t stream) {
    constexpr int V = 16 / IO::bytes;
    const int64_t nchunks = (L + kConvVecT - 1) / kConvVecT;
    const int64_t total = B * nchunks * (D / V);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    switch (K) {
        case 1: conv1d_silu_vec_kernel<IO, 1><<<blocks, 256, 0, stream>>>(L, D, nchunks, total, x, w, bias, u); break;
        case 2: conv1d_silu_vec_kernel<IO, 2><<<blocks, 256, 0, stream>>>(L, D, nchunks, total, x, w, bias, u); break;
        case 3: conv1d_silu_vec_kernel<IO, 3><<<blocks, 256, 0, stream>>>(L, D, nchunks, total, x, w, bias, u); break;
        default: conv1d_silu_vec_kernel<IO, 4><<<blocks, 256, 0, stream>>>(L, D, nchunks, total, x, w, bias, u); break;
    }
}

}  // namespace

hipError_t launch_conv1d_silu(int64_t B, int64_t L, int64_t D, int K, int io_dtype,
                              const void *x, const float *w, const float *bias, void *u,
                              hipStream_t stream) {
    const int64_t es = io_dtype == SSM_BF16 ? 2 : 4, V = 16 / es;
    auto al = [](const void *v) { return ((uintptr_t)v % 16) == 0; };
    if (D % V == 0 && al(x) && al(u)) {
        if (io_dtype == SSM_BF16)
            launch_conv_vec<io_bf16>(B, L, D, K, x, w, bias, u, stream);
        else
            launch_conv_vec<io_f32>(B, L, D, K, x, w, bias, u, stream);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((D + 255) / 256), (unsigned)((L + kConvTChunk - 1) / kConvTChunk),
              (unsigned)B);
    if (io_dtype == SSM_BF16)
        conv1d_silu_kernel<io_bf16><<<grid, 256, 0, stream>>>(L, D, K, x, w, bias, u);
    else
        conv1d_silu_kernel<io_f32><<<grid, 256, 0, stream>>>(L, D, K, x, w, bias, u);
    return hipGetLastError();
}

}  // namespace ssm
