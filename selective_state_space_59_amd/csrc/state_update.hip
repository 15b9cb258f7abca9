// state_update.hip -- one decode step of the selective SSM on gfx950.
//
// The recurrent mode of eq. (2a)/(2b) on the paper summary page "Mamba:
// Linear-Time Sequence Modeling with Selective State Spaces" (sec. 4b), with
// the ZOH of eq. (4), the skip of "14.1 SSM(State Space Models)과 Mamba
// 아키텍처의 부상" sec. 3.1 and the SiLU gate of sec. 4a, on a state kept
// between tokens ("2. Mamba 상세": ssm_state):
//   state[b,d,n] <- exp(dt A) state + Bbar x;   y = (sum_n C state + D x) silu(z)
//
// HBM-bound: the fp32 state is read and written once.  Four lanes share one
// channel, each holding four consecutive state entries, so a wave streams 16
// channels x 64 bytes of state contiguously; the four partial read-outs are
// summed with two cross-lane butterflies.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kLanesPerChannel = 4;
constexpr int kPerLane = SSM_MAX_DSTATE / kLanesPerChannel;  // 4 state entries per lane

struct UpdateParams {
    int64_t B, D;
    int N, softplus;
    float *state;
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *Dskip, *dbias;
    void *y;
};

template <typename IO, bool VEC>
__global__ __launch_bounds__(256) void state_update_kernel(UpdateParams p) {
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ch = gtid / kLanesPerChannel;  // b * D + d
    const int j = (int)(gtid % kLanesPerChannel);
    const bool live = ch < p.B * p.D;
    const int64_t chc = live ? ch : 0;
    const int64_t b = chc / p.D, d = chc % p.D;
    const int N = p.N;
    const int n0 = j * kPerLane;

    float dt = load_io<IO>(p.delta, chc);
    if (p.softplus) dt = softplus(dt + (p.dbias ? p.dbias[d] : 0.0f));
    const float u = load_io<IO>(p.x, chc);

    float hs[kPerLane];
    float* sp = p.state + chc * N + n0;
    if (VEC) {
        const float4 v = *reinterpret_cast<const float4 *>(sp);
        hs[0] = v.x; hs[1] = v.y; hs[2] = v.z; hs[3] = v.w;
    } else {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) hs[k] = (n0 + k < N) ? sp[k] : 0.0f;
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int n = n0 + k;
        if (VEC || n < N) {
            const float a = p.A[d * N + n];
            const float bn = load_io<IO>(p.Bm, b * N + n);
            const float cn = load_io<IO>(p.Cm, b * N + n);
            const float e = hw_exp2(dt * a * kLog2e);
            const float coef = (a == 0.0f) ? dt : (e - 1.0f) / a;
            hs[k] = e * hs[k] + coef * (bn * u);
            acc += cn * hs[k];
        }
    }
    if (live) {
        if (VEC) {
            *reinterpret_cast<float4 *>(sp) = make_float4(hs[0], hs[1], hs[2], hs[3]);
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k)
                if (n0 + k < N) sp[k] = hs[k];
        }
    }
    // Sum the four partial read-outs of the channel (lanes 4c..4c+3).
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (live && j == 0) {
        float yv = acc + (p.Dskip ? p.Dskip[d] * u : 0.0f);
        if (p.z) yv *= silu(load_io<IO>(p.z, chc));
        store_io<IO>(p.y, chc, yv);
    }
}

template <typename IO>
hipError_t launch_typed(const UpdateParams &p, bool vec, hipStream_t stream) {
    const int64_t threads = p.B * p.D * kLanesPerChannel;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (vec)
        state_update_kernel<IO, true><<<blocks, 256, 0, stream>>>(p);
    else
        state_update_kernel<IO, false><<<blocks, 256, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const ssm_state_update_args_t &a, hipStream_t stream) {
    UpdateParams p;
    p.B = a.batch;
    p.D = a.dim;
    p.N = (int)a.dstate;
    p.softplus = a.delta_softplus;
    p.state = a.state;
    p.x = a.x;
    p.delta = a.delta;
    p.z = a.z;
    p.Bm = a.Bm;
    p.Cm = a.Cm;
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.y = a.y;
    // Whole float4 rows need N == 16 and a 16-byte aligned state.
    const bool vec = (a.dstate == SSM_MAX_DSTATE) && ((uintptr_t)a.state % 16 == 0);
    if (a.io_dtype == SSM_BF16) return launch_typed<io_bf16>(p, vec, stream);
    return launch_typed<io_f32>(p, vec, stream);
}

}  // namespace ssm
