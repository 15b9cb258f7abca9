// state_update.hip -- one decode step of the selective SSM on gfx950.
//
// The recurrent mode of eq. (2a)/(2b) on the paper summary page "Mamba:
// Linear-Time Sequence Modeling with Selective State Spaces" (sec. 4b), with
// the ZOH of eq. (4), the skip of "14.1 SSM(State Space Models)과 Mamba
// 아키텍처의 부상" sec. 3.1 and the SiLU gate of sec. 4a, on a state kept
// between tokens ("2. Mamba 상세": ssm_state):
//   state[b,d,n] <- exp(dt A) state + Bbar u;   y = (sum_n C state + D u) silu(z)
// with u = x, or, with a conv state (the last K-1 inputs of each channel),
// the causal conv1d + SiLU prologue of sec. 4a on (window, x); the window
// then drops its oldest input and appends x.
//
// HBM-bound: the fp32 state is read and written once; everything else is
// small (x, delta, z, y per channel; B, C per batch row; A and D per channel,
// shared by all batch rows and so served from the caches).  Four lanes share
// one channel, each holding four consecutive state entries, so a wave moves
// 16 channels x 64 bytes of state with one 16-byte access per lane.  A
// workgroup takes 128 channels of one batch row (so the row's B and C are the
// same for all of it) as two rounds of 64, and each thread issues the loads of
// both its quarters before any arithmetic.  The state is streamed with
// non-temporal loads and stores (it is touched once per step).  The four
// partial read-outs of a channel are summed with two DPP quad swaps.
//
// Bbar x: in waves where every |A| >= 1/16, (e^{dt A} - 1) (B x) / A with an
// approximate reciprocal; otherwise dt phi(dt A) B x with
// phi(z) = (e^z - 1) / z, evaluated as a degree-6 series for |z| < 1/4 (no
// cancellation, and phi(0) = 1 covers A = 0) and as (e^z - 1) / z beyond.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kLanesPerChannel = 4;
constexpr int kPerLane = SSM_MAX_DSTATE / kLanesPerChannel;  // 4 state entries per lane
constexpr int kRounds = 2;                                  // quarters per thread
constexpr int kTileChannels = kRounds * 256 / kLanesPerChannel;  // channels per workgroup
constexpr int64_t kMaxGrid = (int64_t)1 << 22;

struct UpdateParams {
    int64_t B, D;
    int N, softplus, K;
    float *state;
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *Dskip, *dbias, *conv_w, *conv_b;
    void *cs;  // conv state (B, K-1, D), io type
    void *y;
};

// Conv prologue of channel (b, d), spread over the 4 lanes of its quad
// (lane j = quarter index): with the taps right-aligned to width 4, lane j
// holds tap j and input j, where input 3 is the current x and input j < 3
// the one 3-j steps back (window row K-4+j; taps and rows below 0 are 0).
// A quad sum gives every lane the conv output; the window shifts by one
// with a quad permute (lane j takes lane j+1's input) and lanes 0..2 store
// their rows.
struct ConvLane {
    float tap, win, bias;
};
// `win_b` is the window of batch row b (the (K-1, D) slab at b (K-1) D); the
// offsets within it, and within conv_w, fit 32 bits (checked at launch).  The
// window is touched once per step, like the state: non-temporal loads and
// stores.
template <typename IO>
__device__ __forceinline__ ConvLane load_conv(const UpdateParams &p, const char *win_b, int d, int j) {
    constexpr int es = sizeof(typename IO::storage);
    const int r = p.K - 4 + j;  // tap index = window row of this lane
    ConvLane c;
    c.tap = r >= 0 ? p.conv_w[d * p.K + r] : 0.0f;
    c.win = 0.0f;
    if (j < 3 && r >= 0) {
        const char *q = win_b + (uint32_t)(r * (int)p.D + d) * es;
        if constexpr (es == 2) c.win = __uint_as_float((uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(q)) << 16);
        else c.win = __builtin_nontemporal_load(reinterpret_cast<const float *>(q));
    }
    c.bias = (j == 3 && p.conv_b) ? p.conv_b[d] : 0.0f;
    return c;
}
// Lane j's input: the window entry, or x on lane 3.
__device__ __forceinline__ float conv_in(const ConvLane &c, int j, float x) { return j == 3 ? x : c.win; }
__device__ __forceinline__ float quad_sum(float v);
__device__ __forceinline__ float conv_u(const ConvLane &c, float v) {
    return silu(quad_sum(__builtin_fmaf(c.tap, v, c.bias)));
}
// New window row of lane j (j < 3): lane j+1's input (exact: the values came
// from I/O elements).  Every lane of the quad must call this.
__device__ __forceinline__ float conv_shift(float v) {
    return __builtin_amdgcn_update_dpp(0.0f, v, 0xF9, 0xf, 0xf, false);  // quad_perm [1,2,3,3]
}
template <typename IO>
__device__ __forceinline__ void store_window(const UpdateParams &p, char *win_b, int d, int j, float nv) {
    constexpr int es = sizeof(typename IO::storage);
    const int r = p.K - 4 + j;
    if (j < 3 && r >= 0) {
        char *q = win_b + (uint32_t)(r * (int)p.D + d) * es;
        if constexpr (es == 2) __builtin_nontemporal_store(f32_to_bf16_bits(nv), reinterpret_cast<uint16_t *>(q));
        else __builtin_nontemporal_store(nv, reinterpret_cast<float *>(q));
    }
}

// phi(z) = (e^z - 1) / z given e = e^z.
__device__ __forceinline__ float phi_of(float z, float e) {
    const float s = 1.0f + z * (0.5f + z * (1.0f / 6.0f + z * (1.0f / 24.0f +
                    z * (1.0f / 120.0f + z * (1.0f / 720.0f + z * (1.0f / 5040.0f))))));
    const float big = (e - 1.0f) * hw_rcp(z);
    return fabsf(z) < 0.25f ? s : big;
}

// Four consecutive I/O elements as fp32.
template <typename IO>
__device__ __forceinline__ float4 load4_io(const void *p, int64_t i);
template <>
__device__ __forceinline__ float4 load4_io<io_f32>(const void *p, int64_t i) {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
}
template <>
__device__ __forceinline__ float4 load4_io<io_bf16>(const void *p, int64_t i) {
    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    return v;
}

// N = 16 with 16-byte aligned state, A, B and C.  Tile t = (batch row b,
// channel run): round r gives lane l channel d = run * 128 + r * 64 + l / 4
// and entries 4 (l % 4) .. +3 of it.
template <typename IO, bool CONV>
__device__ __forceinline__ void state_update_tile(const UpdateParams &p, int64_t t, int64_t ntiles) {
    constexpr int R = kRounds;
    const int64_t b = t / ntiles;
    const int64_t run = t - b * ntiles;
    const int jq = (int)(threadIdx.x & 3);
    const int dl = (int)(threadIdx.x >> 2);
    float4 st[R], av[R];
    float xv[R], dv[R], zv[R], dsk[R];
    ConvLane cin[R];
    int64_t dd[R];
    constexpr int es = sizeof(typename IO::storage);
    char *win_b = CONV ? static_cast<char *>(p.cs) + b * (p.K - 1) * p.D * es : nullptr;
    // All loads first.
#pragma unroll
    for (int r = 0; r < R; ++r) {
        dd[r] = run * kTileChannels + r * (256 / kLanesPerChannel) + dl;
        const int64_t dc = dd[r] < p.D ? dd[r] : 0;
        const int64_t ch = b * p.D + dc;
        {
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p.state + ch * SSM_MAX_DSTATE + 4 * jq));
            st[r] = make_float4(v.x, v.y, v.z, v.w);
        }
        av[r] = *reinterpret_cast<const float4 *>(p.A + dc * SSM_MAX_DSTATE + 4 * jq);
        xv[r] = load_io<IO>(p.x, ch);
        dv[r] = load_io<IO>(p.delta, ch);
        zv[r] = p.z ? load_io<IO>(p.z, ch) : 0.0f;
        dsk[r] = p.Dskip ? p.Dskip[dc] : 0.0f;
        if (p.softplus) dv[r] = softplus(dv[r] + (p.dbias ? p.dbias[dc] : 0.0f));
        if (CONV) cin[r] = load_conv<IO>(p, win_b, (int)dc, jq);
    }
    const float4 bv = load4_io<IO>(p.Bm, b * SSM_MAX_DSTATE + 4 * jq);
    const float4 cv = load4_io<IO>(p.Cm, b * SSM_MAX_DSTATE + 4 * jq);
    bool big = true;
#pragma unroll
    for (int r = 0; r < R; ++r)
        big = big && fabsf(av[r].x) >= 0.0625f && fabsf(av[r].y) >= 0.0625f &&
              fabsf(av[r].z) >= 0.0625f && fabsf(av[r].w) >= 0.0625f;
    const bool fast = __all(big);
    const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
    const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool live = dd[r] < p.D;
        const int64_t ch = b * p.D + (live ? dd[r] : 0);
        const float dt = dv[r];
        const float vin = CONV ? conv_in(cin[r], jq, xv[r]) : 0.0f;
        const float u = CONV ? conv_u(cin[r], vin) : xv[r];
        const float nwin = CONV ? conv_shift(vin) : 0.0f;
        const float a[4] = {av[r].x, av[r].y, av[r].z, av[r].w};
        float h[4] = {st[r].x, st[r].y, st[r].z, st[r].w};
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float zz = dt * a[i];
            const float e = hw_exp2(zz * kLog2e);
            if (fast) {
                const float qq = (bb[i] * u) * hw_rcp(a[i]);
                h[i] = __builtin_fmaf(e, h[i], __builtin_fmaf(e, qq, -qq));
            } else {
                h[i] = e * h[i] + (dt * phi_of(zz, e)) * (bb[i] * u);
            }
            acc += cc[i] * h[i];
        }
        if (live) {
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v v = {h[0], h[1], h[2], h[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f4v *>(p.state + ch * SSM_MAX_DSTATE + 4 * jq));
        }
        acc = quad_sum(acc);
        // The window was read above by every lane of the quad (loads first).
        if (CONV && live && p.K > 1) store_window<IO>(p, win_b, (int)dd[r], jq, nwin);
        if (live && jq == 0) {
            float yv = acc + dsk[r] * u;
            if (p.z) yv *= silu(zv[r]);
            store_io<IO>(p.y, ch, yv);
        }
    }
}

// One tile per workgroup; a loop over tiles only where they outnumber one
// grid (the loop costs time even when it runs once).
// CONV: the conv prologue runs on the window (conv_k > 0), a compile-time
// choice so that neither path carries the other's branches.
template <typename IO, bool LOOP, bool CONV>
__global__ __launch_bounds__(256) void state_update_vec_kernel(UpdateParams p, int64_t ntiles, int64_t total) {
    if (!LOOP) {
        state_update_tile<IO, CONV>(p, blockIdx.x, ntiles);
        return;
    }
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) state_update_tile<IO, CONV>(p, t, ntiles);
}

// Any N <= 16 and any alignment: one quarter per thread, element loads.
template <typename IO>
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
    const float xin = load_io<IO>(p.x, chc);
    ConvLane cin{0.0f, 0.0f, 0.0f};
    constexpr int es = sizeof(typename IO::storage);
    char *win_b = p.K > 0 ? static_cast<char *>(p.cs) + b * (p.K - 1) * p.D * es : nullptr;
    if (p.K > 0) cin = load_conv<IO>(p, win_b, (int)d, j);
    const float vin = p.K > 0 ? conv_in(cin, j, xin) : 0.0f;
    const float u = p.K > 0 ? conv_u(cin, vin) : xin;
    const float nwin = p.K > 1 ? conv_shift(vin) : 0.0f;

    float hs[kPerLane];
    float *sp = p.state + chc * N + n0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) hs[k] = (n0 + k < N) ? sp[k] : 0.0f;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        const int n = n0 + k;
        if (n < N) {
            const float a = p.A[d * N + n];
            const float bn = load_io<IO>(p.Bm, b * N + n);
            const float cn = load_io<IO>(p.Cm, b * N + n);
            const float zz = dt * a;
            const float e = hw_exp2(zz * kLog2e);
            hs[k] = e * hs[k] + (dt * phi_of(zz, e)) * (bn * u);
            acc += cn * hs[k];
        }
    }
    if (live) {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k)
            if (n0 + k < N) sp[k] = hs[k];
    }
    acc = quad_sum(acc);
    if (live && p.K > 1) store_window<IO>(p, win_b, (int)d, j, nwin);
    if (live && j == 0) {
        float yv = acc + (p.Dskip ? p.Dskip[d] * u : 0.0f);
        if (p.z) yv *= silu(load_io<IO>(p.z, chc));
        store_io<IO>(p.y, chc, yv);
    }
}

template <typename IO>
hipError_t launch_typed(const UpdateParams &p, bool vec, hipStream_t stream) {
    const int64_t nq = p.B * p.D * kLanesPerChannel;
    if (vec) {
        const int64_t ntiles = (p.D + kTileChannels - 1) / kTileChannels;
        const int64_t total = p.B * ntiles;
        const unsigned grid = (unsigned)(total <= kMaxGrid ? total : kMaxGrid);
        if (total <= kMaxGrid) {
            if (p.K > 0) state_update_vec_kernel<IO, false, true><<<grid, 256, 0, stream>>>(p, ntiles, total);
            else state_update_vec_kernel<IO, false, false><<<grid, 256, 0, stream>>>(p, ntiles, total);
        } else {
            if (p.K > 0) state_update_vec_kernel<IO, true, true><<<grid, 256, 0, stream>>>(p, ntiles, total);
            else state_update_vec_kernel<IO, true, false><<<grid, 256, 0, stream>>>(p, ntiles, total);
        }
    } else {
        const unsigned blocks = (unsigned)((nq + 255) / 256);
        state_update_kernel<IO><<<blocks, 256, 0, stream>>>(p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const ssm_state_update_args_t &a, hipStream_t stream) {
    UpdateParams p;
    p.B = a.batch;
    p.D = a.dim;
    p.N = (int)a.dstate;
    p.softplus = a.delta_softplus;
    p.K = (int)a.conv_k;
    p.conv_w = a.conv_w;
    p.conv_b = a.conv_b;
    p.cs = a.conv_state;
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
    // Whole 16-byte quarters need N == 16 and aligned state, A, B and C
    // (B and C rows are 8 bytes per quarter in bf16, 16 in fp32).
    const size_t bc_align = a.io_dtype == SSM_BF16 ? 8 : 16;
    const bool vec = a.dstate == SSM_MAX_DSTATE && (uintptr_t)a.state % 16 == 0 &&
                     (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.Bm % bc_align == 0 &&
                     (uintptr_t)a.Cm % bc_align == 0;
    if (a.io_dtype == SSM_BF16) return launch_typed<io_bf16>(p, vec, stream);
    return launch_typed<io_f32>(p, vec, stream);
}

}  // namespace ssm
