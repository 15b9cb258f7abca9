// scan_bwd.hip -- backward pass of the selective scan (S6) on gfx950.
//
// Gradients of the forward of "Mamba: Linear-Time Sequence Modeling with
// Selective State Spaces" (paper summary page, sec. 4b eq. (4) and (2a)/(2b),
// Algorithm 2, the block of sec. 4a) for a loss with dL/dy = dy and
// dL/dh_final = dh_final.  The page's backward recomputes the states instead
// of storing them (sec. 4c); here:
//   1. a checkpoint pass runs the recurrence forward and stores only the
//      state entering every 16-step block (1/16 of the expanded states): the
//      forward scan kernel's checkpoint variant (launch_scan_ckpt), with its
//      workgroup-staged loads and no read-out.  In training the forward
//      writes them beside y instead, and this pass is skipped;
//   2. the backward kernel walks the blocks from last to first.  Per block it
//      re-runs the 16 steps from the checkpoint, keeping h_{t-1} and
//      exp(dt A) in registers, and then runs the adjoint recurrence
//        lambda_t = C_t gy_t + exp(dt_{t+1} A) lambda_{t+1},  gy = dy silu(z)
//      backwards through them.
//
// Lane layout as in the forward: lane (c, n) of a wave owns state entry n of
// channel c (4 channels per wave, N = 16).  Sums over the 16 entries (the
// read-out C h for dz, and du and ddelta) are transposed through a wave-
// private LDS area so that lane (c, k) sums step k.  dB and dC are sums over
// channels: each workgroup adds its channels in LDS and stores one partial
// per (batch, workgroup, step, entry); a reduction kernel adds the partials of
// the workgroups of a batch row.  dA, dD and the delta bias gradient are
// summed over time per lane and over batch rows by the same reduction.
//
// Derivatives used (B_bar = B (e - 1)/A = dt phi(dt A) B, e = exp(dt A)):
//   d e / d dt = A e,   d B_bar / d dt = B e,   d B_bar / d A = B dt^2 psi(dt A),
//   psi(z) = phi'(z) = (e^z (z - 1) + 1) / z^2 (series near 0).
#include "ssm_device.h"
#include "ssm_internal.h"

#include <algorithm>
#include <utility>

namespace ssm {
namespace {

constexpr int kRowN = 16;            // lanes per row = state entries (N = 16)
constexpr int kStep = 16;            // steps per block
constexpr int kWavesB = 12;          // waves per workgroup (3 per SIMD)
constexpr int kChB = 4 * kWavesB;    // channels per workgroup
// Transpose area of one channel: [16 entries][kTS steps], then padding so
// that the 4 channel areas of a wave start 16 banks apart (336 = 16 mod 32).
constexpr int kTS = kStep + 4;
constexpr int kChArea = kRowN * kTS + 16;
constexpr int kTrWave = 4 * kChArea;          // floats per wave and transpose area
constexpr int kRedWave = 2 * kRowN * kTS;     // per wave: [dB|dC][16 entries][kTS steps]

struct BwdParams {
    int64_t B, L, D, G;              // G: workgroups per batch row
    int softplus;
    int K;                           // conv prologue width, 0 for none
    const float *conv_w, *conv_b;
    const void *cs_in;               // [B][K-1][D] x before t = 0, or NULL (= 0)
    void *dcs;                       // [B][K-1][D] its gradient, or NULL
    float *dU;                       // [B][L][D] dL/du when K > 0 (then dx comes from conv_bwd)
    const void *x, *delta, *Bm, *Cm, *z, *dy;
    const float *A, *Dskip, *dbias, *h0, *dh_final;
    void *dx, *ddelta, *dz;
    float *dh0;
    float *ckpt;      // [nblocks][B][D][16]   state entering each block
    float *partBC;    // [2][B][G][L][16]      per-workgroup sums of dB, dC
    float *partA;     // [B][D][16]
    float *partD;     // [B][D]
    float *partBias;  // [B][D]
};

template <int I>
using icb = std::integral_constant<int, I>;
template <typename F, int... Is>
__device__ __forceinline__ void sfor_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(icb<Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sfor(F &&f) {
    sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// Value of lane K of this lane's 16-lane row (row_newbcast: every lane has a
// source, so no old value is needed and bound_ctrl lets the compiler skip one).
template <int K>
__device__ __forceinline__ float bcast_row(float v) {
    return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + K, 0xf, 0xf, true);
}

// phi(z) = (e^z - 1)/z and psi(z) = phi'(z) = (e^z - phi(z))/z given e = e^z
// and r = 1/z: degree-6 series below |z| = 1/4 (no cancellation), the
// quotients beyond (hardware reciprocal, no division).
__device__ __forceinline__ float phi_f(float zz, float e, float r) {
    const float s = 1.0f + zz * (0.5f + zz * (1.0f / 6.0f + zz * (1.0f / 24.0f +
                    zz * (1.0f / 120.0f + zz * (1.0f / 720.0f + zz * (1.0f / 5040.0f))))));
    return fabsf(zz) < 0.25f ? s : (e - 1.0f) * r;
}
__device__ __forceinline__ float psi_f(float zz, float e, float ph, float r) {
    const float s = 0.5f + zz * (1.0f / 3.0f + zz * (1.0f / 8.0f + zz * (1.0f / 30.0f +
                    zz * (1.0f / 144.0f + zz * (1.0f / 840.0f + zz * (1.0f / 5760.0f))))));
    return fabsf(zz) < 0.25f ? s : (e - ph) * r;
}
__device__ __forceinline__ float sigmoid_f(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }
__device__ __forceinline__ float dsilu_f(float v) {
    const float s = sigmoid_f(v);
    return s * (1.0f + v * (1.0f - s));
}

// Lane setup shared by both kernels.
struct LaneB {
    int64_t b, d;
    int n, c, wave;
    bool valid;
};
__device__ __forceinline__ LaneB lane_setup(const BwdParams &p) {
    LaneB l;
    const int lane = threadIdx.x & 63;
    l.wave = threadIdx.x >> 6;
    l.n = lane & 15;
    l.c = lane >> 4;
    const int64_t g = blockIdx.x;
    l.b = g / p.G;
    l.d = (g % p.G) * kChB + 4 * l.wave + l.c;
    l.valid = l.d < p.D;
    return l;
}

// dt phi(dt A) = (e - 1)/A: in waves where every |A| >= 1/16 (FAST) as
// e/A - 1/A in one fma, otherwise through phi (series near 0).
template <bool FAST>
__device__ __forceinline__ float dtphi(float dt, float a, float ia, float e) {
    if (FAST) return __builtin_fmaf(e, ia, -ia);
    const float zz = dt * a;
    return dt * phi_f(zz, e, hw_rcp(zz));
}

// Raw I/O bits, loaded now and widened later, so that a load can be issued a
// block before its value is used (widening at once would wait for it).
template <typename IO>
__device__ __forceinline__ uint32_t load_bits(const void *p, int64_t i) {
    if constexpr (sizeof(typename IO::storage) == 2) return static_cast<const uint16_t *>(p)[i];
    else return __float_as_uint(static_cast<const float *>(p)[i]);
}
template <typename IO>
__device__ __forceinline__ float bits_f32(uint32_t v) {
    if constexpr (sizeof(typename IO::storage) == 2) return __uint_as_float(v << 16);
    else return __uint_as_float(v);
}

// The own-step inputs of lane (c, n) at step t as raw bits: x at t-3 .. t
// (only x_t without a conv prologue) and delta.  Indices are clamped into the
// tensors and the lanes and window slots outside them are masked when the
// values are used, so no load sits in a branch.
struct OwnRaw {
    uint32_t xr[4];
    uint32_t draw;
    int wm;  // bit j: x_{t-3+j} exists (all 0 for a lane or step outside the tensors)
};
template <typename IO, bool CONV>
__device__ __forceinline__ OwnRaw own_raw(const BwdParams &p, const LaneB &l, int64_t t) {
    OwnRaw r;
    const bool live = l.valid && t < p.L;
    const int64_t tc = live ? t : 0, dc = l.valid ? l.d : 0;
    const int64_t i = (l.b * p.L + tc) * p.D + dc;
    r.xr[3] = load_bits<IO>(p.x, i);
    r.draw = load_bits<IO>(p.delta, i);
    r.wm = live ? 8 : 0;
    r.xr[0] = r.xr[1] = r.xr[2] = 0u;
    if (CONV) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            // before t = 0 the input comes from the entering conv state (the K-1
            // steps before the sequence) or is 0: then the clamped index is step
            // 0's and the slot is masked below
            const int64_t s = tc - 3 + j;
            const bool in = s >= 0;
            const bool hist = !in && p.cs_in != nullptr && s >= -(int64_t)(p.K - 1);
            const void *src = hist ? p.cs_in : p.x;
            const int64_t idx = in ? (l.b * p.L + s) * p.D + dc
                                   : hist ? (l.b * (p.K - 1) + (p.K - 1) + s) * p.D + dc : l.b * p.L * p.D + dc;
            r.xr[j] = load_bits<IO>(src, idx);
            r.wm |= (live && (in || hist)) ? (1 << j) : 0;
        }
    }
    return r;
}
// u and dt from the raw inputs; wr = the conv taps right-aligned to width 4
// (wr[3] weighs x_t; taps past K are 0).
template <typename IO, bool CONV>
__device__ __forceinline__ void own_finish(const BwdParams &p, const OwnRaw &r, const float (&wr)[4], float cb,
                                           float bias, float &u, float &dt) {
    float xw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xw[j] = (r.wm >> j) & 1 ? bits_f32<IO>(r.xr[j]) : 0.0f;
    u = xw[3];
    if (CONV) {
        float c = cb;
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_fmaf(wr[j], xw[j], c);
        u = r.wm ? silu(c) : 0.0f;
    }
    const float raw = r.wm ? bits_f32<IO>(r.draw) : 0.0f;
    dt = p.softplus ? softplus_fast(raw + bias) : raw;  // the forward's softplus, so the states match
    if (!r.wm) dt = 0.0f;
}

// Raw bits of entry n of the B (or C) rows of 16 steps from t0.  Steps past
// the end read the last row instead (no branches): there dt and u are 0, so
// those values reach no output.
template <typename IO>
__device__ __forceinline__ void load_rows_bits(const void *t, const BwdParams &p, const LaneB &l, int64_t t0,
                                               uint32_t (&v)[kStep]) {
#pragma unroll
    for (int k = 0; k < kStep; ++k) {
        const int64_t tk = t0 + k < p.L ? t0 + k : p.L - 1;
        v[k] = load_bits<IO>(t, (l.b * p.L + tk) * kRowN + l.n);
    }
}

// The adjoint's per-step inputs of block jb, as raw bits (see own_raw).  The
// B and C rows (the same for the whole workgroup, so mostly cache hits) are
// read when the block starts: holding them a block ahead does not fit the
// register budget of 3 waves per SIMD.
struct BlockRaw {
    OwnRaw own;
    uint32_t g, z;
    float h;  // the checkpoint
};
template <typename IO, bool CONV>
__device__ __forceinline__ void request_block(const BwdParams &p, const LaneB &l, int64_t jb, BlockRaw &r) {
    const int64_t t = jb * kStep + l.n;
    r.own = own_raw<IO, CONV>(p, l, t);
    const bool live = l.valid && t < p.L;
    const int64_t dc = l.valid ? l.d : 0;
    const int64_t i = (l.b * p.L + (live ? t : 0)) * p.D + dc;
    r.g = load_bits<IO>(p.dy, i);
    r.z = p.z ? load_bits<IO>(p.z, i) : 0u;
    r.h = p.ckpt[((jb * p.B + l.b) * p.D + dc) * kRowN + l.n];
}

// B (or C) tiles in LDS are fp32 [entry n][step k], rows 80 bytes apart
// (16-byte aligned; see the staging below).
constexpr int kBcRow = 80;
// Steps 4 g .. 4 g + 3 of entry n of tile `tensor` (of two consecutive tiles).
__device__ __forceinline__ void bc_quad(const char *bcl, int tensor, int n, int g, float (&v)[4]) {
    const float4 q = reinterpret_cast<const float4 *>(bcl + (tensor * kRowN + n) * kBcRow)[g];
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Sums over the wave's 4 channels (its 4 rows of 16 lanes) of four values
// v[0..3] per lane, for every entry n: row k of the result holds the sum of
// v[k].  v_permlane16_swap exchanges the odd rows of its first operand with
// the even rows of its second, v_permlane32_swap the upper half of the first
// with the lower half of the second; each swap plus an add halves the
// rows still to be added:
//   (v0, v1) -> rows (v0: r0+r1, v1: r0+r1, v0: r2+r3, v1: r2+r3), same for (v2, v3);
//   then the two results -> rows (v0, v1, v2, v3: r0+r1+r2+r3).
// (The swap's two results are taken from a named vector: passed straight
// into a function parameter, both elements read as the first one.)
__device__ __forceinline__ float sum_channels4(const float (&v)[4]) {
    auto u = [](float f) { return __builtin_bit_cast(unsigned, f); };
    auto f = [](unsigned x) { return __builtin_bit_cast(float, x); };
    const u32x2_t a = __builtin_amdgcn_permlane16_swap(u(v[0]), u(v[1]), false, false);
    const float s01 = f(a.x) + f(a.y);
    const u32x2_t b = __builtin_amdgcn_permlane16_swap(u(v[2]), u(v[3]), false, false);
    const float s23 = f(b.x) + f(b.y);
    const u32x2_t c = __builtin_amdgcn_permlane32_swap(u(s01), u(s23), false, false);
    return f(c.x) + f(c.y);
}

// The B and C rows of a block, staged in LDS for the whole workgroup (bf16
// I/O) and widened there once: [tensor][entry n][step k] as fp32, so that the
// lanes read their steps four at a time with no conversion, in the forward
// over the block and again in the adjoint.  Threads 0..255 fetch one 4-byte
// pair of entries each (tensor q / 128, step (q % 128) / 8, entries
// 2 (q % 8), +1) a block ahead and store it during the reduction.
constexpr int kBcLdsBytes = 2 * kRowN * kBcRow;
static_assert(kWavesB * (2 * kTrWave + kRedWave) * 4 + kBcLdsBytes <= 160 * 1024, "LDS of one workgroup");
constexpr int kBcFetchers = 2 * kStep * kRowN / 2;
__device__ __forceinline__ uint32_t bc_fetch(const BwdParams &p, int64_t b, int64_t jb, int q) {
    const int tensor = q >> 7, s = (q & 127) >> 3, part = q & 7;
    const int64_t t = jb * kStep + s;
    const int64_t tc = t < p.L ? t : p.L - 1;  // past the end: the last row (unused there)
    const uint16_t *base = static_cast<const uint16_t *>(tensor ? p.Cm : p.Bm);
    return *reinterpret_cast<const uint32_t *>(base + (b * p.L + tc) * kRowN + 2 * part);
}
__device__ __forceinline__ void bc_store(char *bcl, uint32_t v, int q) {
    const int tensor = q >> 7, s = (q & 127) >> 3, part = q & 7;
    float *col = reinterpret_cast<float *>(bcl + (tensor * kRowN + 2 * part) * kBcRow) + s;
    col[0] = __uint_as_float(v << 16);
    col[kBcRow / 4] = __uint_as_float(v & 0xffff0000u);
}

// Pass 2: the adjoint, blocks from last to first.
// STAGE: B and C through the LDS tile above (bf16 with 4-byte aligned B, C);
// otherwise every lane loads its entries of the 16 rows itself.
template <typename IO, bool FAST, bool CONV, bool STAGE>
__device__ __forceinline__ void bwd_body(const BwdParams &p, const LaneB &l, float *lds, float a, float ia) {
    const int n = l.n, c = l.c;
    // Per wave: two transpose areas (channel c at c * kChArea, [n][k] with
    // stride kTS) and the wave's dB / dC sums [2][16 n][kTS].
    float *tr0 = lds + l.wave * (2 * kTrWave + kRedWave);
    float *tr1 = tr0 + kTrWave;
    float *redw = tr1 + kTrWave;
    float *my0 = tr0 + c * kChArea + n * kTS;  // this lane's row in the areas
    float *my1 = tr1 + c * kChArea + n * kTS;
    const float a2 = a * kLog2e;
    const float dsk = (l.valid && p.Dskip) ? p.Dskip[l.d] : 0.0f;
    const float bias = (l.valid && p.dbias) ? p.dbias[l.d] : 0.0f;
    float lam = (l.valid && p.dh_final) ? p.dh_final[(l.b * p.D + l.d) * kRowN + n] : 0.0f;
    float accA = 0.0f, accD = 0.0f, accBias = 0.0f;
    const int64_t nb = (p.L + kStep - 1) / kStep;
    const int64_t grow = blockIdx.x % p.G;  // workgroup within the batch row
    float wr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float cb = 0.0f;
    if (CONV && l.valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wr[3 - q] = q < p.K ? p.conv_w[l.d * p.K + p.K - 1 - q] : 0.0f;
        cb = p.conv_b ? p.conv_b[l.d] : 0.0f;
    }

    // Block j's inputs as raw bits, requested during block j + 1 once its
    // adjoint is done (then the block's own registers are free), so that they
    // arrive while the sums and the workgroup reduction run.
    BlockRaw nx;
    request_block<IO, CONV>(p, l, nb - 1, nx);
    char *bcl = reinterpret_cast<char *>(lds + kWavesB * (2 * kTrWave + kRedWave));
    const int q = threadIdx.x;
    uint32_t bcv = 0u;
    if (STAGE) {
        if (q < kBcFetchers) bc_store(bcl, bc_fetch(p, l.b, nb - 1, q), q);
        __syncthreads();
    }

    for (int64_t j = nb - 1; j >= 0; --j) {
        const int64_t t0 = j * kStep;
        const int64_t tme = t0 + n;  // this lane's own step
        const bool live = nx.own.wm != 0;  // l.valid && tme < p.L
        // With the B and C tile staged, B and C are read from it where used
        // (in the forward over the block and again in the adjoint), which
        // leaves room for the 16 exp(dt A) of the forward: the adjoint reuses
        // them.
        float u, dt, bv[kStep], cv[kStep], ev[kStep];
        own_finish<IO, CONV>(p, nx.own, wr, cb, bias, u, dt);
        const float raw = live ? bits_f32<IO>(nx.own.draw) : 0.0f;
        if constexpr (!STAGE) {
            uint32_t rb[kStep], rc[kStep];
            load_rows_bits<IO>(p.Bm, p, l, t0, rb);
            load_rows_bits<IO>(p.Cm, p, l, t0, rc);
#pragma unroll
            for (int k = 0; k < kStep; ++k) {
                bv[k] = bits_f32<IO>(rb[k]);
                cv[k] = bits_f32<IO>(rc[k]);
            }
        }
        const float gv = live ? bits_f32<IO>(nx.g) : 0.0f;
        const float zv = (live && p.z) ? bits_f32<IO>(nx.z) : 0.0f;
        // -- forward over the block from its checkpoint ----------------------
        // Only h_{t-1} is kept per step; dt phi(dt A) is formed again, by the
        // same expression, in the adjoint (holding it cost 16 registers and
        // spills).
        float hp[kStep];
        float h = l.valid ? nx.h : 0.0f;
        // B and C of steps g4 .. g4 + 3
        auto bc_group = [&](int g4, float (&bq)[4], float (&cq)[4]) {
            if constexpr (STAGE) {
                bc_quad(bcl, 0, n, g4 / 4, bq);
                bc_quad(bcl, 1, n, g4 / 4, cq);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bq[i] = bv[g4 + i];
                    cq[i] = cv[g4 + i];
                }
            }
        };
        sfor<kStep / 4>([&](auto G) {
            constexpr int g4 = 4 * decltype(G)::value;
            float pk[4], bq[4], cq[4];
            bc_group(g4, bq, cq);
            sfor<4>([&](auto K) {
                constexpr int kk = decltype(K)::value;
                constexpr int k = g4 + kk;
                const float dtk = bcast_row<k>(dt), uk = bcast_row<k>(u);
                const float e = hw_exp2(dtk * a2);
                if constexpr (STAGE) ev[k] = e;
                hp[k] = h;
                h = __builtin_fmaf(e, h, dtphi<FAST>(dtk, a, ia, e) * (bq[kk] * uk));
                pk[kk] = cq[kk] * h;  // partial read-out of step k
            });
            *reinterpret_cast<float4 *>(my0 + g4) = make_float4(pk[0], pk[1], pk[2], pk[3]);
        });
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // lane (c, n) finishes its own step n: y_hat, gy, dz
        float yhat = dsk * u;
#pragma unroll
        for (int i = 0; i < kRowN; ++i) yhat += tr0[c * kChArea + i * kTS + n];
        float gy = gv;
        if (p.z) {
            gy = gv * silu(zv);
            if (l.valid && tme < p.L) store_io<IO>(p.dz, (l.b * p.L + tme) * p.D + l.d, gv * yhat * dsilu_f(zv));
        }
        accD += gy * u;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // -- adjoint over the block, last step first ---------------------------
        sfor<kStep / 4>([&](auto G) {
            constexpr int g4 = kStep - 4 - 4 * decltype(G)::value;  // 12, 8, 4, 0
            float pdu[4], pdt[4], sb[4], sc[4], bq[4], cq[4];
            bc_group(g4, bq, cq);
            sfor<4>([&](auto K) {
                constexpr int kk = 3 - decltype(K)::value;
                constexpr int k = g4 + kk;
                const float gyk = bcast_row<k>(gy), uk = bcast_row<k>(u), dtk = bcast_row<k>(dt);
                const float e = STAGE ? ev[k] : hw_exp2(dtk * a2);
                const float dtph = dtphi<FAST>(dtk, a, ia, e), bk = bq[kk];
                const float hcur = k == kStep - 1 ? h : hp[k + 1 < kStep ? k + 1 : 0];
                const float lt = __builtin_fmaf(cq[kk], gyk, lam);  // dL/dh_t
                const float dabar = lt * hp[k], dbbar = lt * uk;
                const float xb = dbbar * bk;  // dL/dh_t u B
                pdu[kk] = lt * (dtph * bk);
                pdt[kk] = e * __builtin_fmaf(dabar, a, xb);
                if (FAST) {
                    // d B_bar / dA = B (dt e - dt phi) / A: no psi where |A| >= 1/16.  The
                    // difference cancels for small dt A, but the term is then small
                    // next to dt e h (its error is ~1 ulp of B u / A, A >= 1/16).
                    // dL/dA = dt e (dabar + xb / A) - xb dtph / A
                    //       = (dt pdt - xb dtph) / A,  as pdt = e (dabar A + xb):
                    // summed here without the 1/A, which the end applies once.
                    accA = __builtin_fmaf(dtk, pdt[kk], accA);
                    accA = __builtin_fmaf(-xb, dtph, accA);
                } else {
                    const float zz = dtk * a, r = hw_rcp(zz);
                    const float ph = (e - 1.0f) * r;  // phi where |zz| >= 1/4 (psi's series covers the rest)
                    accA = __builtin_fmaf(e * dabar, dtk, accA);
                    accA = __builtin_fmaf(xb * dtk, dtk * psi_f(zz, e, ph, r), accA);
                }
                sb[kk] = dbbar * dtph;
                sc[kk] = gyk * hcur;
                lam = e * lt;
            });
            *reinterpret_cast<float4 *>(my0 + g4) = make_float4(pdu[0], pdu[1], pdu[2], pdu[3]);
            *reinterpret_cast<float4 *>(my1 + g4) = make_float4(pdt[0], pdt[1], pdt[2], pdt[3]);
            // row c of the wave holds the channel sums of step g4 + c
            redw[n * kTS + g4 + c] = sum_channels4(sb);
            redw[(kRowN + n) * kTS + g4 + c] = sum_channels4(sc);
        });
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        request_block<IO, CONV>(p, l, j > 0 ? j - 1 : 0, nx);  // the request after block 0 is not used
        if (STAGE && q < kBcFetchers) bcv = bc_fetch(p, l.b, j > 0 ? j - 1 : 0, q);
        {
            float du = dsk * gy, ddt = 0.0f;
#pragma unroll
            for (int i = 0; i < kRowN; ++i) {
                du += tr0[c * kChArea + i * kTS + n];
                ddt += tr1[c * kChArea + i * kTS + n];
            }
            float draw = ddt;
            if (p.softplus) {
                draw = ddt * sigmoid_f(raw + bias);
                // Steps past the end have dt = 0 but a nonzero ddt where dh_final
                // is given: they must not reach the bias gradient.
                if (live) accBias += draw;
            }
            if (live) {
                const int64_t i = (l.b * p.L + tme) * p.D + l.d;
                if (CONV) p.dU[i] = du;
                else store_io<IO>(p.dx, i, du);
                store_io<IO>(p.ddelta, i, draw);
            }
        }
        // -- dB, dC: add the workgroup's waves ---------------------------------
        __syncthreads();
        // Every wave has read this block's B and C: the next block's replace them.
        if (STAGE && q < kBcFetchers) bc_store(bcl, bcv, q);
        for (int item = threadIdx.x; item < 2 * kStep * kRowN; item += 64 * kWavesB) {
            const int tensor = item / (kStep * kRowN), kn = item % (kStep * kRowN);
            const int k = kn / kRowN, nn = kn % kRowN;
            float s = 0.0f;
            for (int w = 0; w < kWavesB; ++w)
                s += lds[w * (2 * kTrWave + kRedWave) + 2 * kTrWave + (tensor * kRowN + nn) * kTS + k];
            const int64_t t = t0 + k;
            if (t < p.L)
                p.partBC[(((int64_t)tensor * p.B + l.b) * p.G + grow) * p.L * kRowN + t * kRowN + nn] = s;
        }
        __syncthreads();
    }
    if (l.valid) {
        if (p.dh0) p.dh0[(l.b * p.D + l.d) * kRowN + n] = lam;
        p.partA[(l.b * p.D + l.d) * kRowN + n] = FAST ? accA * ia : accA;
    }
    // per-channel sums over the row's own steps
#pragma unroll
    for (int s = 8; s >= 1; s /= 2) {
        accD += __shfl_xor(accD, s, 16);
        accBias += __shfl_xor(accBias, s, 16);
    }
    if (l.valid && n == 0) {
        p.partD[l.b * p.D + l.d] = accD;
        p.partBias[l.b * p.D + l.d] = accBias;
    }
}

template <typename IO, bool CONV, bool STAGE>
__global__ __launch_bounds__(64 * kWavesB) __attribute__((amdgpu_waves_per_eu(3, 3)))
void bwd_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const LaneB l = lane_setup(p);
    const float a = l.valid ? p.A[l.d * kRowN + l.n] : 0.0f;
    const float ia = a != 0.0f ? 1.0f / a : 0.0f;
    if (__all(!l.valid || fabsf(a) >= 0.0625f)) bwd_body<IO, true, CONV, STAGE>(p, l, lds, a, ia);
    else bwd_body<IO, false, CONV, STAGE>(p, l, lds, a, ia);
}

// Through the conv prologue (u = silu(c), c_t = b + sum_k w_k x_{t-K+1+k}):
// one thread per (batch, channel, chunk of kConvChunk steps) walks time with
// rolling windows of x and of dc = du silu'(c), writing
//   dx_s = sum_k dc_{s+K-1-k} w_k            (three steps behind)
// and the chunk's partial sums of dw_k = sum_t dc_t x_{t-K+1+k} and db.  The
// windows are right-aligned to width 4, so no register is indexed by K.
constexpr int kConvChunk = 256;
// With an entering conv state cs (the K-1 inputs before t = 0) the window
// starts from it, and the first chunk also writes the state's gradient dcs
// (the transpose at the negative steps s = -(K-1) .. -1).
template <typename IO>
__global__ void conv_bwd_kernel(const void *x, const float *dU, const float *w, const float *cb, void *dx,
                                float *pw, int64_t B, int64_t L, int64_t D, int K, const void *cs,
                                void *dcs) {
    const int64_t nch = (L + kConvChunk - 1) / kConvChunk;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // d fastest
    if (i >= nch * B * D) return;
    const int64_t d = i % D, bc = i / D, b = bc % B, ch = bc / B;
    const int64_t t0 = ch * kConvChunk, t1 = t0 + kConvChunk < L ? t0 + kConvChunk : L;
    float wr[4], xw[4], dcw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dwr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[3 - j] = j < K ? w[d * K + K - 1 - j] : 0.0f;
    const float bias = cb ? cb[d] : 0.0f;
    const int64_t base = b * L * D + d;
    // Before step t, xw[1..3] hold x_{t-3..t-1}; each step shifts one in.
    xw[0] = 0.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t s = t0 - 3 + j;
        xw[j + 1] = s >= 0 ? load_io<IO>(x, base + s * D)
                  : (cs && s >= -(int64_t)(K - 1)) ? load_io<IO>(cs, (b * (K - 1) + (K - 1) + s) * D + d) : 0.0f;
    }
    float db = 0.0f;
    // Steps in groups of 8 whose 16 loads are issued first (indices clamped into the
    // tensors, values outside them masked), so they overlap.
    constexpr int kG = 8;
    for (int64_t tg = t0; tg < t1 + 3; tg += kG) {
        float xg[kG], ug[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int64_t t = tg + u;
            const int64_t tc = t < L ? t : t0;
            xg[u] = load_io<IO>(x, base + tc * D);
            ug[u] = dU[base + tc * D];
        }
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int64_t t = tg + u;
            if (t >= t1 + 3) break;
            xw[0] = xw[1];
            xw[1] = xw[2];
            xw[2] = xw[3];
            xw[3] = t < L ? xg[u] : 0.0f;
            float dc = 0.0f;
            if (t < L) {
                float c = bias;
#pragma unroll
                for (int j = 0; j < 4; ++j) c = __builtin_fmaf(wr[j], xw[j], c);
                dc = ug[u] * dsilu_f(c);
            }
            if (t < t1) {
                db += dc;
#pragma unroll
                for (int j = 0; j < 4; ++j) dwr[j] = __builtin_fmaf(dc, xw[j], dwr[j]);
            }
            dcw[0] = dcw[1];
            dcw[1] = dcw[2];
            dcw[2] = dcw[3];
            dcw[3] = dc;
            const int64_t s = t - 3;
            if (s >= t0 && s < t1) {
                float v = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) v = __builtin_fmaf(dcw[j], wr[3 - j], v);
                store_io<IO>(dx, base + s * D, v);
            } else if (dcs && s < 0 && s >= -(int64_t)(K - 1)) {
                float v = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) v = __builtin_fmaf(dcw[j], wr[3 - j], v);
                store_io<IO>(dcs, (b * (K - 1) + (K - 1) + s) * D + d, v);
            }
        }
    }
    float *o = pw + ((ch * B + b) * D + d) * 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = dwr[j];
    o[4] = db;
}

// dconv_w (right-aligned partials mapped back to taps 0..K-1) and dconv_b.
__global__ void conv_bwd_reduce_kernel(const float *pw, float *dw, float *db, int64_t nparts, int64_t D, int K) {
    const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= D) return;
    // four independent running sums over the partials (a fixed order), so their loads overlap
    float acc[4][5] = {};
    int64_t q = 0;
    for (; q + 4 <= nparts; q += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 5; ++j) acc[u][j] += pw[((q + u) * D + d) * 5 + j];
    for (; q < nparts; ++q)
#pragma unroll
        for (int j = 0; j < 5; ++j) acc[0][j] += pw[(q * D + d) * 5 + j];
    float s[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) s[j] = (acc[0][j] + acc[1][j]) + (acc[2][j] + acc[3][j]);
    for (int k = 0; k < K; ++k) dw[d * K + k] = s[4 - K + k];
    if (db) db[d] = s[4];
}

// dB, dC = sums of the workgroup partials of each batch row; fp32 outputs.
__global__ void bwd_reduce_bc_kernel(const float *partBC, float *dB, float *dC, int64_t B, int64_t G,
                                     int64_t L) {
    // 4 consecutive (step, entry) values of one (tensor, batch row) per thread, as 16-byte
    // loads; four independent running sums over the workgroups (a fixed order), so the
    // loads of the G partials overlap instead of waiting one for another.
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t per = B * L * kRowN;  // a multiple of 16
    if (i >= 2 * per) return;
    const int64_t tensor = i / per, r = i % per;
    const int64_t b = r / (L * kRowN), tn = r % (L * kRowN);
    const int64_t gs = L * kRowN / 4;  // float4s between the partials of two workgroups
    const float4 *src = reinterpret_cast<const float4 *>(partBC + (tensor * B + b) * G * L * kRowN + tn);
    float4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    int64_t g = 0;
    for (; g + 4 <= G; g += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 v = src[(g + u) * gs];
            acc[u].x += v.x;
            acc[u].y += v.y;
            acc[u].z += v.z;
            acc[u].w += v.w;
        }
    }
    for (; g < G; ++g) {
        const float4 v = src[g * gs];
        acc[0].x += v.x;
        acc[0].y += v.y;
        acc[0].z += v.z;
        acc[0].w += v.w;
    }
    float *dst = (tensor == 0 ? dB : dC) + r;
    dst[0] = (acc[0].x + acc[1].x) + (acc[2].x + acc[3].x);
    dst[1] = (acc[0].y + acc[1].y) + (acc[2].y + acc[3].y);
    dst[2] = (acc[0].z + acc[1].z) + (acc[2].z + acc[3].z);
    dst[3] = (acc[0].w + acc[1].w) + (acc[2].w + acc[3].w);
}

// dA, dDskip, ddelta_bias = sums over batch rows.
__global__ void bwd_reduce_params_kernel(const float *partA, const float *partD, const float *partBias,
                                         float *dA, float *dD, float *dbias, int64_t B, int64_t D) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over D 16
    if (i >= D * kRowN) return;
    float s = 0.0f;
    for (int64_t b = 0; b < B; ++b) s += partA[b * D * kRowN + i];
    dA[i] = s;
    if (i % kRowN == 0) {
        const int64_t d = i / kRowN;
        float sd = 0.0f, sb = 0.0f;
        for (int64_t b = 0; b < B; ++b) {
            sd += partD[b * D + d];
            sb += partBias[b * D + d];
        }
        if (dD) dD[d] = sd;
        if (dbias) dbias[d] = sb;
    }
}

// dh0 of an empty sequence: dh_final (or 0); dA etc. are 0.
template <typename IO>
__global__ void bwd_empty_kernel(const float *dh_final, float *dh0, int64_t nbdn, float *dA, float *dD,
                                 float *dbias, float *dcw, float *dcb, void *dcs, int64_t ncs, int64_t D,
                                 int N, int K) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (dh0 && i < nbdn) dh0[i] = dh_final ? dh_final[i] : 0.0f;
    if (dcs && i < ncs) store_io<IO>(dcs, i, 0.0f);
    if (i < D * N) dA[i] = 0.0f;
    if (dcw && i < D * K) dcw[i] = 0.0f;
    if (i < D) {
        if (dD) dD[i] = 0.0f;
        if (dbias) dbias[i] = 0.0f;
        if (dcb) dcb[i] = 0.0f;
    }
}

// N < 16: the kernels above run on 16 state entries per channel.  The
// per-entry tensors are copied into 16-wide buffers whose extra entries hold
// B = C = 0, h0 = dh_final = 0 and A = -1; those entries then keep a zero
// state and a zero adjoint, add nothing to any gradient of the real entries,
// and their own gradients are dropped when dA, dB, dC and dh0 are copied
// back to N-wide rows.
//   rows x N (elements of `bytes` bytes) -> rows x 16, extra entries = fill.
template <typename T>
__global__ void pad_rows_kernel(const T *src, T *dst, int64_t rows, int N, T fill) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // rows * 16
    if (i >= rows * kRowN) return;
    const int64_t r = i / kRowN;
    const int n = (int)(i % kRowN);
    dst[i] = n < N ? src[r * N + n] : fill;
}
//   rows x 16 -> rows x N
__global__ void compact_rows_kernel(const float *src, float *dst, int64_t rows, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // rows * N
    if (i >= rows * N) return;
    dst[i] = src[(i / N) * kRowN + i % N];
}

template <typename T>
hipError_t pad_rows(const void *src, void *dst, int64_t rows, int N, T fill, hipStream_t stream) {
    const int64_t n = rows * kRowN;
    pad_rows_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(static_cast<const T *>(src),
                                                                     static_cast<T *>(dst), rows, N, fill);
    return hipGetLastError();
}
hipError_t compact_rows(const float *src, float *dst, int64_t rows, int N, hipStream_t stream) {
    const int64_t n = rows * N;
    compact_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(src, dst, rows, N);
    return hipGetLastError();
}

size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of the 16-wide copies when N < 16 (0 when N == 16).
struct PadLayout {
    size_t B, C, A, h0, dhf, dA, dB, dC, dh0, total;
};
PadLayout pad_layout(const ssm_scan_bwd_args_t &a) {
    PadLayout q{};
    if (a.dstate == kRowN) return q;
    const size_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    const size_t bl = (size_t)(a.batch * a.seqlen) * kRowN, bd = (size_t)(a.batch * a.dim) * kRowN;
    q.B = q.C = r256(bl * es);
    q.A = r256((size_t)a.dim * kRowN * sizeof(float));
    q.h0 = a.h0 ? r256(bd * sizeof(float)) : 0;
    q.dhf = a.dh_final ? r256(bd * sizeof(float)) : 0;
    q.dA = q.A;
    q.dB = q.dC = r256(bl * sizeof(float));
    q.dh0 = a.dh0 ? r256(bd * sizeof(float)) : 0;
    q.total = q.B + q.C + q.A + q.h0 + q.dhf + q.dA + q.dB + q.dC + q.dh0;
    return q;
}

struct BwdLayout {
    int64_t G, nb, nch;
    size_t ckpt, partBC, partA, partD, partBias, dU, pconv, total;
};

BwdLayout bwd_layout(const ssm_scan_bwd_args_t &a) {
    BwdLayout q;
    q.G = (a.dim + kChB - 1) / kChB;
    q.nb = (a.seqlen + kStep - 1) / kStep;
    // (none when the caller passes the forward's checkpoints)
    q.ckpt = a.checkpoints ? 0 : r256((size_t)(q.nb * a.batch * a.dim * kRowN) * sizeof(float));
    q.partBC = r256((size_t)(2 * a.batch * q.G * a.seqlen * kRowN) * sizeof(float));
    q.partA = r256((size_t)(a.batch * a.dim * kRowN) * sizeof(float));
    q.partD = r256((size_t)(a.batch * a.dim) * sizeof(float));
    q.partBias = q.partD;
    q.nch = (a.seqlen + kConvChunk - 1) / kConvChunk;
    q.dU = a.conv_k > 0 ? r256((size_t)(a.batch * a.seqlen * a.dim) * sizeof(float)) : 0;
    q.pconv = a.conv_k > 0 ? r256((size_t)(q.nch * a.batch * a.dim * 5) * sizeof(float)) : 0;
    q.total = q.ckpt + q.partBC + q.partA + q.partD + q.partBias + q.dU + q.pconv;
    return q;
}

template <typename IO>
hipError_t launch_bwd_typed(const BwdParams &p, const ssm_scan_bwd_args_t &a, float *pconv, int64_t nch,
                            hipStream_t stream) {
    const unsigned grid = (unsigned)(p.G * p.B);
    // Pass 1, the checkpoints: the forward scan kernel in its checkpoint
    // variant (staged loads; no read-out), on the 16-entry rows.
    ssm_scan_args_t f{};
    f.batch = p.B;
    f.seqlen = p.L;
    f.dim = p.D;
    f.dstate = kRowN;
    f.io_dtype = a.io_dtype;
    f.delta_softplus = p.softplus;
    f.conv_k = p.K;
    f.x = p.x;
    f.delta = p.delta;
    f.Bm = p.Bm;
    f.Cm = p.Cm;
    f.A = p.A;
    f.delta_bias = p.dbias;
    f.conv_w = p.conv_w;
    f.conv_b = p.conv_b;
    f.h0 = p.h0;
    f.conv_state_in = p.cs_in;
    hipError_t e = a.checkpoints ? hipSuccess : launch_scan_ckpt(f, p.ckpt, stream);
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)(kWavesB * (2 * kTrWave + kRedWave)) * sizeof(float);
    // B and C staged in LDS: bf16 rows read as 4-byte pairs.
    const bool stage = sizeof(typename IO::storage) == 2 && (uintptr_t)p.Bm % 4 == 0 && (uintptr_t)p.Cm % 4 == 0;
    if (stage) {
        constexpr bool kStage = sizeof(typename IO::storage) == 2;
        if (p.K > 0) bwd_kernel<IO, true, kStage><<<grid, 64 * kWavesB, lds + kBcLdsBytes, stream>>>(p);
        else bwd_kernel<IO, false, kStage><<<grid, 64 * kWavesB, lds + kBcLdsBytes, stream>>>(p);
    } else {
        if (p.K > 0) bwd_kernel<IO, true, false><<<grid, 64 * kWavesB, lds, stream>>>(p);
        else bwd_kernel<IO, false, false><<<grid, 64 * kWavesB, lds, stream>>>(p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nbc = 2 * p.B * p.L * kRowN / 4;  // threads: 4 values each
    bwd_reduce_bc_kernel<<<(unsigned)((nbc + 255) / 256), 256, 0, stream>>>(p.partBC, a.dBm, a.dCm, p.B, p.G, p.L);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_reduce_params_kernel<<<(unsigned)((p.D * kRowN + 255) / 256), 256, 0, stream>>>(
        p.partA, p.partD, p.partBias, a.dA, a.dDskip, a.ddelta_bias, p.B, p.D);
    e = hipGetLastError();
    if (e != hipSuccess || p.K == 0) return e;
    const int64_t nthr = nch * p.B * p.D;
    conv_bwd_kernel<IO><<<(unsigned)((nthr + 255) / 256), 256, 0, stream>>>(
        p.x, p.dU, p.conv_w, p.conv_b, p.dx, pconv, p.B, p.L, p.D, p.K, p.cs_in, p.dcs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    conv_bwd_reduce_kernel<<<(unsigned)((p.D + 255) / 256), 256, 0, stream>>>(pconv, a.dconv_w, a.dconv_b,
                                                                              nch * p.B, p.D, p.K);
    return hipGetLastError();
}

}  // namespace

size_t scan_bwd_workspace_bytes(const ssm_scan_bwd_args_t &a) {
    if (a.batch == 0 || a.seqlen == 0) return 0;
    return pad_layout(a).total + bwd_layout(a).total;
}

namespace {
hipError_t launch_scan_bwd16(const ssm_scan_bwd_args_t &a, char *ws, hipStream_t stream);
}

hipError_t launch_scan_bwd(const ssm_scan_bwd_args_t &a, hipStream_t stream) {
    const int N = (int)a.dstate;
    if (a.seqlen == 0) {
        // nothing reads the entering conv state: its gradient is 0
        void *dcs = a.conv_k > 1 ? a.dconv_state_in : nullptr;
        const int64_t ncs = dcs ? a.batch * (a.conv_k - 1) * a.dim : 0;
        const int64_t n = std::max<int64_t>(std::max<int64_t>(a.batch * a.dim * N, ncs),
                                            std::max<int64_t>(a.dim * N, a.dim * a.conv_k));
        const unsigned g = (unsigned)((n + 255) / 256);
        if (a.io_dtype == SSM_BF16)
            bwd_empty_kernel<io_bf16><<<g, 256, 0, stream>>>(a.dh_final, a.dh0, a.batch * a.dim * N, a.dA,
                                                           a.dDskip, a.ddelta_bias, a.dconv_w, a.dconv_b, dcs,
                                                           ncs, a.dim, N, (int)a.conv_k);
        else
            bwd_empty_kernel<io_f32><<<g, 256, 0, stream>>>(a.dh_final, a.dh0, a.batch * a.dim * N, a.dA,
                                                          a.dDskip, a.ddelta_bias, a.dconv_w, a.dconv_b, dcs,
                                                          ncs, a.dim, N, (int)a.conv_k);
        return hipGetLastError();
    }
    char *ws = static_cast<char *>(a.workspace);
    if (N == kRowN) return launch_scan_bwd16(a, ws, stream);
    // 16-wide copies of the per-entry tensors, the kernels, then the gradients back.
    const PadLayout q = pad_layout(a);
    ssm_scan_bwd_args_t b = a;
    b.dstate = kRowN;
    char *w = ws;
    auto take = [&](size_t n) { char *r = n ? w : nullptr; w += n; return r; };
    b.Bm = take(q.B);
    b.Cm = take(q.C);
    b.A = reinterpret_cast<float *>(take(q.A));
    b.h0 = reinterpret_cast<float *>(take(q.h0));
    b.dh_final = reinterpret_cast<float *>(take(q.dhf));
    b.dA = reinterpret_cast<float *>(take(q.dA));
    b.dBm = reinterpret_cast<float *>(take(q.dB));
    b.dCm = reinterpret_cast<float *>(take(q.dC));
    b.dh0 = reinterpret_cast<float *>(take(q.dh0));
    const int64_t bl = a.batch * a.seqlen, bd = a.batch * a.dim;
    hipError_t e;
    if (a.io_dtype == SSM_BF16) {
        if ((e = pad_rows<uint16_t>(a.Bm, const_cast<void *>(b.Bm), bl, N, 0, stream)) != hipSuccess) return e;
        if ((e = pad_rows<uint16_t>(a.Cm, const_cast<void *>(b.Cm), bl, N, 0, stream)) != hipSuccess) return e;
    } else {
        if ((e = pad_rows<float>(a.Bm, const_cast<void *>(b.Bm), bl, N, 0.0f, stream)) != hipSuccess) return e;
        if ((e = pad_rows<float>(a.Cm, const_cast<void *>(b.Cm), bl, N, 0.0f, stream)) != hipSuccess) return e;
    }
    if ((e = pad_rows<float>(a.A, const_cast<float *>(b.A), a.dim, N, -1.0f, stream)) != hipSuccess) return e;
    if (a.h0 && (e = pad_rows<float>(a.h0, const_cast<float *>(b.h0), bd, N, 0.0f, stream)) != hipSuccess)
        return e;
    if (a.dh_final &&
        (e = pad_rows<float>(a.dh_final, const_cast<float *>(b.dh_final), bd, N, 0.0f, stream)) != hipSuccess)
        return e;
    if ((e = launch_scan_bwd16(b, w, stream)) != hipSuccess) return e;
    if ((e = compact_rows(b.dA, a.dA, a.dim, N, stream)) != hipSuccess) return e;
    if ((e = compact_rows(b.dBm, a.dBm, bl, N, stream)) != hipSuccess) return e;
    if ((e = compact_rows(b.dCm, a.dCm, bl, N, stream)) != hipSuccess) return e;
    if (a.dh0 && (e = compact_rows(b.dh0, a.dh0, bd, N, stream)) != hipSuccess) return e;
    return hipSuccess;
}

namespace {
// The backward pass with N == 16 on the workspace `ws` (bwd_layout's size).
hipError_t launch_scan_bwd16(const ssm_scan_bwd_args_t &a, char *ws, hipStream_t stream) {
    const BwdLayout q = bwd_layout(a);
    BwdParams p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.D = a.dim;
    p.G = q.G;
    p.softplus = a.delta_softplus;
    p.K = (int)a.conv_k;
    p.conv_w = a.conv_w;
    p.conv_b = a.conv_b;
    p.cs_in = a.conv_k > 1 ? a.conv_state_in : nullptr;
    p.dcs = a.conv_k > 1 ? a.dconv_state_in : nullptr;
    p.dU = a.conv_k > 0 ? reinterpret_cast<float *>(ws + q.ckpt + q.partBC + q.partA + q.partD + q.partBias)
                        : nullptr;
    p.x = a.x;
    p.delta = a.delta;
    p.Bm = a.Bm;
    p.Cm = a.Cm;
    p.z = a.z;
    p.dy = a.dy;
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.h0 = a.h0;
    p.dh_final = a.dh_final;
    p.dx = a.dx;
    p.ddelta = a.ddelta;
    p.dz = a.dz;
    p.dh0 = a.dh0;
    p.ckpt = a.checkpoints ? const_cast<float *>(a.checkpoints) : reinterpret_cast<float *>(ws);
    p.partBC = reinterpret_cast<float *>(ws + q.ckpt);
    p.partA = reinterpret_cast<float *>(ws + q.ckpt + q.partBC);
    p.partD = reinterpret_cast<float *>(ws + q.ckpt + q.partBC + q.partA);
    p.partBias = reinterpret_cast<float *>(ws + q.ckpt + q.partBC + q.partA + q.partD);
    float *pconv = a.conv_k > 0
                       ? reinterpret_cast<float *>(ws + q.ckpt + q.partBC + q.partA + q.partD + q.partBias + q.dU)
                       : nullptr;
    if (a.io_dtype == SSM_BF16) return launch_bwd_typed<io_bf16>(p, a, pconv, q.nch, stream);
    return launch_bwd_typed<io_f32>(p, a, pconv, q.nch, stream);
}
}  // namespace

}  // namespace ssm
