// ssd.hip -- the SSD (Mamba-2) layer, chunked forward on the gfx950 matrix cores.
//
// "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상", sec. 5.1: with the
// state matrix a scalar times the identity per step and head (A_t = a_t I),
// the layer is the masked product Y = (L o (C B^T)) X, L the causal mask of
// cumulative decays; sec. 5.2: run it in chunks, the quadratic (attention)
// form inside a chunk on the matrix cores and the linear (recurrent) form
// between chunks.  Discretised by ZOH (eq. (4) of "Mamba: Linear-Time
// Sequence Modeling with Selective State Spaces"), which for A = a I gives
// alpha_t = exp(dt_t a) and the input weight w_t = dt_t phi(dt_t a),
// phi(v) = (e^v - 1) / v.  Per chunk of kQ steps (acum = inclusive prefix sum
// of dt a inside the chunk, H the state entering the chunk, (P, N) per head):
//
//   Y[t]  = e^{acum[t]} C_t H^T                                  (entering state)
//         + sum_{s<=t} e^{acum[t]-acum[s]} w_s (C_t . B_s) x_s    (inside the chunk)
//         + Dskip x_t,  then x silu(z_t)
//   H    <- e^{acum[end]} H + sum_s e^{acum[end]-acum[s]} w_s x_s B_s^T
//
// One workgroup of 4 waves owns one (batch, head) and walks its chunks in
// order.  Every product is a 16x16x16 bf16 MFMA with fp32 accumulation:
//   G^T tiles  B_s . C_t   (A = B rows, B = C rows): the result layout is
//              exactly the A operand of the next product, so the masked,
//              scaled tile M goes to LDS only because other waves read it;
//   Y          C H^T + M X (each wave owns 16 of the 64 head channels);
//   state      B^T (w' X) (same 16 channels; the fp32 state stays in the
//              accumulators across chunks, a copy in LDS feeds C H^T).
// x, B and C are bf16 inputs and exact as operands.  The computed operands
// (M, w' X and the state copy) enter as a sum of two bf16 numbers, hi + lo
// with lo = bf16(v - hi), and each such product is two MFMAs: about 16
// significant bits, where a single bf16 rounding (8 bits) would leave errors
// of order 1% in sums that cancel (C.h is a sum of N terms of either sign).
// The state tiles, the outputs and the chunk's inputs never leave the CU
// except as the layer's own inputs and outputs.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kQ = 64;     // chunk length (4 tiles of 16)
constexpr int kP = 64;     // head channels (one 16-wide tile per wave)
constexpr int kPadE = 8;   // row padding, bf16 elements (16 bytes)
constexpr int kThreads = 256;

typedef short ssd_s4 __attribute__((ext_vector_type(4)));
typedef float ssd_f4 __attribute__((ext_vector_type(4)));

template <int N>
struct SsdLds {
    static constexpr int nld = N + kPadE;   // rows of N entries: Bs, Cs, HT
    static constexpr int qld = kQ + kPadE;  // rows of kQ entries: BT, XT, XWT, Mb
    // HT, XWT and Mb hold a hi plane and then a lo plane.
    static constexpr size_t bs = 0;
    static constexpr size_t cs = bs + (size_t)kQ * nld * 2;
    static constexpr size_t ht = cs + (size_t)kQ * nld * 2;
    static constexpr size_t ht_lo = (size_t)kP * nld;  // elements to the lo plane
    static constexpr size_t bt = ht + 2 * (size_t)kP * nld * 2;
    static constexpr size_t xt = bt + (size_t)N * qld * 2;
    static constexpr size_t xwt = xt + (size_t)kP * qld * 2;
    static_assert(kQ == kP, "XWT (kP rows) and Mb (kQ rows) share one lo-plane offset");
    static constexpr size_t q_lo = (size_t)kQ * qld;    // elements to the lo plane (XWT, Mb)
    static constexpr size_t mb = xwt + 2 * (size_t)kP * qld * 2;
    static constexpr size_t dts = mb + 2 * (size_t)kQ * qld * 2;
    static constexpr size_t total = dts + (size_t)kQ * sizeof(float);
};

struct SsdParams {
    int64_t B, L, H, G;
    const uint16_t *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dskip, *dbias, *h0;
    uint16_t *y;
    float *h_final;
    int softplus;
};

__device__ __forceinline__ float bf(uint16_t v) { return bf16_bits_to_f32(v); }

// phi(v) = (e^v - 1) / v with e = e^v; a series where the quotient cancels.
__device__ __forceinline__ float ssd_phi(float v, float e) {
    if (fabsf(v) < 0.25f)
        return 1.0f + v * (0.5f + v * (1.0f / 6 + v * (1.0f / 24 + v * (1.0f / 120 + v * (1.0f / 720)))));
    return (e - 1.0f) / v;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// v ~ hi + lo, both bf16 (4 values): hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void split4(const float (&v)[4], uint2 &hi, uint2 &lo) {
    hi = pack4(v[0], v[1], v[2], v[3]);
    const float h0 = __uint_as_float(hi.x << 16), h1 = __uint_as_float(hi.x & 0xffff0000u);
    const float h2 = __uint_as_float(hi.y << 16), h3 = __uint_as_float(hi.y & 0xffff0000u);
    lo = pack4(v[0] - h0, v[1] - h1, v[2] - h2, v[3] - h3);
}

__device__ __forceinline__ void store_split4(uint16_t *hi_plane, size_t lo_off, const float (&v)[4]) {
    uint2 hi, lo;
    split4(v, hi, lo);
    *reinterpret_cast<uint2 *>(hi_plane) = hi;
    *reinterpret_cast<uint2 *>(hi_plane + lo_off) = lo;
}

#define SSD_MFMA(a, b, c) __builtin_amdgcn_mfma_f32_16x16x16bf16_1k((a), (b), (c), 0, 0, 0)

__device__ __forceinline__ ssd_s4 lds4(const uint16_t *p) {
    return __builtin_bit_cast(ssd_s4, *reinterpret_cast<const uint2 *>(p));
}

// (tile of t, tile of s) pairs of the causal lower triangle of a chunk
__constant__ int8_t kPairT[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kPairS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(SsdParams p) {
    using Lay = SsdLds<N>;
    constexpr int NT = N / 16;
    constexpr int nld = Lay::nld, qld = Lay::qld;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    uint16_t *Bs = reinterpret_cast<uint16_t *>(lds + Lay::bs);
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds + Lay::cs);
    uint16_t *HT = reinterpret_cast<uint16_t *>(lds + Lay::ht);
    uint16_t *BT = reinterpret_cast<uint16_t *>(lds + Lay::bt);
    uint16_t *XT = reinterpret_cast<uint16_t *>(lds + Lay::xt);
    uint16_t *XWT = reinterpret_cast<uint16_t *>(lds + Lay::xwt);
    uint16_t *Mb = reinterpret_cast<uint16_t *>(lds + Lay::mb);
    float *dts = reinterpret_cast<float *>(lds + Lay::dts);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = 4 * (lane >> 4);
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t g = h / (p.H / p.G);
    const int64_t L = p.L;
    const float a = p.A[h];
    const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
    const float dbias = p.dbias ? p.dbias[h] : 0.0f;
    const int pcol = 16 * w + r16;  // this lane's head channel in the wave's tile

    // State tiles of this wave's channels: st[nt][v] is entry n = 16 nt + q4 + v
    // of channel pcol.
    ssd_f4 st[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float v4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            st[nt][v] = p.h0 ? p.h0[(bh * kP + pcol) * N + 16 * nt + q4 + v] : 0.0f;
            v4[v] = st[nt][v];
        }
        store_split4(HT + pcol * nld + 16 * nt + q4, Lay::ht_lo, v4);
    }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kQ;
        // ---- the chunk's inputs into LDS ------------------------------------
        constexpr int PR = N / 8;  // 16-byte pieces per B/C row
        for (int id = tid; id < kQ * PR; id += kThreads) {
            const int s = id / PR, c8 = (id % PR) * 8;
            const int64_t t = t0 + s;
            uint4 vb = make_uint4(0, 0, 0, 0), vc = vb;
            if (t < L) {
                const int64_t off = ((b * L + t) * p.G + g) * N + c8;
                vb = *reinterpret_cast<const uint4 *>(p.Bm + off);
                vc = *reinterpret_cast<const uint4 *>(p.Cm + off);
            }
            *reinterpret_cast<uint4 *>(Bs + s * nld + c8) = vb;
            *reinterpret_cast<uint4 *>(Cs + s * nld + c8) = vc;
            const uint32_t wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                BT[(c8 + 2 * i) * qld + s] = (uint16_t)(wb[i] & 0xffffu);
                BT[(c8 + 2 * i + 1) * qld + s] = (uint16_t)(wb[i] >> 16);
            }
        }
        for (int id = tid; id < kQ * (kP / 8); id += kThreads) {
            const int s = id / (kP / 8), c8 = (id % (kP / 8)) * 8;
            const int64_t t = t0 + s;
            uint4 vx = make_uint4(0, 0, 0, 0);
            if (t < L) vx = *reinterpret_cast<const uint4 *>(p.x + ((b * L + t) * p.H + h) * kP + c8);
            const uint32_t wx[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                XT[(c8 + 2 * i) * qld + s] = (uint16_t)(wx[i] & 0xffffu);
                XT[(c8 + 2 * i + 1) * qld + s] = (uint16_t)(wx[i] >> 16);
            }
        }
        if (tid < kQ) {
            const int64_t t = t0 + tid;
            float dt = 0.0f;
            if (t < L) {
                dt = bf(p.delta[(b * L + t) * p.H + h]);
                if (p.softplus) dt = softplus_fast(dt + dbias);
            }
            dts[tid] = dt;
        }
        __syncthreads();

        // ---- chunk scalars, one copy per wave (lane = step s) ----------------
        const float dtl = dts[lane];
        const float zl = dtl * a;
        float acum = zl;  // inclusive prefix sum of dt a
#pragma unroll
        for (int off = 1; off < 64; off *= 2) {
            const float v = __shfl_up(acum, off, 64);
            if (lane >= off) acum += v;
        }
        const float aend = __shfl(acum, 63, 64);
        const float wl = dtl * ssd_phi(zl, hw_exp2(zl * kLog2e));       // ZOH input weight
        const float fl = hw_exp2((aend - acum) * kLog2e) * wl;         // weight in the end state

        // ---- masked, scaled G^T tiles -> Mb[t][s]; X' = f x -> XWT ----------
        for (int pi = w; pi < 10; pi += 4) {
            const int tb = kPairT[pi], sb = kPairS[pi];
            ssd_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NT; ++kk)
                acc = SSD_MFMA(lds4(Bs + (16 * sb + r16) * nld + 16 * kk + q4),
                               lds4(Cs + (16 * tb + r16) * nld + 16 * kk + q4), acc);
            // lane holds s = 16 sb + q4 + v, t = 16 tb + r16
            const int t = 16 * tb + r16;
            const float at = __shfl(acum, t, 64);
            float m[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = 16 * sb + q4 + v;
                const float as = __shfl(acum, s, 64), ws = __shfl(wl, s, 64);
                m[v] = s <= t ? acc[v] * hw_exp2((at - as) * kLog2e) * ws : 0.0f;
            }
            store_split4(Mb + t * qld + 16 * sb + q4, Lay::q_lo, m);
        }
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const int pp = 16 * w + i;
            const float v = bf(XT[pp * qld + lane]) * fl;
            const uint16_t hi = f32_to_bf16_bits(v);
            XWT[pp * qld + lane] = hi;
            XWT[Lay::q_lo + pp * qld + lane] = f32_to_bf16_bits(v - bf(hi));
        }
        __syncthreads();

        // ---- outputs of this wave's 16 channels --------------------------------
        for (int tb = 0; tb < kQ / 16; ++tb) {
            ssd_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < NT; ++kk) {
                const ssd_s4 cop = lds4(Cs + (16 * tb + r16) * nld + 16 * kk + q4);
                const uint16_t *hp = HT + pcol * nld + 16 * kk + q4;
                acc = SSD_MFMA(cop, lds4(hp), acc);
                acc = SSD_MFMA(cop, lds4(hp + Lay::ht_lo), acc);
            }
            // lane holds t = 16 tb + q4 + v, channel pcol
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] *= hw_exp2(__shfl(acum, 16 * tb + q4 + v, 64) * kLog2e);
            for (int sb = 0; sb <= tb; ++sb) {
                const uint16_t *mp = Mb + (16 * tb + r16) * qld + 16 * sb + q4;
                const ssd_s4 xop = lds4(XT + pcol * qld + 16 * sb + q4);
                acc = SSD_MFMA(lds4(mp), xop, acc);
                acc = SSD_MFMA(lds4(mp + Lay::q_lo), xop, acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 16 * tb + q4 + v;
                const int64_t tt = t0 + t;
                if (tt < L) {
                    const int64_t i = ((b * L + tt) * p.H + h) * kP + pcol;
                    float yv = acc[v] + dsk * bf(XT[pcol * qld + t]);
                    if (p.z) yv *= silu(bf(p.z[i]));
                    p.y[i] = f32_to_bf16_bits(yv);
                }
            }
        }

        // ---- the state entering the next chunk ---------------------------------
        const float dend = hw_exp2(aend * kLog2e);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            ssd_f4 s4v = st[nt] * dend;
#pragma unroll
            for (int kk = 0; kk < kQ / 16; ++kk) {
                const ssd_s4 bop = lds4(BT + (16 * nt + r16) * qld + 16 * kk + q4);
                const uint16_t *xp = XWT + pcol * qld + 16 * kk + q4;
                s4v = SSD_MFMA(bop, lds4(xp), s4v);
                s4v = SSD_MFMA(bop, lds4(xp + Lay::q_lo), s4v);
            }
            st[nt] = s4v;
            const float v4[4] = {s4v[0], s4v[1], s4v[2], s4v[3]};
            store_split4(HT + pcol * nld + 16 * nt + q4, Lay::ht_lo, v4);
        }
        __syncthreads();
    }

    if (p.h_final) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) p.h_final[(bh * kP + pcol) * N + 16 * nt + q4 + v] = st[nt][v];
    }
}

template <int N>
hipError_t launch_n(const SsdParams &p, int64_t B, int64_t H, hipStream_t stream) {
    ssd_chunk_kernel<N><<<(unsigned)(B * H), kThreads, SsdLds<N>::total, stream>>>(p);
    return hipGetLastError();
}

}  // namespace

bool ssd_supported(int64_t headdim, int64_t dstate) {
    return headdim == kP && (dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128);
}

hipError_t launch_ssd_fwd(const ssm_ssd_args_t &a, hipStream_t stream) {
    SsdParams p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.H = a.nheads;
    p.G = a.ngroups;
    p.x = static_cast<const uint16_t *>(a.x);
    p.delta = static_cast<const uint16_t *>(a.delta);
    p.Bm = static_cast<const uint16_t *>(a.Bm);
    p.Cm = static_cast<const uint16_t *>(a.Cm);
    p.z = static_cast<const uint16_t *>(a.z);
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.h0 = a.h0;
    p.y = static_cast<uint16_t *>(a.y);
    p.h_final = a.h_final;
    p.softplus = a.delta_softplus;
    switch (a.dstate) {
        case 16: return launch_n<16>(p, a.batch, a.nheads, stream);
        case 32: return launch_n<32>(p, a.batch, a.nheads, stream);
        case 64: return launch_n<64>(p, a.batch, a.nheads, stream);
        default: return launch_n<128>(p, a.batch, a.nheads, stream);
    }
}

}  // namespace ssm
