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
// One workgroup of 4 waves owns one (batch, head, 32 head channels) and walks
// that head's chunks in order; the two channel halves of a head run as two
// workgroups (they share B and C through the L2).  Every product is a bf16
// MFMA with fp32 accumulation (16x16x32; 16x16x16 for the sums over the
// state entries when N = 16).  Wave w owns the 16 steps
// t in [16 w, 16 w + 16) of each chunk for the outputs and the state entries
// n in [32 w, 32 w + 32) (N = 128; N / 4 in general) for the state:
//   G^T tiles  B_s . C_t for s <= t (A = B rows, B = C rows, the wave's own
//              C rows loaded from memory straight into registers): the result
//              layout is exactly the A operand of the next product, so the
//              causally masked, decayed tile M never leaves the registers;
//   Y          C H^T + M X;
//   state      B^T (w' X); the fp32 state stays in the accumulators across
//              chunks, a copy in LDS feeds C H^T (read before the
//              workgroup's middle barrier, rewritten after it).
// x, B and C are bf16 inputs and exact as operands.  The computed operands
// (M, w' X and the state copy) enter as a sum of two bf16 numbers, hi + lo
// with lo = bf16(v - hi), and each such product is two MFMAs: about 16
// significant bits, where a single bf16 rounding (8 bits) would leave errors
// of order 1% in sums that cancel (C.h is a sum of N terms of either sign).
// The chunk's inputs for the next chunk are loaded into registers while this
// one is computed.  About 60 KB of LDS per workgroup (N = 128): two
// workgroups share a CU.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <algorithm>
#include <type_traits>

namespace ssm {
namespace {

constexpr int kQ = 64;     // chunk length (4 tiles of 16)
constexpr int64_t kMaxHeadDim = 4096;
constexpr int kPT = 32;    // head channels per workgroup (the head dim P is a multiple)
constexpr int kPTL = kPT / 16;  // MFMA column tiles per workgroup
constexpr int kPadE = 8;   // row padding, bf16 elements (16 bytes)
constexpr int kThreads = 256;

typedef short ssd_s4 __attribute__((ext_vector_type(4)));
typedef __bf16 ssd_b8 __attribute__((ext_vector_type(8)));
typedef float ssd_f4 __attribute__((ext_vector_type(4)));

template <int N>
struct SsdLds {
    static constexpr int nld = N + kPadE;    // rows of N entries: Bs, HT
    static constexpr int tld = kPT + kPadE;  // rows of kPT entries: Xs, Zs (Ys)
    static constexpr int qld = kQ + kPadE;   // rows of kQ entries: XWT
    // XT is read 8 bytes at a time only: rows 136 bytes apart put the 16 rows
    // of one read in disjoint 8-byte bank slots (144, as XWT, pairs rows r, r + 8)
    static constexpr int xld = kQ + 4;
    static constexpr size_t bs = 0;
    static constexpr size_t xs = bs + (size_t)kQ * nld * 2;
    static constexpr size_t zs = xs + (size_t)kQ * tld * 2;
    // HT: [hi/lo plane][kPT channels][nld]
    static constexpr size_t ht = zs + (size_t)kQ * tld * 2;
    static constexpr size_t ht_plane = (size_t)kPT * nld;  // elements
    // XWT: [hi/lo plane][kPT channels][qld]; then XT: x transposed, [kPT][xld]
    static constexpr size_t xwt = ht + 2 * ht_plane * 2;
    static constexpr size_t xwt_plane = (size_t)kPT * qld;
    static constexpr size_t xt = xwt + 2 * xwt_plane * 2;
    static constexpr size_t dts = xt + (size_t)kPT * xld * 2;  // 16-byte aligned (32 rows of 136 bytes)
    // per wave: the chunk's prefix sums of dt a (times log2 e), then its ZOH weights (lane = step)
    static constexpr size_t scal = dts + (size_t)kQ * sizeof(float);
    static constexpr size_t total = scal + (size_t)4 * 2 * kQ * sizeof(float);
    static_assert(xt % 16 == 0 && dts % 16 == 0 && scal % 16 == 0, "16-byte aligned LDS arrays");
};

struct SsdParams {
    int64_t B, L, H, G;
    int64_t P;  // head dim, a multiple of kPT
    const uint16_t *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dskip, *dbias, *h0;
    uint16_t *y;
    float *h_final;
    int softplus;
    // Sequence segments (mode 0: one segment, the whole sequence).  Mode 1:
    // each segment from a zero state, writing only its end state and its
    // sum of dt a; mode 2: each segment from its entering state, writing y.
    int mode;  // selects the kernel instance
    int64_t nseg, seg_chunks;
    float *ws_state;  // (nseg, B, H, P, N): end states, then entering states
    float *ws_lsum;   // (nseg, B, H): sum of dt a over the segment
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
// The 16x16x32 form: 8 bf16 of k per lane.  A and B take their k slots from
// the same (lane group, element) positions, so any assignment of the
// contracted index to slots that both operands share gives the same sum.
#define SSD_MFMA32(a, b, c) __builtin_amdgcn_mfma_f32_16x16x32_bf16((a), (b), (c), 0, 0, 0)

__device__ __forceinline__ ssd_s4 lds4(const uint16_t *p) {
    return __builtin_bit_cast(ssd_s4, *reinterpret_cast<const uint2 *>(p));
}

__device__ __forceinline__ ssd_b8 lds8(const uint16_t *p) {
    return __builtin_bit_cast(ssd_b8, *reinterpret_cast<const uint4 *>(p));
}

// Two 4-entry operands side by side as one 8-entry operand.
__device__ __forceinline__ ssd_b8 cat8(ssd_s4 a, ssd_s4 b) {
    struct Pair {
        ssd_s4 a, b;
    } t = {a, b};
    return __builtin_bit_cast(ssd_b8, t);
}

// The state update's contracted index (the 32 steps of a half chunk) in the
// slots of lane group g and element e (slot 8 g + e) is step
//   8 c + 2 (g ^ c) + (e & 1),  c = e >> 1,
// a permutation chosen so that the four lane groups' 2-byte column reads of
// one element fall in four disjoint 32-byte bank ranges (rows 2 apart are 32
// bytes apart in the bank cycle; rows 8 apart, the identity's choice, hit the
// same banks).  The weighted x it pairs with is stored in slot order.
__device__ __forceinline__ int ssd_slot_of_step(int s) {  // s in 0..63
    const int c = (s >> 3) & 3, g = ((s >> 1) & 3) ^ c;
    return (s & 32) + 8 * g + 2 * c + (s & 1);
}
// Row offsets (elements, row stride ld) of the steps of elements 2c, 2c + 1
// for lane group g.
__device__ __forceinline__ void ssd_slot_rows(int g, int ld, int (&off)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) off[c] = (8 * c + 2 * ((g ^ c) & 3)) * ld;
}
// The eight column entries of a lane's slots (p: the half chunk's first row).
__device__ __forceinline__ ssd_b8 col8_slots(const uint16_t *p, const int (&off)[4], int ld) {
    const ssd_s4 a = {(short)p[off[0]], (short)p[off[0] + ld], (short)p[off[1]], (short)p[off[1] + ld]};
    const ssd_s4 b = {(short)p[off[2]], (short)p[off[2] + ld], (short)p[off[3]], (short)p[off[3] + ld]};
    return cat8(a, b);
}

// Inclusive prefix sum over the 64 lanes of a wave: within each row of 16
// lanes by DPP row shifts (lanes shifted in from outside the row read 0),
// then the totals of the rows before, read from lanes 15, 31 and 47.
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const int row = lane >> 4;
    return v + (row >= 1 ? t0 : 0.0f) + (row >= 2 ? t1 : 0.0f) + (row >= 3 ? t2 : 0.0f);
}

// The chunk's inputs in registers between their global load and their LDS
// store, so that the next chunk's loads are in flight during this chunk's
// products.  Each thread owns KB 16-byte pieces of B, and one 16-byte piece
// each of x and z.
template <int N>
struct ChunkRegs {
    static constexpr int PR = N / 8;  // pieces per B row
    static constexpr int KB = (kQ * PR + kThreads - 1) / kThreads;
    uint4 b[KB], x, z;
    uint16_t dt;  // raw bits: converting here would wait for the load
};

// A wave's C rows, the operand of both its products with C (G^T and C H^T),
// loaded from global memory straight into the operand layout: lane (r16, g)
// holds entries 32 kk + 8 g .. + 7 of step 16 w + r16 (N >= 32; entries
// 16 kk + 4 g .. + 3 for N = 16).  Only this wave reads them, so they need no
// LDS copy; rows past the end are 0.
template <int N>
struct CRows {
    static constexpr int K = N >= 32 ? N / 32 : N / 16;
    using Piece = typename std::conditional<(N >= 32), uint4, uint2>::type;
    Piece v[K];
};

template <int N>
__device__ __forceinline__ void fetch_c(const SsdParams &p, int64_t b, int64_t g, int64_t t0, int w, int lane,
                                        CRows<N> &r) {
    using R = CRows<N>;
    const int64_t t = t0 + 16 * w + (lane & 15);
    const int64_t off = ((b * p.L + t) * p.G + g) * N + (N >= 32 ? 8 : 4) * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < R::K; ++kk) {
        r.v[kk] = typename R::Piece{};
        if (t < p.L) r.v[kk] = *reinterpret_cast<const typename R::Piece *>(p.Cm + off + (N >= 32 ? 32 : 16) * kk);
    }
}

template <int N>
__device__ __forceinline__ void fetch_chunk(const SsdParams &p, int64_t b, int64_t h, int64_t g, int pt,
                                            int64_t t0, bool outputs, int tid, ChunkRegs<N> &r) {
    using R = ChunkRegs<N>;
    const int64_t L = p.L;
#pragma unroll
    for (int k = 0; k < R::KB; ++k) {
        const int id = tid + k * kThreads;
        const int s = id / R::PR, c8 = (id % R::PR) * 8;
        const int64_t t = t0 + s;
        r.b[k] = make_uint4(0, 0, 0, 0);
        if (id < kQ * R::PR && t < L) {
            const int64_t off = ((b * L + t) * p.G + g) * N + c8;
            r.b[k] = *reinterpret_cast<const uint4 *>(p.Bm + off);
        }
    }
    {
        static_assert(kQ * (kPT / 8) == kThreads, "one x and one z piece per thread");
        const int s = tid / (kPT / 8), c8 = (tid % (kPT / 8)) * 8;
        const int64_t t = t0 + s;
        r.x = make_uint4(0, 0, 0, 0);
        r.z = r.x;
        if (t < L) {
            const int64_t off = ((b * L + t) * p.H + h) * p.P + kPT * pt + c8;
            r.x = *reinterpret_cast<const uint4 *>(p.x + off);
            if (p.z && outputs) r.z = *reinterpret_cast<const uint4 *>(p.z + off);
        }
    }
    r.dt = 0;  // bf16 zero: the step of a row past the end
    if (tid < kQ && t0 + tid < L) r.dt = p.delta[(b * L + t0 + tid) * p.H + h];
}

template <int N>
__device__ __forceinline__ void store_chunk(const ChunkRegs<N> &r, uint16_t *Bs, uint16_t *Xs, uint16_t *XT,
                                            uint16_t *Zs, float *dts, int tid, bool row_live, int softplus,
                                            float dbias) {
    using R = ChunkRegs<N>;
    using Lay = SsdLds<N>;
#pragma unroll
    for (int k = 0; k < R::KB; ++k) {
        const int id = tid + k * kThreads;
        if (id < kQ * R::PR) {
            const int s = id / R::PR, c8 = (id % R::PR) * 8;
            *reinterpret_cast<uint4 *>(Bs + s * Lay::nld + c8) = r.b[k];
        }
    }
    {
        const int s = tid / (kPT / 8), c8 = (tid % (kPT / 8)) * 8;
        *reinterpret_cast<uint4 *>(Xs + s * Lay::tld + c8) = r.x;
        *reinterpret_cast<uint4 *>(Zs + s * Lay::tld + c8) = r.z;
        // x transposed (channel-major), the k-contiguous operand of M X
        const uint32_t wv[4] = {r.x.x, r.x.y, r.x.z, r.x.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            XT[(c8 + i) * Lay::xld + s] = (uint16_t)(i % 2 ? wv[i / 2] >> 16 : wv[i / 2] & 0xffffu);
    }
    if (tid < kQ) {
        float dt = bf(r.dt);
        if (softplus && row_live) dt = softplus_fast(dt + dbias);
        dts[tid] = dt;
    }
}

template <int N, int MODE>
__global__ __launch_bounds__(kThreads, 2) void ssd_chunk_kernel(SsdParams p) {
    using Lay = SsdLds<N>;
    constexpr int NT = N / 16;       // state tiles of the head
    constexpr int NW = NT / 4;       // state tiles per wave (N >= 64); see below for N < 64
    constexpr int NWT = NW > 0 ? NW : 1;
    constexpr int nld = Lay::nld, tld = Lay::tld, qld = Lay::qld;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    uint16_t *Bs = reinterpret_cast<uint16_t *>(lds + Lay::bs);
    uint16_t *Xs = reinterpret_cast<uint16_t *>(lds + Lay::xs);
    uint16_t *Zs = reinterpret_cast<uint16_t *>(lds + Lay::zs);
    uint16_t *HT = reinterpret_cast<uint16_t *>(lds + Lay::ht);
    uint16_t *XWT = reinterpret_cast<uint16_t *>(lds + Lay::xwt);
    uint16_t *XT = reinterpret_cast<uint16_t *>(lds + Lay::xt);
    float *dts = reinterpret_cast<float *>(lds + Lay::dts);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // this wave's copy of the chunk scalars (written and read by this wave only)
    float *acum_s = reinterpret_cast<float *>(lds + Lay::scal) + 2 * kQ * w;
    float *wl_s = acum_s + kQ;
    const int r16 = lane & 15, q4 = 4 * (lane >> 4);
    const int kslot = ssd_slot_of_step(lane);  // where step `lane` sits in XWT
    int brow[4];
    ssd_slot_rows(lane >> 4, nld, brow);
    const int64_t seg = (int64_t)blockIdx.x % p.nseg;
    const int64_t bhp = (int64_t)blockIdx.x / p.nseg;
    const int pt = (int)(bhp % (p.P / kPT));
    const int64_t bh = bhp / (p.P / kPT);
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t g = h / (p.H / p.G);
    const int64_t L = p.L;
    const float a = p.A[h];
    const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
    const float dbias = p.dbias ? p.dbias[h] : 0.0f;
    const int tb = w;  // this wave's 16-step row tile
    // column tile j: this lane's head channel kPT pt + 16 j + r16 (local 16 j + r16)

    // State tiles of this wave: st[i][j][v] is entry n = 16 nt + q4 + v of
    // local channel 16 j + r16, nt = NW w + i.  (N < 64: waves beyond NT hold
    // nothing.)
    ssd_f4 st[NWT][kPTL];
    auto my_nt = [&](int i) { return NW > 0 ? NW * w + i : w; };
    const bool owns_state = NW > 0 || w < NT;
    constexpr bool outputs = MODE != 1;
    // the entering state: h0 (or 0) for the whole sequence, 0 for a segment's
    // end state, the combined entering state for a segment's outputs
    const float *hin = MODE == 0 ? p.h0 : MODE == 2 ? p.ws_state + seg * p.B * p.H * p.P * N : nullptr;
    const float *hin_bh = hin ? hin + bh * p.P * N : nullptr;
#pragma unroll
    for (int i = 0; i < NWT; ++i)
#pragma unroll
        for (int j = 0; j < kPTL; ++j) {
            const int nt = my_nt(i), pl = 16 * j + r16;
            float v4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (owns_state && hin_bh) {
#pragma unroll
                for (int v = 0; v < 4; ++v) v4[v] = hin_bh[(kPT * pt + pl) * N + 16 * nt + q4 + v];
            }
            st[i][j] = ssd_f4{v4[0], v4[1], v4[2], v4[3]};
            if (owns_state) store_split4(HT + pl * nld + 16 * nt + q4, Lay::ht_plane, v4);
        }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    const int64_t c_begin = seg * p.seg_chunks;
    const int64_t c_end = c_begin + p.seg_chunks < nchunks ? c_begin + p.seg_chunks : nchunks;
    float lsum = 0.0f;  // sum of dt a over this workgroup's chunks
    ChunkRegs<N> regs;
    CRows<N> crow;
    if (c_begin < c_end) {
        fetch_chunk<N>(p, b, h, g, pt, c_begin * kQ, outputs, tid, regs);
        if constexpr (outputs) fetch_c<N>(p, b, g, c_begin * kQ, w, lane, crow);
    }
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = c * kQ;
        store_chunk<N>(regs, Bs, Xs, XT, Zs, dts, tid, t0 + tid < L, p.softplus, dbias);
        __syncthreads();
        // the next chunk's loads fly while this chunk is computed
        if (c + 1 < c_end) fetch_chunk<N>(p, b, h, g, pt, t0 + kQ, outputs, tid, regs);

        // ---- chunk scalars, one copy per wave (lane = step s) ----------------
        const float dtl = dts[lane];
        const float zl = dtl * a;
        const float acum = wave_prefix_sum(zl, lane);  // inclusive prefix sum of dt a
        const float aend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acum), 63));
        lsum += aend;
        const float wl = dtl * ssd_phi(zl, hw_exp2(zl * kLog2e));       // ZOH input weight
        const float fl = hw_exp2((aend - acum) * kLog2e) * wl;         // weight in the end state
        acum_s[lane] = acum * kLog2e;  // kept in log2 units: the readers exponentiate base 2
        wl_s[lane] = wl;

        // ---- X' = f x -> XWT[p][slot of s] (hi, lo): wave w takes channels 8w .. 8w+7
        // of step s = lane, one 16-byte row read (read after the middle barrier)
        {
            static_assert(kPT / 4 == 8, "one 16-byte piece of x per lane");
            const uint4 q = *reinterpret_cast<const uint4 *>(Xs + lane * tld + 8 * w);
            const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int pp = 8 * w + i;
                const uint16_t xb = (uint16_t)(i % 2 ? wv[i / 2] >> 16 : wv[i / 2] & 0xffffu);
                const float v = bf(xb) * fl;
                const uint16_t hi = f32_to_bf16_bits(v);
                XWT[pp * qld + kslot] = hi;
                XWT[Lay::xwt_plane + pp * qld + kslot] = f32_to_bf16_bits(v - bf(hi));
            }
        }

        if constexpr (outputs) {
            // The matrix-core phases (G^T tiles and outputs, the state update) run at a
            // raised wave priority, the staging and barriers around them at the base
            // one, so a CU's two workgroups drift out of phase.  Measured in one
            // process against the same kernel without it: 2-4% faster, outputs
            // bit-identical.
            __builtin_amdgcn_s_setprio(2);
            // ---- this wave's G^T tiles, masked and decayed in place ---------------------
            // Only the s tiles on or below the diagonal are formed (the rest stay 0).
            // The count is a compile-time constant in one copy of the loop per wave
            // index, so the operand loads still run ahead of the MFMAs in
            // straight-line code.
            ssd_f4 gacc[kQ / 16];
    #pragma unroll
            for (int sb = 0; sb < kQ / 16; ++sb) gacc[sb] = ssd_f4{0.0f, 0.0f, 0.0f, 0.0f};
            auto gt_tiles = [&](auto TBc) {
                constexpr int TB = decltype(TBc)::value;
                if constexpr (N >= 32) {
    #pragma unroll
                    for (int kk = 0; kk < N / 32; ++kk) {
                        const ssd_b8 cop = __builtin_bit_cast(ssd_b8, crow.v[kk]);
    #pragma unroll
                        for (int sb = 0; sb <= TB; ++sb)
                            gacc[sb] = SSD_MFMA32(lds8(Bs + (16 * sb + r16) * nld + 32 * kk + 2 * q4), cop, gacc[sb]);
                    }
                } else {
    #pragma unroll
                    for (int kk = 0; kk < NT; ++kk) {
                        const ssd_s4 cop = __builtin_bit_cast(ssd_s4, crow.v[kk]);
    #pragma unroll
                        for (int sb = 0; sb <= TB; ++sb)
                            gacc[sb] = SSD_MFMA(lds4(Bs + (16 * sb + r16) * nld + 16 * kk + q4), cop, gacc[sb]);
                    }
                }
            };
            static_assert(kQ / 16 == 4, "four row tiles per chunk");
            switch (__builtin_amdgcn_readfirstlane(tb)) {
                case 0: gt_tiles(std::integral_constant<int, 0>()); break;
                case 1: gt_tiles(std::integral_constant<int, 1>()); break;
                case 2: gt_tiles(std::integral_constant<int, 2>()); break;
                default: gt_tiles(std::integral_constant<int, 3>()); break;
            }
            // lane holds s = 16 sb + q4 + v, t = 16 tb + r16: M[t][s], the A operand
            // (row t, k = s) of M X as it stands
            ssd_s4 mhi[kQ / 16], mlo[kQ / 16];
            {
                const float at = acum_s[16 * tb + r16];  // log2 units
    #pragma unroll
                for (int sb = 0; sb < kQ / 16; ++sb) {
                    if (sb > tb) {  // above the diagonal (wave-uniform): all zero
                        mhi[sb] = mlo[sb] = ssd_s4{0, 0, 0, 0};
                        continue;
                    }
                    const float4 as4 = *reinterpret_cast<const float4 *>(acum_s + 16 * sb + q4);
                    const float4 ws4 = *reinterpret_cast<const float4 *>(wl_s + 16 * sb + q4);
                    const float as[4] = {as4.x, as4.y, as4.z, as4.w}, ws[4] = {ws4.x, ws4.y, ws4.z, ws4.w};
                    float m[4];
                    if (sb < tb) {  // below the diagonal (wave-uniform): every s <= t
    #pragma unroll
                        for (int v = 0; v < 4; ++v) m[v] = gacc[sb][v] * hw_exp2(at - as[v]) * ws[v];
                    } else {
    #pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int s = 16 * sb + q4 + v;
                            m[v] = s <= 16 * tb + r16 ? gacc[sb][v] * hw_exp2(at - as[v]) * ws[v] : 0.0f;
                        }
                    }
                    uint2 hi, lo;
                    split4(m, hi, lo);
                    mhi[sb] = __builtin_bit_cast(ssd_s4, hi);
                    mlo[sb] = __builtin_bit_cast(ssd_s4, lo);
                }
            }

            // ---- Y for this wave's 16 steps and the workgroup's channels --------------
            {
                ssd_f4 acc[kPTL], acc2[kPTL];
    #pragma unroll
                for (int j = 0; j < kPTL; ++j) acc[j] = acc2[j] = ssd_f4{0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (N >= 32) {
    #pragma unroll
                    for (int kk = 0; kk < N / 32; ++kk) {
                        const ssd_b8 cop = __builtin_bit_cast(ssd_b8, crow.v[kk]);
    #pragma unroll
                        for (int j = 0; j < kPTL; ++j) {
                            const uint16_t *hp = HT + (16 * j + r16) * nld + 32 * kk + 2 * q4;
                            acc[j] = SSD_MFMA32(cop, lds8(hp), acc[j]);
                            acc2[j] = SSD_MFMA32(cop, lds8(hp + Lay::ht_plane), acc2[j]);
                        }
                    }
                } else {
    #pragma unroll
                    for (int kk = 0; kk < NT; ++kk) {
                        const ssd_s4 cop = __builtin_bit_cast(ssd_s4, crow.v[kk]);
    #pragma unroll
                        for (int j = 0; j < kPTL; ++j) {
                            const uint16_t *hp = HT + (16 * j + r16) * nld + 16 * kk + q4;
                            acc[j] = SSD_MFMA(cop, lds4(hp), acc[j]);
                            acc2[j] = SSD_MFMA(cop, lds4(hp + Lay::ht_plane), acc2[j]);
                        }
                    }
                }
                // lane holds t = 16 tb + q4 + v, local channel 16 j + r16
                float dec[4];
                {
                    const float4 a4 = *reinterpret_cast<const float4 *>(acum_s + 16 * tb + q4);
                    dec[0] = hw_exp2(a4.x);
                    dec[1] = hw_exp2(a4.y);
                    dec[2] = hw_exp2(a4.z);
                    dec[3] = hw_exp2(a4.w);
                }
    #pragma unroll
                for (int j = 0; j < kPTL; ++j) {
                    acc[j] += acc2[j];
    #pragma unroll
                    for (int v = 0; v < 4; ++v) acc[j][v] *= dec[v];
                }
                // two s tiles per product: slot (lane group, e) is step 16 sb + q4 + e
                // of the pair's first tile for e < 4, of its second tile for e >= 4
    #pragma unroll
                for (int sp = 0; sp < kQ / 32; ++sp) {  // tiles above the diagonal are 0
                    const int s0 = 32 * sp, s1 = 32 * sp + 16;
                    const ssd_b8 ahi = cat8(mhi[2 * sp], mhi[2 * sp + 1]), alo = cat8(mlo[2 * sp], mlo[2 * sp + 1]);
    #pragma unroll
                    for (int j = 0; j < kPTL; ++j) {
                        const uint16_t *xr = XT + (16 * j + r16) * Lay::xld;
                        const ssd_b8 xop = cat8(lds4(xr + s0 + q4), lds4(xr + s1 + q4));
                        acc[j] = SSD_MFMA32(ahi, xop, acc[j]);
                        acc[j] = SSD_MFMA32(alo, xop, acc[j]);
                    }
                }
                // skip and gate; the result replaces the gate entry it used
    #pragma unroll
                for (int j = 0; j < kPTL; ++j)
    #pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = 16 * tb + q4 + v, pl = 16 * j + r16;
                        float yv = acc[j][v] + dsk * bf(Xs[t * tld + pl]);
                        if (p.z) yv *= silu(bf(Zs[t * tld + pl]));
                        Zs[t * tld + pl] = f32_to_bf16_bits(yv);
                    }
            }
            // this wave's C rows of the next chunk, in flight until its G^T
            if (c + 1 < c_end) fetch_c<N>(p, b, g, t0 + kQ, w, lane, crow);
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();  // XWT and Ys (in Zs) complete; every read of HT done

        if constexpr (outputs) {
            // ---- outputs leave as 16-byte pieces, one per thread --------------------
            {
                const int t = tid / (kPT / 8), c8 = (tid % (kPT / 8)) * 8;
                const int64_t tt = t0 + t;
                if (tt < L)
                    *reinterpret_cast<uint4 *>(p.y + ((b * L + tt) * p.H + h) * p.P + kPT * pt + c8) =
                        *reinterpret_cast<const uint4 *>(Zs + t * tld + c8);
            }
        }

        // ---- this wave's state tiles for the next chunk ----------------------------
        __builtin_amdgcn_s_setprio(2);
        if (owns_state) {
            const float dend = hw_exp2(aend * kLog2e);
#pragma unroll
            for (int i = 0; i < NWT; ++i)
#pragma unroll
                for (int j = 0; j < kPTL; ++j) st[i][j] *= dend;
            // slot (lane group g, e) holds step 32 kk + 8 c + 2 (g ^ c) + (e & 1), c = e / 2
#pragma unroll
            for (int kk = 0; kk < kQ / 32; ++kk) {
                ssd_b8 bop[NWT];
#pragma unroll
                for (int i = 0; i < NWT; ++i)
                    bop[i] = col8_slots(Bs + 32 * kk * nld + 16 * my_nt(i) + r16, brow, nld);
#pragma unroll
                for (int j = 0; j < kPTL; ++j) {
                    const uint16_t *xp = XWT + (16 * j + r16) * qld + 32 * kk + 2 * q4;
                    const ssd_b8 xhi = lds8(xp), xlo = lds8(xp + Lay::xwt_plane);
#pragma unroll
                    for (int i = 0; i < NWT; ++i) {
                        st[i][j] = SSD_MFMA32(bop[i], xhi, st[i][j]);
                        st[i][j] = SSD_MFMA32(bop[i], xlo, st[i][j]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NWT; ++i)
#pragma unroll
                for (int j = 0; j < kPTL; ++j) {
                    const float v4[4] = {st[i][j][0], st[i][j][1], st[i][j][2], st[i][j][3]};
                    store_split4(HT + (16 * j + r16) * nld + 16 * my_nt(i) + q4, Lay::ht_plane, v4);
                }
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();  // inputs free for the next chunk; HT holds the new state
    }

    // the final state (whole sequence), or a segment's end state and decay
    float *hout = MODE == 0 ? p.h_final : MODE == 1 ? p.ws_state + seg * p.B * p.H * p.P * N : nullptr;
    if (hout && owns_state) {
#pragma unroll
        for (int i = 0; i < NWT; ++i)
#pragma unroll
            for (int j = 0; j < kPTL; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    hout[(bh * p.P + kPT * pt + 16 * j + r16) * N + 16 * my_nt(i) + q4 + v] = st[i][j][v];
    }
    if (MODE == 1 && pt == 0 && tid == 0) p.ws_lsum[seg * p.B * p.H + bh] = lsum;
}

// The segments' entering states: H_0 = h0 (or 0), H_{k+1} = e^{lsum_k} H_k +
// E_k with E_k segment k's end state from a zero start (exact: the layer is
// linear in its entering state).  Slot k of the workspace trades E_k for H_k;
// the last H is the final state.  One thread per state entry.
__global__ __launch_bounds__(256) void ssd_seg_combine_kernel(float *ws_state, const float *ws_lsum, const float *h0,
                                                              float *h_final, int64_t BH, int64_t PN, int64_t nseg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BH * PN) return;
    const int64_t bh = i / PN;
    float hs = h0 ? h0[i] : 0.0f;
    for (int64_t k = 0; k < nseg; ++k) {
        float *slot = ws_state + k * BH * PN + i;
        const float e = *slot;
        *slot = hs;
        hs = __expf(ws_lsum[k * BH + bh]) * hs + e;
    }
    if (h_final) h_final[i] = hs;
}

template <int N>
hipError_t launch_n(const SsdParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)(p.B * p.H * (p.P / kPT) * p.nseg);
    const size_t lds = SsdLds<N>::total;
    if (p.mode == 1)
        ssd_chunk_kernel<N, 1><<<grid, kThreads, lds, stream>>>(p);
    else if (p.mode == 2)
        ssd_chunk_kernel<N, 2><<<grid, kThreads, lds, stream>>>(p);
    else
        ssd_chunk_kernel<N, 0><<<grid, kThreads, lds, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_dstate(const SsdParams &p, int64_t N, hipStream_t stream) {
    switch (N) {
        case 16: return launch_n<16>(p, stream);
        case 32: return launch_n<32>(p, stream);
        case 64: return launch_n<64>(p, stream);
        default: return launch_n<128>(p, stream);
    }
}

// Segments: when the (batch, head, channel half) workgroups would fill at
// most half of the resident slots (two per CU), the sequence is cut into
// segments of at least kMinSegChunks chunks, as many as still run in one
// round (up to kMaxSeg).  The end-state pass and the combine cost about half
// a pass, so fuller launches are left whole.
constexpr int64_t kSlotsWanted = 2 * 256;
constexpr int64_t kMinSegChunks = 4;
constexpr int64_t kMaxSeg = 64;

struct SsdPlan {
    int64_t nseg, seg_chunks;
    size_t ws_state, ws_lsum;
};

SsdPlan ssd_plan(const ssm_ssd_args_t &a) {
    SsdPlan q{1, 0, 0, 0};
    const int64_t nchunks = (a.seqlen + kQ - 1) / kQ;
    q.seg_chunks = nchunks;
    const int64_t wgs = a.batch * a.nheads * (a.headdim / kPT);
    if (wgs > 0 && 2 * wgs <= kSlotsWanted) {
        int64_t s = std::min<int64_t>({kMaxSeg, kSlotsWanted / wgs, nchunks / kMinSegChunks});
        if (s > 1) {
            q.seg_chunks = (nchunks + s - 1) / s;
            q.nseg = (nchunks + q.seg_chunks - 1) / q.seg_chunks;
        }
    }
    if (q.nseg > 1) {
        auto r256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
        q.ws_state = r256((size_t)(q.nseg * a.batch * a.nheads * a.headdim * a.dstate) * sizeof(float));
        q.ws_lsum = r256((size_t)(q.nseg * a.batch * a.nheads) * sizeof(float));
    }
    return q;
}

// ---- decode: one token on a resident state -----------------------------------
//
// The same layer in recurrent mode for one step: per (batch, head, channel p)
// the state row S[p, :] (N fp32) becomes alpha S + w x B and y = (S . C +
// D x) silu(z).  A workgroup takes 2 * 256 / (N / 4) channels of one (batch,
// head), so the step, its decay and weight, and the B and C rows are the same
// for all of its lanes; each lane owns 4 consecutive state entries of one
// channel in each of two rounds (16 bytes, loaded and stored once, both loads
// issued first) and the N / 4 lanes of a channel, one aligned lane group, sum
// their partial S . C by xor shuffles.  Bound by moving the fp32 state
// through HBM.
struct SsdStepParams {
    int64_t B, H, P, G;
    const uint16_t *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dskip, *dbias;
    float *state;
    uint16_t *y;
    int softplus;
};

constexpr int kStepRounds = 2;

// Tile t: channels [tile * 2 CPR, (tile + 1) * 2 CPR) of (batch, head) bh, t = bh * ntiles + tile.
template <int Q4>  // lanes per channel: N = 4 Q4
__device__ __forceinline__ void ssd_step_tile(const SsdStepParams &p, int64_t t, int64_t ntiles) {
    constexpr int N = 4 * Q4;
    constexpr int CPR = 256 / Q4;  // channels per round
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int64_t bh = t / ntiles;
    const int64_t tile = t - bh * ntiles;
    const int64_t h = bh % p.H, b = bh / p.H;
    const int64_t grp = h / (p.H / p.G);
    const int q = threadIdx.x % Q4;
    const int c0 = threadIdx.x / Q4;
    f4v s[kStepRounds];
    int64_t pch[kStepRounds];
#pragma unroll
    for (int r = 0; r < kStepRounds; ++r) {
        pch[r] = tile * (kStepRounds * CPR) + r * CPR + c0;
        const int64_t pc = pch[r] < p.P ? pch[r] : 0;
        s[r] = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p.state + (bh * p.P + pc) * N + 4 * q));
    }
    const uint2 bq = *reinterpret_cast<const uint2 *>(p.Bm + (b * p.G + grp) * N + 4 * q);
    const uint2 cq = *reinterpret_cast<const uint2 *>(p.Cm + (b * p.G + grp) * N + 4 * q);
    float dt = bf(p.delta[bh]);
    if (p.softplus) dt = softplus_fast(dt + (p.dbias ? p.dbias[h] : 0.0f));
    const float za = dt * p.A[h];
    const float e = hw_exp2(za * kLog2e);  // decay of the step
    const float wdt = dt * ssd_phi(za, e);  // ZOH input weight
    const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
    const float bv[4] = {__uint_as_float(bq.x << 16), __uint_as_float(bq.x & 0xffff0000u),
                         __uint_as_float(bq.y << 16), __uint_as_float(bq.y & 0xffff0000u)};
    const float cv[4] = {__uint_as_float(cq.x << 16), __uint_as_float(cq.x & 0xffff0000u),
                         __uint_as_float(cq.y << 16), __uint_as_float(cq.y & 0xffff0000u)};
#pragma unroll
    for (int r = 0; r < kStepRounds; ++r) {
        const bool live = pch[r] < p.P;
        const int64_t ch = bh * p.P + (live ? pch[r] : 0);
        const float u = bf(p.x[ch]);
        const float wu = wdt * u;
        float hn[4];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hn[i] = __builtin_fmaf(e, s[r][i], wu * bv[i]);
            part = __builtin_fmaf(hn[i], cv[i], part);
        }
#pragma unroll
        for (int m = Q4 / 2; m >= 1; m /= 2) part += __shfl_xor(part, m, 64);
        if (live) {
            const f4v o = {hn[0], hn[1], hn[2], hn[3]};
            __builtin_nontemporal_store(o, reinterpret_cast<f4v *>(p.state + ch * N + 4 * q));
            if (q == 0) {
                float yv = part + dsk * u;
                if (p.z) yv *= silu(bf(p.z[ch]));
                p.y[ch] = f32_to_bf16_bits(yv);
            }
        }
    }
}

// One tile per workgroup; a loop over tiles where there are more than one grid
// takes (a loop costs ~9% of the step even when it runs once, so it is kept out
// of the common case).
template <int Q4, bool LOOP>
__global__ __launch_bounds__(256) void ssd_step_kernel(SsdStepParams p, int64_t ntiles, int64_t total) {
    if (!LOOP) {
        ssd_step_tile<Q4>(p, blockIdx.x, ntiles);
        return;
    }
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) ssd_step_tile<Q4>(p, t, ntiles);
}

constexpr int64_t kStepMaxGrid = (int64_t)1 << 22;

template <int Q4>
void launch_step_q4(const SsdStepParams &p, hipStream_t stream) {
    const int64_t per_tile = kStepRounds * (256 / Q4);
    const int64_t ntiles = (p.P + per_tile - 1) / per_tile;
    const int64_t total = p.B * p.H * ntiles;
    if (total <= kStepMaxGrid)
        ssd_step_kernel<Q4, false><<<(unsigned)total, 256, 0, stream>>>(p, ntiles, total);
    else
        ssd_step_kernel<Q4, true><<<(unsigned)kStepMaxGrid, 256, 0, stream>>>(p, ntiles, total);
}

// ---- fp32 I/O: the recurrent form over the whole sequence ---------------------
//
// The matrix-core chunks take bf16 operands, which fp32 inputs do not fit
// without losing the fp32 bound, so fp32 I/O runs the layer in its recurrent
// form ("14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상", sec. 5.1: the
// same map as the quadratic form): sequential in time with the state in
// registers, in fp32 throughout.
//
// A lane holds 8 consecutive state entries (a slice) of one (head, channel)
// pair.  A wave holds Q slices of 64 / Q pairs of one (batch, group), Q = 4
// (2 when N = 16): lane = q (64 / Q) + channel.  The W = N / (8 Q) waves of a
// workgroup hold the other slices of the same pairs, so the workgroup covers
// 64 / Q pairs whole.  A step's B and C entries depend on the slice only.
// Each wave fetches its slices' B and C for 16 steps with Q 16-byte loads per
// lane, a round ahead, and keeps them in a wave-private LDS area from which
// every step reads them as broadcasts (Q addresses per read, in disjoint
// banks).  Per step each lane adds its slice's share of C h into LDS; every
// 16 steps the workgroup adds the shares of each (step, pair) in a fixed
// order and applies the skip and the gate.  Steps past the end run with
// dt = 0 and x = 0, which leaves the state as it is, and store nothing.
struct SsdF32Params {
    int64_t B, L, H, P, G;
    const float *x, *delta, *Bm, *Cm, *z, *A, *Dskip, *dbias, *h0;
    float *y, *h_final;
    int softplus;
};

constexpr int kF32E = 8;   // state entries per lane (a slice)
constexpr int kF32K = 16;  // steps per read-out round
constexpr int kF32U = 4;   // steps whose x and dt are requested together

// Slices per wave, pairs per wave and waves per workgroup for N / 8 slices.
template <int S>
struct F32Shape {
    static constexpr int Q = S < 4 ? S : 4;
    static constexpr int C = 64 / Q;
    static constexpr int W = S / Q;
};

struct F32Lane {
    const float *xl, *zl, *dl, *bw, *cw;
    float *yl;
    float a2, ia, dsk, dbias;
    int lane;
    bool live;
};

// The rounds of 16 steps.  FAST: every pair of the wave has |a| >= 1/16, and
// the input weight (e - 1)/a is one fma with 1/a (as the S6 scan's fast form);
// otherwise dt phi(dt a), series near 0.  Both variants pass the same
// barriers.
template <int S, bool FAST, bool SOFTPLUS>
__device__ __forceinline__ void f32_rounds(const SsdF32Params &p, const F32Lane &l, float (&st)[kF32E],
                                           float (&share)[F32Shape<S>::W][kF32K][64],
                                           float4 (&bcs)[kF32K * F32Shape<S>::Q * 4], int w, float a) {
    using Sh = F32Shape<S>;
    constexpr int Q = Sh::Q, C = Sh::C, W = Sh::W;
    const int64_t L = p.L, HP = p.H * p.P, GN = p.G * kF32E * S;
    const int lane = l.lane, q = lane / C;
    if (L == 0) return;  // the state passes through
    // piece j of this lane's share of the wave's B and C for steps t0 ..
    // t0 + 15: element (j 64 + lane) of bcs, laid out as [step][slice][B lo,
    // B hi, C lo, C hi]
    auto fetch_bc = [&](int64_t t0, int j) -> float4 {
        const int idx = j * 64 + lane;
        const int k = idx / (4 * Q), qq = (idx >> 2) % Q, piece = idx & 3;
        const int64_t t = t0 + k;
        const int64_t tb = t < L ? t : L - 1;  // a step that exists (unused past the end)
        const float *src = ((piece & 2) ? l.cw : l.bw) + tb * GN + kF32E * qq + 4 * (piece & 1);
        return *reinterpret_cast<const float4 *>(src);
    };
    float xs[kF32U], ds[kF32U];
    auto request = [&](int64_t t0) {  // x and raw dt of steps t0 .. t0 + kF32U - 1 (0 past the end)
#pragma unroll
        for (int u = 0; u < kF32U; ++u) {
            const bool in = l.live && t0 + u < L;
            const int64_t tc = in ? t0 + u : 0;
            xs[u] = in ? l.xl[tc * HP] : 0.0f;
            ds[u] = in ? l.dl[tc * p.H] : 0.0f;
        }
    };
    float4 bc_next[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) bc_next[j] = fetch_bc(0, j);
    request(0);
    for (int64_t t0 = 0; t0 < L; t0 += kF32K) {
#pragma unroll
        for (int j = 0; j < Q; ++j) bcs[j * 64 + lane] = bc_next[j];  // wave-private
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < Q; ++j) bc_next[j] = fetch_bc(t0 + kF32K, j);
        // each step's B and C are read from LDS one step ahead of their use
        const float4 *mine = bcs + 4 * q;
        float4 q0 = mine[0], q1 = mine[1], q2 = mine[2], q3 = mine[3];
        for (int k0 = 0; k0 < kF32K; k0 += kF32U) {
            float xc[kF32U], dc[kF32U];
#pragma unroll
            for (int u = 0; u < kF32U; ++u) {
                xc[u] = xs[u];
                dc[u] = ds[u];
            }
            request(t0 + k0 + kF32U);
#pragma unroll
            for (int u = 0; u < kF32U; ++u) {
                const int k = k0 + u;
                const float4 b0 = q0, b1 = q1, c0 = q2, c1 = q3;
                const int kn = k + 1 < kF32K ? k + 1 : k;
                const float4 *nx = mine + kn * 4 * Q;
                q0 = nx[0];
                q1 = nx[1];
                q2 = nx[2];
                q3 = nx[3];
                const float bt[kF32E] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                const float ct[kF32E] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                float dt = dc[u];
                if (SOFTPLUS) dt = t0 + k < L ? softplus_fast(dt + l.dbias) : 0.0f;
                const float e = hw_exp2(dt * l.a2);
                const float wdt = FAST ? __builtin_fmaf(e, l.ia, -l.ia) : dt * ssd_phi(dt * a, e);
                const float wx = wdt * xc[u];
                float part = 0.0f;
#pragma unroll
                for (int i = 0; i < kF32E; ++i) {
                    st[i] = __builtin_fmaf(e, st[i], wx * bt[i]);
                    part = __builtin_fmaf(st[i], ct[i], part);
                }
                share[w][k][lane] = part;
            }
        }
        __syncthreads();
        // y of (step k, pair c): the N / 8 slice shares, waves outer, slices inner
        for (int o = threadIdx.x; o < kF32K * C; o += 64 * W) {
            const int k = o / C, c = o - k * C;
            const int64_t t = t0 + k;
            float sum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww)
#pragma unroll
                for (int qq = 0; qq < Q; ++qq) sum += share[ww][k][qq * C + c];
            // x, z and y of pair c sit c - (lane mod C) channels from this lane's
            const int64_t off = t * HP + (c - (lane % C));
            if (l.live && t < L) {
                float yv = sum + l.dsk * l.xl[off];
                if (l.zl) yv *= silu(l.zl[off]);
                l.yl[off] = yv;
            }
        }
        __syncthreads();
    }
}

template <int S, bool SOFTPLUS>
__global__ __launch_bounds__(64 * F32Shape<S>::W) void ssd_scan_f32_kernel(SsdF32Params p, int64_t ntiles) {
    using Sh = F32Shape<S>;
    constexpr int N = kF32E * S, Q = Sh::Q, C = Sh::C, W = Sh::W;
    __shared__ float share[W][kF32K][64];
    __shared__ float4 bcs[W][kF32K * Q * 4];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // w: uniform
    const int q = lane / C, slice = w * Q + q;
    const int64_t bg = blockIdx.x / ntiles, tile = blockIdx.x - bg * ntiles;
    const int64_t b = bg / p.G, g = bg - b * p.G;
    const int64_t hpg = p.H / p.G;
    const int64_t pair = tile * C + lane % C;  // (head within the group) P + channel
    F32Lane l;
    l.lane = lane;
    l.live = pair < hpg * p.P;
    const int64_t pr = l.live ? pair : 0;
    const int64_t hl = pr / p.P;
    const int64_t h = g * hpg + hl, pc = pr - hl * p.P;
    const int64_t L = p.L, HP = p.H * p.P;
    const float a = p.A[h];
    l.ia = fabsf(a) >= 0.0625f ? 1.0f / a : 0.0f;
    l.a2 = a * kLog2e;
    l.dsk = p.Dskip ? p.Dskip[h] : 0.0f;
    l.dbias = p.dbias ? p.dbias[h] : 0.0f;
    l.xl = p.x + b * L * HP + h * p.P + pc;  // step t at t HP
    l.zl = p.z ? p.z + b * L * HP + h * p.P + pc : nullptr;
    l.yl = p.y + b * L * HP + h * p.P + pc;
    l.dl = p.delta + b * L * p.H + h;  // step t at t H
    l.bw = p.Bm + (b * L * p.G + g) * N + kF32E * Q * w;  // the wave's slices; step t at t G N
    l.cw = p.Cm + (b * L * p.G + g) * N + kF32E * Q * w;
    const int64_t slot = ((b * p.H + h) * p.P + pc) * N + kF32E * slice;  // this lane's entries of h0 / h_final
    float st[kF32E];
#pragma unroll
    for (int i = 0; i < kF32E; ++i) st[i] = (p.h0 && l.live) ? p.h0[slot + i] : 0.0f;
    if (__all(fabsf(a) >= 0.0625f))
        f32_rounds<S, true, SOFTPLUS>(p, l, st, share, bcs[w], w, a);
    else
        f32_rounds<S, false, SOFTPLUS>(p, l, st, share, bcs[w], w, a);
    if (p.h_final && l.live) {
#pragma unroll
        for (int i = 0; i < kF32E; ++i) p.h_final[slot + i] = st[i];
    }
}

template <int S>
hipError_t launch_f32_s(const SsdF32Params &p, hipStream_t stream) {
    using Sh = F32Shape<S>;
    const int64_t ntiles = (p.H / p.G * p.P + Sh::C - 1) / Sh::C;
    const unsigned grid = (unsigned)(p.B * p.G * ntiles);
    if (p.softplus) ssd_scan_f32_kernel<S, true><<<grid, 64 * Sh::W, 0, stream>>>(p, ntiles);
    else ssd_scan_f32_kernel<S, false><<<grid, 64 * Sh::W, 0, stream>>>(p, ntiles);
    return hipGetLastError();
}

hipError_t launch_ssd_f32(const ssm_ssd_args_t &a, hipStream_t stream) {
    SsdF32Params p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.H = a.nheads;
    p.P = a.headdim;
    p.G = a.ngroups;
    p.x = static_cast<const float *>(a.x);
    p.delta = static_cast<const float *>(a.delta);
    p.Bm = static_cast<const float *>(a.Bm);
    p.Cm = static_cast<const float *>(a.Cm);
    p.z = static_cast<const float *>(a.z);
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.h0 = a.h0;
    p.y = static_cast<float *>(a.y);
    p.h_final = a.h_final;
    p.softplus = a.delta_softplus;
    switch (a.dstate) {
        case 16: return launch_f32_s<2>(p, stream);
        case 32: return launch_f32_s<4>(p, stream);
        case 64: return launch_f32_s<8>(p, stream);
        default: return launch_f32_s<16>(p, stream);
    }
}

}  // namespace

bool ssd_step_supported(int64_t dstate) {
    return dstate >= 4 && dstate <= 256 && (dstate & (dstate - 1)) == 0;
}

hipError_t launch_ssd_step(const ssm_ssd_step_args_t &a, hipStream_t stream) {
    SsdStepParams p;
    p.B = a.batch;
    p.H = a.nheads;
    p.P = a.headdim;
    p.G = a.ngroups;
    p.x = static_cast<const uint16_t *>(a.x);
    p.delta = static_cast<const uint16_t *>(a.delta);
    p.Bm = static_cast<const uint16_t *>(a.Bm);
    p.Cm = static_cast<const uint16_t *>(a.Cm);
    p.z = static_cast<const uint16_t *>(a.z);
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.state = a.state;
    p.y = static_cast<uint16_t *>(a.y);
    p.softplus = a.delta_softplus;
    switch (a.dstate / 4) {
        case 1: launch_step_q4<1>(p, stream); break;
        case 2: launch_step_q4<2>(p, stream); break;
        case 4: launch_step_q4<4>(p, stream); break;
        case 8: launch_step_q4<8>(p, stream); break;
        case 16: launch_step_q4<16>(p, stream); break;
        case 32: launch_step_q4<32>(p, stream); break;
        default: launch_step_q4<64>(p, stream); break;
    }
    return hipGetLastError();
}

bool ssd_supported(int64_t headdim, int64_t dstate) {
    return headdim >= kPT && headdim <= kMaxHeadDim && headdim % kPT == 0 &&
           (dstate == 16 || dstate == 32 || dstate == 64 || dstate == 128);
}

size_t ssd_workspace_bytes(const ssm_ssd_args_t &a) {
    if (a.io_dtype == SSM_F32) return 0;  // the recurrent form needs none
    const SsdPlan q = ssd_plan(a);
    return q.ws_state + q.ws_lsum;
}

hipError_t launch_ssd_fwd(const ssm_ssd_args_t &a, hipStream_t stream) {
    if (a.io_dtype == SSM_F32) return launch_ssd_f32(a, stream);
    SsdParams p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.H = a.nheads;
    p.G = a.ngroups;
    p.P = a.headdim;
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
    const SsdPlan q = ssd_plan(a);
    p.nseg = q.nseg;
    p.seg_chunks = q.seg_chunks;
    p.ws_state = nullptr;
    p.ws_lsum = nullptr;
    if (q.nseg <= 1) {
        p.mode = 0;
        return launch_dstate(p, a.dstate, stream);
    }
    char *ws = static_cast<char *>(a.workspace);
    p.ws_state = reinterpret_cast<float *>(ws);
    p.ws_lsum = reinterpret_cast<float *>(ws + q.ws_state);
    p.mode = 1;
    hipError_t e = launch_dstate(p, a.dstate, stream);
    if (e != hipSuccess) return e;
    const int64_t BH = a.batch * a.nheads, PN = a.headdim * a.dstate;
    ssd_seg_combine_kernel<<<(unsigned)((BH * PN + 255) / 256), 256, 0, stream>>>(p.ws_state, p.ws_lsum, a.h0,
                                                                                 a.h_final, BH, PN, q.nseg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.mode = 2;
    return launch_dstate(p, a.dstate, stream);
}

}  // namespace ssm
