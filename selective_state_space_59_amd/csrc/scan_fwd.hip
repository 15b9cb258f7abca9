// scan_fwd.hip -- selective scan (S6) forward on gfx950.
//
// Computes, per batch b, channel d and state index n (paper summary page
// "Mamba: Linear-Time Sequence Modeling with Selective State Spaces",
// sec. 4b eq. (4) and eq. (2a)/(2b), Algorithm 2; the skip of
// "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상" sec. 3.1; the conv
// prologue and gate of the summary page's sec. 4a):
//   Abar = exp(dt A),  Bbar u = (exp(dt A) - 1) / A * B u   (dt B u if A == 0)
//   h    = Abar h + Bbar u,   y = (sum_n C h + D u) * silu(z)
//
// Work decomposition ("row" layout).  One lane owns one (channel, state
// index) chain; a 16-lane row of the wave holds the 16 state entries of one
// channel, so a wave covers 4 channels and every workgroup is one wave.
// With N = 16 the 130M-like layer (B=8, D=1536) becomes 3072 waves and the
// 2.8B-like layer 5120 waves: 3 and 5 per SIMD, evenly spread.
//
// Time advances in blocks of 16 steps.  Within a block:
//   * each lane loads x/delta/z of ITS OWN step (t0 + n) for its channel and
//     computes u (conv prologue) and dt there, once per (t, channel); the
//     conv's 3-step history comes from the neighbouring lanes of the row
//     (and the previous block's lanes 13..15) through DPP shifts;
//   * the recurrence of step k reads dt and u of step k from lane k of the
//     row through a DPP row broadcast folded into the multiply (no memory);
//   * the B and C rows (shared by all channels) reach every row of the wave
//     through the matrix cores: one MFMA with a 0/1 selector matrix copies
//     4 steps x 16 entries of B (or C), loaded from memory as an MFMA
//     operand, into 4 registers of every lane, exactly (bf16 -> fp32 for
//     free), keeping the broadcast off the LDS and the vector ALU;
//   * each lane keeps its 16 partial read-outs C_{t,n} h_{t,n}; they are
//     transposed through LDS so lane (c, j) sums the 16 partials of step
//     t0 + j and applies the skip, the gate and the store.
// Global memory goes through buffer descriptors built once per launch;
// each lane advances a 32-bit offset per block.  Reads past the end of the
// sequence (or of the channel range) return 0 and such writes are dropped,
// so the ragged tail needs no branches.  Inputs are requested two blocks
// ahead.  The (B, L, D, N) state never leaves registers.
//
// Vector-ALU cost per state update (the binding resource): one exp (two
// issue slots on gfx950) and six fp32 ops:
//   zz = dt*A*log2e; e = 2^zz; bu = B*u; q = bu/A; bx = e*q - q (fused);
//   h = e*h + bx (fused); p = C*h.
// bx = fma(e, q, -q) makes dt = 0 hold the state exactly (e = 1 gives 0).
//
// Accuracy: e - 1 inherits the absolute rounding error of e (~1e-7), so the
// fast form above errs by ~1e-7 |B u / A| per step.  Waves in which some
// |A| < 1/16 (including A == 0) instead take the "precise" form
//   Bbar u = dt * phi(dt A) * B u,  phi(z) = (e^z - 1) / z,
// with a degree-6 series for |z| < 1/4 and (e - 1)/z otherwise.
// B and C are broadcast through multiplications by 0 and 1, so they must be
// finite (an infinity would turn neighbouring entries into NaN).
#include "ssm_device.h"
#include "ssm_internal.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace ssm {
namespace {

constexpr int kRow = 16;                     // lanes per row = state entries per channel
constexpr int kChPerWave = 4;                // rows per wave
constexpr int kTB = 16;                      // time steps per block
constexpr int kPStride = kTB + 4;            // padded [n][k] stride of partials
constexpr int kPRow = kRow * kPStride + 16;  // per-channel partial block (336 floats)
constexpr float kFastMinAbsA = 0.0625f;
constexpr uint32_t kOOB = 0xFFFFFFFFu;       // buffer offset that is always out of range
constexpr int kRsrcWord3 = 0x00020000;       // raw, untyped buffer descriptor (gfx9)
// Largest byte range one launch addresses per tensor and batch row: offsets
// are 32-bit; longer sequences are split into launches that chain the state.
constexpr int64_t kMaxRowBytes = 0xFFF00000LL;

struct ScanKernelParams {
    int64_t B, L, D;
    int N, K, softplus;
    int64_t t_begin, t_end;  // rows [t_begin, t_end) of every batch row
    int64_t groups_per_b, ngroups;
    const void *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dskip, *dbias, *conv_w, *conv_b;
    const float *h_in;  // state entering row t_begin, or NULL (= 0)
    void *y;
    float *h_out;       // state after row t_end - 1, or NULL
};

template <int I>
using ic = std::integral_constant<int, I>;

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(ic<Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value of lane K of this lane's 16-lane row (DPP row_newbcast).
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + K, 0xf, 0xf, false);
}
// Lane n receives `cur` of lane n-K of its row, or `prev` of lane n-K+16
// when n < K (the previous block's tail): the x history of the conv.
template <int K>
__device__ __forceinline__ float row_shift_in(float cur, float prev) {
    const float wrap = __builtin_amdgcn_update_dpp(0.0f, prev, 0x120 + K, 0xf, 0xf, false);  // row_ror:K
    return __builtin_amdgcn_update_dpp(wrap, cur, 0x110 + K, 0xf, 0xf, false);               // row_shr:K
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber them so that consecutive channel groups, which share cache
// lines of x/delta/z/y and the same B/C rows, run on the same XCD.
__device__ __forceinline__ int64_t xcd_group(int64_t bid, int64_t nblocks) {
    constexpr int64_t kXcd = 8;
    const int64_t full = nblocks - nblocks % kXcd;
    if (bid >= full) return bid;
    return (bid % kXcd) * (full / kXcd) + bid / kXcd;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t byte_off,
                                                       int64_t records) {
    const char *p = static_cast<const char *>(base) + byte_off;
    const uint32_t n = (uint32_t)(records < 0 ? 0 : records);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, (int)n, kRsrcWord3);
}

// One I/O element from a buffer (0 when out of range), as raw bits.
template <typename IO>
__device__ __forceinline__ uint32_t buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ uint32_t buf_ld<io_bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <>
__device__ __forceinline__ uint32_t buf_ld<io_f32>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <typename IO>
__device__ __forceinline__ float widen(uint32_t raw) {
    if constexpr (std::is_same<IO, io_bf16>::value) return __uint_as_float(raw << 16);
    else return __uint_as_float(raw);
}
template <typename IO>
__device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    if constexpr (std::is_same<IO, io_bf16>::value)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, off,
                                              0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

__device__ __forceinline__ float softplus_fast(float v) {
    // max(v,0) + log(1 + e^-|v|); for tiny w = e^-|v|, log(1+w) ~ w (1 - w/2).
    const float w = hw_exp2(-fabsf(v) * kLog2e);
    const float lg = __builtin_amdgcn_logf(1.0f + w) * 0.69314718055994531f;
    const float small = w * (1.0f - 0.5f * w);
    return fmaxf(v, 0.0f) + (w < 0.0078125f ? small : lg);
}

// phi(z) = (e^z - 1) / z given e = e^z; series for small |z|.
__device__ __forceinline__ float phi_of(float z, float e) {
    const float s = 1.0f + z * (0.5f + z * (1.0f / 6.0f + z * (1.0f / 24.0f +
                    z * (1.0f / 120.0f + z * (1.0f / 720.0f + z * (1.0f / 5040.0f))))));
    const float big = (e - 1.0f) * hw_rcp(z);
    return fabsf(z) < 0.25f ? s : big;
}

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef short mfma_bf16x4 __attribute__((ext_vector_type(4)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));

// Selector operand of the broadcast MFMA (constant per lane).
struct BcastSel {
    mfma_bf16x4 bf;  // bf16: identity 16x16 as the B operand
    float f;         // fp32: A[i][k] = (k == i % 4) as the A operand
};
__device__ __forceinline__ BcastSel make_sel(int lane) {
    BcastSel s;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        s.bf[r] = (4 * (lane >> 4) + r == (lane & 15)) ? (short)0x3F80 : (short)0;
    s.f = ((lane >> 4) == ((lane & 15) & 3)) ? 1.0f : 0.0f;
    return s;
}

// ---------------------------------------------------------------------------
// Workgroup tiles.  A workgroup of W waves covers CH = 4W consecutive
// channels of one batch row.  Per 16-step block it stages in LDS, with wide
// coalesced loads shared by all its waves:
//   own [slot][x|delta|z][16 rows][CH]   raw I/O elements
//   ybuf[slot][16 rows][CH]              raw outputs, stored coalesced
//   bc  [slot][B|C][16 rows][16]         raw B and C rows (zero past N)
// and per wave a partial-sum transpose area.  Slots alternate per block.
// ---------------------------------------------------------------------------
struct Tiles {
    int CH;
    uint32_t own, ybuf, bc, part;    // byte offsets in the dynamic LDS block
    uint32_t own_slot, ybuf_slot, bc_slot, own_tensor;
};

template <typename IO>
__device__ __host__ __forceinline__ Tiles tile_layout(int W) {
    constexpr int es = sizeof(typename IO::storage);
    Tiles t;
    t.CH = 4 * W;
    t.own_tensor = (uint32_t)(kTB * t.CH * es);
    t.own_slot = 3 * t.own_tensor;
    t.ybuf_slot = (uint32_t)(kTB * t.CH * es);
    t.bc_slot = (uint32_t)(2 * kTB * kRow * es);
    t.own = 0;
    t.ybuf = t.own + 2 * t.own_slot;
    t.bc = t.ybuf + 2 * t.ybuf_slot;
    t.part = (t.bc + 2 * t.bc_slot + 15u) & ~15u;
    return t;
}
template <typename IO>
__host__ __forceinline__ size_t tile_lds_bytes(int W) {
    const Tiles t = tile_layout<IO>(W);
    return t.part + (size_t)W * kChPerWave * kPRow * sizeof(float);
}

// Launch-wide addressing of one workgroup.
struct Geo {
    __amdgpu_buffer_rsrc_t rx, rdt, rz, ry, rb, rc;
    uint32_t row_step;   // bytes per block in x/delta/z/y
    uint32_t bc_step;    // bytes per block in B/C
    int64_t D;
    int N, W, d0;
};

// Raw global data of one block held by one thread between its load and its
// copy into LDS.  Every load instruction reads a single tensor, so its
// buffer descriptor is wave-uniform (a per-lane descriptor would turn each
// load into a loop over lanes).
//   own tiles, wide path: thread t < 16 W holds chunk t (row t / W, channels
//     4 (t % W) .. +3) of each of x, delta, z;
//   own tiles, element path: thread t holds element t (row t / CH, channel
//     t % CH) of each of x, delta, z;
//   B/C rows, wide path (N = 16): threads t < 64 hold chunk t (4 elements)
//     of B and of C; element path: elements t + i * threads (< 256) of B, C.
// Which path runs is fixed at compile time: a run-time choice would merge
// the two register sets at the loop back-edge with copies that must wait
// for every load in flight.
struct Fetch {
    uint4 own[3];
    uint4 bcv[2];
    uint32_t bce[8];
};

template <typename IO, bool VEC>
__device__ __forceinline__ void fetch_block(const Geo &g, uint32_t blk_off, uint32_t bc_off,
                                            int tid, int nthreads, Fetch &f) {
    constexpr int es = sizeof(typename IO::storage);
    const int CH = 4 * g.W;
    const __amdgpu_buffer_rsrc_t rs[3] = {g.rx, g.rdt, g.rz};
    if (VEC) {
        const int row = tid / g.W, cc = tid % g.W;
        const int ch = g.d0 + 4 * cc;
        const uint32_t off = (tid < kTB * g.W && ch < g.D)
                                 ? blk_off + (uint32_t)((row * g.D + ch) * es) : kOOB;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if constexpr (es == 2) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs[i], off, 0, 0));
                f.own[i] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                f.own[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs[i], off, 0, 0));
            }
        }
    } else {
        const int row = tid / CH, ci = tid % CH;
        const int ch = g.d0 + ci;
        const uint32_t off = ch < g.D ? blk_off + (uint32_t)((row * g.D + ch) * es) : kOOB;
#pragma unroll
        for (int i = 0; i < 3; ++i) f.own[i].x = buf_ld<IO>(rs[i], off);
    }
    if (VEC) {
        const uint32_t off = tid < 64 ? bc_off + (uint32_t)(tid * 4 * es) : kOOB;
        if constexpr (es == 2) {
            const uint2 b = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(g.rb, off, 0, 0));
            const uint2 c = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(g.rc, off, 0, 0));
            f.bcv[0] = make_uint4(b.x, b.y, 0u, 0u);
            f.bcv[1] = make_uint4(c.x, c.y, 0u, 0u);
        } else {
            f.bcv[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g.rb, off, 0, 0));
            f.bcv[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g.rc, off, 0, 0));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * nthreads;
            const int row = e / kRow, nn = e % kRow;
            const uint32_t off = (e < kTB * kRow && nn < g.N)
                                     ? bc_off + (uint32_t)((row * g.N + nn) * es) : kOOB;
            f.bce[i] = buf_ld<IO>(g.rb, off);
            f.bce[4 + i] = buf_ld<IO>(g.rc, off);
        }
    }
}

template <typename IO, bool VEC>
__device__ __forceinline__ void stage_block(const Geo &g, const Tiles &T, char *lds, int slot,
                                            int tid, int nthreads, const Fetch &f) {
    constexpr int es = sizeof(typename IO::storage);
    const int CH = T.CH;
    char *own = lds + T.own + slot * T.own_slot;
    if (VEC) {
        if (tid < kTB * g.W) {
            const int row = tid / g.W, cc = tid % g.W;
            char *dst = own + (row * CH + 4 * cc) * es;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if constexpr (es == 2)
                    *reinterpret_cast<uint2 *>(dst + i * T.own_tensor) = make_uint2(f.own[i].x, f.own[i].y);
                else
                    *reinterpret_cast<uint4 *>(dst + i * T.own_tensor) = f.own[i];
            }
        }
    } else {
        char *dst = own + tid * es;  // element tid = (row, channel) of each tensor
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if constexpr (es == 2) *reinterpret_cast<uint16_t *>(dst + i * T.own_tensor) = (uint16_t)f.own[i].x;
            else *reinterpret_cast<uint32_t *>(dst + i * T.own_tensor) = f.own[i].x;
        }
    }
    char *bc = lds + T.bc + slot * T.bc_slot;
    char *cc = bc + kTB * kRow * es;
    if (VEC) {
        if (tid < 64) {
            if constexpr (es == 2) {
                *reinterpret_cast<uint2 *>(bc + tid * 8) = make_uint2(f.bcv[0].x, f.bcv[0].y);
                *reinterpret_cast<uint2 *>(cc + tid * 8) = make_uint2(f.bcv[1].x, f.bcv[1].y);
            } else {
                *reinterpret_cast<uint4 *>(bc + tid * 16) = f.bcv[0];
                *reinterpret_cast<uint4 *>(cc + tid * 16) = f.bcv[1];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * nthreads;
            if (e < kTB * kRow) {
                if constexpr (es == 2) {
                    *reinterpret_cast<uint16_t *>(bc + e * es) = (uint16_t)f.bce[i];
                    *reinterpret_cast<uint16_t *>(cc + e * es) = (uint16_t)f.bce[4 + i];
                } else {
                    *reinterpret_cast<uint32_t *>(bc + e * es) = f.bce[i];
                    *reinterpret_cast<uint32_t *>(cc + e * es) = f.bce[4 + i];
                }
            }
        }
    }
}

// Coalesced store of one block of outputs from LDS.
template <typename IO, bool VEC>
__device__ __forceinline__ void store_block(const Geo &g, const Tiles &T, const char *lds,
                                            int slot, uint32_t blk_off, int tid, int nthreads) {
    constexpr int es = sizeof(typename IO::storage);
    const int CH = T.CH;
    const char *yb = lds + T.ybuf + slot * T.ybuf_slot;
    if (VEC) {
        if (tid < kTB * g.W) {
            const int row = tid / g.W, cc = tid % g.W;
            const int ch = g.d0 + 4 * cc;
            const uint32_t off = ch < g.D ? blk_off + (uint32_t)((row * g.D + ch) * es) : kOOB;
            const char *src = yb + (row * CH + 4 * cc) * es;
            if constexpr (es == 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i_t, v), g.ry, off, 0, 0);
            } else {
                const uint4 v = *reinterpret_cast<const uint4 *>(src);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i_t, v), g.ry, off, 0, 0);
            }
        }
    } else {
        const int row = tid / CH, ci = tid % CH;
        const int ch = g.d0 + ci;
        const uint32_t off = ch < g.D ? blk_off + (uint32_t)((row * g.D + ch) * es) : kOOB;
        if constexpr (es == 2)
            __builtin_amdgcn_raw_buffer_store_b16(*reinterpret_cast<const uint16_t *>(yb + tid * es), g.ry, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t *>(yb + tid * es), g.ry, off, 0, 0);
    }
}

// MFMA operand of step group g for this lane, from the staged B or C rows.
//  bf16: row 4g + lane%4, entries 4*(lane/16) .. +3   (A operand, 16x16x16)
//  fp32: row 4g + lane/16, entry lane%16                (B operand, 16x16x4)
template <typename IO>
__device__ __forceinline__ mfma_f32x4 bcast_group(const char *rows, int g, int lane,
                                                  const BcastSel &sel) {
    const mfma_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (std::is_same<IO, io_bf16>::value) {
        const uint2 op = *reinterpret_cast<const uint2 *>(
            rows + ((4 * g + (lane & 3)) * kRow + 4 * (lane >> 4)) * 2);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mfma_bf16x4, op), sel.bf,
                                                         zero, 0, 0, 0);
    } else {
        const float op = *reinterpret_cast<const float *>(
            rows + ((4 * g + (lane >> 4)) * kRow + (lane & 15)) * 4);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(sel.f, op, zero, 0, 0, 0);
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

struct LaneConst {
    float a, a2, ia, dsk, dbias, cb, wp0, wp1, wp2, wp3;
    float iar[kRow];  // 1 / A of every state entry of the lane's channel (0 where A == 0)
};

// One block of one wave: decode the lane's own step from the staged tile,
// run 16 recurrence steps, transpose the partial read-outs, write y to LDS.
template <typename IO, bool CONV, bool FAST, bool TAIL>
__device__ __forceinline__ void compute_block(const ScanKernelParams &p, const Tiles &T,
                                              char *lds, int slot, int64_t t0, int wave, int c,
                                              int n, int lane, const BcastSel &sel,
                                              const LaneConst &k, float &x_prev, float &h) {
    constexpr int es = sizeof(typename IO::storage);
    const int ci = 4 * wave + c;
    const char *own = lds + T.own + slot * T.own_slot + (n * T.CH + ci) * es;
    float xv, dt, zv;
    if constexpr (es == 2) {
        xv = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(own) << 16);
        dt = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(own + T.own_tensor) << 16);
        zv = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(own + 2 * T.own_tensor) << 16);
    } else {
        xv = *reinterpret_cast<const float *>(own);
        dt = *reinterpret_cast<const float *>(own + T.own_tensor);
        zv = *reinterpret_cast<const float *>(own + 2 * T.own_tensor);
    }
    float u = xv;
    if (CONV) {
        const float xm1 = row_shift_in<1>(xv, x_prev);
        const float xm2 = row_shift_in<2>(xv, x_prev);
        const float xm3 = row_shift_in<3>(xv, x_prev);
        u = silu(k.cb + k.wp0 * xm3 + k.wp1 * xm2 + k.wp2 * xm1 + k.wp3 * xv);
        x_prev = xv;
    }
    if (p.softplus) dt = softplus_fast(dt + k.dbias);
    if (TAIL && t0 + n >= p.t_end) {  // past the end: the state must not move
        dt = 0.0f;
        u = 0.0f;
    }
    const char *brows = lds + T.bc + slot * T.bc_slot;
    const char *crows = brows + kTB * kRow * es;
    float *prow = reinterpret_cast<float *>(lds + T.part) + (wave * kChPerWave + c) * kPRow;

    // Steps in groups of four: one broadcast MFMA each for B and C per
    // group, one 128-bit LDS write of the group's four partial read-outs.
    static_for<kTB / 4>([&](auto G) {
        constexpr int gi = decltype(G)::value;
        constexpr int g4 = 4 * gi;
        const mfma_f32x4 Bk = bcast_group<IO>(brows, gi, lane, sel);
        const mfma_f32x4 Ck = bcast_group<IO>(crows, gi, lane, sel);
        float pk[4];
        static_for<4>([&](auto K) {
            constexpr int kk = decltype(K)::value;
            constexpr int kx = g4 + kk;
            const float dtk = row_bcast<kx>(dt);
            const float uk = row_bcast<kx>(u);
            const float e = hw_exp2(dtk * k.a2);
            const float bu = uk * Bk[kk];
            float bx;
            if (FAST) {
                bx = __builtin_fmaf(e, bu, -bu);  // h holds A h here
            } else {
                bx = (dtk * phi_of(dtk * k.a, e)) * bu;
            }
            h = __builtin_fmaf(e, h, bx);
            pk[kk] = Ck[kk] * h;
        });
        *reinterpret_cast<float4 *>(&prow[n * kPStride + g4]) = make_float4(pk[0], pk[1], pk[2], pk[3]);
    });
    wave_sync();
    float part[kRow];
#pragma unroll
    for (int j = 0; j < kRow; ++j) part[j] = prow[j * kPStride + n];
    float acc;
    if (FAST) {
        // The fast form keeps g = A h, so C h = (C g) / A per entry.
        float s0 = part[0] * k.iar[0], s1 = part[1] * k.iar[1];
#pragma unroll
        for (int j = 2; j < kRow; j += 2) {
            s0 = __builtin_fmaf(part[j], k.iar[j], s0);
            s1 = __builtin_fmaf(part[j + 1], k.iar[j + 1], s1);
        }
        acc = s0 + s1;
    } else {
#pragma unroll
        for (int w = kRow / 2; w >= 1; w /= 2)
#pragma unroll
            for (int j = 0; j < w; ++j) part[j] += part[j + w];
        acc = part[0];
    }
    float yv = acc + k.dsk * u;
    if (p.z) yv *= silu(zv);
    char *ydst = lds + T.ybuf + slot * T.ybuf_slot + (n * T.CH + ci) * es;
    if constexpr (es == 2)
        *reinterpret_cast<uint16_t *>(ydst) = __builtin_bit_cast(uint16_t, (__bf16)yv);
    else
        *reinterpret_cast<float *>(ydst) = yv;
    wave_sync();  // the next block rewrites the partials
}

template <typename IO, bool CONV, bool VEC, bool FAST>
__device__ __forceinline__ void scan_tiles_body(const ScanKernelParams &p, const Geo &geo,
                                                const Tiles &T, char *lds, int wave, int c,
                                                int n, const LaneConst &k, float &h,
                                                float x_prev) {
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & 63;
    const BcastSel sel = make_sel(lane);
    const int64_t rows = p.t_end - p.t_begin;
    const int64_t nblocks = (rows + kTB - 1) / kTB;

    // Tile j is requested three blocks before it is computed (two blocks of
    // latency budget), copied into LDS slot j % 2 one block before, and its
    // outputs leave LDS one block after.  Unrolled by two so the two fetch
    // register sets alternate without copies.  The loop has a single exit
    // at its bottom (the last one or two blocks run after it): an exit in
    // the middle would route through the back-edge once the control flow is
    // structured, and the load counters merged there would force a wait for
    // every prefetch in flight.  Prefetches past the last block read zeros
    // or unused rows and are never consumed.
    Fetch f0, f1;
    fetch_block<IO, VEC>(geo, 0, 0, tid, nthreads, f0);
    fetch_block<IO, VEC>(geo, geo.row_step, geo.bc_step, tid, nthreads, f1);
    stage_block<IO, VEC>(geo, T, lds, 0, tid, nthreads, f0);
    fetch_block<IO, VEC>(geo, 2 * geo.row_step, 2 * geo.bc_step, tid, nthreads, f0);
    uint32_t ro = 0, bo = 0;  // offsets of block j
    int64_t j = 0;
    for (; j + 2 < nblocks; j += 2) {
        // -- block j (slot 0); f1 holds block j+1, f0 block j+2 --------------
        __syncthreads();
        if (j > 0) store_block<IO, VEC>(geo, T, lds, 1, ro - geo.row_step, tid, nthreads);
        compute_block<IO, CONV, FAST, false>(p, T, lds, 0, p.t_begin + j * kTB, wave, c, n, lane, sel, k,
                                      x_prev, h);
        stage_block<IO, VEC>(geo, T, lds, 1, tid, nthreads, f1);
        // Keep the refill of f1 after its copy into LDS, so the new data can
        // land in the same registers.
        __builtin_amdgcn_sched_barrier(0);
        fetch_block<IO, VEC>(geo, ro + 3 * geo.row_step, bo + 3 * geo.bc_step, tid, nthreads, f1);
        // -- block j+1 (slot 1); f0 holds block j+2, f1 block j+3 ------------
        __syncthreads();
        store_block<IO, VEC>(geo, T, lds, 0, ro, tid, nthreads);
        compute_block<IO, CONV, FAST, false>(p, T, lds, 1, p.t_begin + (j + 1) * kTB, wave, c, n, lane,
                                      sel, k, x_prev, h);
        stage_block<IO, VEC>(geo, T, lds, 0, tid, nthreads, f0);
        __builtin_amdgcn_sched_barrier(0);
        fetch_block<IO, VEC>(geo, ro + 4 * geo.row_step, bo + 4 * geo.bc_step, tid, nthreads, f0);
        ro += 2 * geo.row_step;
        bo += 2 * geo.bc_step;
    }
    // One or two blocks remain; block j sits in slot 0 and f1 holds j+1.
    __syncthreads();
    if (j > 0) store_block<IO, VEC>(geo, T, lds, 1, ro - geo.row_step, tid, nthreads);
    compute_block<IO, CONV, FAST, true>(p, T, lds, 0, p.t_begin + j * kTB, wave, c, n, lane, sel, k,
                                  x_prev, h);
    if (j + 1 < nblocks) {
        stage_block<IO, VEC>(geo, T, lds, 1, tid, nthreads, f1);
        __syncthreads();
        store_block<IO, VEC>(geo, T, lds, 0, ro, tid, nthreads);
        compute_block<IO, CONV, FAST, true>(p, T, lds, 1, p.t_begin + (j + 1) * kTB, wave, c, n, lane,
                                      sel, k, x_prev, h);
        __syncthreads();
        store_block<IO, VEC>(geo, T, lds, 1, ro + geo.row_step, tid, nthreads);
    } else {
        __syncthreads();
        store_block<IO, VEC>(geo, T, lds, 0, ro, tid, nthreads);
    }
}

// blockDim.x = 64 W; workgroup g covers channels [4 W q, 4 W q + 4 W) of
// batch row g / groups_per_b, with q = g % groups_per_b.
// Register budget: the bf16 wide-tile variants (the 130M- and 2.8B-like
// layers) must fit 5 waves per SIMD (<= 96 VGPRs) so a 2.8B-like layer
// (5120 waves) is resident at once; the others may use up to 128.
template <typename IO, bool VEC>
constexpr int kMinWavesPerEU = (VEC && std::is_same<IO, io_bf16>::value) ? 5 : 4;

template <typename IO, bool CONV, bool VEC>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(kMinWavesPerEU<IO, VEC>, 8)))
void scan_tiles_kernel(ScanKernelParams p) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int es = sizeof(typename IO::storage);
    const int W = blockDim.x / 64;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x & 63;
    const int c = lane / kRow, n = lane % kRow;
    const int64_t grp = xcd_group(blockIdx.x, gridDim.x);
    const int64_t b = grp / p.groups_per_b;
    const int d0 = (int)((grp % p.groups_per_b) * 4 * W);
    const int64_t d = d0 + 4 * wave + c;
    const bool dvalid = d < p.D;
    const bool live = dvalid && n < p.N;
    const int64_t D = p.D, N = p.N;
    const int64_t rows = p.t_end - p.t_begin;
    const Tiles T = tile_layout<IO>(W);

    Geo geo;
    const int64_t xbase = (b * p.L + p.t_begin) * D * es;
    const int64_t xrec = rows * D * es;
    geo.rx = rsrc(p.x, xbase, xrec);
    geo.rdt = rsrc(p.delta, xbase, xrec);
    // Without a gate the descriptor has no records: loads return 0.
    geo.rz = p.z ? rsrc(p.z, xbase, xrec) : rsrc(p.x, 0, 0);
    geo.ry = rsrc(p.y, xbase, xrec);
    const int64_t bbase = (b * p.L + p.t_begin) * N * es;
    geo.rb = rsrc(p.Bm, bbase, rows * N * es);
    geo.rc = rsrc(p.Cm, bbase, rows * N * es);
    geo.row_step = (uint32_t)(kTB * D * es);
    geo.bc_step = (uint32_t)(kTB * N * es);
    geo.D = D;
    geo.N = (int)N;
    geo.W = W;
    geo.d0 = d0;

    LaneConst k;
    k.a = live ? p.A[d * N + n] : 0.0f;
    k.a2 = k.a * kLog2e;
    k.ia = (k.a != 0.0f) ? 1.0f / k.a : 0.0f;
    static_for<kRow>([&](auto J) { k.iar[decltype(J)::value] = row_bcast<decltype(J)::value>(k.ia); });
    k.dsk = (p.Dskip && dvalid) ? p.Dskip[d] : 0.0f;
    k.dbias = (p.dbias && dvalid) ? p.dbias[d] : 0.0f;
    k.wp0 = k.wp1 = k.wp2 = k.wp3 = k.cb = 0.0f;
    if (CONV && dvalid) {
        // Taps right-aligned to width 4: wp3 weighs the current token.
        const int K = p.K;
        const float *w = p.conv_w + d * K;
        k.wp3 = w[K - 1];
        if (K >= 2) k.wp2 = w[K - 2];
        if (K >= 3) k.wp1 = w[K - 3];
        if (K >= 4) k.wp0 = w[K - 4];
        if (p.conv_b) k.cb = p.conv_b[d];
    }
    float h = (live && p.h_in) ? p.h_in[(b * D + d) * N + n] : 0.0f;
    // Conv history entering the launch: x at rows t_begin - 16 + n (only the
    // last three lanes of a row are used).
    float x_prev = 0.0f;
    if (CONV && p.t_begin > 0 && dvalid && n >= kRow - 3) {
        const int64_t t = p.t_begin - kRow + n;
        x_prev = t >= 0 ? load_io<IO>(p.x, (b * p.L + t) * D + d) : 0.0f;
    }
    // Wave-uniform choice of the update form (see the file comment).
    const bool fast = __all(!live || fabsf(k.a) >= kFastMinAbsA);
    if (fast) {
        // The fast form carries g = A h (the 1/A moves to the read-out).
        h *= k.a;
        scan_tiles_body<IO, CONV, VEC, true>(p, geo, T, lds, wave, c, n, k, h, x_prev);
        h *= k.ia;
    } else {
        scan_tiles_body<IO, CONV, VEC, false>(p, geo, T, lds, wave, c, n, k, h, x_prev);
    }
    if (p.h_out && live) p.h_out[(b * D + d) * N + n] = h;
}

__global__ void copy_or_zero_kernel(const float *src, float *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// Waves per workgroup: the workgroups should spread evenly over the 256 CUs
// (each CU holds up to 20 waves of this kernel).  Among W = 1..16 pick the
// one whose busiest CU carries the least work, preferring wider tiles.
int choose_waves(int64_t batch, int64_t dim) {
    constexpr int64_t kCUs = 256, kMaxWavesPerCU = 20;
    int best = 1;
    double best_cost = 1e300;
    for (int W = 1; W <= 16; ++W) {
        const int64_t per_row = (dim + 4 * W - 1) / (4 * W);
        const int64_t groups = per_row * batch;
        const int64_t per_cu = (groups + kCUs - 1) / kCUs;            // workgroups on the busiest CU
        const int64_t fit = std::max<int64_t>(1, kMaxWavesPerCU / W); // resident at once
        const int64_t rounds = (per_cu + fit - 1) / fit;
        // busiest-CU work in wave-blocks, plus a small penalty for narrow tiles
        const double cost = (double)(rounds * std::min(per_cu, fit) * W) * (1.0 + 0.02 * (16 - W));
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = W;
        }
    }
    return best;
}

template <typename IO, bool VEC>
hipError_t launch_typed(const ScanKernelParams &p, int W, hipStream_t stream) {
    const unsigned grid = (unsigned)p.ngroups;
    const size_t lds = tile_lds_bytes<IO>(W);
    if (p.K > 0)
        scan_tiles_kernel<IO, true, VEC><<<grid, 64 * W, lds, stream>>>(p);
    else
        scan_tiles_kernel<IO, false, VEC><<<grid, 64 * W, lds, stream>>>(p);
    return hipGetLastError();
}

// Rows one launch may cover (a multiple of two blocks).  The prefetch
// addresses up to four blocks past the last row, so 64 rows of offset
// headroom are kept below the 32-bit limit.
int64_t rows_per_launch(const ssm_scan_args_t &a) {
    const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    int64_t r = kMaxRowBytes / (a.dim * es) - 4 * kTB;
    r -= r % (2 * kTB);
    return r;
}

}  // namespace

size_t scan_workspace_bytes(const ssm_scan_args_t &a) {
    // A sequence too long for one launch is split; the state between the
    // launches lives in the workspace.
    if (a.seqlen <= rows_per_launch(a)) return 0;
    return (size_t)(a.batch * a.dim * a.dstate) * sizeof(float);
}

hipError_t launch_scan_fwd(const ssm_scan_args_t &a, hipStream_t stream) {
    ScanKernelParams p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.D = a.dim;
    p.N = (int)a.dstate;
    p.K = (int)a.conv_k;
    p.softplus = a.delta_softplus;
    const int W = choose_waves(a.batch, a.dim);
    p.groups_per_b = (a.dim + 4 * W - 1) / (4 * W);
    p.ngroups = p.groups_per_b * a.batch;
    p.x = a.x;
    p.delta = a.delta;
    p.Bm = a.Bm;
    p.Cm = a.Cm;
    p.z = a.z;
    p.A = a.A;
    p.Dskip = a.Dskip;
    p.dbias = a.delta_bias;
    p.conv_w = a.conv_w;
    p.conv_b = a.conv_b;
    p.y = a.y;
    if (p.ngroups > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    const int64_t chunk = rows_per_launch(a);
    if (chunk < 2 * kTB || a.dim * es > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // Wide (4-element) chunks need D % 4 == 0, N = 16 and aligned tensors.
    auto al = [&](const void *q) { return ((uintptr_t)q % (4 * es)) == 0; };
    const bool vec = (a.dim % 4 == 0) && a.dstate == kRow && al(a.x) && al(a.delta) && al(a.y) &&
                     (!a.z || al(a.z)) && al(a.Bm) && al(a.Cm);
    float *carry = static_cast<float *>(a.workspace);
    hipError_t e = hipSuccess;
    for (int64_t t = 0; t < a.seqlen && e == hipSuccess; t += chunk) {
        const bool first = t == 0, last = t + chunk >= a.seqlen;
        p.t_begin = t;
        p.t_end = last ? a.seqlen : t + chunk;
        p.h_in = first ? a.h0 : carry;
        p.h_out = last ? a.h_final : carry;
        if (a.io_dtype == SSM_BF16)
            e = vec ? launch_typed<io_bf16, true>(p, W, stream) : launch_typed<io_bf16, false>(p, W, stream);
        else
            e = vec ? launch_typed<io_f32, true>(p, W, stream) : launch_typed<io_f32, false>(p, W, stream);
    }
    return e;
}

hipError_t launch_empty_scan_state(const ssm_scan_args_t &a, hipStream_t stream) {
    if (!a.h_final) return hipSuccess;
    const int64_t n = a.batch * a.dim * a.dstate;
    if (n == 0) return hipSuccess;
    copy_or_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a.h0, a.h_final, n);
    return hipGetLastError();
}

}  // namespace ssm
