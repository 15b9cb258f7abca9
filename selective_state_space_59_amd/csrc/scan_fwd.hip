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
// Work decomposition.  One lane owns one (channel, state index) chain; a
// 16-lane row of the wave holds the 16 state entries of one channel, so a
// wave covers 4 channels and the (B, L, D, N) state never leaves registers.
// A workgroup of W waves covers 4W consecutive channels of one batch row;
// with N = 16 the 130M-like layer (B=8, D=1536) is 3072 waves and the
// 2.8B-like layer 5120.  Few-channel long sequences are cut into segments
// scanned at once (see launch_scan_fwd).
//
// Time advances in blocks of 16 steps.  Per block:
//   * x, delta, z ([16 rows][4W channels]) and the B, C rows ([16][16]) are
//     staged in LDS with 16-byte loads, each wave holding one load duty so
//     every load reads one tensor through a wave-uniform buffer descriptor;
//     reads past the data return 0 and such writes are dropped, so ragged
//     edges need no branches;
//   * each lane decodes x, delta, z of ITS OWN step (t0 + n) for its
//     channel and computes u (conv prologue, its 3-step history from the
//     neighbouring lanes through DPP shifts) and dt there, once per
//     (t, channel);
//   * the recurrence of step k reads dt of step k from lane k of the row
//     through a DPP row broadcast folded into the multiply;
//   * two products of the step loop run on the matrix cores, 4 steps x 16
//     entries x 4 channels per MFMA: u B (bf16 I/O without the conv
//     prologue: a 4x4x4 bf16 MFMA on the raw u and B, exact) and the
//     read-out weights C x (x = 1/A in the fast form, 1 otherwise; see
//     WSel).  Otherwise B reaches every row through a 0/1 selector MFMA and
//     u B is a vector product with u of step k read through a DPP row
//     broadcast;
//   * each lane's 16 states h_{t,n} are transposed through LDS, so lane
//     (c, j) sums the 16 states of step t0 + j times their weights and
//     applies the skip and the gate; y goes out through LDS with coalesced
//     16-byte stores;
//   * optionally (training) the state entering the block is stored as the
//     backward's checkpoint of that block; the backward's own first pass is
//     this kernel with that store and no outputs (kCkptPass).
// The block loop is software-pipelined: loads run four blocks ahead through
// a three-slot LDS ring, a block's read-outs are summed and its y stored
// during the next block, and the MFMAs run one step group ahead.
//
// Vector-ALU cost per state update (the binding resource): one exp (a
// quarter-rate transcendental on gfx950), dt A, and two fused fp32 ops in
// the fast form, which carries g = A h, plus one fused op of the read-out sum:
//   e = 2^(dt A log2e); bx = e*bu - bu; g = e*g + bx; y += g * w.
// bx = fma(e, bu, -bu) makes dt = 0 hold the state exactly (e = 1 gives 0).
// With the conv prologue, or fp32 I/O, bu = u*B adds one more.
//
// Accuracy: e - 1 inherits the absolute rounding error of e (~1e-7), so the
// fast form errs by ~1e-7 |B u / A| per step.  Waves in which some
// |A| < 1/16 (including A == 0) instead carry h and take the "precise" form
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
    const void *cs_in;  // conv state (B, K-1, D): x before row 0, or NULL (= 0)
    void *y;
    float *h_out;       // state after row t_end - 1, or NULL
    // The state entering every 16-step block, [nblocks][B][D][16] (entry
    // n < N at n), or NULL.  ckpt_only launches (the backward's first pass)
    // write these and no outputs.
    float *ckpt;
    int ckpt_only;
    // Sequence segments (see launch_segmented): mode 0 scans [t_begin, t_end)
    // as one piece; mode 1 scans every segment of seg_len rows from a zero
    // state (the first from h_in) and records its end state, its sum of dt
    // and its head length; mode 2 re-scans the heads of segments 1.. from
    // their true entering states.
    int mode, nseg;
    int64_t seg_len;
    float *ws_hend;        // [nseg][B][D][N]  end state of each segment (mode 1)
    float *ws_stot;        // [nseg][B][D]     sum of dt over each segment (mode 1)
    int *ws_head;          // [nseg][ngroups]  head blocks of each segment (mode 1 -> 2)
    const float *ws_hin;   // [nseg][B][D][N]  state entering each segment (mode 2)
};

// Rows [t0, t1) a workgroup scans (its segment of the launch's rows).
struct Span {
    int64_t t0, t1;
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
    // row_newbcast: every lane has a source, so no old value is needed
    return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + K, 0xf, 0xf, true);
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

// Selector operands of the broadcast MFMA (constant per lane).
//  bf16 (16x16x16): the selector of step group g is the A operand
//    A[i][k] = (k == 4g + i % 4): lane l holds the one-hot of l % 4 when
//    l / 16 == g, zeros otherwise;
//  fp32 (16x16x4): A[i][k] = (k == i % 4).
struct BcastSel {
    mfma_bf16x4 bf[4];
    float f;
};
__device__ __forceinline__ BcastSel make_sel(int lane) {
    BcastSel s;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s.bf[g][r] = ((lane >> 4) == g && r == (lane & 3)) ? (short)0x3F80 : (short)0;
    s.f = ((lane >> 4) == ((lane & 15) & 3)) ? 1.0f : 0.0f;
    return s;
}

// ---------------------------------------------------------------------------
// Workgroup tiles.  A workgroup of W waves covers CH = 4W consecutive
// channels of one batch row.  Per 16-step block it stages in LDS, with wide
// coalesced loads shared by all its waves:
//   own [3 slots][x|delta|z][16 rows][CH + pad]  raw I/O elements
//   bc  [3 slots][B|C][16 rows][16]               raw B and C rows (zero past N);
//                                                 bf16 entry-major, [16 entries][20] (16 steps used)
//   ybuf[2][16 rows][CH + pad]                    raw outputs, stored coalesced
// and per wave a partial-sum transpose area.  The row pad puts the 16 time
// steps that the 16 lanes of a wave row read (or write) on distinct banks;
// the planes of one slot are a fixed distance apart (sized for W = 16), so
// a lane reaches its x, delta and z with one address.
// ---------------------------------------------------------------------------
constexpr int kSlots = 3;
constexpr int kMaxW = 16;

// Row stride in dwords: a multiple of 4 (16-byte chunks) that is 4 mod 8,
// so the 16 time steps a wave row reads fall on two-way-shared banks at
// worst.
template <typename IO>
__device__ __host__ constexpr int row_dwords(int W) {
    const int data = (4 * W * (int)sizeof(typename IO::storage) + 3) / 4;
    const int s = (data + 3) / 4 * 4;
    return s % 8 == 0 ? s + 4 : s;
}
template <typename IO>
constexpr uint32_t kPlane = (uint32_t)kTB * 4u * row_dwords<IO>(kMaxW);
// Staged B and C tiles of one block (B first, then C, in each ring slot).
// bf16 B is entry-major with rows of 20 elements (40 bytes = 10 dwords): the
// 16 lanes that read one 8-byte piece each (the same steps of the 16
// entries) then hit 16 distinct bank pairs.  bf16 C is step-major with rows
// of 24 elements (48 bytes = 12 dwords): the lanes that read one 16-byte
// piece each (the same entries of 8 steps) then hit 32 distinct banks.
// fp32 B and C are step-major ([16 steps][16 entries]).
constexpr uint32_t kBcRowBytes = 40;
constexpr uint32_t kCRowBytes = 48;
template <typename IO>
constexpr uint32_t kBTile = sizeof(typename IO::storage) == 2 ? kRow * kBcRowBytes : kTB * kRow * 4;
template <typename IO>
constexpr uint32_t kCTile = sizeof(typename IO::storage) == 2 ? kTB * kCRowBytes : kTB * kRow * 4;

struct Tiles {
    int CH;
    uint32_t rs;                   // bytes per staged row
    uint32_t own, bc, ybuf, part;  // byte offsets in the dynamic LDS block
    uint32_t own_slot, bc_slot, ybuf_slot;
};

template <typename IO>
__device__ __host__ __forceinline__ Tiles tile_layout(int W) {
    constexpr int es = sizeof(typename IO::storage);
    Tiles t;
    t.CH = 4 * W;
    t.rs = 4u * (uint32_t)row_dwords<IO>(W);
    t.own_slot = 3 * kPlane<IO>;
    t.bc_slot = kBTile<IO> + kCTile<IO>;
    t.ybuf_slot = kTB * t.rs;
    t.own = 0;
    t.bc = t.own + kSlots * t.own_slot;
    t.ybuf = t.bc + kSlots * t.bc_slot;
    t.part = (t.ybuf + 2 * t.ybuf_slot + 15u) & ~15u;
    return t;
}
template <typename IO>
__host__ __forceinline__ size_t tile_lds_bytes(int W) {
    const Tiles t = tile_layout<IO>(W);
    // partials, then one int per wave for the head-length reduction
    return t.part + (size_t)W * kChPerWave * kPRow * sizeof(float) + kMaxW * sizeof(int);
}

// Launch-wide addressing of one workgroup.
struct Geo {
    __amdgpu_buffer_rsrc_t rx, rdt, rz, ry, rb, rc;  // element path
    uint32_t row_step;   // bytes per block in x/delta/z/y
    uint32_t bc_step;    // bytes per block in B/C
    int64_t D;
    int N, W, d0;
};

// Wide path: how the block moves between global memory and LDS.  Each wave
// has one duty, so every load instruction reads one tensor through a
// wave-uniform descriptor and each thread holds one 16-byte chunk:
//   waves [0, a), [a, 2a), [2a, 3a): chunk q of x, delta, z, with
//     q = (wave - role a) * 64 + lane < 16 CH / cw  (row q / (CH / cw),
//     channels cw (q % (CH / cw)) .. +cw-1; cw = 16 / element size);
//   wave 3a: chunk lane of the 16 B rows; wave 3a + 1: of the C rows;
//   the x waves also carry the matching chunks of y from LDS to memory.
// a = ceil(16 CH / cw / 64).  The launch picks W so that 3a + 2 <= W.
struct Duty {
    const char *gbase;  // tensor of the duty at the launch's first row (uniform)
    uint32_t grec;      // its bytes in this launch (uniform; < 4 GiB per launch)
    uint32_t step;      // its bytes per block (uniform)
    uint32_t goff;      // the thread's chunk within a block, or kOOB
    uint32_t lds;       // LDS offset of the chunk within a slot of the own or bc area
    int to_bc;          // the duty fills the bc area (uniform)
    int scatter;        // bf16 B rows: the chunk is written entry-major (uniform)
    int ystore;         // the wave stores y chunks (uniform)
    uint32_t ylds;      // ybuf offset of the thread's y chunk
};

template <typename IO>
__device__ __forceinline__ constexpr int chunk_ch() {
    return 16 / (int)sizeof(typename IO::storage);
}
template <typename IO>
__device__ __forceinline__ int duty_waves(int W) {  // a
    return (kTB * 4 * W / chunk_ch<IO>() + 63) / 64;
}

template <typename IO>
__device__ __forceinline__ Duty make_duty(const ScanKernelParams &p, const Span &sp,
                                          const Tiles &T, int64_t b, int d0, int wave, int lane) {
    constexpr int es = sizeof(typename IO::storage);
    constexpr int cw = chunk_ch<IO>();
    const int W = T.CH / 4;
    const int a = duty_waves<IO>(W);
    const int per_row = T.CH / cw;  // chunks per staged row
    const int64_t D = p.D, N = p.N, rows = sp.t1 - sp.t0;
    const int role = wave < 3 * a ? wave / a : 3 + (wave - 3 * a);  // uniform
    Duty d;
    d.to_bc = __builtin_amdgcn_readfirstlane(role == 3 || role == 4 ? 1 : 0);
    d.scatter = __builtin_amdgcn_readfirstlane(es == 2 && role == 3 ? 1 : 0);
    d.ystore = __builtin_amdgcn_readfirstlane(role == 0 ? 1 : 0);
    d.goff = kOOB;
    d.lds = 0;
    d.ylds = 0;
    if (role < 3) {
        const void *src = role == 0 ? p.x : role == 1 ? p.delta : p.z;
        const int64_t base = (b * p.L + sp.t0) * D * es;
        d.gbase = static_cast<const char *>(src ? src : p.x) + base;
        d.grec = src ? (uint32_t)(rows * D * es) : 0u;  // no gate: every z read gives 0
        d.step = (uint32_t)(kTB * D * es);
        const int q = (wave - role * a) * 64 + lane;
        const int row = q / per_row, ck = q % per_row;
        const int64_t ch = d0 + (int64_t)ck * cw;
        if (q < kTB * per_row && ch < D) d.goff = (uint32_t)((row * D + ch) * es);
        if (q < kTB * per_row) {
            d.lds = (uint32_t)role * kPlane<IO> + (uint32_t)(row * T.rs + ck * 16);
            d.ylds = (uint32_t)(row * T.rs + ck * 16);
        }
    } else {
        const void *src = role == 3 ? p.Bm : p.Cm;
        const int64_t base = (b * p.L + sp.t0) * N * es;
        d.gbase = static_cast<const char *>(src) + base;
        d.grec = role <= 4 ? (uint32_t)(rows * N * es) : 0u;
        d.step = (uint32_t)(kTB * N * es);
        if (role <= 4 && lane * 16 < kTB * kRow * es) {
            d.goff = (uint32_t)(lane * 16);
            // bf16: the chunk is entries 8 (lane % 2) .. +7 of step lane / 2;
            // B stores it entry-major (see stage_block), C into its step row
            if (es != 2) d.lds = (role == 3 ? 0u : kBTile<IO>) + (uint32_t)(lane * 16);
            else if (role == 3) d.lds = (uint32_t)(8 * (lane % 2) * kBcRowBytes + (lane / 2) * es);
            else d.lds = kBTile<IO> + (uint32_t)((lane / 2) * kCRowBytes + 16 * (lane % 2));
        }
    }
    d.grec = __builtin_amdgcn_readfirstlane(d.grec);
    d.step = __builtin_amdgcn_readfirstlane(d.step);
    return d;
}

// max(a - b, 0) on the scalar unit (the compiler forms this saturating
// difference on the vector ALU otherwise, one more vector op per use).
__device__ __forceinline__ uint32_t scalar_sat_sub(uint32_t a, uint32_t b) {
    uint32_t r;
    asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=s"(r) : "s"(a), "s"(b) : "scc");
    return r;
}

// Buffer descriptor of the duty's tensor for block jb (rebased on the
// block, so the per-lane offsets stay fixed; scalar arithmetic only).
// 32-bit scalar arithmetic: a launch spans less than 4 GiB per tensor, and a
// prefetch past the end gets no records.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t duty_rsrc(const Duty &d, uint32_t jb) {
    const uint32_t off = jb * d.step;
    const uint32_t rem = scalar_sat_sub(d.grec, off);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(d.gbase + off), (short)0, (int)rem,
                                             kRsrcWord3);
}

// Raw global data of one block held by one thread between its load and its
// copy into LDS.  Which layout is used is fixed at compile time: a run-time
// choice would merge two register sets at the loop back-edge with copies
// that must wait for every load in flight.
//   wide path: the thread's 16-byte chunk of its duty;
//   element path: element t (row t / CH, channel t % CH) of each of x,
//     delta, z, and elements t + i * threads (< 256) of the B and C rows.
template <bool VEC>
struct Fetch;
template <>
struct Fetch<true> {
    uint4 v;
};
template <>
struct Fetch<false> {
    uint32_t own[3];
    uint32_t bce[8];
};

template <typename IO, bool VEC>
__device__ __forceinline__ void fetch_block(const Geo &g, const Duty &d, uint32_t jb, int tid,
                                            int nthreads, Fetch<VEC> &f) {
    constexpr int es = sizeof(typename IO::storage);
    if constexpr (VEC) {
        f.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(duty_rsrc(d, jb), d.goff, 0, 0));
    } else {
        const uint32_t blk_off = (uint32_t)(jb * g.row_step), bc_off = (uint32_t)(jb * g.bc_step);
        const int CH = 4 * g.W;
        const __amdgpu_buffer_rsrc_t rs[3] = {g.rx, g.rdt, g.rz};
        const int row = tid / CH, ci = tid % CH;
        const int ch = g.d0 + ci;
        const uint32_t off = ch < g.D ? blk_off + (uint32_t)((row * g.D + ch) * es) : kOOB;
#pragma unroll
        for (int i = 0; i < 3; ++i) f.own[i] = buf_ld<IO>(rs[i], off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * nthreads;
            const int brow = e / kRow, nn = e % kRow;
            const uint32_t boff = (e < kTB * kRow && nn < g.N)
                                      ? bc_off + (uint32_t)((brow * g.N + nn) * es) : kOOB;
            f.bce[i] = buf_ld<IO>(g.rb, boff);
            f.bce[4 + i] = buf_ld<IO>(g.rc, boff);
        }
    }
}

template <typename IO, bool VEC>
__device__ __forceinline__ void stage_block(const Geo &g, const Duty &d, const Tiles &T, char *lds,
                                            int slot, int tid, int nthreads, const Fetch<VEC> &f) {
    constexpr int es = sizeof(typename IO::storage);
    if constexpr (VEC) {
        // Lanes without a chunk (or past the channel range) write nothing:
        // channels past D are never stored, so their staged values do not matter.
        char *base = lds + (d.to_bc ? T.bc + slot * T.bc_slot : T.own + slot * T.own_slot);
        if (d.goff != kOOB) {
            if (es == 2 && d.scatter) {
                // bf16 B/C rows go in entry-major: 8 entries of one step, a
                // column of the [n][t] tile.
                char *dst = base + d.lds;
                const uint32_t w[4] = {f.v.x, f.v.y, f.v.z, f.v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint16_t *>(dst + e * kBcRowBytes) = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
            } else {
                *reinterpret_cast<uint4 *>(base + d.lds) = f.v;
            }
        }
    } else {
        char *own = lds + T.own + slot * T.own_slot;
        char *bc = lds + T.bc + slot * T.bc_slot;
        char *cc = bc + kBTile<IO>;
        const int row = tid / T.CH, ci = tid % T.CH;
        char *dst = own + row * T.rs + ci * es;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if constexpr (es == 2) *reinterpret_cast<uint16_t *>(dst + i * kPlane<IO>) = (uint16_t)f.own[i];
            else *reinterpret_cast<uint32_t *>(dst + i * kPlane<IO>) = f.own[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * nthreads;
            if (e < kTB * kRow) {
                if constexpr (es == 2) {
                    const int te = (e % kRow) * kBcRowBytes + (e / kRow) * es;  // entry-major
                    const int tc = (e / kRow) * kCRowBytes + (e % kRow) * es;   // step-major
                    *reinterpret_cast<uint16_t *>(bc + te) = (uint16_t)f.bce[i];
                    *reinterpret_cast<uint16_t *>(cc + tc) = (uint16_t)f.bce[4 + i];
                } else {
                    *reinterpret_cast<uint32_t *>(bc + e * es) = f.bce[i];
                    *reinterpret_cast<uint32_t *>(cc + e * es) = f.bce[4 + i];
                }
            }
        }
    }
}

// Outputs of block jb from ybuf half `par` to global memory.  The LDS read
// is issued by read_ybuf early and the store made later by store_y, so the
// read latency is hidden.
template <bool VEC>
struct YChunk;
template <>
struct YChunk<true> {
    uint4 v;
};
template <>
struct YChunk<false> {
    uint32_t v;
};
template <typename IO, bool VEC>
__device__ __forceinline__ YChunk<VEC> read_ybuf(const Duty &d, const Tiles &T, const char *lds,
                                                 int par, int tid) {
    constexpr int es = sizeof(typename IO::storage);
    const char *yb = lds + T.ybuf + par * T.ybuf_slot;
    YChunk<VEC> y;
    if constexpr (VEC) {
        y.v = *reinterpret_cast<const uint4 *>(yb + d.ylds);
    } else {
        const char *src = yb + (tid / T.CH) * T.rs + (tid % T.CH) * es;
        if constexpr (es == 2) y.v = *reinterpret_cast<const uint16_t *>(src);
        else y.v = *reinterpret_cast<const uint32_t *>(src);
    }
    return y;
}
template <typename IO, bool VEC>
__device__ __forceinline__ void store_y(const ScanKernelParams &p, const Geo &g, const Duty &d,
                                        const YChunk<VEC> &y, uint32_t jb, int tid) {
    constexpr int es = sizeof(typename IO::storage);
    if constexpr (VEC) {
        const uint32_t off = jb * d.step;
        const uint32_t rem = scalar_sat_sub(d.grec, off);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char *>(p.y) + (d.gbase - static_cast<const char *>(p.x)) + off, (short)0,
            (int)rem, kRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i_t, y.v), r, d.goff, 0, 0);
    } else {
        const int CH = 4 * g.W;
        const int row = tid / CH, ci = tid % CH;
        const int ch = g.d0 + ci;
        const uint32_t off = ch < g.D ? (uint32_t)(jb * g.row_step) + (uint32_t)((row * g.D + ch) * es) : kOOB;
        if constexpr (es == 2)
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)y.v, g.ry, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(y.v, g.ry, off, 0, 0);
    }
}

// Two products of the step loop can run on the matrix cores.  (dt A stays
// on the vector ALU: a 4x4x1 MFMA per step group, whose A-block broadcast
// hands every lane of a row the dt of steps 4g..4g+3, measured no faster than
// the 16 multiplies with dt read from lane k through a DPP row broadcast.)
//
// u B of steps 4g..4g+3, where u is a bf16 input (bf16 I/O without the conv
// prologue: u is x itself).  4x4x4 bf16 MFMA: a wave is 16 blocks of 4
// lanes, and the A operand of every block of a wave row is broadcast from
// the row's block g (CBSZ 2, ABID g).  Lane (c, t) gives its u at position t % 4
// of four (zeros elsewhere, udiag), so that block's A is the diagonal of
// u_{4g..4g+3}; lane (c, n) gives steps 4g..4g+3 of B's entry n as the B
// operand.  Register r of lane (c, n) holds u_{4g+r} B_{4g+r,n}: one exact
// product of two bf16 values.
// (The element path, which holds more registers per block, keeps the
// broadcast below.)
template <typename IO, bool CONV, bool VEC>
constexpr bool kBuMfma = std::is_same<IO, io_bf16>::value && !CONV && VEC;

__device__ __forceinline__ uint2 make_udiag(float u, uint32_t m0, uint32_t m1) {
    const uint32_t b = __builtin_bit_cast(uint32_t, u);  // a widened bf16: low half is 0
    const uint32_t two = b | (b >> 16);
    return make_uint2(two & m0, two & m1);
}
template <int G>
__device__ __forceinline__ mfma_f32x4 bu_group(uint2 udiag, uint2 bsteps) {
    const mfma_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mfma_bf16x4, udiag),
                                                  __builtin_bit_cast(mfma_bf16x4, bsteps), zero, 2, G, 0);
}

// Otherwise (conv prologue, or fp32 I/O) B reaches every wave row through a
// 0/1 selector MFMA and u B is a vector-ALU product.  Operands of one block's
// B rows held by a lane:
//  bf16 broadcast: staged entry-major ([n][t]), steps 4*(lane/16) .. +3 of
//        entry lane%16 (each value read once);
//  bf16 u B MFMA: steps 4g .. 4g+3 of entry lane%16, for g = 0..3;
//  fp32: per step group g, row 4g + lane/16, entry lane%16.
template <typename IO>
struct BcBlock;
template <>
struct BcBlock<io_bf16> {
    uint2 v;
};
template <>
struct BcBlock<io_f32> {
    float v[4];
};
template <typename IO, bool MF>
struct BOp {
    BcBlock<IO> v;
};
template <>
struct BOp<io_bf16, true> {
    uint2 g[4];
};
template <typename IO, bool MF>
__device__ __forceinline__ BOp<IO, MF> load_bop(const char *rows, int lane) {
    BOp<IO, MF> o;
    if constexpr (MF) {
        const char *r = rows + (lane & 15) * kBcRowBytes;
#pragma unroll
        for (int g = 0; g < 4; ++g) o.g[g] = *reinterpret_cast<const uint2 *>(r + 8 * g);
    } else if constexpr (std::is_same<IO, io_bf16>::value) {
        o.v.v = *reinterpret_cast<const uint2 *>(rows + (lane & 15) * kBcRowBytes + 8 * (lane >> 4));
    } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
            o.v.v[g] = *reinterpret_cast<const float *>(rows + ((4 * g + (lane >> 4)) * kRow + (lane & 15)) * 4);
    }
    return o;
}
// Broadcast of rows 4g..4g+3 to every wave row: register r of lane l gets
// entry l%16 of row 4g + r (0/1 selector, exact).
template <typename IO>
__device__ __forceinline__ mfma_f32x4 bcast(const BcBlock<IO> &op, const BcastSel &sel, int g) {
    const mfma_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (std::is_same<IO, io_bf16>::value)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sel.bf[g], __builtin_bit_cast(mfma_bf16x4, op.v),
                                                         zero, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x4f32(sel.f, op.v[g], zero, 0, 0, 0);
}

// Read-out weights.  After the transpose, lane (c, t) sums over the entries
// n of its channel the states of step t times w_n = C_{t,n} x_n, where x_n is
// 1/A_n in the fast form (which carries g = A h) and 1 otherwise.  The
// weights come from four MFMAs per block, one per entry group q; register r
// of group q holds w for entry 4q + r:
//  bf16 (16x16x16): D[4c + r][t] = sum_k X[4c + r][k] Y[k][t] with
//     Y[4s + i][t] = C_{t,4q+i} for every K block s (each lane reads entries
//     4q..4q+3 of its step row t), and X[4c + r][4s + i] = part s of x_{c,4q+r}
//     when i == r and s < 3, 0 otherwise.  x is cut into three bf16 parts
//     (hi, mid, lo: each the leading 8 bits of what the previous parts left),
//     which add up to x exactly, so each product is exact and w is x C
//     rounded in the MFMA's fp32 sums;
//  fp32 (16x16x4): Y[k][t] = C_{t,4q+k}, X[4c + r][k] = x_{c,4q+r} when k == r.
// X is constant per wave (WSel).
template <typename IO>
struct WSel;
template <>
struct WSel<io_bf16> {
    mfma_bf16x4 q[4];
};
template <>
struct WSel<io_f32> {
    float q[4];
};
template <typename IO>
struct COp;
template <>
struct COp<io_bf16> {
    uint4 v[2];  // entries 0..15 of step lane % 16
};
template <>
struct COp<io_f32> {
    float v[4];  // entry 4q + lane / 16 of step lane % 16, q = 0..3
};

// x of (channel cw0 + (lane % 16) / 4, entry 4q + lane % 4), the entry a lane
// gives to the A operand of the weight MFMAs.
template <bool FAST>
__device__ __forceinline__ float weight_x(const ScanKernelParams &p, int64_t cw0, int lane, int q) {
    const int64_t dd = cw0 + (lane & 15) / 4;
    const int e = 4 * q + (lane & 3);
    if (dd >= p.D || e >= p.N) return 0.0f;
    if (!FAST) return 1.0f;
    const float a = p.A[dd * p.N + e];
    return a != 0.0f ? 1.0f / a : 0.0f;
}
__device__ __forceinline__ uint32_t lead8(float v) {  // leading 8 significant bits of v
    return __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u;
}
template <typename IO, bool FAST>
__device__ __forceinline__ WSel<IO> make_wsel(const ScanKernelParams &p, int64_t cw0, int lane) {
    WSel<IO> w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float x = weight_x<FAST>(p, cw0, lane, q);
        if constexpr (std::is_same<IO, io_bf16>::value) {
            const uint32_t hi = lead8(x);
            const float r1 = x - __builtin_bit_cast(float, hi);
            const uint32_t mid = lead8(r1);
            const uint32_t lo = lead8(r1 - __builtin_bit_cast(float, mid));
            const int s = lane >> 4;
            const uint32_t part = s == 0 ? hi : s == 1 ? mid : s == 2 ? lo : 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) w.q[q][i] = i == (lane & 3) ? (short)(part >> 16) : (short)0;
        } else {
            w.q[q] = (lane >> 4) == (lane & 3) ? x : 0.0f;
        }
    }
    return w;
}
template <typename IO>
__device__ __forceinline__ COp<IO> load_cop(const char *ctile, int lane) {
    COp<IO> o;
    if constexpr (std::is_same<IO, io_bf16>::value) {
        const char *r = ctile + (lane & 15) * kCRowBytes;
        o.v[0] = *reinterpret_cast<const uint4 *>(r);
        o.v[1] = *reinterpret_cast<const uint4 *>(r + 16);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o.v[q] = *reinterpret_cast<const float *>(ctile + ((lane & 15) * kRow + 4 * q + (lane >> 4)) * 4);
    }
    return o;
}
template <typename IO, int Q>
__device__ __forceinline__ mfma_f32x4 weight_group(const WSel<IO> &ws, const COp<IO> &co) {
    const mfma_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (std::is_same<IO, io_bf16>::value) {
        const uint4 v = co.v[Q / 2];
        const uint2 y = Q % 2 == 0 ? make_uint2(v.x, v.y) : make_uint2(v.z, v.w);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ws.q[Q], __builtin_bit_cast(mfma_bf16x4, y), zero, 0,
                                                         0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(ws.q[Q], co.v[Q], zero, 0, 0, 0);
    }
}

struct LaneConst {
    float a, a2, ia, dsk, dbias, cb, wp0, wp1, wp2, wp3;
    bool live;     // the lane holds a real (channel, entry)
    bool dvalid;   // the lane's channel is real
    // A checkpoint slab entry (b D + d) 16 + n as the workgroup's uniform part
    // (b D + d0) 16 and the lane's part ((d - d0) 16 + n, below 2^10): the
    // store then takes a scalar base and a fixed lane offset.
    int64_t ckpt_wg;
    uint32_t ckpt_lane;
};

// Read-out of one step: lane (c, t) reads the 16 states of step t that the
// lanes of its row transposed into prow, and sums them times the weights.
__device__ __forceinline__ void load_partials(const float *prow, int n, float (&part)[kRow]) {
#pragma unroll
    for (int i = 0; i < kRow; ++i) part[i] = prow[i * kPStride + n];
}
__device__ __forceinline__ float sum_partials(const float (&part)[kRow], const mfma_f32x4 (&w)[4]) {
    float s0 = part[0] * w[0][0], s1 = part[1] * w[0][1];
#pragma unroll
    for (int i = 2; i < kRow; i += 2) {
        s0 = __builtin_fmaf(part[i], w[i / 4][i % 4], s0);
        s1 = __builtin_fmaf(part[i + 1], w[i / 4][(i + 1) % 4], s1);
    }
    return s0 + s1;
}

// Per-lane values carried from one block to the next.
struct Carry {
    float own[3];          // x, delta, z of this lane's step in the current block
    float u_prev, z_prev;  // u and z of this lane's step in the previous block
    float x_prev;          // conv history: x of the previous block (lanes 13..15 used)
    float h;               // state (A h in the fast form)
    float acc;             // read-out sum C h of this lane's step in the previous block
    float dsum;            // segment pass: this lane's dt summed since the last check
    float scum;            // segment pass: sum of dt of the channel up to the last check
    int head;              // segment pass: blocks until the entering state is forgotten, or -1
};

// The segment pass checks whether the entering state has been forgotten every
// kHeadCheck blocks (a head is then a multiple of that many blocks; checking
// less often only lengthens heads, which stays exact).
constexpr int kHeadCheck = 8;

// Sum over the 16 lanes of a row (every lane gets it): four rotations.
__device__ __forceinline__ float row_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x128, 0xf, 0xf, false);  // row_ror:8
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x124, 0xf, 0xf, false);  // row_ror:4
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x122, 0xf, 0xf, false);  // row_ror:2
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x121, 0xf, 0xf, false);  // row_ror:1
    return v;
}

// exp2 of anything below this is exactly 0 in fp32: once A log2(e) sum(dt)
// is below it for every state entry, the state a segment started from no
// longer reaches its outputs.
constexpr float kForgetExp2 = -160.0f;

template <typename IO>
__device__ __forceinline__ void read_own(const Tiles &T, const char *lds, int slot, int n, int ci,
                                         float (&v)[3]) {
    constexpr int es = sizeof(typename IO::storage);
    const char *src = lds + T.own + slot * T.own_slot + n * T.rs + ci * es;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if constexpr (es == 2) v[i] = widen<IO>(*reinterpret_cast<const uint16_t *>(src + i * kPlane<IO>));
        else v[i] = *reinterpret_cast<const float *>(src + i * kPlane<IO>);
    }
}

// Workgroup barrier of the wide block loop.  Every LDS operation that other
// waves depend on (the staging and ybuf writes, and the reads of a ring slot
// that a later block overwrites) has completed before it; only the wave's
// last SSM_PART_READ_OPS LDS instructions, the read-back of its own states (a
// wave-private area, reused only by this wave's next block), may still be in
// flight.  LDS instructions of one wave complete in order, so waiting until
// at most that many are outstanding covers all the earlier ones.  The
// read-back is at least SSM_PART_READ_OPS instructions (16 values, read at most
// two per instruction), and no LDS or scalar-memory instruction is issued
// between it and this barrier.
#define SSM_PART_READ_OPS 6
#define SSM_STR_(x) #x
#define SSM_STR(x) SSM_STR_(x)
__device__ __forceinline__ void wave_barrier() {
    asm volatile("s_waitcnt lgkmcnt(" SSM_STR(SSM_PART_READ_OPS) ")\n\ts_barrier" ::: "memory");
}

// Kernel variants (a template argument): the whole rows of a launch; a
// sequence segment's first pass (also recording what the combine needs); the
// backward's checkpoints (the state entering every block, no outputs).
constexpr int kWhole = 0, kSegPass = 1, kCkptPass = 2;

// Per-wave constants of the matrix-core products.
template <typename IO>
struct WaveOps {
    BcastSel sel;      // 0/1 selectors of the B broadcast
    WSel<IO> ws;       // read-out weight factors
    uint32_t um0, um1; // udiag masks: the half of the 4 x bf16 A operand that holds u
};

// One 16-step block of one wave, software-pipelined across blocks:
//   * right after the workgroup barrier, the LDS reads whose results are
//     needed later are issued: the next block's own inputs and B tile
//     (staged before this barrier) and the outputs two blocks back;
//   * the previous block's outputs are finished from its read-out sum, which
//     that block left in registers, so nothing after the barrier waits for
//     LDS before the step loop;
//   * the 16 recurrence steps run on this block's B tile, read one block
//     earlier; their states are transposed through the wave's own LDS area
//     and read back at once, with this block's C rows;
//   * block j+2 is copied from registers into LDS, block j+4 is requested
//     from global memory, the read-out weights are formed and the states
//     are summed.
// PAR = j % 2 selects the ybuf halves; SLOT = j % 3 when it is known at
// compile time; TAIL masks steps past the sequence end; STAGE is off in the
// last block.
template <typename IO, bool CONV, bool VEC, bool FAST, int KIND, bool TAIL, int PAR, bool STAGE,
          int SLOT = -1>
__device__ __forceinline__ void block_iter(const ScanKernelParams &p, const Span &sp, const Geo &geo,
                                           const Tiles &T, char *lds, int wave, int c, int n,
                                           int lane, const WaveOps<IO> &ops, const LaneConst &k,
                                           const Duty &du, int j, int s_run, Fetch<VEC> &f,
                                           BOp<IO, kBuMfma<IO, CONV, VEC>> &bop, Carry &cy) {
    constexpr bool MF = kBuMfma<IO, CONV, VEC>;
    constexpr bool STATS = KIND == kSegPass, CKPT = KIND == kCkptPass;
    constexpr int es = sizeof(typename IO::storage);
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int ci = 4 * wave + c;
    // LDS slot of this block: fixed at compile time (SLOT >= 0: every LDS offset
    // of the block is then an immediate) or the scalar s_run
    const int s_cur = SLOT >= 0 ? SLOT : s_run;
    const int s_next = s_cur == kSlots - 1 ? 0 : s_cur + 1;
    const int s_stage = s_next == kSlots - 1 ? 0 : s_next + 1;
    float *prow = reinterpret_cast<float *>(lds + T.part) + (wave * kChPerWave + c) * kPRow;

    // (A checkpoint launch reads no states back before its barrier.)
    if constexpr (VEC && !CKPT) wave_barrier();
    else __syncthreads();
    if (CKPT || p.ckpt) {
        // the state entering this block (the fast form carries A h)
        if (k.dvalid)
            (p.ckpt + (sp.t0 / kTB + j) * (p.B * p.D * kRow) + k.ckpt_wg)[k.ckpt_lane] = FAST ? cy.h * k.ia : cy.h;
    }
    // Wave priority (wide path): the recurrence steps run at a raised priority,
    // the LDS and memory phases around them at the base one, so a SIMD's
    // waves drift apart in phase and one wave's step loop issues while the
    // others wait on LDS.  Measured in one process against the same kernel
    // without it: 1-5% faster, outputs bit-identical.
    if constexpr (VEC && !CKPT) __builtin_amdgcn_s_setprio(0);
    // -- LDS reads of later blocks first ------------------------------------------
    float own_next[3];
    read_own<IO>(T, lds, s_next, n, ci, own_next);
    YChunk<VEC> yst;
    if constexpr (!CKPT) yst = read_ybuf<IO, VEC>(du, T, lds, PAR, tid);
    const BOp<IO, MF> bop_n = load_bop<IO, MF>(lds + T.bc + s_next * T.bc_slot, lane);

    // -- this block's inputs ---------------------------------------------------
    const float xv = cy.own[0];
    float dt = cy.own[1];
    const float zv = cy.own[2];
    float u = xv;
    if (CONV) {
        const float xm1 = row_shift_in<1>(xv, cy.x_prev);
        const float xm2 = row_shift_in<2>(xv, cy.x_prev);
        const float xm3 = row_shift_in<3>(xv, cy.x_prev);
        u = silu(k.cb + k.wp0 * xm3 + k.wp1 * xm2 + k.wp2 * xm1 + k.wp3 * xv);
        cy.x_prev = xv;
    }
    if (p.softplus) dt = softplus_fast(dt + k.dbias);
    if (TAIL && sp.t0 + j * kTB + n >= sp.t1) {  // past the end: the state must not move
        dt = 0.0f;
        u = 0.0f;
    }
    if constexpr (STATS) {
        // Decay of the entering state through the blocks so far: exp(A sum(dt)).
        cy.dsum += dt;
        if ((j & (kHeadCheck - 1)) == kHeadCheck - 1) {
            cy.scum += row_sum(cy.dsum);
            cy.dsum = 0.0f;
            if (cy.head < 0 && __all(!k.live || k.a2 * cy.scum < kForgetExp2)) cy.head = (int)j + 1;
        }
    }

    // -- outputs of block j-1 (lane (c, n) finishes its step n) ---------------
    if constexpr (!CKPT) {
        float yv = cy.acc + k.dsk * cy.u_prev;
        if (p.z) yv *= silu(cy.z_prev);
        char *ydst = lds + T.ybuf + (1 - PAR) * T.ybuf_slot + n * T.rs + ci * es;
        if constexpr (es == 2)
            *reinterpret_cast<uint16_t *>(ydst) = __builtin_bit_cast(uint16_t, (__bf16)yv);
        else
            *reinterpret_cast<float *>(ydst) = yv;
    }
    // -- outputs of block j-2 leave ----------------------------------------------
    if constexpr (!CKPT)
        if (j >= 2 && (!VEC || du.ystore)) store_y<IO, VEC>(p, geo, du, yst, j - 2, tid);

    // -- the 16 steps ----------------------------------------------------------
    // Steps in groups of four: the group's u B (or B) comes from an MFMA
    // issued one group ahead, so the matrix cores' latency is hidden, and the
    // group's four states leave with one 128-bit LDS write.
    uint2 ud = make_uint2(0u, 0u);
    if constexpr (MF) ud = make_udiag(u, ops.um0, ops.um1);
    auto bu_of = [&](auto G) -> mfma_f32x4 {
        constexpr int g = decltype(G)::value;
        if constexpr (MF) return bu_group<g>(ud, bop.g[g]);
        else return bcast<IO>(bop.v, ops.sel, g);
    };
    if constexpr (VEC && !CKPT) __builtin_amdgcn_s_setprio(2);
    mfma_f32x4 Bn = bu_of(ic<0>{});
    static_for<kTB / 4>([&](auto G) {
        constexpr int gi = decltype(G)::value;
        constexpr int g4 = 4 * gi;
        const mfma_f32x4 Bk = Bn;
        if constexpr (gi + 1 < kTB / 4) {
            Bn = bu_of(ic<gi + 1>{});
        }
        float pk[4];
        static_for<4>([&](auto K) {
            constexpr int kk = decltype(K)::value;
            constexpr int kx = g4 + kk;
            const float e = hw_exp2(row_bcast<kx>(dt) * k.a2);
            float bu;
            if constexpr (MF) bu = Bk[kk];
            else bu = row_bcast<kx>(u) * Bk[kk];
            float bx;
            if (FAST) {
                bx = __builtin_fmaf(e, bu, -bu);  // h holds A h here
            } else {
                const float dtk = row_bcast<kx>(dt);
                bx = (dtk * phi_of(dtk * k.a, e)) * bu;
            }
            cy.h = __builtin_fmaf(e, cy.h, bx);
            pk[kk] = cy.h;
        });
        if constexpr (!CKPT)
            *reinterpret_cast<float4 *>(&prow[n * kPStride + g4]) = make_float4(pk[0], pk[1], pk[2], pk[3]);
    });
    // The states are this wave's own: they are read back (LDS operations of
    // one wave complete in order) after this block's C rows and the staging
    // writes, so that the reads may still be in flight at the next barrier
    // (wide path; see wave_barrier).  The element path reads C after
    // staging (its fetch registers are live until then).
    if constexpr (VEC && !CKPT) __builtin_amdgcn_s_setprio(0);
    float part[kRow];
    COp<IO> cop;
    if constexpr (CKPT) {
    } else if constexpr (VEC) {
        cop = load_cop<IO>(lds + T.bc + s_cur * T.bc_slot + kBTile<IO>, lane);
    } else {
        load_partials(prow, n, part);
    }

    cy.u_prev = u;
    cy.z_prev = zv;
#pragma unroll
    for (int i = 0; i < 3; ++i) cy.own[i] = own_next[i];
    bop = bop_n;

    if (STAGE) {
        __builtin_amdgcn_sched_barrier(0);
        stage_block<IO, VEC>(geo, du, T, lds, s_stage, tid, nthreads, f);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (VEC && !CKPT) {
        load_partials(prow, n, part);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (STAGE) {
        // Keep the refill after the copy, so the new data can land in the
        // same registers.
        fetch_block<IO, VEC>(geo, du, j + 4, tid, nthreads, f);
    }
    if constexpr (VEC && !CKPT) __builtin_amdgcn_s_setprio(0);  // the read-out sums too
    if constexpr (!CKPT) {
        if constexpr (!VEC) cop = load_cop<IO>(lds + T.bc + s_cur * T.bc_slot + kBTile<IO>, lane);
        const mfma_f32x4 w[4] = {weight_group<IO, 0>(ops.ws, cop), weight_group<IO, 1>(ops.ws, cop),
                                 weight_group<IO, 2>(ops.ws, cop), weight_group<IO, 3>(ops.ws, cop)};
        cy.acc = sum_partials(part, w);
    }
}

template <typename IO, bool CONV, bool VEC, bool FAST, int KIND>
__device__ __forceinline__ void scan_tiles_body(const ScanKernelParams &p, const Span &sp, const Geo &geo,
                                                const Tiles &T, char *lds, int64_t b, int wave,
                                                int c, int n, const LaneConst &k, Carry &cy) {
    constexpr bool STATS = KIND == kSegPass, CKPT = KIND == kCkptPass;
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int lane = tid & 63;
    const int ci = 4 * wave + c;
    WaveOps<IO> ops;
    ops.sel = make_sel(lane);
    ops.ws = make_wsel<IO, FAST>(p, geo.d0 + 4 * wave, lane);
    ops.um0 = (n & 3) == 0 ? 0x0000FFFFu : (n & 3) == 1 ? 0xFFFF0000u : 0u;
    ops.um1 = (n & 3) == 2 ? 0x0000FFFFu : (n & 3) == 3 ? 0xFFFF0000u : 0u;
    const int64_t rows = sp.t1 - sp.t0;
    const int nblocks = (int)((rows + kTB - 1) / kTB);

    // Block j is requested four blocks ahead, copied into LDS slot j % 3
    // two blocks ahead, and its outputs leave LDS two blocks later.  Two
    // fetch register sets alternate (the loop is unrolled by two).  The loop
    // has a single exit at its bottom: an exit in the middle would route
    // through the back-edge once the control flow is structured, and the
    // load counters merged there would force a wait for every prefetch in
    // flight.  Prefetches past the last block read zeros or unused rows and
    // are never consumed.
    const Duty du = make_duty<IO>(p, sp, T, b, geo.d0, __builtin_amdgcn_readfirstlane(wave), lane);
    Fetch<VEC> fa, fb;
    fetch_block<IO, VEC>(geo, du, 0, tid, nthreads, fa);
    fetch_block<IO, VEC>(geo, du, 1, tid, nthreads, fb);
    stage_block<IO, VEC>(geo, du, T, lds, 0, tid, nthreads, fa);
    fetch_block<IO, VEC>(geo, du, 2, tid, nthreads, fa);
    stage_block<IO, VEC>(geo, du, T, lds, 1, tid, nthreads, fb);
    fetch_block<IO, VEC>(geo, du, 3, tid, nthreads, fb);
    __syncthreads();
    read_own<IO>(T, lds, 0, n, ci, cy.own);
    BOp<IO, kBuMfma<IO, CONV, VEC>> bop = load_bop<IO, kBuMfma<IO, CONV, VEC>>(lds + T.bc, lane);
    cy.u_prev = 0.0f;
    cy.z_prev = 0.0f;
    cy.acc = 0.0f;

    int s = 0;  // LDS slot of block j
    int j = 0;
    // Six blocks per iteration (wide path): the ring slot (j % 3) and the ybuf
    // half (j % 2) are then compile-time constants, so no LDS address is
    // computed per block.  The element path holds more registers per block and
    // keeps the two-block loop.
    if constexpr (VEC) for (; j + 6 < nblocks; j += 6) {
        block_iter<IO, CONV, VEC, FAST, KIND, false, 0, true, 0>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j, 0, fa, bop, cy);
        block_iter<IO, CONV, VEC, FAST, KIND, false, 1, true, 1>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j + 1, 0, fb, bop, cy);
        block_iter<IO, CONV, VEC, FAST, KIND, false, 0, true, 2>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j + 2, 0, fa, bop, cy);
        block_iter<IO, CONV, VEC, FAST, KIND, false, 1, true, 0>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j + 3, 0, fb, bop, cy);
        block_iter<IO, CONV, VEC, FAST, KIND, false, 0, true, 1>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j + 4, 0, fa, bop, cy);
        block_iter<IO, CONV, VEC, FAST, KIND, false, 1, true, 2>(p, sp, geo, T, lds, wave, c, n, lane, ops,
                                                                k, du, j + 5, 0, fb, bop, cy);
    }
    // The remaining blocks (j % 6 == 0, so the slot is 0 again): pairs with the
    // slot kept scalar (it is the same for the whole workgroup).
    auto advance = [&]() { s = __builtin_amdgcn_readfirstlane(s == kSlots - 1 ? 0 : s + 1); };
    for (; j + 2 < nblocks; j += 2) {
        block_iter<IO, CONV, VEC, FAST, KIND, false, 0, true>(p, sp, geo, T, lds, wave, c, n, lane, ops, k,
                                                        du, j, s, fa, bop, cy);
        advance();
        block_iter<IO, CONV, VEC, FAST, KIND, false, 1, true>(p, sp, geo, T, lds, wave, c, n, lane, ops, k,
                                                        du, j + 1, s, fb, bop, cy);
        advance();
    }
    // One or two blocks remain (j is even).
    int last_par;
    if (j + 1 < nblocks) {
        block_iter<IO, CONV, VEC, FAST, KIND, false, 0, true>(p, sp, geo, T, lds, wave, c, n, lane, ops, k,
                                                        du, j, s, fa, bop, cy);
        advance();
        block_iter<IO, CONV, VEC, FAST, KIND, true, 1, false>(p, sp, geo, T, lds, wave, c, n, lane, ops, k,
                                                        du, j + 1, s, fb, bop, cy);
        last_par = 1;
    } else {
        block_iter<IO, CONV, VEC, FAST, KIND, true, 0, false>(p, sp, geo, T, lds, wave, c, n, lane, ops, k,
                                                        du, j, s, fa, bop, cy);
        last_par = 0;
    }
    if constexpr (STATS) {
        // the dt of the blocks since the last check
        cy.scum += row_sum(cy.dsum);
        if (cy.head < 0 && __all(!k.live || k.a2 * cy.scum < kForgetExp2)) cy.head = nblocks;
    }
    if constexpr (CKPT) return;
    // Outputs of the last block and of the one before it.
    constexpr int es = sizeof(typename IO::storage);
    const int jl = nblocks - 1;
    __syncthreads();  // every wave has read ybuf[last_par] for its store
    {
        float yv = cy.acc + k.dsk * cy.u_prev;
        if (p.z) yv *= silu(cy.z_prev);
        char *ydst = lds + T.ybuf + last_par * T.ybuf_slot + n * T.rs + ci * es;
        if constexpr (es == 2)
            *reinterpret_cast<uint16_t *>(ydst) = __builtin_bit_cast(uint16_t, (__bf16)yv);
        else
            *reinterpret_cast<float *>(ydst) = yv;
    }
    __syncthreads();
    if (!VEC || du.ystore) {
        const YChunk<VEC> y1 = read_ybuf<IO, VEC>(du, T, lds, 1 - last_par, tid);
        const YChunk<VEC> y0 = read_ybuf<IO, VEC>(du, T, lds, last_par, tid);
        if (jl >= 1) store_y<IO, VEC>(p, geo, du, y1, jl - 1, tid);
        store_y<IO, VEC>(p, geo, du, y0, jl, tid);
    }
}

// blockDim.x = 64 W; workgroup g covers channels [4 W q, 4 W q + 4 W) of
// batch row g / groups_per_b, with q = g % groups_per_b.
// Register budget: the wide path 4 waves per SIMD (<= 128 VGPRs; a 96-VGPR
// budget, 5 waves per SIMD, spilled in the conv variants and ran slower on
// every measured layer), the element path 3 (<= 168 VGPRs: it holds more
// registers per block and spilled in its block loop at 128).
template <bool VEC>
constexpr int kWavesPerSimd = VEC ? 4 : 3;

template <typename IO, bool CONV, bool VEC, int KIND>
__global__ __launch_bounds__(256 * kWavesPerSimd<VEC>)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<VEC>, 8)))
void scan_tiles_kernel(ScanKernelParams p) {
    constexpr bool STATS = KIND == kSegPass;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int es = sizeof(typename IO::storage);
    const int W = blockDim.x / 64;
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x & 63;
    const int c = lane / kRow, n = lane % kRow;
    const int64_t gid = xcd_group(blockIdx.x, gridDim.x);
    const int64_t grp = gid % p.ngroups;
    const int64_t b = grp / p.groups_per_b;
    const int d0 = (int)((grp % p.groups_per_b) * 4 * W);
    const int64_t d = d0 + 4 * wave + c;
    const bool dvalid = d < p.D;
    const bool live = dvalid && n < p.N;
    const int64_t D = p.D, N = p.N;
    const int64_t BDN = p.B * D * N;

    // This workgroup's rows and states (segments shift them; all uniform).
    Span sp{p.t_begin, p.t_end};
    const float *h_in = p.h_in;
    float *h_out = p.h_out;
    int64_t seg = 0;
    if (p.mode != 0) {
        seg = gid / p.ngroups + (p.mode == 2 ? 1 : 0);
        sp.t0 = p.t_begin + seg * p.seg_len;
        sp.t1 = std::min(p.t_end, sp.t0 + p.seg_len);
        if (p.mode == 1) {
            h_in = seg == 0 ? p.h_in : nullptr;
            h_out = p.ws_hend + seg * BDN;
        } else {
            const int head = p.ws_head[seg * p.ngroups + grp];
            sp.t1 = std::min(sp.t1, sp.t0 + (int64_t)head * kTB);
            h_in = p.ws_hin + seg * BDN;
            h_out = nullptr;
        }
    }
    const int64_t rows = sp.t1 - sp.t0;
    const Tiles T = tile_layout<IO>(W);

    Geo geo;
    const int64_t xbase = (b * p.L + sp.t0) * D * es;
    const int64_t xrec = rows * D * es;
    geo.rx = rsrc(p.x, xbase, xrec);
    geo.rdt = rsrc(p.delta, xbase, xrec);
    // Without a gate the descriptor has no records: loads return 0.
    geo.rz = p.z ? rsrc(p.z, xbase, xrec) : rsrc(p.x, 0, 0);
    geo.ry = rsrc(p.y, xbase, xrec);
    const int64_t bbase = (b * p.L + sp.t0) * N * es;
    geo.rb = rsrc(p.Bm, bbase, rows * N * es);
    geo.rc = rsrc(p.Cm, bbase, rows * N * es);
    geo.row_step = (uint32_t)(kTB * D * es);
    geo.bc_step = (uint32_t)(kTB * N * es);
    geo.D = D;
    geo.N = (int)N;
    geo.W = W;
    geo.d0 = d0;

    LaneConst k;
    k.live = live;
    k.dvalid = dvalid;
    k.ckpt_wg = (b * D + d0) * kRow;
    k.ckpt_lane = (uint32_t)((4 * wave + c) * kRow + n);
    k.a = live ? p.A[d * N + n] : 0.0f;
    k.a2 = k.a * kLog2e;
    k.ia = (k.a != 0.0f) ? 1.0f / k.a : 0.0f;
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
    Carry cy;
    cy.h = (live && h_in) ? h_in[(b * D + d) * N + n] : 0.0f;
    cy.scum = 0.0f;
    cy.dsum = 0.0f;
    cy.head = -1;
    // Conv history entering the rows: x at rows t0 - 16 + n (only the last
    // three lanes of a row are used); before row 0 it comes from the
    // entering conv state, or is 0.
    cy.x_prev = 0.0f;
    if (CONV && dvalid && n >= kRow - 3) {
        const int64_t t = sp.t0 - kRow + n;
        if (t >= 0)
            cy.x_prev = load_io<IO>(p.x, (b * p.L + t) * D + d);
        else if (p.cs_in && t >= -(int64_t)(p.K - 1))
            cy.x_prev = load_io<IO>(p.cs_in, (b * (p.K - 1) + (p.K - 1) + t) * D + d);
    }
    // Wave-uniform choice of the update form (see the file comment).
    const bool fast = __all(!live || fabsf(k.a) >= kFastMinAbsA);
    if (rows > 0) {
        if (fast) {
            // The fast form carries g = A h (the 1/A moves to the read-out).
            cy.h *= k.a;
            scan_tiles_body<IO, CONV, VEC, true, KIND>(p, sp, geo, T, lds, b, wave, c, n, k, cy);
            cy.h *= k.ia;
        } else {
            scan_tiles_body<IO, CONV, VEC, false, KIND>(p, sp, geo, T, lds, b, wave, c, n, k, cy);
        }
    }
    if (h_out && live) h_out[(b * D + d) * N + n] = cy.h;
    if constexpr (STATS) {
        // Sum of dt per channel, and the workgroup's head length: the most
        // blocks any of its waves needs before the entering state is gone.
        if (dvalid && n == 0) p.ws_stot[(seg * p.B + b) * D + d] = cy.scum;
        const int nblk = (int)((rows + kTB - 1) / kTB);
        int *kred = reinterpret_cast<int *>(lds + T.part + (size_t)W * kChPerWave * kPRow * sizeof(float));
        __syncthreads();
        if (lane == 0) kred[wave] = cy.head < 0 ? nblk : cy.head;
        __syncthreads();
        if (threadIdx.x == 0) {
            int m = 0;
            for (int w = 0; w < W; ++w) m = std::max(m, kred[w]);
            p.ws_head[seg * p.ngroups + grp] = m;
        }
    }
}

// State entering every segment and after the last one: segment 0 ran from
// the true state; segment s > 0 from zero, so its true end state is
// exp(A sum(dt)) times its entering state plus its local end state.
__global__ void seg_combine_kernel(const float *A, const float *hend, const float *stot,
                                   float *hin, float *h_final, int64_t B, int64_t D, int N,
                                   int nseg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t BDN = B * D * N;
    if (i >= BDN) return;
    const int64_t bd = i / N;
    const int64_t d = bd % D;
    const float a2 = A[d * N + i % N] * kLog2e;
    float h = hend[i];
    for (int s = 1; s < nseg; ++s) {
        hin[s * BDN + i] = h;
        h = __builtin_amdgcn_exp2f(a2 * stot[s * B * D + bd]) * h + hend[s * BDN + i];
    }
    if (h_final) h_final[i] = h;
}

// Conv state after the scan, per (batch, channel): x at rows L-(K-1)..L-1,
// from the entering conv state (or 0) where the row is negative.  Raw bit
// copies; each thread reads its whole window before writing, so the state
// may be updated in place.
template <typename T>
__global__ void conv_state_out_kernel(const T *x, const T *cs_in, T *cs_out, int64_t B, int64_t L,
                                      int64_t D, int K) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // b * D + d
    if (i >= B * D) return;
    const int64_t b = i / D, d = i % D;
    T v[SSM_MAX_CONV_K - 1];
#pragma unroll
    for (int k = 0; k < SSM_MAX_CONV_K - 1; ++k) {
        if (k >= K - 1) break;
        const int64_t t = L - (K - 1) + k;
        v[k] = t >= 0 ? x[(b * L + t) * D + d] : cs_in ? cs_in[(b * (K - 1) + (K - 1) + t) * D + d] : T(0);
    }
#pragma unroll
    for (int k = 0; k < SSM_MAX_CONV_K - 1; ++k) {
        if (k >= K - 1) break;
        cs_out[(b * (K - 1) + k) * D + d] = v[k];
    }
}

hipError_t launch_conv_state_out(const ssm_scan_args_t &a, hipStream_t stream) {
    if (!a.conv_state_out || a.conv_k < 2 || a.batch == 0) return hipSuccess;
    const int64_t n = a.batch * a.dim;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (a.io_dtype == SSM_BF16)
        conv_state_out_kernel<uint16_t><<<blocks, 256, 0, stream>>>(
            static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.conv_state_in),
            static_cast<uint16_t *>(a.conv_state_out), a.batch, a.seqlen, a.dim, (int)a.conv_k);
    else
        conv_state_out_kernel<uint32_t><<<blocks, 256, 0, stream>>>(
            static_cast<const uint32_t *>(a.x), static_cast<const uint32_t *>(a.conv_state_in),
            static_cast<uint32_t *>(a.conv_state_out), a.batch, a.seqlen, a.dim, (int)a.conv_k);
    return hipGetLastError();
}

__global__ void copy_or_zero_kernel(const float *src, float *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// Waves per workgroup: the workgroups should spread evenly over the 256 CUs.
// A CU holds 4 x kWavesPerSimd waves of this kernel and 160 KiB of LDS.
// Among the allowed W pick the one whose busiest CU carries the least work,
// preferring wider tiles.  The wide path needs 3 ceil(W / cw) + 2 <= W waves
// for its load duties (cw = channels per 16-byte chunk) and, for bf16, an
// even W so that every workgroup's channel range starts on a 16-byte
// boundary.
bool wide_w_ok(int W, int64_t es) {
    const int cw = (int)(16 / es);
    if (es == 2 && W % 2 != 0) return false;
    return 3 * ((W + cw - 1) / cw) + 2 <= W;
}

int choose_waves(int64_t batch, int64_t dim, bool wide, int64_t es) {
    constexpr int64_t kCUs = 256, kLdsPerCU = 160 * 1024;
    const int64_t waves_per_cu = 4 * (wide ? kWavesPerSimd<true> : kWavesPerSimd<false>);
    int best = 0;
    double best_cost = 1e300;
    for (int W = 1; W <= std::min<int64_t>(kMaxW, waves_per_cu); ++W) {
        if (wide && !wide_w_ok(W, es)) continue;
        const int64_t lds = (int64_t)(es == 2 ? tile_lds_bytes<io_bf16>(W) : tile_lds_bytes<io_f32>(W));
        const int64_t per_row = (dim + 4 * W - 1) / (4 * W);
        const int64_t groups = per_row * batch;
        const int64_t per_cu = (groups + kCUs - 1) / kCUs;  // workgroups on the busiest CU
        const int64_t fit = std::max<int64_t>(1, std::min(waves_per_cu / W, kLdsPerCU / lds));  // resident at once
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
    const int64_t copies = p.mode == 0 ? 1 : p.mode == 1 ? p.nseg : p.nseg - 1;
    const unsigned grid = (unsigned)(p.ngroups * copies);
    const size_t lds = tile_lds_bytes<IO>(W);
    if (p.mode == 1) {
        if (p.K > 0)
            scan_tiles_kernel<IO, true, VEC, kSegPass><<<grid, 64 * W, lds, stream>>>(p);
        else
            scan_tiles_kernel<IO, false, VEC, kSegPass><<<grid, 64 * W, lds, stream>>>(p);
    } else if (p.ckpt_only) {
        if (p.K > 0)
            scan_tiles_kernel<IO, true, VEC, kCkptPass><<<grid, 64 * W, lds, stream>>>(p);
        else
            scan_tiles_kernel<IO, false, VEC, kCkptPass><<<grid, 64 * W, lds, stream>>>(p);
    } else {
        if (p.K > 0)
            scan_tiles_kernel<IO, true, VEC, kWhole><<<grid, 64 * W, lds, stream>>>(p);
        else
            scan_tiles_kernel<IO, false, VEC, kWhole><<<grid, 64 * W, lds, stream>>>(p);
    }
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

// Sequence segments.  With few (batch, channel) pairs the scan alone cannot
// fill the GPU (one wave per 4 channels); a long sequence is then cut into
// S segments scanned at the same time:
//   1. every segment is scanned from a zero state (the first from the true
//      one), writing y, its end state, its sum of dt and the number of
//      blocks after which exp(A sum(dt)) is exactly 0 in fp32 for all its
//      state entries (its "head");
//   2. the true entering states follow in one pass over the segments:
//      h_in(s+1) = exp(A sum_s(dt)) h_in(s) + h_end(s);
//   3. the heads of segments 1.. are scanned again from their true entering
//      states, overwriting y there.  Past the head the zero-start outputs
//      already are the true ones: the entering state's share has decayed to 0.
// The extra work is the heads (short when A dt is not tiny; a whole segment
// when some A is 0).
constexpr int64_t kMinSegRows = 2048;
constexpr int64_t kMaxSegs = 64;
constexpr int64_t kWaveTarget = 4096;  // about 4 waves per SIMD

struct Plan {
    int W, nseg;
    int64_t chunk, seg_len, groups_per_b, ngroups;
    bool vec;
    size_t ws_carry, ws_hend, ws_hin, ws_stot, ws_head, total;
};

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

Plan make_plan(const ssm_scan_args_t &a, bool segments = true) {
    Plan q;
    const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    // Wide (16-byte chunk) staging needs whole chunks per row, N = 16 and
    // 16-byte aligned tensors; otherwise elements are staged one by one.
    auto al = [](const void *v) { return ((uintptr_t)v % 16) == 0; };
    q.vec = (a.dim % (16 / es) == 0) && a.dstate == kRow && al(a.x) && al(a.delta) &&
            al(a.y) && (!a.z || al(a.z)) && al(a.Bm) && al(a.Cm);
    q.chunk = rows_per_launch(a);
    const int64_t rows = std::min(a.seqlen, q.chunk);  // rows of the longest launch
    const int64_t waves = a.batch * ((a.dim + 3) / 4);
    int64_t S = 1;
    if (segments && waves * 2 < kWaveTarget)
        S = std::max<int64_t>(1, std::min({kMaxSegs, kWaveTarget / std::max<int64_t>(waves, 1),
                                           rows / kMinSegRows}));
    q.nseg = (int)S;
    q.seg_len = S > 1 ? ((rows + S - 1) / S + kTB - 1) / kTB * kTB : rows;
    q.W = choose_waves(a.batch * S, a.dim, q.vec, es);
    q.groups_per_b = q.W ? (a.dim + 4 * q.W - 1) / (4 * q.W) : 0;
    q.ngroups = q.groups_per_b * a.batch;
    const size_t bdn = (size_t)(a.batch * a.dim * a.dstate) * sizeof(float);
    q.ws_carry = a.seqlen > q.chunk ? round256(bdn) : 0;
    q.ws_hend = S > 1 ? round256(bdn * S) : 0;
    q.ws_hin = S > 1 ? round256(bdn * S) : 0;
    q.ws_stot = S > 1 ? round256((size_t)(a.batch * a.dim) * sizeof(float) * S) : 0;
    q.ws_head = S > 1 ? round256((size_t)q.ngroups * sizeof(int) * S) : 0;
    q.total = q.ws_carry + q.ws_hend + q.ws_hin + q.ws_stot + q.ws_head;
    return q;
}

hipError_t launch_pass(const ssm_scan_args_t &a, const ScanKernelParams &p, const Plan &q,
                       hipStream_t stream) {
    if (a.io_dtype == SSM_BF16)
        return q.vec ? launch_typed<io_bf16, true>(p, q.W, stream) : launch_typed<io_bf16, false>(p, q.W, stream);
    return q.vec ? launch_typed<io_f32, true>(p, q.W, stream) : launch_typed<io_f32, false>(p, q.W, stream);
}

}  // namespace

size_t scan_workspace_bytes(const ssm_scan_args_t &a) {
    // A sequence too long for one launch is split; the state between the
    // launches lives in the workspace, and so do the segment records.
    return make_plan(a).total;
}

hipError_t launch_scan_fwd(const ssm_scan_args_t &a, hipStream_t stream) {
    const Plan q = make_plan(a);
    const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    if (q.W == 0 || q.ngroups * q.nseg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (q.chunk < 2 * kTB || a.dim * es > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ScanKernelParams p;
    p.B = a.batch;
    p.L = a.seqlen;
    p.D = a.dim;
    p.N = (int)a.dstate;
    p.K = (int)a.conv_k;
    p.softplus = a.delta_softplus;
    p.groups_per_b = q.groups_per_b;
    p.ngroups = q.ngroups;
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
    p.cs_in = a.conv_k > 0 ? a.conv_state_in : nullptr;
    p.y = a.y;
    p.ckpt = a.checkpoints;
    p.ckpt_only = 0;
    p.mode = 0;
    p.nseg = 1;
    p.seg_len = q.seg_len;
    char *ws = static_cast<char *>(a.workspace);
    float *carry = reinterpret_cast<float *>(ws);
    p.ws_hend = reinterpret_cast<float *>(ws + q.ws_carry);
    float *hin = reinterpret_cast<float *>(ws + q.ws_carry + q.ws_hend);
    p.ws_hin = hin;
    p.ws_stot = reinterpret_cast<float *>(ws + q.ws_carry + q.ws_hend + q.ws_hin);
    p.ws_head = reinterpret_cast<int *>(ws + q.ws_carry + q.ws_hend + q.ws_hin + q.ws_stot);
    hipError_t e = hipSuccess;
    for (int64_t t = 0; t < a.seqlen && e == hipSuccess; t += q.chunk) {
        const bool first = t == 0, last = t + q.chunk >= a.seqlen;
        p.t_begin = t;
        p.t_end = last ? a.seqlen : t + q.chunk;
        p.h_in = first ? a.h0 : carry;
        p.h_out = last ? a.h_final : carry;
        const int64_t nseg = q.nseg > 1 ? (p.t_end - p.t_begin + q.seg_len - 1) / q.seg_len : 1;
        if (nseg <= 1) {
            p.mode = 0;
            p.nseg = 1;
            e = launch_pass(a, p, q, stream);
            continue;
        }
        p.nseg = (int)nseg;
        p.mode = 1;
        e = launch_pass(a, p, q, stream);
        if (e != hipSuccess) break;
        const int64_t bdn = a.batch * a.dim * a.dstate;
        seg_combine_kernel<<<(unsigned)((bdn + 255) / 256), 256, 0, stream>>>(
            a.A, p.ws_hend, p.ws_stot, hin, p.h_out, a.batch, a.dim, (int)a.dstate, p.nseg);
        e = hipGetLastError();
        if (e != hipSuccess) break;
        p.mode = 2;
        e = launch_pass(a, p, q, stream);
    }
    // The conv state is written after every pass has read the entering one
    // (it may be the same tensor).
    if (e == hipSuccess) e = launch_conv_state_out(a, stream);
    return e;
}

hipError_t launch_scan_ckpt(const ssm_scan_args_t &a, float *ckpt, hipStream_t stream) {
    const Plan q = make_plan(a, false);
    const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
    if (q.W == 0 || q.ngroups > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (q.chunk < 2 * kTB || a.dim * es > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ScanKernelParams p{};
    p.B = a.batch;
    p.L = a.seqlen;
    p.D = a.dim;
    p.N = (int)a.dstate;
    p.K = (int)a.conv_k;
    p.softplus = a.delta_softplus;
    p.groups_per_b = q.groups_per_b;
    p.ngroups = q.ngroups;
    p.x = a.x;
    p.delta = a.delta;
    p.Bm = a.Bm;
    p.Cm = a.Cm;
    p.z = nullptr;
    p.A = a.A;
    p.Dskip = nullptr;
    p.dbias = a.delta_bias;
    p.conv_w = a.conv_w;
    p.conv_b = a.conv_b;
    p.cs_in = a.conv_k > 0 ? a.conv_state_in : nullptr;
    p.y = nullptr;
    p.ckpt = ckpt;
    p.ckpt_only = 1;
    p.mode = 0;
    p.nseg = 1;
    p.seg_len = q.seg_len;
    // Launches start on block boundaries (q.chunk is a multiple of 32 rows),
    // so the state between two launches is the checkpoint of the second's
    // first block: each launch leaves it there and the next one starts from it.
    const int64_t slab = a.batch * a.dim * (int64_t)kRow;
    hipError_t e = hipSuccess;
    for (int64_t t = 0; t < a.seqlen && e == hipSuccess; t += q.chunk) {
        const bool first = t == 0, last = t + q.chunk >= a.seqlen;
        p.t_begin = t;
        p.t_end = last ? a.seqlen : t + q.chunk;
        p.h_in = first ? a.h0 : ckpt + (t / kTB) * slab;
        p.h_out = last ? nullptr : ckpt + (p.t_end / kTB) * slab;
        e = launch_pass(a, p, q, stream);
    }
    return e;
}

hipError_t launch_empty_scan_state(const ssm_scan_args_t &a, hipStream_t stream) {
    const int64_t n = a.batch * a.dim * a.dstate;
    if (a.h_final && n > 0) {
        copy_or_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a.h0, a.h_final, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_conv_state_out(a, stream);
}

}  // namespace ssm
