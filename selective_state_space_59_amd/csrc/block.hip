// block.hip -- one Mamba (S6) block with its pre-norm residual, on gfx950.
//
// The block of "Mamba: Linear-Time Sequence Modeling with Selective State
// Spaces" (paper summary page, sec. 4a, the table of tensor shapes): RMSNorm,
// the expanding Linear (x and gate halves), Conv1d + SiLU, the selective SSM
// (Algorithm 2, with the x_proj / dt_proj projections of s_B, s_C, s_Delta and
// softplus for tau_Delta), the SiLU gate, the output Linear and the residual:
//
//   hn = RMSNorm(h)                          rmsnorm_kernel (here)
//   x = hn W_in[:D]^T, z = hn W_in[D:]^T     two GEMMs (hipBLASLt, bf16 -> bf16)
//   u = silu(causal conv1d(x))               launch_conv1d_silu
//   xdbl = u W_x^T = [dt_low | B | C]        one GEMM, (R + 2N) outputs per row
//   dt = softplus(dt_low W_dt^T + dt_bias)   dtproj_kernel (here, MFMA); it also
//                                            unpacks B and C into dense rows
//   y = S6(u, dt, A, B, C, D) * silu(z)      launch_scan_fwd
//   h_out = h + y W_out^T                    one GEMM, the residual as its beta C
//
// The big GEMMs are plain library contractions: y = x W^T with W row-major
// (out, in) is the column-major "TN" product D = W^T' x' (m = out, n = rows,
// k = in), fp32 accumulation, bf16 in and out.  dt_proj has a short inner
// dimension (the rank R) and a full-width output, so it is bound by writing
// dt; it runs in its own kernel with the bias and softplus in its epilogue,
// which takes the softplus out of the scan's ALU-bound loop.  Every
// intermediate is stored in bf16 in the caller's workspace.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <new>

struct ssm_block_plan {
    ssm_block_dims_t dims;
    hipblasLtHandle_t lt;
    struct Gemm {
        hipblasLtMatmulDesc_t op;
        hipblasLtMatrixLayout_t a, b, c;
        hipblasLtMatmulAlgo_t algo;
        size_t ws;
    } g[4];
    // byte offsets in the workspace
    size_t o_hn, o_x, o_z, o_u, o_xdbl, o_b, o_c, o_dl, o_y, o_scan, o_lt, total;
    size_t scan_ws, lt_ws;
};

namespace ssm {
namespace {

constexpr size_t kLtWorkspace = 32u << 20;  // hipBLASLt scratch offered to the heuristics

enum GemmId { kGx = 0, kGz, kGxdbl, kGout };

// RMSNorm over the last axis, one wave per row: h / sqrt(mean(h^2) + eps) * w.
// The row (d_model a multiple of 8, 16-byte aligned) is read in 16-byte
// groups of 8; up to NR groups per lane (NR chosen at launch from the row
// length, at most 8) stay in registers between the sum of squares and the
// scaling, and a longer row is read a second time.

__device__ __forceinline__ void bf16x8(const uint4 &q, float (&v)[8]) {
    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(wv[i] << 16);
        v[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 norm8(const uint4 &q, const float *w, float scale) {
    float v[8];
    bf16x8(q, v);
    const float4 w0 = *reinterpret_cast<const float4 *>(w), w1 = *reinterpret_cast<const float4 *>(w + 4);
    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i] * scale * ww[2 * i], v[2 * i + 1] * scale * ww[2 * i + 1]);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int kNormRegs>
__device__ __forceinline__ void rmsnorm_row(const uint16_t *h, const float *w, uint16_t *out, int64_t row,
                                            int64_t dm, float eps, int lane) {
    const uint4 *hr = reinterpret_cast<const uint4 *>(h + row * dm);
    uint4 *orow = reinterpret_cast<uint4 *>(out + row * dm);
    const int64_t groups = dm / 8;
    uint4 keep[kNormRegs];
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < kNormRegs; ++r) {
        const int64_t gi = lane + 64 * r;
        keep[r] = gi < groups ? hr[gi] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < kNormRegs; ++r) {
        float v[8];
        bf16x8(keep[r], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[i], v[i], acc);
    }
    for (int64_t gi = lane + 64 * kNormRegs; gi < groups; gi += 64) {
        float v[8];
        bf16x8(hr[gi], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(v[i], v[i], acc);
    }
#pragma unroll
    for (int s = 32; s >= 1; s /= 2) acc += __shfl_xor(acc, s, 64);
    const float scale = 1.0f / sqrtf(acc / (float)dm + eps);
#pragma unroll
    for (int r = 0; r < kNormRegs; ++r) {
        const int64_t gi = lane + 64 * r;
        if (gi < groups) orow[gi] = norm8(keep[r], w + 8 * gi, scale);
    }
    for (int64_t gi = lane + 64 * kNormRegs; gi < groups; gi += 64) orow[gi] = norm8(hr[gi], w + 8 * gi, scale);
}

template <int kNormRegs>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t *h, const float *w, uint16_t *out,
                                                      int64_t rows, int64_t dm, float eps) {
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; row < rows;
         row += (int64_t)gridDim.x * (blockDim.x / 64))
        rmsnorm_row<kNormRegs>(h, w, out, row, dm, eps, lane);
}

// dt = softplus(dt_low W_dt^T + dt_bias) over all rows, with dt_low the first
// R entries of each xdbl row (row stride ldx), W_dt (D, R) row-major; and the
// B, C entries of each row copied to dense (M, N) arrays.
//
// A wave owns 64 rows x 64 channels as 4 x 4 tiles of the 16x16x16 bf16 MFMA:
// the A operand is W_dt (tile row = channel), the B operand dt_low (tile
// column = row), so each lane ends with 4 consecutive channels of one row.
// The rank is walked in steps of 16 (entries past R read as 0): for R <= 64
// all operand loads are issued at once, a longer rank loads the next step's
// operands before this step's MFMAs.  WIDE loads 4 entries at once (R and ldx
// multiples of 4); otherwise entry by entry.  The finished tile goes through
// LDS so that each lane stores 16 contiguous bytes of one row (a wave writes
// 8 whole 128-byte row segments per store).
constexpr int kDtRows = 64;   // rows per workgroup
constexpr int kDtCh = 256;    // channels per workgroup (64 per wave)

typedef short dt_bf16x4 __attribute__((ext_vector_type(4)));
typedef float dt_f32x4 __attribute__((ext_vector_type(4)));

template <bool WIDE>
__device__ __forceinline__ dt_bf16x4 dt_operand(const uint16_t *rowp, bool row_ok, int k, int R) {
    if (WIDE) {
        if (!row_ok || k >= R) return dt_bf16x4{0, 0, 0, 0};
        return __builtin_bit_cast(dt_bf16x4, *reinterpret_cast<const uint2 *>(rowp + k));
    }
    dt_bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (row_ok && k + i < R) ? (short)rowp[k + i] : (short)0;
    return v;
}

template <bool WIDE>
__global__ __launch_bounds__(256) void dtproj_kernel(const uint16_t *__restrict__ xdbl, int64_t ldx,
                                                     const uint16_t *__restrict__ w_dt,
                                                     const float *__restrict__ bias, uint16_t *__restrict__ dt,
                                                     uint16_t *__restrict__ Bo, uint16_t *__restrict__ Co,
                                                     int64_t M, int64_t D, int R, int N) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * kDtRows;
    const int64_t d0 = (int64_t)blockIdx.y * kDtCh + wave * 64;
    const int r16 = lane & 15, kq = 4 * (lane >> 4);

    // B and C of this row block, shared out over all its channel blocks (a
    // few entries per thread, loads issued before the stores).
    {
        const int per = 2 * N, total = kDtRows * per;
        const int stride = (int)gridDim.y * blockDim.x;
        const int first = (int)blockIdx.y * blockDim.x + threadIdx.x;
        constexpr int kMaxPer = 4;
        for (int e0 = first; e0 < total; e0 += kMaxPer * stride) {
            uint16_t v[kMaxPer];
            int64_t dst[kMaxPer];
#pragma unroll
            for (int i = 0; i < kMaxPer; ++i) {
                const int e = e0 + i * stride;
                const int r = e / per, c = e % per;
                const int64_t m = m0 + r;
                dst[i] = -1;
                if (e < total && m < M) {
                    v[i] = xdbl[m * ldx + R + c];
                    dst[i] = c < N ? m * N + c : -(m * N + (c - N)) - 2;
                }
            }
#pragma unroll
            for (int i = 0; i < kMaxPer; ++i) {
                if (dst[i] >= 0) Bo[dst[i]] = v[i];
                else if (dst[i] <= -2) Co[-dst[i] - 2] = v[i];
            }
        }
    }

    const uint16_t *arow[4], *brow[4];
    bool aok[4], bok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t d = d0 + 16 * i + r16, m = m0 + 16 * i + r16;
        aok[i] = d < D;
        bok[i] = m < M;
        arow[i] = w_dt + (aok[i] ? d : 0) * R;
        brow[i] = xdbl + (bok[i] ? m : 0) * ldx;
    }
    dt_f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = dt_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (R <= 64) {
        // the whole rank in one round trip: every operand load issued first
        dt_bf16x4 a[4][4], b[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[s][i] = dt_operand<WIDE>(arow[i], aok[i], 16 * s + kq, R);
                b[s][i] = dt_operand<WIDE>(brow[i], bok[i], 16 * s + kq, R);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (16 * s >= R) break;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
        }
    } else {
        dt_bf16x4 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = dt_operand<WIDE>(arow[i], aok[i], kq, R);
            b[i] = dt_operand<WIDE>(brow[i], bok[i], kq, R);
        }
        for (int k0 = 0; k0 < R; k0 += 16) {
            dt_bf16x4 an[4], bn[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                an[i] = dt_operand<WIDE>(arow[i], aok[i], k0 + 16 + kq, R);
                bn[i] = dt_operand<WIDE>(brow[i], bok[i], k0 + 16 + kq, R);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = an[i];
                b[i] = bn[i];
            }
        }
    }
    // Each wave stages its 64 x 64 outputs through its own LDS area, 32 rows at
    // a time (18 KB per workgroup: six workgroups fit a CU, so the launch runs
    // in one round), and stores them as 16-byte pieces.
    __shared__ __attribute__((aligned(16))) uint16_t stage[4][32][72];
    float4 bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t d = d0 + 16 * i + kq;
        bb[i] = d < D ? *reinterpret_cast<const float4 *>(bias + d) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int c8 = (lane & 7) * 8;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const dt_f32x4 v = acc[i][2 * half + jj];
                const uint32_t lo = pack_bf16x2(softplus_fast(v[0] + bb[i].x), softplus_fast(v[1] + bb[i].y));
                const uint32_t hi = pack_bf16x2(softplus_fast(v[2] + bb[i].z), softplus_fast(v[3] + bb[i].w));
                *reinterpret_cast<uint2 *>(&stage[wave][16 * jj + r16][16 * i + kq]) = make_uint2(lo, hi);
            }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int row = 8 * s + (lane >> 3);
            const int64_t m = m0 + 32 * half + row, d = d0 + c8;
            if (m < M && d < D)
                *reinterpret_cast<uint4 *>(dt + m * D + d) = *reinterpret_cast<const uint4 *>(&stage[wave][row][c8]);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // reads done before the next half's writes
    }
}

size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }

bool gemm_setup(hipblasLtHandle_t lt, ssm_block_plan::Gemm &g, int64_t out, int64_t in, int64_t rows,
                hipblasLtMatmulPreference_t pref) {
    if (hipblasLtMatmulDescCreate(&g.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
    hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
    if (hipblasLtMatrixLayoutCreate(&g.a, HIP_R_16BF, in, out, in) != HIPBLAS_STATUS_SUCCESS) return false;
    if (hipblasLtMatrixLayoutCreate(&g.b, HIP_R_16BF, in, rows, in) != HIPBLAS_STATUS_SUCCESS) return false;
    if (hipblasLtMatrixLayoutCreate(&g.c, HIP_R_16BF, out, rows, out) != HIPBLAS_STATUS_SUCCESS) return false;
    hipblasLtMatmulHeuristicResult_t res;
    int count = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(lt, g.op, g.a, g.b, g.c, g.c, pref, 1, &res, &count) !=
            HIPBLAS_STATUS_SUCCESS || count < 1)
        return false;
    g.algo = res.algo;
    g.ws = res.workspaceSize;
    return true;
}

hipError_t gemm_run(const ssm_block_plan &p, const ssm_block_plan::Gemm &g, const void *w, const void *in,
                    void *out, const void *cin, char *lt_ws, hipStream_t stream) {
    const float alpha = 1.0f, beta = cin ? 1.0f : 0.0f;
    const hipblasStatus_t s = hipblasLtMatmul(p.lt, g.op, &alpha, w, g.a, in, g.b, &beta, cin ? cin : out, g.c,
                                              out, g.c, &g.algo, lt_ws, p.lt_ws, stream);
    return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorUnknown;
}

void plan_free(ssm_block_plan *p) {
    for (auto &g : p->g) {
        if (g.op) hipblasLtMatmulDescDestroy(g.op);
        if (g.a) hipblasLtMatrixLayoutDestroy(g.a);
        if (g.b) hipblasLtMatrixLayoutDestroy(g.b);
        if (g.c) hipblasLtMatrixLayoutDestroy(g.c);
    }
    if (p->lt) hipblasLtDestroy(p->lt);
    delete p;
}

}  // namespace

ssm_status_t block_plan_create(const ssm_block_dims_t &d, ssm_block_plan **out) {
    ssm_block_plan *p = new (std::nothrow) ssm_block_plan();
    if (!p) return SSM_ERR_HIP;
    p->dims = d;
    const int64_t M = d.batch * d.seqlen, D = d.d_inner, N = d.dstate, R = d.dt_rank, dm = d.d_model;
    // workspace layout (bf16 tensors, each 256-aligned)
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += r256(bytes); return at; };
    p->o_hn = take((size_t)(M * dm) * 2);
    p->o_x = take((size_t)(M * D) * 2);
    p->o_z = take((size_t)(M * D) * 2);
    p->o_u = take((size_t)(M * D) * 2);
    p->o_xdbl = take((size_t)(M * (R + 2 * N)) * 2);
    p->o_b = take((size_t)(M * N) * 2);
    p->o_c = take((size_t)(M * N) * 2);
    p->o_dl = take((size_t)(M * D) * 2);
    p->o_y = take((size_t)(M * D) * 2);
    // The scan's own workspace, sized with pointers aligned like the real ones.
    ssm_scan_args_t sa = {};
    sa.batch = d.batch;
    sa.seqlen = d.seqlen;
    sa.dim = D;
    sa.dstate = N;
    sa.io_dtype = SSM_BF16;
    sa.delta_softplus = 0;
    sa.x = sa.delta = sa.Bm = sa.Cm = sa.z = reinterpret_cast<const void *>((uintptr_t)256);
    sa.y = reinterpret_cast<void *>((uintptr_t)256);
    p->scan_ws = scan_workspace_bytes(sa);
    p->o_scan = take(p->scan_ws);
    p->lt_ws = kLtWorkspace;
    p->o_lt = take(p->lt_ws);
    p->total = o;

    // hipBLASLt ends the process when no device is present: check first.
    int ndev = 0, dev = -1;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1 || hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        plan_free(p);
        return SSM_ERR_HIP;
    }
    if (hipblasLtCreate(&p->lt) != HIPBLAS_STATUS_SUCCESS) {
        p->lt = nullptr;
        plan_free(p);
        return SSM_ERR_HIP;
    }
    hipblasLtMatmulPreference_t pref;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) {
        plan_free(p);
        return SSM_ERR_HIP;
    }
    const uint64_t wsmax = kLtWorkspace;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax, sizeof(wsmax));
    const int64_t shapes[4][2] = {{D, dm}, {D, dm}, {R + 2 * N, D}, {dm, D}};  // (out, in)
    bool ok = true;
    for (int i = 0; i < 4 && ok; ++i) ok = gemm_setup(p->lt, p->g[i], shapes[i][0], shapes[i][1], M, pref);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) {
        plan_free(p);
        return SSM_ERR_UNSUPPORTED;
    }
    *out = p;
    return SSM_OK;
}

void block_plan_destroy(ssm_block_plan *p) {
    if (p) plan_free(p);
}

size_t block_workspace_bytes(const ssm_block_plan &p) { return p.total; }

const ssm_block_dims_t &block_dims(const ssm_block_plan &p) { return p.dims; }

hipError_t launch_block_fwd(const ssm_block_plan &p, const ssm_block_weights_t &w, const void *h_in, void *h_out,
                            void *workspace, hipStream_t stream) {
    const ssm_block_dims_t &d = p.dims;
    const int64_t M = d.batch * d.seqlen, D = d.d_inner, N = d.dstate, R = d.dt_rank, dm = d.d_model;
    char *ws = static_cast<char *>(workspace);
    char *lt_ws = ws + p.o_lt;
    uint16_t *hn = reinterpret_cast<uint16_t *>(ws + p.o_hn);
    {
        // grid-stride rows: at most 65536 workgroups of 4 rows
        const unsigned blocks = (unsigned)std::min<int64_t>((M + 3) / 4, 65536);
        const auto *hi = static_cast<const uint16_t *>(h_in);
        const int64_t per_lane = (dm / 8 + 63) / 64;
        if (per_lane <= 1)
            rmsnorm_kernel<1><<<blocks, 256, 0, stream>>>(hi, w.norm_w, hn, M, dm, w.norm_eps);
        else if (per_lane <= 2)
            rmsnorm_kernel<2><<<blocks, 256, 0, stream>>>(hi, w.norm_w, hn, M, dm, w.norm_eps);
        else if (per_lane <= 4)
            rmsnorm_kernel<4><<<blocks, 256, 0, stream>>>(hi, w.norm_w, hn, M, dm, w.norm_eps);
        else
            rmsnorm_kernel<8><<<blocks, 256, 0, stream>>>(hi, w.norm_w, hn, M, dm, w.norm_eps);
    }
    hipError_t e = hipGetLastError();
    const char *w_in = static_cast<const char *>(w.w_in);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGx], w_in, hn, ws + p.o_x, nullptr, lt_ws, stream);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGz], w_in + (size_t)(D * dm) * 2, hn, ws + p.o_z, nullptr, lt_ws, stream);
    if (e == hipSuccess)
        e = launch_conv1d_silu(d.batch, d.seqlen, D, (int)d.conv_k, SSM_BF16, ws + p.o_x, w.conv_w, w.conv_b,
                               ws + p.o_u, stream);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGxdbl], w.w_x, ws + p.o_u, ws + p.o_xdbl, nullptr, lt_ws, stream);
    if (e == hipSuccess) {
        const int64_t ldx = R + 2 * N;
        const dim3 grid((unsigned)((M + kDtRows - 1) / kDtRows), (unsigned)((D + kDtCh - 1) / kDtCh));
        const auto *xd = reinterpret_cast<const uint16_t *>(ws + p.o_xdbl);
        const auto *wdt = static_cast<const uint16_t *>(w.w_dt);
        auto *dto = reinterpret_cast<uint16_t *>(ws + p.o_dl);
        auto *bo = reinterpret_cast<uint16_t *>(ws + p.o_b);
        auto *co = reinterpret_cast<uint16_t *>(ws + p.o_c);
        if (R % 4 == 0 && ldx % 4 == 0)
            dtproj_kernel<true><<<grid, 256, 0, stream>>>(xd, ldx, wdt, w.dt_bias, dto, bo, co, M, D, (int)R, (int)N);
        else
            dtproj_kernel<false><<<grid, 256, 0, stream>>>(xd, ldx, wdt, w.dt_bias, dto, bo, co, M, D, (int)R, (int)N);
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        ssm_scan_args_t sa = {};
        sa.batch = d.batch;
        sa.seqlen = d.seqlen;
        sa.dim = D;
        sa.dstate = N;
        sa.io_dtype = SSM_BF16;
        sa.delta_softplus = 0;  // dt arrives with its bias and softplus applied
        sa.x = ws + p.o_u;
        sa.delta = ws + p.o_dl;
        sa.Bm = ws + p.o_b;
        sa.Cm = ws + p.o_c;
        sa.z = ws + p.o_z;
        sa.A = w.A;
        sa.Dskip = w.Dskip;
        sa.y = ws + p.o_y;
        sa.workspace = p.scan_ws ? ws + p.o_scan : nullptr;
        sa.workspace_bytes = p.scan_ws;
        e = launch_scan_fwd(sa, stream);
    }
    if (e == hipSuccess) e = gemm_run(p, p.g[kGout], w.w_out, ws + p.o_y, h_out, h_in, lt_ws, stream);
    return e;
}

}  // namespace ssm
