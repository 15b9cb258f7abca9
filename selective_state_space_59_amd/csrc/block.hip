// block.hip -- one Mamba (S6) block with its pre-norm residual, on gfx950.
//
// The block of "Mamba: Linear-Time Sequence Modeling with Selective State
// Spaces" (paper summary page, sec. 4a, the table of tensor shapes): RMSNorm,
// the expanding Linear (x and gate halves), Conv1d + SiLU, the selective SSM
// (Algorithm 2, with the x_proj / dt_proj projections of s_B, s_C, s_Delta and
// softplus for tau_Delta), the SiLU gate, the output Linear and the residual:
//
//   hn = RMSNorm(h)                        rmsnorm_kernel (here)
//   x = hn W_in[:D]^T, z = hn W_in[D:]^T   two GEMMs (hipBLASLt, bf16 -> bf16)
//   u = silu(causal conv1d(x))             launch_conv1d_silu
//   dt_low, B, C = u W_x^T (R, N, N rows)  three GEMMs
//   delta = dt_low W_dt^T                  one GEMM
//   y = S6(u, softplus(delta + dt_bias), A, B, C, D) * silu(z)   launch_scan_fwd
//   h_out = h + y W_out^T                  one GEMM, the residual as its beta C
//
// The GEMMs are plain library contractions: y = x W^T with W row-major (out,
// in) is the column-major "TN" product D = W^T' x' (m = out, n = rows, k = in),
// fp32 accumulation, bf16 in and out.  Every intermediate is stored in bf16 in
// the caller's workspace.
#include "ssm_device.h"
#include "ssm_internal.h"

#include <hipblaslt/hipblaslt.h>

#include <new>

struct ssm_block_plan {
    ssm_block_dims_t dims;
    hipblasLtHandle_t lt;
    struct Gemm {
        hipblasLtMatmulDesc_t op;
        hipblasLtMatrixLayout_t a, b, c;
        hipblasLtMatmulAlgo_t algo;
        size_t ws;
    } g[7];
    // byte offsets in the workspace
    size_t o_hn, o_x, o_z, o_u, o_dtl, o_b, o_c, o_dl, o_y, o_scan, o_lt, total;
    size_t scan_ws, lt_ws;
};

namespace ssm {
namespace {

constexpr size_t kLtWorkspace = 32u << 20;  // hipBLASLt scratch offered to the heuristics

enum GemmId { kGx = 0, kGz, kGdtl, kGb, kGc, kGdt, kGout };

// RMSNorm over the last axis (one wave per row): h / sqrt(mean(h^2) + eps) * w.
__global__ void rmsnorm_kernel(const uint16_t *h, const float *w, uint16_t *out, int64_t rows, int64_t dm,
                               float eps) {
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const uint16_t *hr = h + row * dm;
    float acc = 0.0f;
    for (int64_t i = lane; i < dm; i += 64) {
        const float v = bf16_bits_to_f32(hr[i]);
        acc = __builtin_fmaf(v, v, acc);
    }
#pragma unroll
    for (int s = 32; s >= 1; s /= 2) acc += __shfl_xor(acc, s, 64);
    const float scale = 1.0f / sqrtf(acc / (float)dm + eps);
    for (int64_t i = lane; i < dm; i += 64)
        out[row * dm + i] = f32_to_bf16_bits(bf16_bits_to_f32(hr[i]) * scale * w[i]);
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
    p->o_dtl = take((size_t)(M * R) * 2);
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
    sa.delta_softplus = 1;
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
    const int64_t shapes[7][2] = {{D, dm}, {D, dm}, {R, D}, {N, D}, {N, D}, {D, R}, {dm, D}};  // (out, in)
    bool ok = true;
    for (int i = 0; i < 7 && ok; ++i) ok = gemm_setup(p->lt, p->g[i], shapes[i][0], shapes[i][1], M, pref);
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
    rmsnorm_kernel<<<(unsigned)((M + 3) / 4), 256, 0, stream>>>(static_cast<const uint16_t *>(h_in), w.norm_w, hn,
                                                               M, dm, w.norm_eps);
    hipError_t e = hipGetLastError();
    const char *w_in = static_cast<const char *>(w.w_in);
    const char *w_x = static_cast<const char *>(w.w_x);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGx], w_in, hn, ws + p.o_x, nullptr, lt_ws, stream);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGz], w_in + (size_t)(D * dm) * 2, hn, ws + p.o_z, nullptr, lt_ws, stream);
    if (e == hipSuccess)
        e = launch_conv1d_silu(d.batch, d.seqlen, D, (int)d.conv_k, SSM_BF16, ws + p.o_x, w.conv_w, w.conv_b,
                               ws + p.o_u, stream);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGdtl], w_x, ws + p.o_u, ws + p.o_dtl, nullptr, lt_ws, stream);
    if (e == hipSuccess)
        e = gemm_run(p, p.g[kGb], w_x + (size_t)(R * D) * 2, ws + p.o_u, ws + p.o_b, nullptr, lt_ws, stream);
    if (e == hipSuccess)
        e = gemm_run(p, p.g[kGc], w_x + (size_t)((R + N) * D) * 2, ws + p.o_u, ws + p.o_c, nullptr, lt_ws, stream);
    if (e == hipSuccess) e = gemm_run(p, p.g[kGdt], w.w_dt, ws + p.o_dtl, ws + p.o_dl, nullptr, lt_ws, stream);
    if (e == hipSuccess) {
        ssm_scan_args_t sa = {};
        sa.batch = d.batch;
        sa.seqlen = d.seqlen;
        sa.dim = D;
        sa.dstate = N;
        sa.io_dtype = SSM_BF16;
        sa.delta_softplus = 1;
        sa.x = ws + p.o_u;
        sa.delta = ws + p.o_dl;
        sa.Bm = ws + p.o_b;
        sa.Cm = ws + p.o_c;
        sa.z = ws + p.o_z;
        sa.A = w.A;
        sa.Dskip = w.Dskip;
        sa.delta_bias = w.dt_bias;
        sa.y = ws + p.o_y;
        sa.workspace = p.scan_ws ? ws + p.o_scan : nullptr;
        sa.workspace_bytes = p.scan_ws;
        e = launch_scan_fwd(sa, stream);
    }
    if (e == hipSuccess) e = gemm_run(p, p.g[kGout], w.w_out, ws + p.o_y, h_out, h_in, lt_ws, stream);
    return e;
}

}  // namespace ssm
