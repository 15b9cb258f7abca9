// ssm_api.cpp -- the C ABI declared in include/ssm.h: argument checking,
// dispatch to the kernel launchers, status strings.  Nothing here allocates
// device memory or keeps state between calls (apart from the per-thread text
// of the last error and the block plans the caller creates and destroys).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <climits>

#include "ssm_internal.h"

namespace {

thread_local char g_last_error[512] = "";

ssm_status_t fail(ssm_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

ssm_status_t ok() {
    g_last_error[0] = '\0';
    return SSM_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    const char *name;
};

Range range(const void *p, int64_t count, int64_t elem, const char *name) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p ? lo + (uintptr_t)(count * elem) : lo, name};
}

bool overlaps(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;  // empty or absent
    return a.lo < b.hi && b.lo < a.hi;
}

int64_t io_bytes(int32_t dt) { return dt == SSM_BF16 ? 2 : 4; }

bool aligned(const void *p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

// Products of non-negative sizes that must stay far from int64 overflow.
bool mul_ok(int64_t a, int64_t b, int64_t c = 1) {
    const int64_t lim = (int64_t)1 << 60;
    if (a == 0 || b == 0 || c == 0) return true;
    if (a > lim / b) return false;
    const int64_t ab = a * b;
    return ab <= lim / c;
}

// Elements of a checkpoint buffer, (ceil(L / SSM_SCAN_BLOCK), B, D, SSM_MAX_DSTATE),
// or -1 where that product is too large.
int64_t checkpoint_elems(int64_t B, int64_t L, int64_t D) {
    const int64_t nblk = (L + SSM_SCAN_BLOCK - 1) / SSM_SCAN_BLOCK;
    if (!mul_ok(B, D) || !mul_ok(nblk, B * D, SSM_MAX_DSTATE)) return -1;
    return nblk * B * D * SSM_MAX_DSTATE;
}

ssm_status_t check_scan_sizes(const ssm_scan_args_t *a) {
    if (!a) return fail(SSM_ERR_NULL_ARG, "args is NULL");
    if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", a->io_dtype);
    if (a->batch < 0 || a->seqlen < 0)
        return fail(SSM_ERR_BAD_SHAPE, "negative batch (%lld) or seqlen (%lld)",
                    (long long)a->batch, (long long)a->seqlen);
    if (a->dim < 1) return fail(SSM_ERR_BAD_SHAPE, "dim must be >= 1 (got %lld)", (long long)a->dim);
    if (a->dstate < 1) return fail(SSM_ERR_BAD_SHAPE, "dstate must be >= 1 (got %lld)", (long long)a->dstate);
    if (a->dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_UNSUPPORTED, "dstate %lld exceeds SSM_MAX_DSTATE (%d)",
                    (long long)a->dstate, SSM_MAX_DSTATE);
    if (a->conv_k < 0) return fail(SSM_ERR_BAD_SHAPE, "conv_k must be >= 0");
    if (a->conv_k > SSM_MAX_CONV_K)
        return fail(SSM_ERR_UNSUPPORTED, "conv_k %lld exceeds SSM_MAX_CONV_K (%d)",
                    (long long)a->conv_k, SSM_MAX_CONV_K);
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
    if (!mul_ok(a->batch, a->seqlen, a->dim) || !mul_ok(a->batch, a->seqlen, a->dstate) ||
        !mul_ok(a->batch, a->dim, a->dstate))
        return fail(SSM_ERR_BAD_SHAPE, "sizes overflow");
    if (a->checkpoints && checkpoint_elems(a->batch, a->seqlen, a->dim) < 0)
        return fail(SSM_ERR_BAD_SHAPE, "checkpoint sizes overflow");
    return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_last_error_message(void) { return g_last_error; }

const char *ssm_status_string(ssm_status_t s) {
    switch (s) {
        case SSM_OK: return "SSM_OK: success";
        case SSM_ERR_NULL_ARG: return "SSM_ERR_NULL_ARG: a required pointer is NULL";
        case SSM_ERR_BAD_SHAPE: return "SSM_ERR_BAD_SHAPE: a size is negative or inconsistent";
        case SSM_ERR_BAD_DTYPE: return "SSM_ERR_BAD_DTYPE: unknown io_dtype";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: size or option beyond what the kernels support";
        case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output overlaps another argument";
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing, too small or misaligned";
        case SSM_ERR_HIP: return "SSM_ERR_HIP: the HIP runtime reported an error";
        case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: a pointer is not aligned to its element size";
    }
    return "unknown ssm_status_t";
}

size_t ssm_selective_scan_workspace_size(const ssm_scan_args_t *a) {
    if (check_scan_sizes(a) != SSM_OK) return (size_t)-1;
    if (a->batch == 0 || a->seqlen == 0) return 0;
    return ssm::scan_workspace_bytes(*a);
}

}  // extern "C"

namespace {

// The checks and launch of both scan entry points.  With `noalloc` the
// workspace comes from the library's scratch array and the caller passes none.
ssm_status_t scan_fwd(const ssm_scan_args_t *a, void *stream, bool noalloc) {
    ssm_status_t s = check_scan_sizes(a);
    if (s != SSM_OK) return s;
    const int64_t B = a->batch, L = a->seqlen, D = a->dim, N = a->dstate, K = a->conv_k;
    const int64_t es = io_bytes(a->io_dtype);
    const bool work = B > 0 && L > 0;
    if (work) {
        if (!a->x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
        if (!a->delta) return fail(SSM_ERR_NULL_ARG, "delta is NULL");
        if (!a->Bm) return fail(SSM_ERR_NULL_ARG, "Bm is NULL");
        if (!a->Cm) return fail(SSM_ERR_NULL_ARG, "Cm is NULL");
        if (!a->A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
        if (!a->y) return fail(SSM_ERR_NULL_ARG, "y is NULL");
        if (K > 0 && !a->conv_w) return fail(SSM_ERR_NULL_ARG, "conv_w is NULL but conv_k > 0");
    }
    if (K == 0 && (a->conv_w || a->conv_b || a->conv_state_in || a->conv_state_out))
        return fail(SSM_ERR_BAD_SHAPE, "conv_w/conv_b/conv state given but conv_k == 0");
    const void *io_ptrs[] = {a->x, a->delta, a->Bm, a->Cm, a->z, a->y, a->conv_state_in,
                             a->conv_state_out};
    for (const void *p : io_ptrs)
        if (!aligned(p, es)) return fail(SSM_ERR_ALIGN, "an io_dtype pointer is not %lld-byte aligned", (long long)es);
    const void *f_ptrs[] = {a->A, a->Dskip, a->delta_bias, a->conv_w, a->conv_b, a->h0, a->h_final,
                            a->checkpoints};
    for (const void *p : f_ptrs)
        if (!aligned(p, 4)) return fail(SSM_ERR_ALIGN, "an fp32 pointer is not 4-byte aligned");

    const int64_t csn = B * (K > 0 ? K - 1 : 0) * D;  // elements of a conv state
    const Range csi = range(a->conv_state_in, csn, es, "conv_state_in");
    const Range inputs[] = {
        range(a->x, B * L * D, es, "x"),          range(a->delta, B * L * D, es, "delta"),
        range(a->Bm, B * L * N, es, "Bm"),        range(a->Cm, B * L * N, es, "Cm"),
        range(a->z, B * L * D, es, "z"),          range(a->A, D * N, 4, "A"),
        range(a->Dskip, D, 4, "Dskip"),           range(a->delta_bias, D, 4, "delta_bias"),
        range(a->conv_w, D * K, 4, "conv_w"),     range(a->conv_b, D, 4, "conv_b"),
        range(a->h0, B * D * N, 4, "h0"),
        csi,
    };
    const Range y = range(a->y, B * L * D, es, "y");
    const Range hf = range(a->h_final, B * D * N, 4, "h_final");
    const Range cso = range(a->conv_state_out, csn, es, "conv_state_out");
    // The conv state may be updated in place (the same tensor in and out).
    const bool cs_in_place = a->conv_state_out != nullptr && a->conv_state_out == a->conv_state_in;
    for (const Range &r : inputs) {
        if (overlaps(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
        if (overlaps(hf, r)) return fail(SSM_ERR_ALIAS, "h_final overlaps %s", r.name);
        if (!(cs_in_place && &r == &inputs[sizeof(inputs) / sizeof(inputs[0]) - 1]) && overlaps(cso, r))
            return fail(SSM_ERR_ALIAS, "conv_state_out overlaps %s", r.name);
    }
    if (overlaps(y, hf)) return fail(SSM_ERR_ALIAS, "y overlaps h_final");
    if (overlaps(cso, y) || overlaps(cso, hf)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps an output");
    const int64_t nck = a->checkpoints ? checkpoint_elems(B, L, D) : 0;  // >= 0 (checked above)
    const Range ck = range(a->checkpoints, nck, 4, "checkpoints");
    for (const Range &r : inputs)
        if (overlaps(ck, r)) return fail(SSM_ERR_ALIAS, "checkpoints overlap %s", r.name);
    if (overlaps(ck, y) || overlaps(ck, hf) || overlaps(ck, cso))
        return fail(SSM_ERR_ALIAS, "checkpoints overlap an output");

    const size_t need = work ? ssm::scan_workspace_bytes(*a) : 0;
    if (noalloc) {
        if (a->workspace || a->workspace_bytes)
            return fail(SSM_ERR_WORKSPACE, "the no-allocation scan takes no workspace (use its scratch array)");
        if (need > (size_t)SSM_NOALLOC_SCRATCH_BYTES)
            return fail(SSM_ERR_WORKSPACE, "these sizes need %zu bytes of workspace; the no-allocation "
                        "scan has %zu (use ssm_selective_scan_fwd with a workspace)",
                        need, (size_t)SSM_NOALLOC_SCRATCH_BYTES);
    } else if (need > 0) {
        if (!a->workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", need);
        if (a->workspace_bytes < need)
            return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", a->workspace_bytes, need);
        if (!aligned(a->workspace, 256)) return fail(SSM_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        const Range ws = range(a->workspace, (int64_t)need, 1, "workspace");
        for (const Range &r : inputs)
            if (overlaps(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
        if (overlaps(ws, y) || overlaps(ws, hf) || overlaps(ws, cso) || overlaps(ws, ck))
            return fail(SSM_ERR_ALIAS, "workspace overlaps an output");
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (B == 0) return ok();
    if (L == 0) {
        e = ssm::launch_empty_scan_state(*a, st);
    } else if (noalloc && need > 0) {
        ssm_scan_args_t b = *a;
        e = ssm::noalloc_scratch(st, &b.workspace);
        if (e != hipSuccess)
            return fail(SSM_ERR_HIP, "scratch array address: %s", hipGetErrorString(e));
        b.workspace_bytes = SSM_NOALLOC_SCRATCH_BYTES;
        e = ssm::launch_scan_fwd(b, st);
    } else {
        e = ssm::launch_scan_fwd(*a, st);
    }
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

ssm_status_t ssm_selective_scan_fwd(const ssm_scan_args_t *a, void *stream) {
    return scan_fwd(a, stream, false);
}

ssm_status_t ssm_selective_scan_fwd_noalloc(const ssm_scan_args_t *a, void *stream) {
    return scan_fwd(a, stream, true);
}

ssm_status_t ssm_causal_conv1d_silu(int64_t B, int64_t L, int64_t D, int64_t K, int32_t io_dtype,
                                    const void *x, const float *w, const float *bias, void *u,
                                    void *stream) {
    if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", io_dtype);
    if (B < 0 || L < 0) return fail(SSM_ERR_BAD_SHAPE, "negative batch or seqlen");
    if (D < 1) return fail(SSM_ERR_BAD_SHAPE, "dim must be >= 1");
    if (K < 1) return fail(SSM_ERR_BAD_SHAPE, "k must be >= 1");
    if (K > SSM_MAX_CONV_K) return fail(SSM_ERR_UNSUPPORTED, "k %lld exceeds SSM_MAX_CONV_K (%d)", (long long)K, SSM_MAX_CONV_K);
    if (!mul_ok(B, L, D)) return fail(SSM_ERR_BAD_SHAPE, "sizes overflow");
    const int64_t es = io_bytes(io_dtype);
    if (B == 0 || L == 0) return ok();
    if (!x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
    if (!w) return fail(SSM_ERR_NULL_ARG, "w is NULL");
    if (!u) return fail(SSM_ERR_NULL_ARG, "u is NULL");
    if (!aligned(x, es) || !aligned(u, es) || !aligned(w, 4) || !aligned(bias, 4))
        return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
    const Range ur = range(u, B * L * D, es, "u");
    if (overlaps(ur, range(x, B * L * D, es, "x")) || overlaps(ur, range(w, D * K, 4, "w")) ||
        overlaps(ur, range(bias, D, 4, "bias")))
        return fail(SSM_ERR_ALIAS, "u overlaps an input");
    hipError_t e = ssm::launch_conv1d_silu(B, L, D, (int)K, io_dtype, x, w, bias, u,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

ssm_status_t ssm_state_update(const ssm_state_update_args_t *a, void *stream) {
    if (!a) return fail(SSM_ERR_NULL_ARG, "args is NULL");
    if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", a->io_dtype);
    if (a->batch < 0) return fail(SSM_ERR_BAD_SHAPE, "negative batch");
    if (a->dim < 1) return fail(SSM_ERR_BAD_SHAPE, "dim must be >= 1");
    if (a->dstate < 1) return fail(SSM_ERR_BAD_SHAPE, "dstate must be >= 1");
    if (a->dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_UNSUPPORTED, "dstate %lld exceeds SSM_MAX_DSTATE (%d)", (long long)a->dstate, SSM_MAX_DSTATE);
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
    if (!mul_ok(a->batch, a->dim, a->dstate)) return fail(SSM_ERR_BAD_SHAPE, "sizes overflow");
    if (a->conv_k < 0) return fail(SSM_ERR_BAD_SHAPE, "conv_k must be >= 0");
    if (a->conv_k > SSM_MAX_CONV_K)
        return fail(SSM_ERR_UNSUPPORTED, "conv_k %lld exceeds SSM_MAX_CONV_K (%d)", (long long)a->conv_k, SSM_MAX_CONV_K);
    if (a->conv_k == 0 && (a->conv_w || a->conv_b || a->conv_state))
        return fail(SSM_ERR_BAD_SHAPE, "conv_w/conv_b/conv_state given but conv_k == 0");
    if (a->conv_k > 0 && a->dim > ((int64_t)1 << 28))
        return fail(SSM_ERR_UNSUPPORTED, "dim %lld with a conv window exceeds 2^28", (long long)a->dim);
    const int64_t B = a->batch, D = a->dim, N = a->dstate, K = a->conv_k;
    const int64_t es = io_bytes(a->io_dtype);
    if (B == 0) return ok();
    if (!a->state) return fail(SSM_ERR_NULL_ARG, "state is NULL");
    if (!a->x) return fail(SSM_ERR_NULL_ARG, "x is NULL");
    if (!a->delta) return fail(SSM_ERR_NULL_ARG, "delta is NULL");
    if (!a->Bm) return fail(SSM_ERR_NULL_ARG, "Bm is NULL");
    if (!a->Cm) return fail(SSM_ERR_NULL_ARG, "Cm is NULL");
    if (!a->A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
    if (!a->y) return fail(SSM_ERR_NULL_ARG, "y is NULL");
    if (K > 0 && !a->conv_w) return fail(SSM_ERR_NULL_ARG, "conv_w is NULL but conv_k > 0");
    if (K > 1 && !a->conv_state) return fail(SSM_ERR_NULL_ARG, "conv_state is NULL but conv_k > 1");
    const void *io_ptrs[] = {a->x, a->delta, a->z, a->Bm, a->Cm, a->y, a->conv_state};
    for (const void *p : io_ptrs)
        if (!aligned(p, es)) return fail(SSM_ERR_ALIGN, "an io_dtype pointer is not %lld-byte aligned", (long long)es);
    const void *f_ptrs[] = {a->state, a->A, a->Dskip, a->delta_bias, a->conv_w, a->conv_b};
    for (const void *p : f_ptrs)
        if (!aligned(p, 4)) return fail(SSM_ERR_ALIGN, "an fp32 pointer is not 4-byte aligned");
    const Range st = range(a->state, B * D * N, 4, "state");
    const Range y = range(a->y, B * D, es, "y");
    const Range inputs[] = {
        range(a->x, B * D, es, "x"),   range(a->delta, B * D, es, "delta"),
        range(a->z, B * D, es, "z"),   range(a->Bm, B * N, es, "Bm"),
        range(a->Cm, B * N, es, "Cm"), range(a->A, D * N, 4, "A"),
        range(a->Dskip, D, 4, "Dskip"), range(a->delta_bias, D, 4, "delta_bias"),
        range(a->conv_w, D * K, 4, "conv_w"), range(a->conv_b, D, 4, "conv_b"),
    };
    const Range cs = range(K > 1 ? a->conv_state : nullptr, B * (K > 0 ? K - 1 : 0) * D, es, "conv_state");
    for (const Range &r : inputs) {
        if (overlaps(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
        if (overlaps(st, r)) return fail(SSM_ERR_ALIAS, "state overlaps %s", r.name);
        if (overlaps(cs, r)) return fail(SSM_ERR_ALIAS, "conv_state overlaps %s", r.name);
    }
    if (overlaps(y, st)) return fail(SSM_ERR_ALIAS, "y overlaps state");
    if (overlaps(cs, y) || overlaps(cs, st)) return fail(SSM_ERR_ALIAS, "conv_state overlaps an output");
    hipError_t e = ssm::launch_state_update(*a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

static ssm_status_t check_bwd(const ssm_scan_bwd_args_t *a, size_t *need_out) {
    if (!a) return fail(SSM_ERR_NULL_ARG, "args is NULL");
    if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", a->io_dtype);
    if (a->batch < 0 || a->seqlen < 0)
        return fail(SSM_ERR_BAD_SHAPE, "negative batch (%lld) or seqlen (%lld)", (long long)a->batch,
                    (long long)a->seqlen);
    if (a->dim < 1) return fail(SSM_ERR_BAD_SHAPE, "dim must be >= 1");
    if (a->dstate < 1) return fail(SSM_ERR_BAD_SHAPE, "dstate must be >= 1");
    if (a->dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_UNSUPPORTED, "dstate %lld exceeds SSM_MAX_DSTATE (%d)", (long long)a->dstate,
                    SSM_MAX_DSTATE);
    if (a->conv_k < 0) return fail(SSM_ERR_BAD_SHAPE, "conv_k must be >= 0");
    if (a->conv_k > SSM_MAX_CONV_K)
        return fail(SSM_ERR_UNSUPPORTED, "conv_k %lld exceeds SSM_MAX_CONV_K (%d)", (long long)a->conv_k, SSM_MAX_CONV_K);
    if (a->conv_k == 0 && (a->conv_w || a->conv_b || a->dconv_w || a->dconv_b))
        return fail(SSM_ERR_BAD_SHAPE, "conv weights or their gradients given but conv_k == 0");
    if (a->conv_k < 2 && (a->conv_state_in || a->dconv_state_in))
        return fail(SSM_ERR_BAD_SHAPE, "a conv state or its gradient given but conv_k < 2");
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
    // (the backward's checkpoints, in its workspace or the caller's, must be addressable too)
    if (!mul_ok(a->batch, a->seqlen, a->dim) || !mul_ok(a->batch, a->seqlen, a->dstate) ||
        !mul_ok(a->batch, a->dim, a->dstate) || checkpoint_elems(a->batch, a->seqlen, a->dim) < 0)
        return fail(SSM_ERR_BAD_SHAPE, "sizes overflow");
    const int64_t B = a->batch, L = a->seqlen, D = a->dim, N = a->dstate, K = a->conv_k;
    const int64_t es = io_bytes(a->io_dtype);
    *need_out = (B > 0) ? ssm::scan_bwd_workspace_bytes(*a) : 0;
    if (B == 0) return SSM_OK;
    if (!a->A) return fail(SSM_ERR_NULL_ARG, "A is NULL");
    if (!a->dA) return fail(SSM_ERR_NULL_ARG, "dA is NULL");
    if (K > 0 && !a->conv_w) return fail(SSM_ERR_NULL_ARG, "conv_w is NULL but conv_k > 0");
    if (K > 0 && !a->dconv_w) return fail(SSM_ERR_NULL_ARG, "dconv_w is NULL but conv_k > 0");
    if (L > 0) {
        const struct { const void *p; const char *name; } req[] = {
            {a->x, "x"}, {a->delta, "delta"}, {a->Bm, "Bm"}, {a->Cm, "Cm"}, {a->dy, "dy"},
            {a->dx, "dx"}, {a->ddelta, "ddelta"}, {a->dBm, "dBm"}, {a->dCm, "dCm"}};
        for (const auto &r : req)
            if (!r.p) return fail(SSM_ERR_NULL_ARG, "%s is NULL", r.name);
        if (a->z && !a->dz) return fail(SSM_ERR_NULL_ARG, "dz is NULL but z is given");
    }
    if (!a->z && a->dz) return fail(SSM_ERR_BAD_SHAPE, "dz given without z");
    const void *io_ptrs[] = {a->x, a->delta, a->Bm, a->Cm, a->z, a->dy, a->dx, a->ddelta, a->dz,
                             a->conv_state_in, a->dconv_state_in};
    for (const void *p : io_ptrs)
        if (!aligned(p, es)) return fail(SSM_ERR_ALIGN, "an io_dtype pointer is not %lld-byte aligned", (long long)es);
    const void *f_ptrs[] = {a->A, a->Dskip, a->delta_bias, a->h0, a->dh_final, a->dA, a->dBm, a->dCm,
                            a->dDskip, a->ddelta_bias, a->dh0, a->conv_w, a->conv_b, a->dconv_w, a->dconv_b,
                            a->checkpoints};
    for (const void *p : f_ptrs)
        if (!aligned(p, 4)) return fail(SSM_ERR_ALIGN, "an fp32 pointer is not 4-byte aligned");
    const int64_t nck = a->checkpoints ? checkpoint_elems(B, L, D) : 0;
    if (nck < 0) return fail(SSM_ERR_BAD_SHAPE, "checkpoint sizes overflow");
    const Range inputs[] = {
        range(a->x, B * L * D, es, "x"),          range(a->delta, B * L * D, es, "delta"),
        range(a->Bm, B * L * N, es, "Bm"),        range(a->Cm, B * L * N, es, "Cm"),
        range(a->z, B * L * D, es, "z"),          range(a->dy, B * L * D, es, "dy"),
        range(a->A, D * N, 4, "A"),               range(a->Dskip, D, 4, "Dskip"),
        range(a->delta_bias, D, 4, "delta_bias"), range(a->h0, B * D * N, 4, "h0"),
        range(a->dh_final, B * D * N, 4, "dh_final"), range(a->conv_w, D * K, 4, "conv_w"),
        range(a->conv_b, D, 4, "conv_b"),
        range(a->conv_state_in, B * (K > 0 ? K - 1 : 0) * D, es, "conv_state_in"),
        range(a->checkpoints, nck, 4, "checkpoints"),
    };
    const Range outputs[] = {
        range(a->dx, B * L * D, es, "dx"),        range(a->ddelta, B * L * D, es, "ddelta"),
        range(a->dz, B * L * D, es, "dz"),        range(a->dA, D * N, 4, "dA"),
        range(a->dBm, B * L * N, 4, "dBm"),       range(a->dCm, B * L * N, 4, "dCm"),
        range(a->dDskip, D, 4, "dDskip"),         range(a->ddelta_bias, D, 4, "ddelta_bias"),
        range(a->dh0, B * D * N, 4, "dh0"),         range(a->dconv_w, D * K, 4, "dconv_w"),
        range(a->dconv_b, D, 4, "dconv_b"),
        range(a->dconv_state_in, B * (K > 0 ? K - 1 : 0) * D, es, "dconv_state_in"),
    };
    const int nout = (int)(sizeof(outputs) / sizeof(outputs[0]));
    for (int i = 0; i < nout; ++i) {
        for (const Range &r : inputs)
            if (overlaps(outputs[i], r)) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outputs[i].name, r.name);
        for (int k = i + 1; k < nout; ++k)
            if (overlaps(outputs[i], outputs[k]))
                return fail(SSM_ERR_ALIAS, "%s overlaps %s", outputs[i].name, outputs[k].name);
    }
    if (*need_out > 0) {
        if (!a->workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", *need_out);
        if (a->workspace_bytes < *need_out)
            return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", a->workspace_bytes, *need_out);
        if (!aligned(a->workspace, 256)) return fail(SSM_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        const Range ws = range(a->workspace, (int64_t)*need_out, 1, "workspace");
        for (const Range &r : inputs)
            if (overlaps(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
        for (const Range &r : outputs)
            if (overlaps(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
    }
    return SSM_OK;
}

size_t ssm_selective_scan_bwd_workspace_size(const ssm_scan_bwd_args_t *a) {
    if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 1 || a->dstate < 1 || a->dstate > SSM_MAX_DSTATE ||
        !mul_ok(a->batch, a->seqlen, a->dim) || !mul_ok(a->batch, a->dim, a->dstate) ||
        checkpoint_elems(a->batch, a->seqlen, a->dim) < 0)
        return (size_t)-1;
    return a->batch > 0 ? ssm::scan_bwd_workspace_bytes(*a) : 0;
}

ssm_status_t ssm_selective_scan_bwd(const ssm_scan_bwd_args_t *a, void *stream) {
    size_t need = 0;
    const ssm_status_t s = check_bwd(a, &need);
    if (s != SSM_OK) return s;
    if (a->batch == 0) return ok();
    const hipError_t e = ssm::launch_scan_bwd(*a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

ssm_status_t ssm_block_plan_create(const ssm_block_dims_t *d, ssm_block_plan_t **plan) {
    if (!plan) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
    *plan = nullptr;
    if (!d) return fail(SSM_ERR_NULL_ARG, "dims is NULL");
    if (d->batch < 1 || d->seqlen < 1 || d->d_model < 1 || d->d_inner < 1 || d->dstate < 1 || d->dt_rank < 1)
        return fail(SSM_ERR_BAD_SHAPE, "block sizes must all be >= 1");
    if (d->dstate > SSM_MAX_DSTATE)
        return fail(SSM_ERR_UNSUPPORTED, "dstate %lld exceeds SSM_MAX_DSTATE (%d)", (long long)d->dstate,
                    SSM_MAX_DSTATE);
    if (d->d_model % 8 != 0 || d->d_inner % 8 != 0)
        return fail(SSM_ERR_UNSUPPORTED, "d_model and d_inner must be multiples of 8 (got %lld, %lld)",
                    (long long)d->d_model, (long long)d->d_inner);
    if (d->conv_k < 1 || d->conv_k > SSM_MAX_CONV_K)
        return fail(SSM_ERR_UNSUPPORTED, "conv_k must be 1..%d (got %lld)", SSM_MAX_CONV_K, (long long)d->conv_k);
    // hipBLASLt takes 32-bit sizes; the largest operands stay well inside them.
    const int64_t M = d->batch * d->seqlen;
    if (!mul_ok(d->batch, d->seqlen, 4 * (d->d_model + d->d_inner)) || M >= ((int64_t)1 << 30) ||
        d->d_model > INT32_MAX / 4 || d->d_inner > INT32_MAX / 4 || d->dt_rank > d->d_inner)
        return fail(SSM_ERR_BAD_SHAPE, "block sizes out of range (dt_rank <= d_inner, B*L < 2^30)");
    ssm_block_plan *p = nullptr;
    const ssm_status_t s = ssm::block_plan_create(*d, &p);
    if (s != SSM_OK) return fail(s, "could not set up the block's GEMMs (hipBLASLt handle or algorithm)");
    *plan = p;
    return ok();
}

size_t ssm_block_workspace_size(const ssm_block_plan_t *plan) {
    return plan ? ssm::block_workspace_bytes(*plan) : 0;
}

void ssm_block_plan_destroy(ssm_block_plan_t *plan) { ssm::block_plan_destroy(plan); }

ssm_status_t ssm_block_fwd(const ssm_block_plan_t *plan, const ssm_block_weights_t *w, const void *h_in,
                           void *h_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!plan || !w || !h_in || !h_out) return fail(SSM_ERR_NULL_ARG, "plan, weights, h_in and h_out are required");
    if (!w->norm_w || !w->w_in || !w->conv_w || !w->w_x || !w->w_dt || !w->dt_bias || !w->A || !w->w_out)
        return fail(SSM_ERR_NULL_ARG, "a required weight is NULL (only conv_b and Dskip are optional)");
    if (!(w->norm_eps > 0.0f) || !(w->norm_eps < 1e30f)) return fail(SSM_ERR_BAD_SHAPE, "norm_eps must be > 0");
    const ssm_block_dims_t &d = ssm::block_dims(*plan);
    const int64_t M = d.batch * d.seqlen, D = d.d_inner, N = d.dstate, R = d.dt_rank, dm = d.d_model;
    const void *bf[] = {w->w_in, w->w_x, w->w_dt, w->w_out, h_in, h_out, w->norm_w, w->dt_bias};
    for (const void *v : bf)
        if (!aligned(v, 16))
            return fail(SSM_ERR_ALIGN, "bf16 tensors, norm_w and dt_bias must be 16-byte aligned");
    const void *f4[] = {w->norm_w, w->conv_w, w->conv_b, w->dt_bias, w->A, w->Dskip};
    for (const void *v : f4)
        if (!aligned(v, 4)) return fail(SSM_ERR_ALIGN, "fp32 tensors must be 4-byte aligned");
    const size_t need = ssm::block_workspace_bytes(*plan);
    if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(SSM_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    const Range hi = range(h_in, M * dm, 2, "h_in"), ho = range(h_out, M * dm, 2, "h_out");
    if (h_in != h_out && overlaps(hi, ho)) return fail(SSM_ERR_ALIAS, "h_out overlaps h_in (other than in place)");
    const Range inputs[] = {hi,
                            range(w->norm_w, dm, 4, "norm_w"),
                            range(w->w_in, 2 * D * dm, 2, "w_in"),
                            range(w->conv_w, D * d.conv_k, 4, "conv_w"),
                            range(w->conv_b, D, 4, "conv_b"),
                            range(w->w_x, (R + 2 * N) * D, 2, "w_x"),
                            range(w->w_dt, D * R, 2, "w_dt"),
                            range(w->dt_bias, D, 4, "dt_bias"),
                            range(w->A, D * N, 4, "A"),
                            range(w->Dskip, D, 4, "Dskip"),
                            range(w->w_out, dm * D, 2, "w_out")};
    const Range ws = range(workspace, (int64_t)need, 1, "workspace");
    for (const Range &r : inputs) {
        if (overlaps(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
        if (&r != &inputs[0] && overlaps(ho, r)) return fail(SSM_ERR_ALIAS, "h_out overlaps %s", r.name);
    }
    if (overlaps(ws, ho)) return fail(SSM_ERR_ALIAS, "workspace overlaps h_out");
    const hipError_t e = ssm::launch_block_fwd(*plan, *w, h_in, h_out, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

namespace {
ssm_status_t check_ssd_sizes(const ssm_ssd_args_t *a) {
    if (!a) return fail(SSM_ERR_NULL_ARG, "args is NULL");
    if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", a->io_dtype);
    if (a->batch < 0 || a->seqlen < 0) return fail(SSM_ERR_BAD_SHAPE, "negative batch or seqlen");
    if (a->nheads < 1 || a->headdim < 1 || a->ngroups < 1 || a->dstate < 1)
        return fail(SSM_ERR_BAD_SHAPE, "nheads, headdim, ngroups and dstate must be >= 1");
    if (a->nheads % a->ngroups != 0)
        return fail(SSM_ERR_BAD_SHAPE, "ngroups (%lld) must divide nheads (%lld)", (long long)a->ngroups,
                    (long long)a->nheads);
    if (!ssm::ssd_supported(a->headdim, a->dstate))
        return fail(SSM_ERR_UNSUPPORTED,
                    "SSD needs headdim a multiple of 32 up to 4096 and dstate 16, 32, 64 or 128 (got %lld, %lld)",
                    (long long)a->headdim, (long long)a->dstate);
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
    const int64_t B = a->batch, L = a->seqlen, H = a->nheads, P = a->headdim, G = a->ngroups, N = a->dstate;
    if (!mul_ok(B, L, H * P) || !mul_ok(B, L, G * N) || !mul_ok(B, H, P * N))
        return fail(SSM_ERR_BAD_SHAPE, "sizes overflow");
    // one workgroup of 256 threads per (batch, head, 32 channels): the launch holds < 2^32 threads
    if (B * H * (P / 32) > ((int64_t)1 << 23))
        return fail(SSM_ERR_UNSUPPORTED, "batch * nheads * headdim / 32 (%lld) exceeds 2^23",
                    (long long)(B * H * (P / 32)));
    return SSM_OK;
}
}  // namespace

size_t ssm_ssd_workspace_size(const ssm_ssd_args_t *a) {
    if (check_ssd_sizes(a) != SSM_OK) return (size_t)-1;
    if (a->batch == 0 || a->seqlen == 0) return 0;
    return ssm::ssd_workspace_bytes(*a);
}

ssm_status_t ssm_ssd_fwd(const ssm_ssd_args_t *a, void *stream) {
    {
        const ssm_status_t s = check_ssd_sizes(a);
        if (s != SSM_OK) return s;
    }
    const int64_t B = a->batch, L = a->seqlen, H = a->nheads, P = a->headdim, G = a->ngroups, N = a->dstate;
    if (!a->A) return fail(SSM_ERR_NULL_ARG, "A is required");
    if (B * L > 0 && (!a->x || !a->delta || !a->Bm || !a->Cm || !a->y))
        return fail(SSM_ERR_NULL_ARG, "x, delta, Bm, Cm and y are required");
    const int64_t es = io_bytes(a->io_dtype);
    if (a->io_dtype == SSM_BF16) {
        const void *a16[] = {a->x, a->Bm, a->Cm, a->z, a->y};
        for (const void *v : a16)
            if (!aligned(v, 16)) return fail(SSM_ERR_ALIGN, "x, Bm, Cm, z and y must be 16-byte aligned");
        if (!aligned(a->delta, 2)) return fail(SSM_ERR_ALIGN, "delta must be 2-byte aligned");
    } else {
        // fp32: the B and C rows are read as 16-byte groups of 4 entries
        if (!aligned(a->Bm, 16) || !aligned(a->Cm, 16))
            return fail(SSM_ERR_ALIGN, "fp32 Bm and Cm must be 16-byte aligned");
        const void *a4io[] = {a->x, a->z, a->y, a->delta};
        for (const void *v : a4io)
            if (!aligned(v, 4)) return fail(SSM_ERR_ALIGN, "fp32 x, z, y and delta must be 4-byte aligned");
    }
    const void *a4[] = {a->A, a->Dskip, a->delta_bias, a->h0, a->h_final};
    for (const void *v : a4)
        if (!aligned(v, 4)) return fail(SSM_ERR_ALIGN, "fp32 tensors must be 4-byte aligned");
    if (a->io_dtype == SSM_F32 && (!aligned(a->h0, 16) || !aligned(a->h_final, 16)))
        return fail(SSM_ERR_ALIGN, "with fp32 I/O h0 and h_final must be 16-byte aligned");
    const Range inputs[] = {range(a->x, B * L * H * P, es, "x"), range(a->delta, B * L * H, es, "delta"),
                            range(a->A, H, 4, "A"), range(a->Bm, B * L * G * N, es, "Bm"),
                            range(a->Cm, B * L * G * N, es, "Cm"), range(a->Dskip, H, 4, "Dskip"),
                            range(a->z, B * L * H * P, es, "z"), range(a->delta_bias, H, 4, "delta_bias"),
                            range(a->h0, B * H * P * N, 4, "h0")};
    const Range y = range(a->y, B * L * H * P, es, "y"), hf = range(a->h_final, B * H * P * N, 4, "h_final");
    for (const Range &r : inputs) {
        if (overlaps(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
        if (overlaps(hf, r)) return fail(SSM_ERR_ALIAS, "h_final overlaps %s", r.name);
    }
    if (overlaps(y, hf)) return fail(SSM_ERR_ALIAS, "h_final overlaps y");
    if (B == 0) return ok();
    const size_t need = L > 0 ? ssm::ssd_workspace_bytes(*a) : 0;
    if (need > 0) {
        if (!a->workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", need);
        if (a->workspace_bytes < need)
            return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", a->workspace_bytes, need);
        if (!aligned(a->workspace, 256)) return fail(SSM_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        const Range ws = range(a->workspace, (int64_t)need, 1, "workspace");
        for (const Range &r : inputs)
            if (overlaps(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", r.name);
        if (overlaps(ws, y) || overlaps(ws, hf)) return fail(SSM_ERR_ALIAS, "workspace overlaps an output");
    }
    const hipError_t e = ssm::launch_ssd_fwd(*a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

ssm_status_t ssm_ssd_step(const ssm_ssd_step_args_t *a, void *stream) {
    if (!a) return fail(SSM_ERR_NULL_ARG, "args is NULL");
    if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16)
        return fail(SSM_ERR_BAD_DTYPE, "io_dtype %d is not SSM_F32 or SSM_BF16", a->io_dtype);
    if (a->batch < 0) return fail(SSM_ERR_BAD_SHAPE, "negative batch");
    if (a->nheads < 1 || a->headdim < 1 || a->ngroups < 1 || a->dstate < 1)
        return fail(SSM_ERR_BAD_SHAPE, "nheads, headdim, ngroups and dstate must be >= 1");
    if (a->nheads % a->ngroups != 0) return fail(SSM_ERR_BAD_SHAPE, "ngroups must divide nheads");
    if (a->io_dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "the SSD step takes bf16 I/O");
    if (!ssm::ssd_step_supported(a->dstate))
        return fail(SSM_ERR_UNSUPPORTED, "dstate must be a power of two from 4 to 256 (got %lld)",
                    (long long)a->dstate);
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
    const int64_t B = a->batch, H = a->nheads, P = a->headdim, G = a->ngroups, N = a->dstate;
    if (!mul_ok(B, H, P * N) || B * H * P * (N / 4) > ((int64_t)1 << 31))
        return fail(SSM_ERR_BAD_SHAPE, "sizes out of range (B*H*P*N/4 <= 2^31)");
    if (B == 0) return ok();
    if (!a->state || !a->x || !a->delta || !a->A || !a->Bm || !a->Cm || !a->y)
        return fail(SSM_ERR_NULL_ARG, "state, x, delta, A, Bm, Cm and y are required");
    if (!aligned(a->state, 16)) return fail(SSM_ERR_ALIGN, "state must be 16-byte aligned");
    if (!aligned(a->Bm, 8) || !aligned(a->Cm, 8)) return fail(SSM_ERR_ALIGN, "Bm and Cm must be 8-byte aligned");
    const void *a2[] = {a->x, a->delta, a->z, a->y};
    for (const void *v : a2)
        if (!aligned(v, 2)) return fail(SSM_ERR_ALIGN, "bf16 tensors must be 2-byte aligned");
    const void *a4[] = {a->A, a->Dskip, a->delta_bias};
    for (const void *v : a4)
        if (!aligned(v, 4)) return fail(SSM_ERR_ALIGN, "fp32 tensors must be 4-byte aligned");
    const Range inputs[] = {range(a->x, B * H * P, 2, "x"), range(a->delta, B * H, 2, "delta"),
                            range(a->A, H, 4, "A"), range(a->Bm, B * G * N, 2, "Bm"),
                            range(a->Cm, B * G * N, 2, "Cm"), range(a->Dskip, H, 4, "Dskip"),
                            range(a->z, B * H * P, 2, "z"), range(a->delta_bias, H, 4, "delta_bias")};
    const Range st = range(a->state, B * H * P * N, 4, "state"), y = range(a->y, B * H * P, 2, "y");
    for (const Range &r : inputs) {
        if (overlaps(st, r)) return fail(SSM_ERR_ALIAS, "state overlaps %s", r.name);
        if (overlaps(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps %s", r.name);
    }
    if (overlaps(y, st)) return fail(SSM_ERR_ALIAS, "y overlaps the state");
    const hipError_t e = ssm::launch_ssd_step(*a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
