/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * The library computes the Mamba-1 selective state-space layer (S6) on one
 * GPU with hand-written HIP kernels:
 *   - ssm_selective_scan_fwd: the whole-sequence scan (prefill), optionally
 *     with a fused depthwise causal conv1d + SiLU prologue and a final-state
 *     output;
 *   - ssm_state_update: one recurrent (decode) step on a resident state;
 *   - ssm_causal_conv1d_silu: the conv prologue on its own;
 *   - ssm_selective_scan_bwd: the gradients of the scan (training);
 *   - ssm_block_fwd: a whole Mamba block around the scan (with a plan);
 *   - ssm_ssd_fwd: the SSD (Mamba-2) layer, chunked on the matrix cores;
 *   - ssm_ssd_step: one decode step of that layer on a resident state.
 *
 * The operations are defined on these pages (cited by title and section):
 *   [P1] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *        (paper summary page): sec. 4a (Mamba block: Conv1d -> SiLU -> SSM,
 *        output x SiLU(gate)), sec. 4b eq. (1a)/(1b), eq. (4) (ZOH),
 *        eq. (2a)/(2b) (recurrence), Algorithm 2 (S6 shapes), sec. 4d (A
 *        diagonal and real, N = 16, E = 2).
 *   [P2] "2. Mamba 상세" (EulerStack mixer tutorial): d_conv: 4 and the
 *        ssm_state kept between inference steps.
 *   [P4] "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상": sec. 3.1
 *        (y = C h + D x, the D skip), sec. 3.2 (ZOH), sec. 4.1 (Delta =
 *        softplus(parameter + projection)), sec. 5.1/5.2 (SSD, chunks).
 *
 * Conventions common to every entry point
 *   - Every tensor pointer is a DEVICE pointer into memory the caller owns
 *     (e.g. a torch tensor's data_ptr()).  The library allocates no device
 *     memory of its own, keeps no state between calls and never frees caller
 *     memory; the one exception is the block plan (ssm_block_plan_create),
 *     which holds a hipBLASLt handle until ssm_block_plan_destroy.
 *   - Tensors are dense and row-major with the last index fastest; element
 *     strides are implied by the shapes.  Pointers must be aligned to their
 *     element size (2 bytes for bf16, 4 for fp32).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls are asynchronous with respect to the host: they enqueue
 *     kernels on `stream` and return.  Faults inside a kernel surface at the
 *     caller's next synchronisation on that stream.
 *   - Argument checking is complete before any HIP call: on an error the
 *     function returns a status other than SSM_OK, enqueues nothing and
 *     writes nothing.  ssm_last_error_message() then describes the failure
 *     (per calling thread).  After launching, a launch failure reported by
 *     the runtime returns SSM_ERR_HIP.
 *   - No C++ exception crosses this interface.  All entry points are
 *     re-entrant and thread-safe; calls that write the same output memory
 *     concurrently race, as with any kernel.
 *   - Sizes: a batch or sequence length of 0 is a valid empty call and
 *     returns SSM_OK without launching (the final state, if requested, is
 *     then a copy of h0, or zeros).  Negative sizes give SSM_ERR_BAD_SHAPE.
 *   - Arithmetic is fp32 throughout, on fp32 or bf16 inputs; bf16 results
 *     are rounded to nearest even.  State, A, D, bias and conv weights are
 *     always fp32.
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 10
#define SSM_MAX_DSTATE 16 /* largest N the kernels hold in registers */
#define SSM_MAX_CONV_K 4  /* largest conv1d kernel width */

typedef enum ssm_status {
    SSM_OK = 0,
    SSM_ERR_NULL_ARG = 1,    /* a required pointer is NULL                   */
    SSM_ERR_BAD_SHAPE = 2,   /* a negative or inconsistent size              */
    SSM_ERR_BAD_DTYPE = 3,   /* io_dtype is not one of ssm_dtype_t           */
    SSM_ERR_UNSUPPORTED = 4, /* N or K above the compiled maximum, bad flags */
    SSM_ERR_ALIAS = 5,       /* an output overlaps an input or another output*/
    SSM_ERR_WORKSPACE = 6,   /* workspace missing, too small or misaligned  */
    SSM_ERR_HIP = 7,         /* the HIP runtime reported an error            */
    SSM_ERR_ALIGN = 8        /* a pointer is not aligned to its element size */
} ssm_status_t;

typedef enum ssm_dtype {
    SSM_F32 = 0, /* IEEE binary32 */
    SSM_BF16 = 1 /* bfloat16 (upper half of a binary32) */
} ssm_dtype_t;

/*
 * Arguments of the selective scan, [P1] Algorithm 2 with the gate of sec. 4a
 * and the skip of [P4] sec. 3.1.  Per batch b, channel d and state index n:
 *
 *   u[b,t,d]   = x[b,t,d], or, when conv_w != NULL, the fused prologue
 *                silu(sum_{k<K} conv_w[d,k] x[b,t-(K-1)+k,d] + conv_b[d])
 *                ([P1] sec. 4a, [P2] d_conv), where x at negative times
 *                comes from conv_state_in, or is 0 without it.
 *   dt[b,t,d]  = delta[b,t,d], or softplus(delta[b,t,d] + delta_bias[d])
 *                when delta_softplus != 0 ([P1] Algorithm 2).
 *   Abar       = exp(dt A[d,n])                                 (eq. 4)
 *   Bbar       = (dt A[d,n])^-1 (exp(dt A[d,n]) - 1) dt Bm[b,t,n]  (eq. 4),
 *                = dt Bm[b,t,n] where A[d,n] == 0 (the limit)
 *   h[b,d,n]   = Abar h[b,d,n] + Bbar u[b,t,d], from h0 (or 0)  (eq. 2a)
 *   y[b,t,d]   = (sum_n Cm[b,t,n] h[b,d,n] + Dskip[d] u[b,t,d])
 *                * silu(z[b,t,d])                               (eq. 2b, 4a)
 *   h_final    = h after the last time step.
 *
 * Conv state (the prefill -> decode handoff of the conv window, kept between
 * inference calls like the SSM state of [P2]): a (B, K-1, D) io_dtype tensor
 * holding, for every batch row and channel, the K-1 most recent inputs x,
 * oldest first (row k is time -(K-1)+k relative to the next token).
 * conv_state_in gives x at times -(K-1)..-1 of this call; conv_state_out
 * receives x at times L-(K-1)..L-1 (from conv_state_in, or 0, where that time
 * is negative), which is the window ssm_state_update expects for the next
 * token.  Both are raw copies of the inputs, bit for bit.
 */
typedef struct ssm_scan_args {
    int64_t batch;          /* B >= 0                                         */
    int64_t seqlen;         /* L >= 0                                         */
    int64_t dim;            /* D >= 1 (channels, E*d_model in the block)      */
    int64_t dstate;         /* N, 1 <= N <= SSM_MAX_DSTATE                    */
    int32_t io_dtype;       /* ssm_dtype_t of x, delta, Bm, Cm, z and y       */
    int32_t delta_softplus; /* 0: delta is the step; 1: softplus(delta+bias) */
    int64_t conv_k;         /* 0: no prologue; 1..SSM_MAX_CONV_K: fused conv  */
    const void *x;          /* (B,L,D) io_dtype, required                     */
    const void *delta;      /* (B,L,D) io_dtype, required                     */
    const void *Bm;         /* (B,L,N) io_dtype, required; shared by channels */
    const void *Cm;         /* (B,L,N) io_dtype, required; shared by channels */
    const void *z;          /* (B,L,D) io_dtype gate, or NULL (no gate)       */
    const float *A;         /* (D,N) fp32, required; any finite value         */
    const float *Dskip;     /* (D) fp32, or NULL (no skip term)               */
    const float *delta_bias;/* (D) fp32, or NULL (= 0); used with softplus    */
    const float *conv_w;    /* (D,conv_k) fp32; required iff conv_k > 0       */
    const float *conv_b;    /* (D) fp32, or NULL (= 0)                        */
    const float *h0;        /* (B,D,N) fp32 initial state, or NULL (= 0)      */
    void *y;                /* (B,L,D) io_dtype output; required              */
    float *h_final;         /* (B,D,N) fp32 output, or NULL (not written)     */
    void *workspace;        /* device scratch of workspace_bytes, 256-aligned */
    size_t workspace_bytes; /* >= ssm_selective_scan_workspace_size(args)     */
    const void *conv_state_in; /* (B,K-1,D) io_dtype, or NULL (= 0); only with conv_k > 0 */
    void *conv_state_out;   /* (B,K-1,D) io_dtype output, or NULL; only with conv_k > 0;
                               may be exactly conv_state_in (updated in place)    */
    float *checkpoints;     /* (ceil(L/SSM_SCAN_BLOCK), B, D, SSM_MAX_DSTATE) fp32
                               output, or NULL: see below                         */
} ssm_scan_args_t;

/*
 * Checkpoints (for training: the forward hands them to the backward, which
 * then does not recompute them).  checkpoints[j][b][d][n] is the state
 * h[b,d,n] entering time step SSM_SCAN_BLOCK * j (the state after step
 * SSM_SCAN_BLOCK * j - 1, or h0 for j = 0), for n < N; entries n >= N are 0.
 * Where the scan splits a long sequence into segments run at the same time,
 * each segment but the first is scanned from a zero state and its first
 * blocks again from its true entering state, up to the block after which
 * exp(A times the segment's sum of dt) is below 2^-160 for every entry; the
 * states from there on are the zero-start ones, which differ from the true
 * states by that factor times the entering state.  Must not overlap any
 * other argument or the workspace.
 */
#define SSM_SCAN_BLOCK 16

/*
 * Bytes of device workspace ssm_selective_scan_fwd needs for these sizes and
 * options (0 when none is needed; only the size fields, io_dtype and the
 * optional-output flags are read, pointers may be NULL).  The workspace holds
 * per-chunk carries of the split sequence; its contents on entry do not
 * matter and on return are unspecified.  Two calls in flight at once need
 * two workspaces.  Returns (size_t)-1 for invalid sizes.
 */
size_t ssm_selective_scan_workspace_size(const ssm_scan_args_t *args);

/*
 * Enqueue the selective scan described above on `stream`.
 * y must not overlap any input; h_final must not overlap any input or y.
 * h0 may be NULL; when given it may not overlap h_final (copy first to scan
 * in place).  conv_state_out must not overlap any other argument except that
 * it may be the same tensor as conv_state_in.  Returns SSM_OK or an error
 * status (see the conventions).
 */
ssm_status_t ssm_selective_scan_fwd(const ssm_scan_args_t *args, void *stream);

/* Bytes of the device scratch array behind ssm_selective_scan_fwd_noalloc (32 MiB). */
#define SSM_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * ssm_selective_scan_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It computes exactly what ssm_selective_scan_fwd computes, with
 * the same kernels, but its workspace is a device array of
 * SSM_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends (a 1M-token sequence at D = 1024 needs about 2 MiB).
 * args->workspace must be NULL and args->workspace_bytes 0.  The caller still
 * passes every input and output.
 *
 * Errors: besides those of ssm_selective_scan_fwd, SSM_ERR_WORKSPACE when
 * ssm_selective_scan_workspace_size(args) exceeds SSM_NOALLOC_SCRATCH_BYTES
 * (before any HIP call) or a workspace is passed; SSM_ERR_HIP if the array's
 * address cannot be obtained on the stream's device.  The call allocates
 * nothing; the first call on a device looks up the array's address there.
 *
 * Every call on one device shares that device's array, and the array keeps
 * whatever the last call left in it (no call depends on its contents on
 * entry).  Calls that may overlap in time on one device -- on different
 * streams, or from different threads without ordering -- race on it: order
 * them on one stream, or use ssm_selective_scan_fwd with separate workspaces.
 */
ssm_status_t ssm_selective_scan_fwd_noalloc(const ssm_scan_args_t *args, void *stream);

/*
 * Depthwise causal conv1d + SiLU, the prologue of [P1] sec. 4a with the
 * width of [P2] (d_conv: 4):
 *   u[b,t,d] = silu(sum_{k<K} w[d,k] x[b,t-(K-1)+k,d] + bias[d]),
 * x at negative times taken as 0 (zero left padding; w[d,K-1] weighs the
 * current token).  x and u: (B,L,D) of io_dtype; w: (D,K) fp32; bias: (D)
 * fp32 or NULL.  1 <= K <= SSM_MAX_CONV_K.  u must not overlap x.
 */
ssm_status_t ssm_causal_conv1d_silu(int64_t batch, int64_t seqlen, int64_t dim, int64_t k,
                                    int32_t io_dtype, const void *x, const float *w,
                                    const float *bias, void *u, void *stream);

/*
 * One decode step, [P1] eq. (2a)/(2b) in recurrent mode on a state kept
 * between calls ([P2] ssm_state), for every batch row b and channel d:
 *   u           = x[b,d], or with conv_k > 0 the prologue of [P1] sec. 4a on
 *                 the window (conv_state[b,0..K-2,d], x[b,d]):
 *                 silu(sum_{k<K-1} conv_w[d,k] conv_state[b,k,d]
 *                      + conv_w[d,K-1] x[b,d] + conv_b[d]);
 *                 the window then drops its oldest row and appends x[b,d]
 *   dt          = delta[b,d] or softplus(delta[b,d] + delta_bias[d])
 *   state[b,d,n] <- exp(dt A[d,n]) state[b,d,n] + Bbar(dt, A[d,n], Bm[b,n]) u
 *   y[b,d]      = (sum_n Cm[b,n] state[b,d,n] + Dskip[d] u) * silu(z[b,d])
 * with Bbar as in the scan.  The state and the conv state are read and
 * written IN PLACE; the conv state has the layout of the scan's
 * conv_state_out, so a prefill hands over to decode directly.
 */
typedef struct ssm_state_update_args {
    int64_t batch;          /* B >= 0                                     */
    int64_t dim;            /* D >= 1                                     */
    int64_t dstate;         /* N, 1 <= N <= SSM_MAX_DSTATE                */
    int32_t io_dtype;       /* ssm_dtype_t of x, delta, z, Bm, Cm, y      */
    int32_t delta_softplus; /* as in ssm_scan_args                        */
    float *state;           /* (B,D,N) fp32, updated in place; required   */
    const void *x;          /* (B,D) io_dtype, required                   */
    const void *delta;      /* (B,D) io_dtype, required                   */
    const void *z;          /* (B,D) io_dtype, or NULL (no gate)          */
    const void *Bm;         /* (B,N) io_dtype, required                   */
    const void *Cm;         /* (B,N) io_dtype, required                   */
    const float *A;         /* (D,N) fp32, required                       */
    const float *Dskip;     /* (D) fp32, or NULL                          */
    const float *delta_bias;/* (D) fp32, or NULL                          */
    void *y;                /* (B,D) io_dtype output; must not overlap any input or the state */
    int64_t conv_k;         /* 0: no prologue; 1..SSM_MAX_CONV_K: causal conv1d + SiLU on x
                               (then D <= 2^28, else SSM_ERR_UNSUPPORTED) */
    const float *conv_w;    /* (D,conv_k) fp32; required iff conv_k > 0   */
    const float *conv_b;    /* (D) fp32, or NULL (= 0)                    */
    void *conv_state;       /* (B,conv_k-1,D) io_dtype, updated in place; required iff
                               conv_k > 1; must not overlap any other argument */
} ssm_state_update_args_t;

ssm_status_t ssm_state_update(const ssm_state_update_args_t *args, void *stream);

/*
 * Backward pass of the selective scan: the gradients of a scalar loss with
 * dL/dy = dy and dL/dh_final = dh_final through the forward defined above
 * ([P1] eq. (4), (2a)/(2b), sec. 4a; the states are recomputed from
 * checkpoints instead of stored, as [P1] sec. 4c does).  With
 * lambda_t = dL/dh_t and gy_t = dy_t silu(z_t):
 *   lambda_t = C_t gy_t + exp(dt_{t+1} A) lambda_{t+1}  (lambda_{L-1} adds dh_final)
 *   dx       = sum_n lambda Bbar + Dskip gy;   ddelta by the chain rule through
 *              exp(dt A), Bbar and the softplus;   dz = dy (C h + D u) silu'(z);
 *   dA, dDskip, ddelta_bias summed over batch and time; dBm, dCm summed over
 *   channels; dh0 = exp(dt_0 A) lambda_0;
 *   with the conv prologue (u = silu(c), c the causal conv of x): dc = du
 *   silu'(c), dx = the conv's transpose applied to dc, dconv_w and dconv_b
 *   summed over batch and time; with a conv state entering the sequence
 *   (the forward's conv_state_in) its rows are read at negative times and
 *   dconv_state_in is the conv's transpose at those times.
 * 1 <= N <= SSM_MAX_DSTATE.  The kernels hold 16 state entries per channel;
 * for N < 16 the workspace also holds 16-wide copies of Bm, Cm, A, h0 and
 * dh_final (extra entries B = C = 0, h0 = dh_final = 0, A = -1, whose state
 * and adjoint stay 0) and of the gradients dA, dBm, dCm and dh0, which are
 * copied back to N-wide rows.  The forward's input fields have the same
 * meaning and shapes as in ssm_scan_args_t.
 */
typedef struct ssm_scan_bwd_args {
    int64_t batch, seqlen, dim, dstate; /* as in ssm_scan_args_t (1 <= N <= 16) */
    int32_t io_dtype;       /* of x, delta, Bm, Cm, z, dy, dx, ddelta, dz      */
    int32_t delta_softplus; /* as in ssm_scan_args_t                           */
    int64_t conv_k;         /* 0 or 1..SSM_MAX_CONV_K, as in ssm_scan_args_t   */
    const void *x, *delta, *Bm, *Cm, *z;            /* forward inputs            */
    const float *A, *Dskip, *delta_bias, *conv_w, *conv_b, *h0;
    const void *dy;         /* (B,L,D) io_dtype, required                      */
    const float *dh_final;  /* (B,D,N) fp32, or NULL (= 0)                     */
    void *dx;               /* (B,L,D) io_dtype output, required               */
    void *ddelta;           /* (B,L,D) io_dtype output (w.r.t. the raw delta)  */
    void *dz;               /* (B,L,D) io_dtype output; required iff z         */
    float *dA;              /* (D,N) fp32 output, required                     */
    float *dBm, *dCm;       /* (B,L,N) fp32 outputs, required                  */
    float *dDskip;          /* (D) fp32 output, or NULL (not written)          */
    float *ddelta_bias;     /* (D) fp32 output, or NULL; 0 without softplus    */
    float *dconv_w;         /* (D,conv_k) fp32 output; required iff conv_k > 0 */
    float *dconv_b;         /* (D) fp32 output, or NULL; only with conv_k > 0  */
    float *dh0;             /* (B,D,N) fp32 output, or NULL                    */
    void *workspace;        /* device scratch, 256-aligned                     */
    size_t workspace_bytes; /* >= ssm_selective_scan_bwd_workspace_size(args)  */
    const void *conv_state_in; /* (B,K-1,D) io_dtype: the inputs before t = 0 the
                                  forward's conv read (its conv_state_in), or
                                  NULL (= 0); only with conv_k > 1          */
    void *dconv_state_in;   /* (B,K-1,D) io_dtype output: its gradient, or NULL;
                               only with conv_k > 1                            */
    const float *checkpoints; /* (ceil(L/SSM_SCAN_BLOCK), B, D, SSM_MAX_DSTATE) fp32: the
                                 checkpoints an ssm_selective_scan_fwd call wrote for the
                                 same x, delta, A, Bm, h0, delta options, conv weights
                                 and conv_state_in; or NULL, and the backward computes
                                 them (in its workspace, which is then larger) */
} ssm_scan_bwd_args_t;

/* Workspace bytes ssm_selective_scan_bwd needs ((size_t)-1 for invalid sizes). */
size_t ssm_selective_scan_bwd_workspace_size(const ssm_scan_bwd_args_t *args);

/*
 * Enqueue the backward pass on `stream`.  Outputs must not overlap any input,
 * each other or the workspace.  Every output given is overwritten.  Returns
 * SSM_OK or an error status (see the conventions).
 */
ssm_status_t ssm_selective_scan_bwd(const ssm_scan_bwd_args_t *args, void *stream);

/*
 * One Mamba block with its pre-norm residual, the block of [P1] sec. 4a (the
 * table of tensor shapes: RMSNorm, the expanding Linear to x and the gate z,
 * Conv1d -> SiLU, the selective SSM, x SiLU(z), the output Linear, + input),
 * with the projections of [P1] Algorithm 2 (s_B, s_C = Linear_N, s_Delta a
 * low-rank Linear of rank R followed by Linear_D; the page's Linear_1 +
 * Broadcast_D is R = 1 with W_dt = 1) and tau_Delta = softplus:
 *   hn = RMSNorm(h) (eps = norm_eps, weight norm_w)
 *   x = hn W_in[0:D]^T, z = hn W_in[D:2D]^T, u = silu(conv1d(x))
 *   dt_low = u W_x[0:R]^T, B = u W_x[R:R+N]^T, C = u W_x[R+N:R+2N]^T
 *   delta = dt_low W_dt^T;  y = S6(u, softplus(delta + dt_bias), A, B, C, D) * silu(z)
 *   h_out = h + y W_out^T
 * I/O and intermediates are bf16 (products accumulate in fp32; the step
 * softplus(delta + dt_bias) is formed in fp32 and stored in bf16); norm_w,
 * conv weights, dt_bias, A and Dskip are fp32.  in_proj, x_proj and out_proj
 * run in hipBLASLt, dt_proj in the library's own kernel.
 *
 * Usage: create a plan for the sizes (this creates a hipBLASLt handle and
 * picks the GEMM algorithms; host memory only, needs the GPU), query its
 * device workspace size, call ssm_block_fwd any number of times, destroy.
 */
typedef struct ssm_block_dims {
    int64_t batch, seqlen;  /* B >= 1, L >= 1                                  */
    int64_t d_model;        /* model width, a multiple of 8                    */
    int64_t d_inner;        /* D = E * d_model (SSM channels), a multiple of 8 */
    int64_t dstate;         /* N, 1 <= N <= SSM_MAX_DSTATE                     */
    int64_t dt_rank;        /* R >= 1                                          */
    int64_t conv_k;         /* 1..SSM_MAX_CONV_K                               */
} ssm_block_dims_t;

typedef struct ssm_block_weights {
    const float *norm_w;    /* (d_model) fp32                                  */
    const void *w_in;       /* (2 D, d_model) bf16: rows of x, then of z       */
    const float *conv_w;    /* (D, conv_k) fp32                                */
    const float *conv_b;    /* (D) fp32, or NULL                               */
    const void *w_x;        /* (R + 2N, D) bf16: rows of dt_low, B, C          */
    const void *w_dt;       /* (D, R) bf16                                     */
    const float *dt_bias;   /* (D) fp32                                        */
    const float *A;         /* (D, N) fp32                                     */
    const float *Dskip;     /* (D) fp32, or NULL                               */
    const void *w_out;      /* (d_model, D) bf16                               */
    float norm_eps;         /* > 0, e.g. 1e-5                                  */
} ssm_block_weights_t;

typedef struct ssm_block_plan ssm_block_plan_t;

/*
 * Plan for these sizes.  Returns SSM_OK and *plan, or an error and *plan =
 * NULL: SSM_ERR_NULL_ARG, SSM_ERR_BAD_SHAPE (a size < 1, dt_rank > d_inner,
 * B*L >= 2^30), SSM_ERR_UNSUPPORTED (dstate, conv_k or a width not a multiple
 * of 8; or hipBLASLt offers no algorithm), SSM_ERR_HIP (no device, or the
 * handle could not be created).  The plan belongs to the device current at
 * creation.
 */
ssm_status_t ssm_block_plan_create(const ssm_block_dims_t *dims, ssm_block_plan_t **plan);

/* Device workspace bytes ssm_block_fwd needs with this plan (0 for NULL). */
size_t ssm_block_workspace_size(const ssm_block_plan_t *plan);

/*
 * h_out = the block applied to h_in, both (B, L, d_model) bf16.  h_out may be
 * h_in itself (updated in place) but may not overlap it otherwise or any
 * weight; nothing may overlap the workspace (256-aligned, >=
 * ssm_block_workspace_size).  bf16 tensors (h_in, h_out, w_in, w_x, w_dt,
 * w_out), norm_w and dt_bias must be 16-byte aligned, the other fp32 ones
 * 4-byte aligned.  The plan may be
 * shared by calls on different streams only with separate workspaces.
 * Errors: SSM_ERR_NULL_ARG (plan, h_in, h_out or a required weight NULL),
 * SSM_ERR_BAD_SHAPE (norm_eps <= 0), SSM_ERR_ALIGN, SSM_ERR_WORKSPACE,
 * SSM_ERR_ALIAS, SSM_ERR_HIP (a launch or hipBLASLt call failed).
 */
ssm_status_t ssm_block_fwd(const ssm_block_plan_t *plan, const ssm_block_weights_t *weights,
                           const void *h_in, void *h_out, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Release a plan (NULL is ignored). */
void ssm_block_plan_destroy(ssm_block_plan_t *plan);

/*
 * The SSD (Mamba-2) layer: [P4] sec. 5.1 restricts the state matrix to a
 * scalar times the identity per step and head, A_t = a_t I, which makes the
 * layer the masked product Y = (L o (C B^T)) X with L the causal mask of
 * cumulative decays; sec. 5.2 evaluates it chunk by chunk (the quadratic form
 * inside a chunk on the matrix cores, the recurrence between chunks).  With
 * the ZOH rule of [P1] eq. (4) for A = a I, per batch b, head h, head channel
 * p, state entry n and step t (g = h / (H / G) the head's group):
 *   dt      = delta[b,t,h], or softplus(delta[b,t,h] + delta_bias[h])
 *   S[p,n] <- exp(dt A[h]) S[p,n] + (exp(dt A[h]) - 1) / A[h] Bm[b,t,g,n] x[b,t,h,p]
 *             (the weight is dt where dt A[h] == 0), from h0 (or 0)
 *   y[b,t,h,p] = (sum_n Cm[b,t,g,n] S[p,n] + Dskip[h] x[b,t,h,p]) * silu(z[b,t,h,p])
 * The state layout (B, H, P, N) is the scan's (B, D, N) with D = H P.
 * This version: headdim P a multiple of 32 up to 4096, dstate N in
 * {16, 32, 64, 128}, batch * nheads * P / 32 <= 2^23; other values give
 * SSM_ERR_UNSUPPORTED.  bf16 I/O runs the chunked form below.  fp32 I/O runs
 * the recurrent form (the same map, [P4] sec. 5.1) sequentially in time with
 * the state in registers, in fp32 throughout, and needs no workspace; its
 * Bm, Cm, h0 and h_final must be 16-byte aligned.  Products run in bf16 on the matrix
 * cores with fp32 accumulation; the state is fp32 (its bf16 copy feeds the
 * product with C).
 */
typedef struct ssm_ssd_args {
    int64_t batch, seqlen;  /* B >= 0, L >= 0                                  */
    int64_t nheads;         /* H >= 1                                          */
    int64_t headdim;        /* P, a multiple of 32 (<= 4096)                   */
    int64_t ngroups;        /* G >= 1, divides H: heads of a group share B, C  */
    int64_t dstate;         /* N (16, 32, 64 or 128)                           */
    int32_t io_dtype;       /* of x, delta, Bm, Cm, z, y: SSM_BF16 or SSM_F32  */
    int32_t delta_softplus; /* 0: delta is the step; 1: softplus(delta + bias) */
    const void *x;          /* (B,L,H,P) io_dtype, required                    */
    const void *delta;      /* (B,L,H) io_dtype, required                      */
    const float *A;         /* (H) fp32, required; any finite value            */
    const void *Bm, *Cm;    /* (B,L,G,N) io_dtype, required                    */
    const float *Dskip;     /* (H) fp32, or NULL                               */
    const void *z;          /* (B,L,H,P) io_dtype gate, or NULL                */
    const float *delta_bias;/* (H) fp32, or NULL                               */
    const float *h0;        /* (B,H,P,N) fp32 initial state, or NULL (= 0)     */
    void *y;                /* (B,L,H,P) io_dtype output, required             */
    float *h_final;         /* (B,H,P,N) fp32 output, or NULL                  */
    void *workspace;        /* device scratch of workspace_bytes, 256-aligned  */
    size_t workspace_bytes; /* >= ssm_ssd_workspace_size(args)                 */
} ssm_ssd_args_t;

/*
 * Bytes of device workspace ssm_ssd_fwd needs (0 when none; only the size
 * fields are read).  With few (batch, head) pairs the sequence is cut into
 * segments that run at once: each segment's end state from a zero start,
 * then the entering states by the recurrence over segments, then each
 * segment's outputs from its entering state.  The workspace holds those
 * states; its contents on entry do not matter.  (size_t)-1 for invalid sizes.
 */
size_t ssm_ssd_workspace_size(const ssm_ssd_args_t *args);

/*
 * Enqueue the SSD layer on `stream`.  x, Bm, Cm, z and y must be 16-byte
 * aligned, delta 2-byte, the fp32 tensors 4-byte.  y, h_final and the
 * workspace must not overlap any input or each other.  L == 0 copies h0 (or zeros) to h_final;
 * the (B,L,...) pointers may then be NULL.
 */
ssm_status_t ssm_ssd_fwd(const ssm_ssd_args_t *args, void *stream);

/*
 * One decode step of the SSD layer: the recurrence above ([P4] sec. 5.1, the
 * state matrix a_t I per step; the recurrent mode of [P1] sec. 4b used for
 * decoding) for a single token on a state kept between calls (updated IN
 * PLACE), for every batch b, head h, head channel p and state entry n
 * (g = h / (H / G)):
 *   dt = delta[b,h] (or softplus(delta[b,h] + delta_bias[h]))
 *   state[b,h,p,n] <- exp(dt A[h]) state[b,h,p,n] + w(dt, A[h]) Bm[b,g,n] x[b,h,p]
 *   y[b,h,p] = (sum_n Cm[b,g,n] state[b,h,p,n] + Dskip[h] x[b,h,p]) * silu(z[b,h,p])
 * with w the ZOH weight of ssm_ssd_fwd; the state layout is that function's
 * h0/h_final, so a prefill hands over to decode directly.  bf16 I/O; any
 * head dim; dstate a power of two from 4 to 256.
 */
typedef struct ssm_ssd_step_args {
    int64_t batch, nheads, headdim, ngroups, dstate; /* B >= 0, H, P, G | H, N */
    int32_t io_dtype;       /* of x, delta, Bm, Cm, z, y: SSM_BF16 or SSM_F32  */
    int32_t delta_softplus; /* as in ssm_ssd_args_t                            */
    float *state;           /* (B,H,P,N) fp32, updated in place; 16-byte aligned */
    const void *x;          /* (B,H,P) bf16, required                          */
    const void *delta;      /* (B,H) bf16, required                            */
    const float *A;         /* (H) fp32, required                              */
    const void *Bm, *Cm;    /* (B,G,N) bf16, required; 8-byte aligned          */
    const float *Dskip;     /* (H) fp32, or NULL                               */
    const void *z;          /* (B,H,P) bf16 gate, or NULL                      */
    const float *delta_bias;/* (H) fp32, or NULL                               */
    void *y;                /* (B,H,P) bf16 output; must not overlap any input or the state */
} ssm_ssd_step_args_t;

ssm_status_t ssm_ssd_step(const ssm_ssd_step_args_t *args, void *stream);

/* Static description of a status code (never NULL). */
const char *ssm_status_string(ssm_status_t status);

/* Description of the last failure returned on the calling thread ("" if none). */
const char *ssm_last_error_message(void);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MI355X_H */
