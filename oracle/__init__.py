"""fp64 CPU oracle for the selective scan (S6): test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never loads it and shares no code with it.

The arithmetic lives in ``ssm_oracle.c`` (plain nested loops in double
precision, written from eq. (1)-(4), Algorithm 2 and sec. 4a of the paper
summary page "Mamba: Linear-Time Sequence Modeling with Selective State
Spaces", and sec. 3.1 of "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상"
for the D skip term).  This module only compiles it with gcc (``-O2``, no
fast-math) and marshals numpy arrays through ctypes.

Every array is converted to contiguous float64 first, so bf16/fp32 inputs are
widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c into libssm_oracle.so (gcc -O2 -fopenmp)."""
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_selective_scan_f64.argtypes = [I64, I64, I64, I64,
                                                  P, P, P, P, P, P, P, P, I, P, P, I64,
                                                  P, P, P, P, P, I]
        lib.oracle_selective_scan_f64.restype = I
        lib.oracle_causal_conv1d_silu_f64.argtypes = [I64, I64, I64, I64, P, P, P, P, I]
        lib.oracle_causal_conv1d_silu_f64.restype = I
        lib.oracle_state_update_f64.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, P, P, I,
                                                P, P, I64, P, P, I]
        lib.oracle_state_update_f64.restype = I
        lib.oracle_selective_scan_bwd_f64.argtypes = [I64, I64, I64, I64,
                                                      P, P, P, P, P, P, P, P, I, P, P, I64,
                                                      P, P, P, P,
                                                      P, P, P, P, P, P, P, P, P, P, P, P, I]
        lib.oracle_selective_scan_bwd_f64.restype = I
        lib.oracle_ssd_f64.argtypes = [I64, I64, I64, I64, I64, I64,
                                       P, P, P, P, P, P, P, P, I, P, P, P, I]
        lib.oracle_ssd_f64.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit() and int(n) > 0:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def selective_scan(x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                   delta_softplus: bool = False, conv_w=None, conv_b=None, h0=None,
                   conv_state_in=None, return_conv_state: bool = False,
                   nthreads: Optional[int] = None):
    """Return (y, h_final), or (y, h_final, conv_state_out), in float64.

    x, delta, z: (B, L, D); A: (D, N); Bm, Cm: (B, L, N); Dskip, delta_bias,
    conv_b: (D,); conv_w: (D, K); h0: (B, D, N); conv_state_in and the
    returned conv state: (B, K-1, D), the inputs before t = 0 (zeros when
    None) and the last K-1 inputs.
    """
    x = _f64(x)
    Bsz, L, D = x.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (Bsz, L, D))
    A = _f64(A, (D, N))
    Bm = _f64(Bm, (Bsz, L, N))
    Cm = _f64(Cm, (Bsz, L, N))
    Dskip = _f64(Dskip, (D,))
    z = _f64(z, (Bsz, L, D))
    delta_bias = _f64(delta_bias, (D,))
    conv_w = _f64(conv_w)
    K = 0 if conv_w is None else conv_w.shape[1]
    if conv_w is not None:
        conv_w = _f64(conv_w, (D, K))
    conv_b = _f64(conv_b, (D,))
    h0 = _f64(h0, (Bsz, D, N))
    if (conv_state_in is not None or return_conv_state) and conv_w is None:
        raise ValueError("a conv state needs conv_w")
    cs_in = _f64(conv_state_in, (Bsz, K - 1, D))
    cs_out = np.zeros((Bsz, max(K - 1, 0), D), np.float64) if return_conv_state else None
    y = np.zeros((Bsz, L, D), np.float64)
    hf = np.zeros((Bsz, D, N), np.float64)
    rc = _load().oracle_selective_scan_f64(
        Bsz, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
        _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(conv_w), _ptr(conv_b), K,
        _ptr(cs_in), _ptr(cs_out), _ptr(h0), _ptr(y), _ptr(hf), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_selective_scan_f64 rejected the sizes")
    return (y, hf, cs_out) if return_conv_state else (y, hf)


def causal_conv1d_silu(x, w, bias=None, nthreads: Optional[int] = None):
    """u = silu(causal depthwise conv1d(x, w) + bias); x (B,L,D), w (D,K)."""
    x = _f64(x)
    Bsz, L, D = x.shape
    w = _f64(w)
    K = w.shape[1]
    w = _f64(w, (D, K))
    bias = _f64(bias, (D,))
    u = np.zeros_like(x)
    rc = _load().oracle_causal_conv1d_silu_f64(Bsz, L, D, K, _ptr(x), _ptr(w), _ptr(bias),
                                               _ptr(u), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_causal_conv1d_silu_f64 rejected the sizes")
    return u


def state_update(state, x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                 delta_softplus: bool = False, conv_w=None, conv_b=None, conv_state=None,
                 nthreads: Optional[int] = None):
    """One decode step.  Returns (y, new_state), or with conv_w given
    (y, new_state, new_conv_state); the inputs are not modified.

    state: (B, D, N); x, delta, z: (B, D); A: (D, N); Bm, Cm: (B, N);
    conv_w: (D, K); conv_b: (D,); conv_state: (B, K-1, D), the previous K-1
    inputs, oldest first.
    """
    st = _f64(state).copy()
    Bsz, D, N = st.shape
    x = _f64(x, (Bsz, D))
    delta = _f64(delta, (Bsz, D))
    A = _f64(A, (D, N))
    Bm = _f64(Bm, (Bsz, N))
    Cm = _f64(Cm, (Bsz, N))
    Dskip = _f64(Dskip, (D,))
    z = _f64(z, (Bsz, D))
    delta_bias = _f64(delta_bias, (D,))
    K = 0
    cs = None
    if conv_w is not None:
        conv_w = _f64(conv_w)
        K = conv_w.shape[1]
        conv_w = _f64(conv_w, (D, K))
        cs = (_f64(conv_state, (Bsz, K - 1, D)).copy() if conv_state is not None
              else np.zeros((Bsz, K - 1, D), np.float64))
    elif conv_state is not None or conv_b is not None:
        raise ValueError("conv_state/conv_b need conv_w")
    conv_b = _f64(conv_b, (D,))
    y = np.zeros((Bsz, D), np.float64)
    rc = _load().oracle_state_update_f64(Bsz, D, N, _ptr(st), _ptr(x), _ptr(delta), _ptr(A),
                                         _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
                                         _ptr(delta_bias), int(bool(delta_softplus)),
                                         _ptr(conv_w), _ptr(conv_b), K, _ptr(cs), _ptr(y),
                                         int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_state_update_f64 rejected the sizes")
    return (y, st, cs) if conv_w is not None else (y, st)


def selective_scan_bwd(x, delta, A, Bm, Cm, dy, Dskip=None, z=None, delta_bias=None,
                       delta_softplus: bool = False, conv_w=None, conv_b=None, h0=None,
                       dh_final=None, conv_state_in=None, nthreads: Optional[int] = None):
    """Gradients of selective_scan for a loss with dL/dy = dy and dL/dh_final = dh_final.

    Returns a dict with dx, ddelta (B,L,D), dA (D,N), dBm, dCm (B,L,N) and, for the
    optional inputs that were given, dz, dDskip, ddelta_bias, dconv_w, dconv_b, dh0 and
    dconv_state_in (B,K-1,D), the gradient of the conv state entering the sequence.
    """
    x = _f64(x)
    Bsz, L, D = x.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (Bsz, L, D))
    Bm = _f64(Bm, (Bsz, L, N))
    Cm = _f64(Cm, (Bsz, L, N))
    Dskip = _f64(Dskip, (D,))
    z = _f64(z, (Bsz, L, D))
    delta_bias = _f64(delta_bias, (D,))
    conv_w = _f64(conv_w)
    K = 0 if conv_w is None else conv_w.shape[1]
    conv_b = _f64(conv_b, (D,))
    h0 = _f64(h0, (Bsz, D, N))
    dy = _f64(dy, (Bsz, L, D))
    dh_final = _f64(dh_final, (Bsz, D, N))
    if conv_state_in is not None and conv_w is None:
        raise ValueError("a conv state needs conv_w")
    conv_state_in = _f64(conv_state_in, (Bsz, max(K - 1, 0), D))
    out = dict(dx=np.zeros((Bsz, L, D)), ddelta=np.zeros((Bsz, L, D)), dA=np.zeros((D, N)),
               dBm=np.zeros((Bsz, L, N)), dCm=np.zeros((Bsz, L, N)))
    if z is not None:
        out["dz"] = np.zeros((Bsz, L, D))
    if Dskip is not None:
        out["dDskip"] = np.zeros(D)
    if delta_softplus:
        out["ddelta_bias"] = np.zeros(D)
    if conv_w is not None:
        out["dconv_w"] = np.zeros((D, K))
        out["dconv_b"] = np.zeros(D)
    if h0 is not None:
        out["dh0"] = np.zeros((Bsz, D, N))
    if conv_state_in is not None:
        out["dconv_state_in"] = np.zeros((Bsz, K - 1, D))
    g = lambda k: _ptr(out.get(k))
    rc = _load().oracle_selective_scan_bwd_f64(
        Bsz, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(conv_w), _ptr(conv_b), K,
        _ptr(conv_state_in), _ptr(h0), _ptr(dy), _ptr(dh_final), g("dx"), g("ddelta"), g("dz"),
        g("dA"), g("dBm"), g("dCm"), g("dDskip"), g("ddelta_bias"), g("dconv_w"), g("dconv_b"),
        g("dh0"), g("dconv_state_in"), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_selective_scan_bwd_f64 rejected the sizes")
    return out


def round_bf16(a):
    """Round to the nearest bfloat16 (ties to even) by way of float32, the precision in
    which the GPU path holds a value before it stores it as bf16; returned as float64."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    nan = np.isnan(a32)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def _softplus(v):
    """softplus(v) = log(1 + e^v), tau_Delta of Algorithm 2 on the paper summary page
    "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (written as
    log(e^0 + e^v) so that large v does not overflow)."""
    return np.logaddexp(0.0, v)


def rms_norm(h, weight, eps=1e-5):
    """RMSNorm over the last axis: h / sqrt(mean(h^2) + eps) * weight."""
    h = _f64(h)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * _f64(weight)


def mamba_block_fwd(h, norm_w, w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, Dskip, w_out,
                    eps=1e-5, bf16=True, perturb=None, nthreads: Optional[int] = None):
    """One Mamba (S6) block with its pre-norm residual, in float64:

      hn = RMSNorm(h);  x, z = hn W_in[:D]^T, hn W_in[D:]^T        (in_proj, split)
      u = silu(causal conv1d(x))                                    (the block's Conv1d)
      dt_low, B, C = u W_x^T split as (R, N, N)                     (x_proj)
      delta = dt_low W_dt^T;  y = S6(u, softplus(delta + dt_bias), A, B, C, D) * silu(z)
      h_out = h + y W_out^T                                         (out_proj + residual)

    The block of the paper summary page "Mamba: Linear-Time Sequence Modeling with
    Selective State Spaces" (sec. 4a; the projections and dt_rank of Algorithm 2).
    Shapes: h (B,L,d_model); norm_w (d_model,); w_in (2D, d_model); conv_w (D,K); conv_b (D,);
    w_x (R+2N, D); w_dt (D, R); dt_bias (D,); A (D,N); Dskip (D,); w_out (d_model, D).

    bf16=True rounds the output of every operation of that list to bf16 (the block's
    activations are bf16 tensors between its operations): hn, x, z, u, the x_proj outputs
    dt_low, B, C, the step dt = softplus(dt_low W_dt^T + dt_bias) (the tau_Delta of
    Algorithm 2 is one operation), y and h_out.  bf16=False rounds nothing.
    perturb, if given, is applied after that rounding to every one of those tensors and to
    the two values inside an operation, the conv output before its SiLU and the step before
    its softplus; it is how the error bound of `mamba_block_error_bound` is exercised.
    """
    r = round_bf16 if bf16 else (lambda v: v)
    if perturb is not None:
        rr = r
        r = lambda v: perturb(rr(v))
    q = perturb if perturb is not None else (lambda v: v)
    h = _f64(h)
    D = w_in.shape[0] // 2
    N = A.shape[1]
    R = w_dt.shape[1]
    w_in, w_x, w_dt, w_out = (_f64(v) for v in (w_in, w_x, w_dt, w_out))
    hn = r(rms_norm(h, norm_w, eps))
    x = r(hn @ w_in[:D].T)
    z = r(hn @ w_in[D:].T)
    if perturb is None:
        u = r(causal_conv1d_silu(x, conv_w, conv_b, nthreads=nthreads))
    else:
        c = q(_causal_conv1d(x, conv_w, conv_b))
        u = r(c / (1.0 + np.exp(-c)))
    xd = u @ w_x.T
    dt_low, Bm, Cm = r(xd[..., :R]), r(xd[..., R:R + N]), r(xd[..., R + N:])
    dt = r(_softplus(q(dt_low @ w_dt.T + _f64(dt_bias))))
    y, _ = selective_scan(u, dt, A, Bm, Cm, Dskip=Dskip, z=z, nthreads=nthreads)
    return r(h + r(y) @ w_out.T)


def _causal_conv1d(x, w, b=None):
    """c[t] = sum_k w[k] x[t-K+1+k] (+ b), zero before t = 0 (the conv orientation of the
    scan's prologue); x (B,L,D), w (D,K)."""
    x = _f64(x)
    w = _f64(w)
    K = w.shape[1]
    L = x.shape[1]
    c = np.zeros_like(x) if b is None else np.broadcast_to(_f64(b), x.shape).copy()
    for k in range(K):
        s = K - 1 - k                    # tap k reads x s steps back
        if s < L:
            c[:, s:, :] += w[:, k] * x[:, :L - s, :]
    return c


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits), round to nearest
U_F32 = 2.0 ** -24   # unit roundoff of fp32


def mamba_block_error_bound(h, norm_w, w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, Dskip,
                            w_out, eps=1e-5, lam=10.0):
    """(h_out, tol, sigma): the block of `mamba_block_fwd` in float64 with no rounding; a
    per-element tolerance for an implementation that stores the block's intermediates in
    bf16; and the standard deviation of its error that the tolerance is built from.

    Error model.  The implementation may round to bf16 the output of any operation of the
    block (hn, x, z, the conv output before and after its SiLU, dt_low, B, C, the step
    before and after its softplus, y: relative error at most U_BF16 each) and rounds h_out
    to bf16; inside an operation it works in fp32 (a sum of K terms errs by at most
    K U_F32 of the sum of their magnitudes; exp, SiLU and softplus by a few U_F32; the ZOH
    input weight (e^{dt a} - 1)/a by a few U_F32 of 1/|a|, since e^{dt a} - 1 cancels
    for small dt a).

    Propagation.  As in probabilistic rounding error analysis, each rounding error is
    taken as an independent zero-mean variable, uniform on [-u|v|, u|v|] (variance
    u^2 v^2 / 3); to first order the output error is a linear combination of them, and its
    variance is carried through the block: a projection v W^T maps variances by W^2, an
    elementwise function by its squared derivative, and the recurrence of eq. (2a) on the
    paper summary page "Mamba: Linear-Time Sequence Modeling with Selective State
    Spaces" (sec. 4b) carries the state variance by A_bar^2 and adds the squared
    sensitivities of h_t to dt_t (a A_bar h + A_bar B u), B_t and u_t.  The fp32 terms
    are added as if they were roundings of the same size.

    tol = lam * sigma + U_BF16 |h_out|: lam standard deviations of the first-order error
    plus the rounding of h_out itself, which every bf16 output carries.
    """
    ub, uf = U_BF16, U_F32
    h = _f64(h)
    Bsz, L, dm = h.shape
    D = w_in.shape[0] // 2
    A = _f64(A)
    N = A.shape[1]
    R = w_dt.shape[1]
    K = conv_w.shape[1]
    w_in, w_x, w_dt, w_out, conv_w = (_f64(v) for v in (w_in, w_x, w_dt, w_out, conv_w))
    conv_b = None if conv_b is None else _f64(conv_b)
    Dsk = _f64(Dskip)
    third = 1.0 / 3.0
    rnd = lambda v, u: third * (u * v) ** 2          # variance of one rounding of v

    def lin(v, var_v, W, rounded=True):
        """v W^T and its error variance (K = W's inner size)."""
        o = v @ W.T
        var = var_v @ (W * W).T + rnd(np.abs(v) @ np.abs(W).T, W.shape[1] * uf)
        return o, var + (rnd(o, ub) if rounded else 0.0)

    # RMSNorm (sum of squares over d_model, a square root and a division, then the weight)
    hn = rms_norm(h, norm_w, eps)
    var_hn = rnd(hn, (dm + 8) * uf) + rnd(hn, ub)
    x, var_x = lin(hn, var_hn, w_in[:D])
    z, var_z = lin(hn, var_hn, w_in[D:])
    # causal conv1d, then SiLU with derivative s(c)(1 + c(1 - s(c)))
    c = _causal_conv1d(x, conv_w, conv_b)
    var_c = (_causal_conv1d(var_x, conv_w * conv_w)
             + rnd(_causal_conv1d(np.abs(x), np.abs(conv_w),
                                  None if conv_b is None else np.abs(conv_b)), (K + 1) * uf)
             + rnd(c, ub))
    sg = 1.0 / (1.0 + np.exp(-c))
    u = c * sg
    du = sg * (1.0 + c * (1.0 - sg))
    var_u = du * du * var_c + rnd(u, 4 * uf) + rnd(u, ub)
    # x_proj
    xd, var_xd = lin(u, var_u, w_x)
    dt_low, Bm, Cm = xd[..., :R], xd[..., R:R + N], xd[..., R + N:]
    v_dl, v_B, v_C = var_xd[..., :R], var_xd[..., R:R + N], var_xd[..., R + N:]
    # dt_proj + bias, then softplus (derivative: the logistic function)
    pre, var_pre = lin(dt_low, v_dl, w_dt, rounded=False)
    pre = pre + _f64(dt_bias)
    var_pre += rnd(_f64(dt_bias), uf) + rnd(pre, ub)
    dt = _softplus(pre)
    sig = 1.0 / (1.0 + np.exp(-pre))
    var_dt = sig * sig * var_pre + rnd(dt, 4 * uf) + rnd(dt, ub)
    # the recurrence per (b, d, n), in the order of eq. (2a)/(2b); the terms that do not
    # depend on the state are formed for a chunk of steps at once
    hs = np.zeros((Bsz, D, N))
    var_hs = np.zeros((Bsz, D, N))
    y = np.zeros((Bsz, L, D))
    var_y = np.zeros((Bsz, L, D))
    a = A[None, None, :, :]
    a_nz = a != 0.0
    inv_a = np.where(a_nz, 1.0 / np.where(a_nz, np.abs(a), 1.0), 0.0)
    T = max(8, min(512, (1 << 18) // max(1, Bsz * D * N)))
    for t0 in range(0, L, T):
        t1 = min(L, t0 + T)
        dtt = dt[:, t0:t1, :, None]
        ut, vut = u[:, t0:t1, :, None], var_u[:, t0:t1, :, None]
        Bt, vBt = Bm[:, t0:t1, None, :], v_B[:, t0:t1, None, :]
        Ct, vCt = Cm[:, t0:t1, None, :], v_C[:, t0:t1, None, :]
        za = dtt * a
        ab = np.exp(za)
        w = np.where(a_nz, np.expm1(za) / np.where(a_nz, a, 1.0), dtt)
        bu = Bt * ut
        wbu = w * bu
        src = ((w * ut) ** 2 * vBt + (w * Bt) ** 2 * vut + rnd(wbu, 4 * uf)
               + rnd(bu * inv_a, 4 * uf))
        ab2, aab, abbu = ab * ab, a * ab, ab * bu
        rel = third * ((np.abs(za) + 4) * uf) ** 2 * ab2      # rounding of A_bar h, per h^2
        vdt = var_dt[:, t0:t1, :, None]
        H = np.empty_like(ab)
        VH = np.empty_like(ab)
        for k in range(t1 - t0):
            sens = aab[:, k] * hs + abbu[:, k]
            var_hs = (ab2[:, k] * var_hs + sens * sens * vdt[:, k] + src[:, k]
                      + rel[:, k] * hs * hs)
            hs = ab[:, k] * hs + wbu[:, k]
            H[:, k] = hs
            VH[:, k] = var_hs
        us = u[:, t0:t1]
        ys = (Ct * H).sum(-1) + Dsk * us
        var_ys = ((Ct * Ct * VH + H * H * vCt).sum(-1) + Dsk * Dsk * var_u[:, t0:t1]
                  + rnd(np.abs(Ct * H).sum(-1) + np.abs(Dsk * us), (N + 2) * uf))
        zt = z[:, t0:t1]
        sz_sig = 1.0 / (1.0 + np.exp(-zt))
        sz = zt * sz_sig
        dsz = sz_sig * (1.0 + zt * (1.0 - sz_sig))
        yt = ys * sz
        y[:, t0:t1] = yt
        var_y[:, t0:t1] = (sz * sz * var_ys + (ys * dsz) ** 2 * var_z[:, t0:t1]
                           + rnd(yt, 4 * uf) + rnd(yt, ub))
    # out_proj + residual
    o, var_o = lin(y, var_y, w_out, rounded=False)
    out = h + o
    var_out = var_o + rnd(np.abs(h), (D + 1) * uf)
    sigma = np.sqrt(var_out)
    return out, lam * sigma + ub * np.abs(out), sigma


def ssd(x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None, delta_softplus: bool = False,
        h0=None, nthreads: Optional[int] = None):
    """The SSD (Mamba-2) layer in recurrent mode, in float64 (``oracle_ssd_f64``): per head a
    scalar A_t = a_t I ("14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상", sec. 5.1),
    discretised by ZOH (eq. (4) of the paper summary page "Mamba: Linear-Time Sequence
    Modeling with Selective State Spaces").  Returns (y, h_final).

    x, z: (B, L, H, P); delta: (B, L, H); A, Dskip, delta_bias: (H,); Bm, Cm: (B, L, G, N)
    with H a multiple of G (head h reads group h // (H // G)); h0, h_final: (B, H, P, N).
    """
    x = _f64(x)
    Bsz, L, H, P = x.shape
    Bm = _f64(Bm)
    G, N = Bm.shape[2], Bm.shape[3]
    delta = _f64(delta, (Bsz, L, H))
    A = _f64(A, (H,))
    Bm = _f64(Bm, (Bsz, L, G, N))
    Cm = _f64(Cm, (Bsz, L, G, N))
    Dskip = _f64(Dskip, (H,))
    z = _f64(z, (Bsz, L, H, P))
    delta_bias = _f64(delta_bias, (H,))
    h0 = _f64(h0, (Bsz, H, P, N))
    y = np.zeros((Bsz, L, H, P), np.float64)
    hf = np.zeros((Bsz, H, P, N), np.float64)
    rc = _load().oracle_ssd_f64(Bsz, L, H, P, G, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm),
                                _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(delta_bias),
                                int(bool(delta_softplus)), _ptr(h0), _ptr(y), _ptr(hf),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_ssd_f64 rejected the sizes")
    return y, hf


def ssd_quadratic(x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None):
    """The same layer in its quadratic ("attention") mode, float64 numpy: per (batch, head)
    Y = (L o (C B^T)) (w X) + D X, the duality form of sec. 5.1 of "14.1 SSM(State Space
    Models)과 Mamba 아키텍처의 부상", with L[t, s] = prod_{r=s+1..t} alpha_r for s <= t and 0
    above the diagonal (the causal mask of cumulative decays), alpha_t = exp(dt_t a) and
    w_s the ZOH input weight.  An entering state h0 adds (prod_{r<=t} alpha_r) C_t h0.
    Returns (y, h_final) like ``ssd``; delta is the step itself (no softplus here).
    """
    x = _f64(x)
    Bsz, L, H, P = x.shape
    Bm = _f64(Bm)
    G, N = Bm.shape[2], Bm.shape[3]
    delta = _f64(delta, (Bsz, L, H))
    A = _f64(A, (H,))
    Cm = _f64(Cm, (Bsz, L, G, N))
    hpg = H // G
    y = np.zeros((Bsz, L, H, P))
    hf = np.zeros((Bsz, H, P, N))
    t_idx = np.arange(L)
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            za = delta[b, :, h] * A[h]                       # dt_t a, (L,)
            w = np.where(za == 0.0, delta[b, :, h], np.expm1(za) / np.where(za == 0.0, 1.0, A[h]))
            cs = np.concatenate([[0.0], np.cumsum(za)])      # cs[t+1] = sum_{r<=t} dt_r a
            # log L[t, s] = sum_{r=s+1..t} dt_r a = cs[t+1] - cs[s+1]
            logm = cs[1:, None] - cs[None, 1:]
            causal = t_idx[:, None] >= t_idx[None, :]
            mask = np.where(causal, np.exp(np.where(causal, logm, 0.0)), 0.0)
            M = mask * (Cm[b, :, g, :] @ Bm[b, :, g, :].T)   # (L, L)
            Xw = w[:, None] * x[b, :, h, :]                  # (L, P)
            yb = M @ Xw
            decay_in = np.exp(cs[1:])                        # prod_{r<=t} alpha_r
            if h0 is not None:
                yb += decay_in[:, None] * (Cm[b, :, g, :] @ _f64(h0)[b, h].T)
            if Dskip is not None:
                yb += _f64(Dskip)[h] * x[b, :, h, :]
            if z is not None:
                zz = _f64(z)[b, :, h, :]
                yb *= zz / (1.0 + np.exp(-zz))
            y[b, :, h, :] = yb
            # final state: sum_s (prod_{r=s+1..L-1} alpha_r) w_s x_s B_s^T (+ decayed h0)
            tail = np.exp(cs[L] - cs[1:]) if L else np.zeros(0)
            hfin = (tail[:, None] * Xw).T @ Bm[b, :, g, :]   # (P, N)
            if h0 is not None:
                hfin += np.exp(cs[L]) * _f64(h0)[b, h]
            hf[b, h] = hfin
    return y, hf
