"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (scipy's ZOH discretisation and ODE solver, numpy's convolution,
torch's conv1d / silu / softplus), a closed form, a hand-worked example, an
invariant, or brute force.  Page references name the page's title and the
section or equation:

  [P1] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
       (paper summary page)
  [P2] "2. Mamba 상세" (EulerStack mixer tutorial)
  [P4] "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상"
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.integrate import solve_ivp
from scipy.signal import cont2discrete
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng


def _rand_problem(rng, B=2, L=9, D=3, N=4, gate=True, skip=True, h0=True):
    x = rng.standard_normal((B, L, D))
    delta = np.log1p(np.exp(rng.standard_normal((B, L, D)) - 1.0))
    A = -rng.uniform(0.2, 3.0, size=(D, N))
    Bm = rng.standard_normal((B, L, N))
    Cm = rng.standard_normal((B, L, N))
    Dskip = rng.standard_normal(D) if skip else None
    z = rng.standard_normal((B, L, D)) if gate else None
    hinit = rng.standard_normal((B, D, N)) if h0 else None
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=z, h0=hinit)


def _zoh_scipy(a, b, dt):
    """ZOH of the scalar system h' = a h + b x via scipy's matrix-exponential route."""
    Ad, Bd, _, _, _ = cont2discrete((np.array([[a]]), np.array([[b]]), np.array([[1.0]]),
                                     np.array([[0.0]])), dt, method="zoh")
    return Ad[0, 0], Bd[0, 0]


# ---------------------------------------------------------------- Pi-1: LTI mode
def test_lti_case_equals_convolution_with_zoh_kernel():
    """[P1] sec. 4b, eq. (2) and its convolution mode K = (CB, CAB, ...), y = x * K;
    [P4] sec. 3.3.  Constant Delta, B, C, no gate, zero start: y = x * Kbar + D x, with
    (Abar, Bbar) from scipy's ZOH of the diagonal system and the convolution by numpy."""
    rng = RNG(11)
    L, D, N = 40, 2, 5
    A = -rng.uniform(0.3, 2.5, size=(D, N))
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    dts = np.array([0.37, 0.05])
    Dskip = rng.standard_normal(D)
    x = rng.standard_normal((1, L, D))
    delta = np.broadcast_to(dts, (1, L, D)).copy()
    Bm = np.broadcast_to(Bv, (1, L, N)).copy()
    Cm = np.broadcast_to(Cv, (1, L, N)).copy()
    y, _ = oracle.selective_scan(x, delta, A, Bm, Cm, Dskip=Dskip)
    for d in range(D):
        Ad, Bd, Cd, Dd, _ = cont2discrete((np.diag(A[d]), Bv[:, None], Cv[None, :],
                                           np.zeros((1, 1))), dts[d], method="zoh")
        K = np.empty(L)
        P = np.eye(N)
        for k in range(L):
            K[k] = (Cd @ P @ Bd)[0, 0]
            P = Ad @ P
        ref = np.convolve(x[0, :, d], K)[:L] + Dskip[d] * x[0, :, d]
        np.testing.assert_allclose(y[0, :, d], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- Pi-2: Theorem 1 (eq. 5)
def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = v.split()
    return vals


def test_theorem1_worked_example():
    """[P1] sec. 4b Theorem 1, eq. (5): N=1, A=-1, B=1, Delta=softplus(s) gives the
    gated RNN h_t = (1-g_t) h_{t-1} + g_t x_t with g_t = sigmoid(s_t).  Hand-worked
    dyadic example in tests/golden/theorem1_gated_rnn.txt."""
    g = _read_golden("theorem1_gated_rnn.txt")
    s = np.array([{"0": 0.0, "ln3": math.log(3), "-ln3": -math.log(3),
                   "ln7": math.log(7)}[v] for v in g["s"]])
    x = np.array([float(v) for v in g["x"]])
    href = np.array([float(v) for v in g["h"]])
    L = len(s)
    y, hf = oracle.selective_scan(x.reshape(1, L, 1), s.reshape(1, L, 1),
                                  np.array([[-1.0]]), np.ones((1, L, 1)), np.ones((1, L, 1)),
                                  delta_softplus=True)
    np.testing.assert_allclose(y[0, :, 0], href, rtol=1e-14, atol=1e-14)
    assert abs(hf[0, 0, 0] - href[-1]) < 1e-14


def test_theorem1_random_gates():
    """Same theorem on a long random sequence, against the closed form with scipy's
    expit for the gate; the softplus is applied by the oracle (delta_softplus) with a
    per-channel bias, the parameterisation Delta = softplus(Parameter + s(x)) of
    [P1] Algorithm 2 / [P4] sec. 4.1."""
    rng = RNG(2)
    L, D = 300, 3
    s = 2.0 * rng.standard_normal((1, L, D))
    bias = rng.standard_normal(D)
    x = rng.standard_normal((1, L, D))
    y, _ = oracle.selective_scan(x, s, -np.ones((D, 1)), np.ones((1, L, 1)), np.ones((1, L, 1)),
                                 delta_bias=bias, delta_softplus=True)
    gt = expit(s[0] + bias)
    h = np.zeros(D)
    for t in range(L):
        h = (1.0 - gt[t]) * h + gt[t] * x[0, t]
        np.testing.assert_allclose(y[0, t], h, rtol=1e-12, atol=1e-12)


# --------------------------------------------------- Pi-3: brute force, L <= 4
@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_bruteforce_expanded_recurrence(L):
    """[P1] eq. (2a)/(2b) unrolled by hand: h_t = prod_{r<=t} Abar_r h0 +
    sum_{s<=t} prod_{s<r<=t} Abar_r Bbar_s u_s, with every (Abar, Bbar) from scipy's
    ZOH per (t, n); plus the skip and the gate, both from torch."""
    rng = RNG(100 + L)
    D, N = 3, 3
    p = _rand_problem(rng, B=1, L=L, D=D, N=N)
    y, hf = oracle.selective_scan(**p)
    for d in range(D):
        for t in range(L):
            acc = 0.0
            for n in range(N):
                pairs = [_zoh_scipy(p["A"][d, n], p["Bm"][0, s, n], p["delta"][0, s, d])
                         for s in range(t + 1)]
                term = p["h0"][0, d, n]
                for s in range(t + 1):
                    term *= pairs[s][0]
                for s in range(t + 1):
                    prod = pairs[s][1] * p["x"][0, s, d]
                    for r in range(s + 1, t + 1):
                        prod *= pairs[r][0]
                    term += prod
                acc += p["Cm"][0, t, n] * term
                if t == L - 1:
                    assert abs(hf[0, d, n] - term) <= 1e-12 * (1 + abs(term))
            zt = torch.tensor(p["z"][0, t, d], dtype=torch.float64)
            ref = (acc + p["Dskip"][d] * p["x"][0, t, d]) * torch.nn.functional.silu(zt).item()
            assert abs(y[0, t, d] - ref) <= 1e-12 * (1 + abs(ref))


# ---------------------------------------------------- Pi-4: Delta = 0 holds state
def test_zero_step_holds_state_bit_exactly():
    """[P1] sec. 4b (small Delta keeps the state, Abar -> I) and Q6: with Delta = 0
    exactly, Abar = 1 and Bbar = 0, so the state never moves and y_t = C_t h0 + D u_t."""
    rng = RNG(4)
    p = _rand_problem(rng, B=2, L=17, D=4, N=5, gate=False)
    p["delta"][:] = 0.0
    y, hf = oracle.selective_scan(**p)
    assert np.array_equal(hf, p["h0"])
    ref = np.einsum("bln,bdn->bld", p["Cm"], p["h0"]) + p["Dskip"] * p["x"]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)


# --------------------------------------- Pi-5: strongly negative A*Delta resets
def test_large_step_resets_state():
    """[P1] sec. 4b (large Delta resets the state, Abar -> 0) and Q6: with Delta = 1e3
    and A <= -1, exp(Delta A) underflows to 0 and Bbar = -B/A, so h_t = -B_t u_t / A,
    independent of the past."""
    rng = RNG(5)
    p = _rand_problem(rng, B=1, L=12, D=3, N=4, gate=False, skip=False)
    p["A"] = -rng.uniform(1.0, 5.0, size=(3, 4))
    p["delta"][:] = 1e3
    _, hf = oracle.selective_scan(**p)
    y, _ = oracle.selective_scan(**p)
    href = -p["Bm"][0, -1][None, :] * p["x"][0, -1][:, None] / p["A"]
    np.testing.assert_allclose(hf[0], href, rtol=1e-13, atol=0)
    yref = np.einsum("ln,ldn->ld", p["Cm"][0],
                     -p["Bm"][0][:, None, :] * p["x"][0][:, :, None] / p["A"][None])
    np.testing.assert_allclose(y[0], yref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------- Pi-6: chunked == unchunked
@pytest.mark.parametrize("split", [1, 7, 20])
def test_chunked_equals_unchunked(split):
    """The carried state makes a scan resumable (the state kept for inference in [P2],
    the recurrent mode of [P1] eq. (2)): scanning [0, s) then [s, L) from the first
    part's final state reproduces the single scan exactly."""
    rng = RNG(6)
    p = _rand_problem(rng, B=2, L=21, D=3, N=4)
    y, hf = oracle.selective_scan(**p)
    a = {k: (v[:, :split] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
    b = {k: (v[:, split:] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
    y1, h1 = oracle.selective_scan(**a)
    b["h0"] = h1
    y2, h2 = oracle.selective_scan(**b)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, hf)


# ---------------------------------------------- Pi-7: ZOH solves the ODE exactly
@pytest.mark.parametrize("a,dt", [(-1.0, 0.1), (-7.5, 0.3), (-0.01, 2.0), (0.0, 0.7), (0.8, 0.4)])
def test_zoh_step_matches_ode_integration(a, dt):
    """[P1] eq. (1a) and eq. (4), [P4] sec. 3.2: one recurrence step with the input held
    constant over [0, Delta] equals the ODE h' = a h + b x integrated over Delta
    (scipy solve_ivp, rtol 1e-12).  Includes a = 0, where Bbar takes the limit Delta*b."""
    h0, b, x = 0.7, -1.3, 2.1
    y, hf = oracle.selective_scan(np.full((1, 1, 1), x), np.full((1, 1, 1), dt),
                                  np.full((1, 1), a), np.full((1, 1, 1), b), np.ones((1, 1, 1)),
                                  h0=np.full((1, 1, 1), h0))
    sol = solve_ivp(lambda t, h: a * h + b * x, (0.0, dt), [h0], rtol=1e-12, atol=1e-14)
    assert abs(hf[0, 0, 0] - sol.y[0, -1]) < 1e-10
    assert abs(y[0, 0, 0] - sol.y[0, -1]) < 1e-10


# --------------------------------------------- Pi-8: associativity of the combine
def test_affine_combine_any_tree_order():
    """[P1] Q4 and [P4] sec. 4.2: h_t = Abar_t h_{t-1} + Bbar_t x_t is an associative
    composition of affine maps (a1,b1) then (a2,b2) = (a1 a2, a2 b1 + b2), so any
    bracketing (random trees here) gives the oracle's sequential final state."""
    rng = RNG(8)
    L, N = 37, 3
    p = _rand_problem(rng, B=1, L=L, D=1, N=N, gate=False)
    _, hf = oracle.selective_scan(**p)

    def combine(l, r):
        return (l[0] * r[0], r[0] * l[1] + r[1])

    def tree(items):
        if len(items) == 1:
            return items[0]
        cut = int(rng.integers(1, len(items)))
        return combine(tree(items[:cut]), tree(items[cut:]))

    for _ in range(5):
        for n in range(N):
            pairs = [(1.0, p["h0"][0, 0, n])]  # the initial state as a constant map
            for t in range(L):
                a, bb = _zoh_scipy(p["A"][0, n], p["Bm"][0, t, n], p["delta"][0, t, 0])
                pairs.append((a, bb * p["x"][0, t, 0]))
            agg = tree(pairs)
            assert abs(agg[1] - hf[0, 0, n]) <= 1e-12 * (1 + abs(hf[0, 0, n]))


# ----------------------------- Pi-9: linearity, causality, channel independence
def test_linearity_in_input_and_initial_state():
    """[P1] eq. (2a)/(2b): without the gate, y is linear in (u, h0) for fixed Delta, B, C."""
    rng = RNG(9)
    p = _rand_problem(rng, B=1, L=15, D=3, N=4, gate=False)
    q = dict(p)
    q["x"] = rng.standard_normal(p["x"].shape)
    q["h0"] = rng.standard_normal(p["h0"].shape)
    al, be = 0.7, -1.9
    r = dict(p)
    r["x"] = al * p["x"] + be * q["x"]
    r["h0"] = al * p["h0"] + be * q["h0"]
    yp, hp = oracle.selective_scan(**p)
    yq, hq = oracle.selective_scan(**q)
    yr, hr = oracle.selective_scan(**r)
    np.testing.assert_allclose(yr, al * yp + be * yq, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hr, al * hp + be * hq, rtol=1e-11, atol=1e-11)


def test_causality_and_channel_independence():
    """Outputs at t depend only on inputs at s <= t (the recurrence runs forward), and
    channels/batches are independent (Algorithm 2: A per channel, B and C per batch)."""
    rng = RNG(10)
    p = _rand_problem(rng, B=2, L=14, D=4, N=3)
    y, _ = oracle.selective_scan(**p)
    q = {k: (None if v is None else v.copy()) for k, v in p.items()}
    for k in ("x", "delta", "Bm", "Cm", "z"):
        q[k][:, 9:] = rng.standard_normal(q[k][:, 9:].shape) + (1.0 if k == "delta" else 0.0)
    q["delta"] = np.abs(q["delta"])
    yq, _ = oracle.selective_scan(**q)
    assert np.array_equal(yq[:, :9], y[:, :9])
    perm = np.array([2, 0, 3, 1])
    r = dict(p)
    for k in ("x", "delta", "z"):
        r[k] = p[k][:, :, perm]
    r["A"], r["Dskip"], r["h0"] = p["A"][perm], p["Dskip"][perm], p["h0"][:, perm]
    yr, _ = oracle.selective_scan(**r)
    assert np.array_equal(yr, y[:, :, perm])
    yb, _ = oracle.selective_scan(**{k: (v[1:] if k in ("x", "delta", "Bm", "Cm", "z", "h0")
                                         else v) for k, v in p.items()})
    assert np.array_equal(yb[0], y[1])


# ---------------------------------------------------- Pi-10: decode == scan
def test_decode_steps_equal_scan():
    """[P1] eq. (2) in recurrent mode (one O(N) update per token) and the carried
    ssm_state of [P2]: 64 state_update steps reproduce a scan over L = 64."""
    rng = RNG(12)
    p = _rand_problem(rng, B=3, L=64, D=5, N=4)
    y, hf = oracle.selective_scan(**p)
    st = p["h0"].copy()
    for t in range(64):
        yt, st = oracle.state_update(st, p["x"][:, t], p["delta"][:, t], p["A"], p["Bm"][:, t],
                                     p["Cm"][:, t], Dskip=p["Dskip"], z=p["z"][:, t])
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(st, hf, rtol=1e-15, atol=1e-15)


# ----------------------------------------------------- Pi-11: Euler limit
def test_small_step_tends_to_euler():
    """[P1] sec. 4b, eq. (4) note: as Delta -> 0, Bbar -> Delta B (Euler); the relative
    gap is Delta*a/2 to first order."""
    a, b = -2.3, 0.9
    for dt in (1e-2, 1e-4, 1e-6):
        y, _ = oracle.selective_scan(np.ones((1, 1, 1)), np.full((1, 1, 1), dt),
                                     np.full((1, 1), a), np.full((1, 1, 1), b), np.ones((1, 1, 1)))
        ratio = y[0, 0, 0] / (dt * b)
        assert abs(ratio - 1.0 - dt * a / 2) < (dt * a) ** 2


# ------------------------------------------------------- A = 0 integrator
def test_zero_A_integrates():
    """Reading of eq. (4) at A = 0 (the removable singularity): Bbar = Delta B, Abar = 1,
    so h is the running sum of Delta_t B_t u_t (numpy cumsum)."""
    rng = RNG(13)
    p = _rand_problem(rng, B=1, L=25, D=2, N=3, gate=False, skip=False, h0=False)
    p["A"][:] = 0.0
    y, hf = oracle.selective_scan(**p)
    inc = p["delta"][0][:, :, None] * p["Bm"][0][:, None, :] * p["x"][0][:, :, None]
    h = np.cumsum(inc, axis=0)
    np.testing.assert_allclose(hf[0], h[-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[0], np.einsum("ln,ldn->ld", p["Cm"][0], h), rtol=1e-12,
                               atol=1e-12)


# ----------------------------------- Pi-12/13: conv prologue, gate, softplus
def test_conv_prologue_matches_torch_conv1d():
    """[P1] sec. 4a (Conv1d -> SiLU before the SSM) and [P2] (d_conv: 4): depthwise
    causal conv, zero left padding, w[:, K-1] on the current token, then SiLU; checked
    against torch conv1d(padding=K-1, groups=D) in float64."""
    rng = RNG(14)
    for K in (1, 2, 4):
        x = rng.standard_normal((2, 19, 5))
        w = 0.5 * rng.standard_normal((5, K))
        bias = rng.standard_normal(5)
        u = oracle.causal_conv1d_silu(x, w, bias)
        xt = torch.tensor(x).transpose(1, 2)
        ref = torch.nn.functional.conv1d(xt, torch.tensor(w)[:, None, :], torch.tensor(bias),
                                         padding=K - 1, groups=5)[..., :19]
        ref = torch.nn.functional.silu(ref).transpose(1, 2).numpy()
        np.testing.assert_allclose(u, ref, rtol=1e-13, atol=1e-13)


def test_fused_conv_equals_conv_then_scan():
    """The scan with the conv prologue equals the standalone conv followed by the scan
    on its output (the block order of [P1] sec. 4a)."""
    rng = RNG(15)
    p = _rand_problem(rng, B=2, L=23, D=3, N=4)
    w = 0.5 * rng.standard_normal((3, 4))
    cb = rng.standard_normal(3)
    y1, h1 = oracle.selective_scan(**p, conv_w=w, conv_b=cb)
    q = dict(p)
    q["x"] = oracle.causal_conv1d_silu(p["x"], w, cb)
    y2, h2 = oracle.selective_scan(**q)
    np.testing.assert_allclose(y1, y2, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(h1, h2, rtol=1e-15, atol=1e-15)


# ------------------------------- conv state carried between calls (f1)
def _with_history(rng, K, B=2, L=13, D=3, N=4):
    p = _rand_problem(rng, B=B, L=L, D=D, N=N)
    w = 0.5 * rng.standard_normal((D, K))
    cb = rng.standard_normal(D)
    hist = rng.standard_normal((B, K - 1, D))
    return p, w, cb, hist


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv_history_matches_torch_conv1d_on_concatenation(K):
    """A scan entering with a conv state: the K-1 inputs before t = 0 take the place
    of the zero padding of [P1] sec. 4a's causal conv.  Checked against torch conv1d
    on the concatenated sequence (history, then x), whose last L outputs feed a scan
    without prologue."""
    rng = RNG(40 + K)
    p, w, cb, hist = _with_history(rng, K)
    y1, h1 = oracle.selective_scan(**p, conv_w=w, conv_b=cb, conv_state_in=hist)
    xx = np.concatenate([hist, p["x"]], axis=1)
    xt = torch.tensor(xx).transpose(1, 2)
    u = torch.nn.functional.conv1d(xt, torch.tensor(w)[:, None, :], torch.tensor(cb),
                                   padding=K - 1, groups=3)[..., K - 1:K - 1 + 13]
    u = torch.nn.functional.silu(u).transpose(1, 2).numpy()
    q = dict(p)
    q["x"] = u
    y2, h2 = oracle.selective_scan(**q)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("K,L", [(1, 5), (2, 0), (2, 7), (4, 0), (4, 1), (4, 2), (4, 3), (4, 17)])
def test_conv_state_out_is_the_last_inputs(K, L):
    """The conv state after a scan is its last K-1 inputs, reaching back into the
    entering state when L < K-1 (numpy slicing of the concatenated inputs)."""
    rng = RNG(50 + 10 * K + L)
    p, w, cb, hist = _with_history(rng, K, L=L)
    for h in (hist, None):
        _, _, cs = oracle.selective_scan(**p, conv_w=w, conv_b=cb, conv_state_in=h,
                                         return_conv_state=True)
        prev = h if h is not None else np.zeros_like(hist)
        ref = np.concatenate([prev, p["x"]], axis=1)[:, prev.shape[1] + L - (K - 1):]
        assert cs.shape == (2, K - 1, 3)
        assert np.array_equal(cs, ref)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_decode_with_conv_state_equals_scan(K):
    """Decode with the conv state of [P2] (a rolling window of the last K-1 inputs):
    40 steps reproduce a scan over the same 40 tokens that enters with the same conv
    state and h0 -- every y, the final h and the final window."""
    rng = RNG(60 + K)
    p, w, cb, hist = _with_history(rng, K, B=3, L=40, D=5, N=4)
    y, hf, cs_ref = oracle.selective_scan(**p, conv_w=w, conv_b=cb, conv_state_in=hist,
                                          return_conv_state=True)
    st, cs = p["h0"].copy(), hist.copy()
    for t in range(40):
        yt, st, cs = oracle.state_update(st, p["x"][:, t], p["delta"][:, t], p["A"],
                                         p["Bm"][:, t], p["Cm"][:, t], Dskip=p["Dskip"],
                                         z=p["z"][:, t], conv_w=w, conv_b=cb, conv_state=cs)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st, hf, rtol=1e-14, atol=1e-14)
    assert np.array_equal(cs, cs_ref)


@pytest.mark.parametrize("split", [1, 2, 3, 9])
def test_chunked_prefill_hands_over_conv_state(split):
    """Chunked prefill: a scan over [0, s) returning (h, conv state), then a scan over
    [s, L) entering with both, equals one scan over [0, L) -- bit for bit, since the
    second chunk's conv reads the same inputs from the handed-over state."""
    rng = RNG(70 + split)
    K = 4
    p, w, cb, hist = _with_history(rng, K, L=14)
    seq = ("x", "delta", "Bm", "Cm", "z")
    y, hf, cs = oracle.selective_scan(**p, conv_w=w, conv_b=cb, conv_state_in=hist,
                                      return_conv_state=True)
    a = {k: (v[:, :split] if k in seq else v) for k, v in p.items()}
    ya, ha, csa = oracle.selective_scan(**a, conv_w=w, conv_b=cb, conv_state_in=hist,
                                        return_conv_state=True)
    b = {k: (v[:, split:] if k in seq else v) for k, v in p.items()}
    b["h0"] = ha
    yb, hb, csb = oracle.selective_scan(**b, conv_w=w, conv_b=cb, conv_state_in=csa,
                                        return_conv_state=True)
    assert np.array_equal(np.concatenate([ya, yb], axis=1), y)
    assert np.array_equal(hb, hf)
    assert np.array_equal(csb, cs)


def test_gate_is_silu_of_z():
    """[P1] sec. 4a: the SSM output is multiplied by SiLU(gate); torch silu in float64."""
    rng = RNG(16)
    p = _rand_problem(rng, B=1, L=11, D=3, N=2)
    y, _ = oracle.selective_scan(**p)
    q = dict(p)
    q["z"] = None
    y0, _ = oracle.selective_scan(**q)
    g = torch.nn.functional.silu(torch.tensor(p["z"])).numpy()
    np.testing.assert_allclose(y, y0 * g, rtol=1e-14, atol=1e-14)


def test_delta_softplus_matches_torch():
    """[P1] Algorithm 2 (tau_Delta = softplus) with the per-channel bias of [P4] sec. 4.1:
    the oracle's activation equals torch softplus in float64, including large arguments."""
    rng = RNG(17)
    p = _rand_problem(rng, B=1, L=13, D=3, N=2)
    raw = 15.0 * rng.standard_normal(p["delta"].shape)
    raw[0, 3, 1], raw[0, 5, 2] = 800.0, -800.0   # exp() overflows / underflows here
    bias = rng.standard_normal(3)
    q = dict(p)
    q["delta"] = raw
    y1, h1 = oracle.selective_scan(**q, delta_bias=bias, delta_softplus=True)
    q["delta"] = torch.nn.functional.softplus(torch.tensor(raw + bias)).numpy()
    y2, h2 = oracle.selective_scan(**q)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-13, atol=1e-13)


def test_no_skip_no_gate_no_h0_defaults():
    """Optional inputs default to: no skip term, no gate, zero initial state."""
    rng = RNG(18)
    p = _rand_problem(rng, B=1, L=6, D=2, N=2, gate=False, skip=False, h0=False)
    y, _ = oracle.selective_scan(**p)
    q = dict(p)
    q["Dskip"] = np.zeros(2)
    q["h0"] = np.zeros((1, 2, 2))
    y2, _ = oracle.selective_scan(**q)
    assert np.array_equal(y, y2)


def test_empty_sequence():
    """L = 0 is a valid empty scan: no outputs, and the final state is the start state."""
    rng = RNG(19)
    h0 = rng.standard_normal((1, 2, 3))
    y, hf = oracle.selective_scan(np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), -np.ones((2, 3)),
                                  np.zeros((1, 0, 3)), np.zeros((1, 0, 3)), h0=h0)
    assert y.shape == (1, 0, 2)
    assert np.array_equal(hf, h0)
