"""Seeded random configurations of the scan and the decode step against the
fp64 oracle (needs an MI355X).

Each case draws its own shape and options from a numpy generator seeded by
the case index: batch, length, channels, state size, I/O dtype, conv taps,
Delta softplus with a bias, an entering state, gate and skip, and a diagonal
A that mixes the S4D-real rows -(n+1) with random negative rates, entries
below 1/16 in magnitude, zeros and small positive rates (so both ZOH forms
of the kernels run, sometimes inside one wave).  A few cases are long
sequences on few channels, which the launch scans as concurrent segments;
in fp32 these draw decaying rates only (see _random_A).
Every output element and every final-state entry is compared with the
tolerance of the hand-written cases: |got - ref| <= tol (1 + |ref|), tol =
1e-4 for fp32 I/O and 1e-2 for bf16 I/O.
"""
import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, oracle_scan, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _random_A(rng, D, N, L, f32=False):
    A = -(np.arange(1, N + 1, dtype=np.float64))[None, :].repeat(D, 0)
    kind = rng.integers(0, 4)
    if f32 and L > 1500:
        # Entries that never or barely decay integrate thousands of fp32
        # roundings: a plain sequential fp32 scan then errs by up to 2e-4 of
        # 1 + |y| against the fp64 oracle on these inputs, past the 1e-4 bound
        # that is stated for fp32 I/O.  Long fp32 rows get decaying rates only
        # (undecaying entries are covered in bf16 here and in fp32 on short
        # rows and in the hand-written segment case).
        kind = min(kind, 1)
    if kind >= 1:   # random negative rates on some rows
        rows = rng.random(D) < 0.5
        A[rows] = -rng.uniform(0.05, 8.0, size=(int(rows.sum()), N))
    if kind >= 2:   # small magnitudes and zeros scattered over the matrix
        m = rng.random((D, N))
        A[m < 0.05] = 0.0
        small = (m >= 0.05) & (m < 0.12)
        A[small] = -rng.uniform(0.0, 0.06, size=int(small.sum()))
    if kind == 3 and L <= 800:   # a few slowly growing modes on short sequences
        m = rng.random((D, N)) < 0.02
        A[m] = rng.uniform(0.0, 0.01, size=int(m.sum()))
    return torch.tensor(A, dtype=torch.float32, device=DEV)


def _scan_case(i):
    rng = np.random.default_rng(7000 + i)
    if i % 6 == 5:   # long sequence, few channels: segmented launch
        B, L, D = int(rng.integers(1, 3)), int(rng.integers(4096, 9000)), int(rng.integers(1, 48))
    else:
        B, L, D = int(rng.integers(1, 5)), int(rng.integers(1, 700)), int(rng.integers(1, 320))
    N = int(rng.choice([16, 16, 16, int(rng.integers(1, 17))]))
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    conv_k = int(rng.choice([0, 0, 4, int(rng.integers(1, 5))]))
    softplus = bool(rng.random() < 0.3)
    opts = dict(gate=bool(rng.random() < 0.8), skip=bool(rng.random() < 0.8),
                h0=bool(rng.random() < 0.5), conv_k=conv_k,
                delta_shift=float(rng.uniform(0.5, 3.5)))
    return B, L, D, N, dt, softplus, opts


SCAN_CASES = list(range(36))


@pytest.mark.parametrize("i", SCAN_CASES)
def test_random_scan_config(i):
    B, L, D, N, dt, softplus, opts = _scan_case(i)
    print("case", i, B, L, D, N, dt, softplus, opts, flush=True)
    rng = np.random.default_rng(9000 + i)
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=100 + i, device=DEV, **opts)
    inp["A"] = _random_A(rng, D, N, L, f32=dt == torch.float32)
    kw = {}
    if softplus:
        # raw Delta of either sign before the softplus, plus a per-channel bias
        raw = torch.tensor(rng.normal(-1.0, 1.5, size=(B, L, D)), dtype=torch.float32, device=DEV)
        inp["delta"] = raw.to(dt).contiguous()
        kw = dict(delta_softplus=True,
                  delta_bias=torch.tensor(rng.normal(0.0, 0.5, size=D), dtype=torch.float32,
                                          device=DEV))
    y, hf = ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                   Dskip=inp.get("Dskip"), z=inp.get("z"),
                                   conv_w=inp.get("conv_w"), conv_b=inp.get("conv_b"),
                                   h0=inp.get("h0"), return_final_state=True, **kw)
    torch.cuda.synchronize()
    yr, hr = oracle_scan(inp, **kw)
    assert_close(to64(y), yr, TOL[dt], "y")
    assert_close(to64(hf), hr, TOL[dt], "h_final")


@pytest.mark.parametrize("i", list(range(16)))
def test_random_state_update_config(i):
    rng = np.random.default_rng(8000 + i)
    B, D = int(rng.integers(1, 40)), int(rng.integers(1, 700))
    N = int(rng.choice([16, 16, int(rng.integers(1, 17))]))
    dt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    steps = int(rng.integers(1, 6))
    K = int(rng.choice([0, 0, 4, int(rng.integers(2, 5))]))
    softplus = bool(rng.random() < 0.3)
    print("case", i, B, D, N, dt, steps, K, softplus, flush=True)
    inp = W.make_decode_inputs(B, D, N, steps, io_dtype=dt, seed=300 + i, device=DEV,
                               gate=bool(rng.random() < 0.8), skip=bool(rng.random() < 0.8))
    A = _random_A(rng, D, N, steps)
    bias = (torch.tensor(rng.normal(0.0, 0.5, size=D), dtype=torch.float32, device=DEV)
            if softplus else None)
    conv_w = conv_b = cs = None
    if K:
        conv_w = torch.tensor(rng.normal(0.0, 0.5, size=(D, K)), dtype=torch.float32, device=DEV)
        conv_b = torch.tensor(rng.normal(0.0, 0.5, size=D), dtype=torch.float32, device=DEV)
        cs = torch.tensor(rng.normal(size=(B, K - 1, D)), dtype=torch.float32, device=DEV).to(dt)
    st = inp["state0"].clone()
    cs_dev = None if cs is None else cs.clone()
    ref = to64(inp["state0"])
    ref_cs = to64(cs)
    for t in range(steps):
        y = ssm.state_update(st, inp["x"][t], inp["delta"][t], A, inp["Bm"][t], inp["Cm"][t],
                             Dskip=inp["Dskip"], z=None if inp["z"] is None else inp["z"][t],
                             delta_bias=bias, delta_softplus=softplus,
                             conv_w=conv_w, conv_b=conv_b, conv_state=cs_dev)
        torch.cuda.synchronize()
        out = oracle.state_update(ref, to64(inp["x"][t]), to64(inp["delta"][t]), to64(A),
                                  to64(inp["Bm"][t]), to64(inp["Cm"][t]), Dskip=to64(inp["Dskip"]),
                                  z=None if inp["z"] is None else to64(inp["z"][t]),
                                  delta_bias=to64(bias), delta_softplus=softplus,
                                  conv_w=to64(conv_w), conv_b=to64(conv_b), conv_state=ref_cs)
        if K:
            yr, ref, ref_cs = out
            # the window holds raw inputs: the device copy is exact
            np.testing.assert_array_equal(to64(cs_dev), ref_cs)
        else:
            yr, ref = out
        assert_close(to64(y), yr, TOL[dt], "y step %d" % t)
    assert_close(to64(st), ref, TOL[dt], "state")


# ---- backward -----------------------------------------------------------------
# Per-element gradients at the forward's bound; the sums over batch, time or
# channels (dA, dB, dC, dDskip, the Delta bias, the conv taps and bias) at the
# same tol scaled by 1 + |ref| + mean|ref| (the scale of the backward's own
# tests: a sum with cancellation can be far smaller than its terms).
BWD_PER_ELEM = ("dx", "ddelta", "dz", "dh0", "dconv_state_in")


def _check_grads(g, ref, dt):
    for k, r in ref.items():
        got = to64(g[k])
        assert got.shape == r.shape, (k, got.shape, r.shape)
        assert np.all(np.isfinite(got)), k
        scale = 0.0 if k in BWD_PER_ELEM else float(np.mean(np.abs(r)))
        err = np.abs(got - r) / (1.0 + np.abs(r) + scale)
        worst = float(err.max()) if err.size else 0.0
        assert worst <= TOL[dt], (k, worst)


@pytest.mark.parametrize("i", list(range(16)))
def test_random_backward_config(i):
    rng = np.random.default_rng(6000 + i)
    B, L, D = int(rng.integers(1, 4)), int(rng.integers(1, 300)), int(rng.integers(1, 200))
    N = int(rng.choice([16, 16, int(rng.integers(1, 17))]))
    dt = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    K = int(rng.choice([0, 0, 4, int(rng.integers(1, 5))]))
    softplus = bool(rng.random() < 0.4)
    h0, dhf_on = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    print("case", i, B, L, D, N, dt, K, softplus, h0, dhf_on, flush=True)
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=200 + i, device=DEV, h0=h0, conv_k=K,
                             gate=bool(rng.random() < 0.8), skip=bool(rng.random() < 0.8))
    inp["A"] = _random_A(rng, D, N, L, f32=dt == torch.float32)
    bias = None
    if softplus:
        raw = torch.tensor(rng.normal(-1.0, 1.5, size=(B, L, D)), dtype=torch.float32, device=DEV)
        inp["delta"] = raw.to(dt).contiguous()
        bias = torch.tensor(rng.normal(0.0, 0.4, size=D), dtype=torch.float32, device=DEV)
    conv_b = (torch.tensor(rng.normal(0.0, 0.5, size=D), dtype=torch.float32, device=DEV)
              if K and rng.random() < 0.5 else None)
    dy = torch.tensor(rng.normal(size=(B, L, D)), dtype=torch.float32, device=DEV).to(dt)
    dhf = (torch.tensor(rng.normal(size=(B, D, N)), dtype=torch.float32, device=DEV)
           if dhf_on else None)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias,
                               delta_softplus=softplus, h0=inp["h0"], dh_final=dhf,
                               conv_w=inp["conv_w"], conv_b=conv_b)
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]),
                                    to64(inp["Bm"]), to64(inp["Cm"]), to64(dy),
                                    Dskip=to64(inp["Dskip"]), z=to64(inp["z"]),
                                    delta_bias=to64(bias), delta_softplus=softplus,
                                    h0=to64(inp["h0"]), dh_final=to64(dhf),
                                    conv_w=to64(inp["conv_w"]), conv_b=to64(conv_b))
    _check_grads(g, ref, dt)


# ---- SSD (Mamba-2) layer --------------------------------------------------------
@pytest.mark.parametrize("i", list(range(16)))
def test_random_ssd_config(i):
    rng = np.random.default_rng(5000 + i)
    N = int(rng.choice([16, 32, 64, 128]))
    P = int(rng.choice([32, 64, 64, 96, 128]))
    G = int(rng.choice([1, 1, 2]))
    H = G * int(rng.integers(1, 5))
    if i % 4 == 3:   # few (batch, head) pairs on a long row: segmented
        B, L = 1, int(rng.integers(1500, 4000))
    else:
        B, L = int(rng.integers(1, 4)), int(rng.integers(1, 400))
    dt = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    softplus = bool(rng.random() < 0.3)
    print("case", i, B, L, H, P, G, N, dt, softplus, flush=True)
    inp = W.make_ssd_inputs(B, L, H, P, G, N, seed=400 + i, device=DEV, io_dtype=dt,
                            h0=bool(rng.random() < 0.5), gate=bool(rng.random() < 0.8),
                            skip=bool(rng.random() < 0.8),
                            delta_shift=float(rng.uniform(0.5, 3.0)))
    A = -rng.uniform(0.05, 6.0, size=H)
    if rng.random() < 0.3:
        A[rng.integers(0, H)] = 0.0 if L <= 800 else -0.01
    inp["A"] = torch.tensor(A, dtype=torch.float32, device=DEV)
    bias = None
    if softplus:
        raw = torch.tensor(rng.normal(-1.0, 1.0, size=(B, L, H)), dtype=torch.float32, device=DEV)
        inp["delta"] = raw.to(dt).contiguous()
        bias = torch.tensor(rng.normal(0.0, 0.4, size=H), dtype=torch.float32, device=DEV)
    y, hf = ssm.ssd_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                        z=inp["z"], delta_bias=bias, delta_softplus=softplus, h0=inp["h0"],
                        return_final_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd(to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]),
                        to64(inp["Cm"]), Dskip=to64(inp["Dskip"]), z=to64(inp["z"]),
                        delta_bias=to64(bias), delta_softplus=softplus, h0=to64(inp["h0"]))
    assert_close(to64(y), yr, TOL[dt], "y")
    assert_close(to64(hf), hr, TOL[dt], "h_final")
