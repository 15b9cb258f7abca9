"""Parity of the backward pass (gradients) against the fp64 oracle (needs an MI355X).

Tolerance.  The forward's bound |got - ref| <= tol (1 + |ref|), tol = 1e-4 for
fp32 and 1e-2 for bf16 I/O, holds per element for the per-element gradients
(dx, ddelta, dz, dh0; bf16 ones are rounded to bf16).  The gradients that are
sums over many terms (dA over batch and time, dB and dC over channels, dDskip
and the delta bias over batch and time; fp32 outputs accumulated in fp32) are
held to the same tol, scaled by (1 + |ref| + s) with s the mean absolute entry
of that gradient, since a sum with cancellation can be small next to its
terms.  Measured: every sum within ~2e-6 of that scale.
"""
import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_SUM = TOL
PER_ELEM = ("dx", "ddelta", "dz", "dh0", "dconv_state_in")


def _check(name, got, ref, tol, scale=0.0):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref) / (1.0 + np.abs(ref) + scale)
    worst = float(err.max()) if err.size else 0.0
    print("  %-12s worst scaled error %.2e (tol %.0e)" % (name, worst, tol), flush=True)
    if worst > tol:
        bad = np.argwhere(err > tol)
        idx = tuple(bad[0])
        print("  %s: %d elements over; first %s got %r ref %r; last %s" % (
            name, len(bad), idx, got[idx], ref[idx], tuple(bad[-1])), flush=True)
    assert worst <= tol, (name, worst)


def _run(inp, dt, softplus=False, bias=None, dh_final=None, rows=None):
    dy = torch.randn(inp["x"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(5)).to(dt)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias,
                               delta_softplus=softplus, h0=inp["h0"], dh_final=dh_final)
    torch.cuda.synchronize()
    sel = (lambda t: t) if rows is None else (lambda t: None if t is None else t[rows])
    ref = oracle.selective_scan_bwd(
        to64(sel(inp["x"])), to64(sel(inp["delta"])), to64(inp["A"]), to64(sel(inp["Bm"])),
        to64(sel(inp["Cm"])), to64(sel(dy)), Dskip=to64(inp["Dskip"]), z=to64(sel(inp["z"])),
        delta_bias=to64(bias), delta_softplus=softplus, h0=to64(sel(inp["h0"])),
        dh_final=to64(sel(dh_final)))
    return g, ref


CASES = [
    # name, B, L, D, dtype, extra
    ("small_f32", 1, 37, 20, torch.float32, dict(h0=True)),
    ("ragged_bf16", 2, 100, 70, torch.bfloat16, dict(h0=True)),
    ("block_f32", 3, 64, 64, torch.float32, {}),
    ("nogate_noskip_f32", 2, 45, 33, torch.float32, dict(gate=False, skip=False)),
    ("L1_f32", 2, 1, 40, torch.float32, dict(h0=True)),
    ("wide_bf16", 2, 130, 300, torch.bfloat16, {}),
]


@pytest.mark.parametrize("name,B,L,D,dt,extra", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(name, B, L, D, dt, extra):
    print("case", name, flush=True)
    inp = W.make_scan_inputs(B, L, D, 16, io_dtype=dt, seed=500 + L + D, device=DEV, **extra)
    dhf = torch.randn(B, D, 16, device=DEV, generator=torch.Generator(DEV).manual_seed(6))
    g, ref = _run(inp, dt, dh_final=dhf)
    for k, r in ref.items():
        if k in PER_ELEM:
            _check(k, to64(g[k]), r, TOL[dt])
        else:
            _check(k, to64(g[k]), r, TOL_SUM[dt], float(np.mean(np.abs(r))))


def test_bwd_softplus_bias_and_zero_A():
    inp = W.make_scan_inputs(2, 70, 48, 16, io_dtype=torch.float32, seed=531, device=DEV, h0=True)
    g0 = torch.Generator(DEV).manual_seed(7)
    inp["delta"] = (torch.randn(inp["delta"].shape, device=DEV, generator=g0) - 1.0).contiguous()
    A = inp["A"].clone()
    A[:, 0] = 0.0
    A[5, 3] = 0.02
    inp["A"] = A
    bias = 0.3 * torch.randn(48, device=DEV, generator=g0)
    g, ref = _run(inp, torch.float32, softplus=True, bias=bias)
    for k, r in ref.items():
        if k in PER_ELEM:
            _check(k, to64(g[k]), r, TOL[torch.float32])
        else:
            _check(k, to64(g[k]), r, TOL_SUM[torch.float32], float(np.mean(np.abs(r))))


def test_bwd_softplus_bias_with_final_state_gradient_ragged():
    """Softplus with a bias, a gradient on the final state and a length that ends inside a
    16-step block: the steps past the end (dt = 0) carry dh_final back unchanged and must
    add nothing to the bias gradient."""
    inp = W.make_scan_inputs(2, 70, 40, 16, io_dtype=torch.float32, seed=533, device=DEV, h0=True)
    g0 = torch.Generator(DEV).manual_seed(8)
    inp["delta"] = (torch.randn(inp["delta"].shape, device=DEV, generator=g0) - 1.0).contiguous()
    bias = 0.3 * torch.randn(40, device=DEV, generator=g0)
    dhf = torch.randn(2, 40, 16, device=DEV, generator=g0)
    g, ref = _run(inp, torch.float32, softplus=True, bias=bias, dh_final=dhf)
    for k, r in ref.items():
        if k in PER_ELEM:
            _check(k, to64(g[k]), r, TOL[torch.float32])
        else:
            _check(k, to64(g[k]), r, TOL_SUM[torch.float32], float(np.mean(np.abs(r))))


def test_bwd_empty_sequence():
    inp = W.make_scan_inputs(2, 0, 32, 16, io_dtype=torch.float32, seed=532, device=DEV, h0=True)
    dhf = torch.randn(2, 32, 16, device=DEV)
    g, _ = _run(inp, torch.float32, dh_final=dhf)
    assert torch.equal(g["dh0"], dhf) and torch.count_nonzero(g["dA"]) == 0


def test_bwd_130m_layer_sampled_batch_row():
    """The 130M-like layer (B=8, L=2048, D=1536, bf16) in full; the oracle checks batch
    row 5 on every channel (dx, ddelta, dz, dB, dC of that row)."""
    cfg = W.C2_130M
    print("config", cfg.name, flush=True)
    inp = W.make_config_inputs(cfg, device=DEV)
    dt = cfg.io_dtype
    dy = torch.randn(inp["x"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(5)).to(dt)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"])
    torch.cuda.synchronize()
    r = slice(5, 6)
    ref = oracle.selective_scan_bwd(to64(inp["x"][r]), to64(inp["delta"][r]), to64(inp["A"]),
                                    to64(inp["Bm"][r]), to64(inp["Cm"][r]), to64(dy[r]),
                                    Dskip=to64(inp["Dskip"]), z=to64(inp["z"][r]))
    for k in ("dx", "ddelta", "dz"):
        _check(k, to64(g[k][r]), ref[k], TOL[dt])
    for k in ("dBm", "dCm"):
        _check(k, to64(g[k][r]), ref[k], TOL_SUM[dt], float(np.mean(np.abs(ref[k]))))
    del inp, g, dy
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,L,D,K,dt", [(2, 70, 40, 4, torch.float32), (1, 300, 70, 3, torch.bfloat16),
                                        (2, 5, 33, 2, torch.float32), (1, 600, 20, 4, torch.float32),
                                        (2, 257, 64, 4, torch.bfloat16)])
def test_bwd_through_conv_prologue(B, L, D, K, dt):
    """Gradients through the fused causal conv + SiLU prologue (dx via the conv's
    transpose, dconv_w, dconv_b), including sequences spanning several conv chunks."""
    print("conv case", B, L, D, K, dt, flush=True)
    inp = W.make_scan_inputs(B, L, D, 16, io_dtype=dt, seed=600 + L + K, device=DEV, conv_k=K, h0=True)
    inp["conv_b"] = 0.5 * torch.randn(D, device=DEV, generator=torch.Generator(DEV).manual_seed(8))
    dy = torch.randn(inp["x"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(5)).to(dt)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], h0=inp["h0"], conv_w=inp["conv_w"],
                               conv_b=inp["conv_b"])
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]),
                                    to64(inp["Cm"]), to64(dy), Dskip=to64(inp["Dskip"]), z=to64(inp["z"]),
                                    h0=to64(inp["h0"]), conv_w=to64(inp["conv_w"]),
                                    conv_b=to64(inp["conv_b"]))
    assert set(ref) <= set(g)
    for k, r in ref.items():
        if k in PER_ELEM:
            _check(k, to64(g[k]), r, TOL[dt])
        else:
            _check(k, to64(g[k]), r, TOL_SUM[dt], float(np.mean(np.abs(r))))


def _check_all(g, ref, dt):
    assert set(ref) <= set(g), (set(ref), set(g))
    for k, r in ref.items():
        if k in PER_ELEM:
            _check(k, to64(g[k]), r, TOL[dt])
        else:
            _check(k, to64(g[k]), r, TOL_SUM[dt], float(np.mean(np.abs(r))))


@pytest.mark.parametrize("N,dt,conv_k", [(1, torch.float32, 0), (5, torch.float32, 4),
                                         (15, torch.bfloat16, 0), (8, torch.bfloat16, 3)])
def test_bwd_fewer_state_entries(N, dt, conv_k):
    """N < 16: the library pads the per-entry tensors to 16 entries (B = C = 0 there) in
    its workspace and copies dA, dB, dC and dh0 back; every gradient against the oracle
    at that N, with softplus, h0, a final-state gradient and a ragged length."""
    print("case N=%d %s K=%d" % (N, dt, conv_k), flush=True)
    B, L, D = 2, 77, 37
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=640 + N, device=DEV, h0=True,
                             conv_k=conv_k)
    g0 = torch.Generator(DEV).manual_seed(9)
    inp["delta"] = (torch.randn(inp["delta"].shape, device=DEV, generator=g0) - 1.0).to(dt)
    bias = 0.3 * torch.randn(D, device=DEV, generator=g0)
    dhf = torch.randn(B, D, N, device=DEV, generator=g0)
    dy = torch.randn(inp["x"].shape, device=DEV, generator=g0).to(dt)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias, delta_softplus=True,
                               h0=inp["h0"], dh_final=dhf, conv_w=inp["conv_w"])
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]),
                                    to64(inp["Bm"]), to64(inp["Cm"]), to64(dy),
                                    Dskip=to64(inp["Dskip"]), z=to64(inp["z"]),
                                    delta_bias=to64(bias), delta_softplus=True,
                                    h0=to64(inp["h0"]), dh_final=to64(dhf),
                                    conv_w=to64(inp["conv_w"]))
    _check_all(g, ref, dt)


@pytest.mark.parametrize("B,L,D,K,dt", [(2, 70, 40, 4, torch.float32), (1, 300, 70, 3, torch.bfloat16),
                                        (2, 2, 33, 4, torch.float32), (1, 600, 24, 2, torch.bfloat16)])
def test_bwd_with_entering_conv_state(B, L, D, K, dt):
    """A conv state entering the sequence (the forward's conv_state_in): read at negative
    times by the recompute and the conv's transpose, which also gives its gradient;
    including a sequence shorter than the state and one over several conv chunks."""
    print("conv state case", B, L, D, K, dt, flush=True)
    inp = W.make_scan_inputs(B, L, D, 16, io_dtype=dt, seed=660 + L + K, device=DEV, conv_k=K, h0=True)
    g0 = torch.Generator(DEV).manual_seed(10)
    cs = torch.randn(B, K - 1, D, device=DEV, generator=g0).to(dt)
    dy = torch.randn(inp["x"].shape, device=DEV, generator=g0).to(dt)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], h0=inp["h0"], conv_w=inp["conv_w"],
                               conv_state_in=cs)
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]),
                                    to64(inp["Bm"]), to64(inp["Cm"]), to64(dy),
                                    Dskip=to64(inp["Dskip"]), z=to64(inp["z"]), h0=to64(inp["h0"]),
                                    conv_w=to64(inp["conv_w"]), conv_state_in=to64(cs))
    assert "dconv_state_in" in ref
    _check_all(g, ref, dt)


def test_bwd_chained_chunks_equal_one_pass():
    """Training on a sequence cut into two calls: the second call's dh0 is the first
    call's dh_final and its dconv_state_in adds to the first call's dx on its last K-1
    rows; the chained gradients equal one backward pass over the whole sequence."""
    B, L1, L2, D, K = 2, 150, 113, 48, 4
    dt = torch.float32
    inp = W.make_scan_inputs(B, L1 + L2, D, 16, io_dtype=dt, seed=680, device=DEV, conv_k=K, h0=True)
    dy = torch.randn(inp["x"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(11))
    kw = dict(Dskip=inp["Dskip"], conv_w=inp["conv_w"])
    cut = lambda t, a, b: t[:, a:b].contiguous()
    full = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                                  z=inp["z"], h0=inp["h0"], **kw)
    # forward of part 1 for the state and the conv state entering part 2
    _, h1, cs1 = ssm.selective_scan_fwd(cut(inp["x"], 0, L1), cut(inp["delta"], 0, L1), inp["A"],
                                        cut(inp["Bm"], 0, L1), cut(inp["Cm"], 0, L1), z=cut(inp["z"], 0, L1),
                                        h0=inp["h0"], return_final_state=True, return_conv_state=True,
                                        **kw)
    g2 = ssm.selective_scan_bwd(cut(inp["x"], L1, L1 + L2), cut(inp["delta"], L1, L1 + L2), inp["A"],
                                cut(inp["Bm"], L1, L1 + L2), cut(inp["Cm"], L1, L1 + L2),
                                cut(dy, L1, L1 + L2), z=cut(inp["z"], L1, L1 + L2), h0=h1,
                                conv_state_in=cs1, **kw)
    g1 = ssm.selective_scan_bwd(cut(inp["x"], 0, L1), cut(inp["delta"], 0, L1), inp["A"],
                                cut(inp["Bm"], 0, L1), cut(inp["Cm"], 0, L1), cut(dy, 0, L1),
                                z=cut(inp["z"], 0, L1), h0=inp["h0"], dh_final=g2["dh0"], **kw)
    torch.cuda.synchronize()
    dx = torch.cat([g1["dx"], g2["dx"]], 1)
    dx[:, L1 - (K - 1):L1] += g2["dconv_state_in"]
    chained = dict(dx=dx, ddelta=torch.cat([g1["ddelta"], g2["ddelta"]], 1),
                   dz=torch.cat([g1["dz"], g2["dz"]], 1), dh0=g1["dh0"],
                   dBm=torch.cat([g1["dBm"], g2["dBm"]], 1), dCm=torch.cat([g1["dCm"], g2["dCm"]], 1),
                   dA=g1["dA"] + g2["dA"], dDskip=g1["dDskip"] + g2["dDskip"],
                   dconv_w=g1["dconv_w"] + g2["dconv_w"])
    for k, v in chained.items():
        r = to64(full[k])
        if k in PER_ELEM:
            _check(k, to64(v), r, TOL[dt])
        else:
            _check(k, to64(v), r, TOL_SUM[dt], float(np.mean(np.abs(r))))


def test_bwd_empty_sequence_conv_state_gradient_is_zero():
    inp = W.make_scan_inputs(2, 0, 32, 16, io_dtype=torch.bfloat16, seed=534, device=DEV, conv_k=4)
    cs = torch.randn(2, 3, 32, device=DEV).to(torch.bfloat16)
    dy = torch.empty_like(inp["x"])
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                               Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"], conv_state_in=cs)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dconv_state_in"]) == 0 and g["dconv_state_in"].shape == cs.shape
