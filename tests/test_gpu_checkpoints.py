"""The forward -> backward handoff of block checkpoints (needs an MI355X).

Training keeps the forward's states for the backward at a coarse grain: the
state entering every 16-step block ("Mamba: Linear-Time Sequence Modeling with
Selective State Spaces", sec. 3.3 and 4c: states are recomputed in the
backward pass instead of stored per step).  A forward given a checkpoint tensor
writes them beside y; a backward given that tensor reads them instead of
running its own first pass.

Checked here:
  * each checkpoint is the state the oracle reaches after that block's prefix
    (the forward's bound for h_final: |got - ref| <= tol (1 + |ref|)), with
    the entries past N zero;
  * gradients from the forward's checkpoints equal those of a backward that
    computes its own, bit for bit where the forward ran the same kernel path
    (N = 16, one unsegmented launch), and within the backward's bound
    otherwise (N < 16, and a long row the forward splits into segments,
    whose checkpoints past each segment's head are the zero-start states).
"""
import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from selective_state_space_59_amd.ssm import SCAN_BLOCK as BLK
from selective_state_space_59_amd.ssm import _scan_args
from tests.gpu_helpers import TOL, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, L, D, N, dt, seed, conv, h0=True):
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=seed, device=DEV, conv_k=4 if conv else 0,
                             h0=h0)
    g = torch.Generator(DEV).manual_seed(seed + 100)
    inp["dy"] = torch.randn((B, L, D), device=DEV, generator=g).to(dt)
    inp["dh_final"] = torch.randn((B, D, N), device=DEV, generator=g)
    return inp


def _fwd(inp, softplus=False, bias=None):
    B, L, D = inp["x"].shape
    ck = torch.full(ssm.checkpoint_shape(B, L, D), float("nan"), device=DEV)
    y, hf = ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                   Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias,
                                   delta_softplus=softplus, conv_w=inp["conv_w"], h0=inp["h0"],
                                   return_final_state=True, checkpoints=ck)
    return y, hf, ck


def _bwd(inp, ck, softplus=False, bias=None):
    return ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"],
                                  Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias,
                                  delta_softplus=softplus, h0=inp["h0"], dh_final=inp["dh_final"],
                                  conv_w=inp["conv_w"], checkpoints=ck)


def _prefix_state(inp, t, softplus=False, bias=None):
    """The oracle's state after the first t steps (h0 for t = 0)."""
    B, L, D = inp["x"].shape
    N = inp["A"].shape[1]
    if t == 0:
        return to64(inp["h0"]) if inp["h0"] is not None else np.zeros((B, D, N))
    cut = lambda k: to64(inp[k][:, :t])
    _, hf = oracle.selective_scan(cut("x"), cut("delta"), to64(inp["A"]), cut("Bm"), cut("Cm"),
                                  delta_bias=to64(bias), delta_softplus=softplus,
                                  conv_w=to64(inp["conv_w"]), h0=to64(inp["h0"]))
    return hf


def _close(name, got, ref, tol, scale=0.0):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref) / (1.0 + np.abs(ref) + scale)
    worst = float(err.max()) if err.size else 0.0
    print("  %-12s worst scaled error %.2e (tol %.0e)" % (name, worst, tol), flush=True)
    assert worst <= tol, (name, worst)


CASES = [
    # name, B, L, D, N, dtype, conv, softplus (h0 is given except in the last case)
    ("bf16_vec", 2, 77, 64, 16, torch.bfloat16, False, False),
    ("bf16_vec_conv", 2, 100, 48, 16, torch.bfloat16, True, True),
    ("f32_vec", 1, 64, 40, 16, torch.float32, False, True),
    ("f32_elem_conv", 2, 45, 37, 16, torch.float32, True, False),
    ("bf16_N5_conv", 1, 50, 24, 5, torch.bfloat16, True, False),
    ("f32_N1", 2, 33, 20, 1, torch.float32, False, False),
    ("bf16_no_h0", 3, 40, 32, 16, torch.bfloat16, True, False),
]


@pytest.mark.parametrize("name,B,L,D,N,dt,conv,softplus", CASES, ids=[c[0] for c in CASES])
def test_checkpoints_are_the_prefix_states(name, B, L, D, N, dt, conv, softplus):
    print("case %s" % name, flush=True)
    inp = _inputs(B, L, D, N, dt, seed=71, conv=conv, h0=not name.endswith("no_h0"))
    bias = torch.randn(D, device=DEV, generator=torch.Generator(DEV).manual_seed(3)) if softplus else None
    y, hf, ck = _fwd(inp, softplus, bias)
    torch.cuda.synchronize()
    c = to64(ck)
    assert c.shape == ((L + BLK - 1) // BLK, B, D, 16)
    assert np.all(c[..., N:] == 0.0), "entries past N must be zero"
    tol = TOL[dt]
    for j in range(c.shape[0]):
        _close("ckpt[%d]" % j, c[j, ..., :N], _prefix_state(inp, j * BLK, softplus, bias), tol)
    # y and h_final are those of a forward without checkpoints
    y2, hf2 = ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                     Dskip=inp["Dskip"], z=inp["z"], delta_bias=bias,
                                     delta_softplus=softplus, conv_w=inp["conv_w"], h0=inp["h0"],
                                     return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(hf, hf2)


GRADS = ("dx", "ddelta", "dz", "dA", "dBm", "dCm", "dDskip", "ddelta_bias", "dh0", "dconv_w",
         "dconv_b")


@pytest.mark.parametrize("name,B,L,D,N,dt,conv,softplus", CASES, ids=[c[0] for c in CASES])
def test_backward_from_forward_checkpoints(name, B, L, D, N, dt, conv, softplus):
    print("case %s" % name, flush=True)
    inp = _inputs(B, L, D, N, dt, seed=73, conv=conv, h0=not name.endswith("no_h0"))
    bias = torch.randn(D, device=DEV, generator=torch.Generator(DEV).manual_seed(4)) if softplus else None
    _, _, ck = _fwd(inp, softplus, bias)
    g1 = _bwd(inp, ck, softplus, bias)
    g0 = _bwd(inp, None, softplus, bias)
    torch.cuda.synchronize()
    assert set(g1) == set(g0)
    if N == 16:
        for k in g0:
            assert torch.equal(g1[k], g0[k]), k
        return
    ref = oracle.selective_scan_bwd(
        to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]), to64(inp["Cm"]),
        to64(inp["dy"]), Dskip=to64(inp["Dskip"]), z=to64(inp["z"]), delta_bias=to64(bias),
        delta_softplus=softplus, h0=to64(inp["h0"]), dh_final=to64(inp["dh_final"]),
        conv_w=to64(inp["conv_w"]))
    tol = TOL[dt]
    for k in GRADS:
        if k not in g1:
            continue
        r = ref[k]
        scale = 0.0 if k in ("dx", "ddelta", "dz", "dh0") else float(np.abs(r).mean())
        _close(k, to64(g1[k]), r, tol, scale)


def test_segmented_forward_checkpoints():
    """One long row: the forward scans it in segments at once.  Its checkpoints
    are the true states up to each segment's head and the zero-start ones after
    it (equal to the true ones up to a 2^-160 share of the entering state)."""
    B, L, D, N = 1, 20000, 64, 16
    dt = torch.bfloat16
    inp = _inputs(B, L, D, N, dt, seed=79, conv=True)
    a, _ = _scan_args(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], None, None, None, False,
                      inp["conv_w"], None, inp["h0"], torch.empty_like(inp["x"]), None)
    assert ssm.lib().ssm_selective_scan_workspace_size(ctypes.byref(a)) > 0, "expected segments"
    _, hf, ck = _fwd(inp)
    g1 = _bwd(inp, ck)
    torch.cuda.synchronize()
    c = to64(ck)
    tol = TOL[dt]
    nblk = c.shape[0]
    rng = np.random.default_rng(5)
    js = sorted(set([0, 1, nblk - 1] + [int(v) for v in rng.choice(nblk, 9, replace=False)]))
    for j in js:
        _close("ckpt[%d]" % j, c[j], _prefix_state(inp, j * BLK), tol)
    ref = oracle.selective_scan_bwd(
        to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]), to64(inp["Cm"]),
        to64(inp["dy"]), Dskip=to64(inp["Dskip"]), z=to64(inp["z"]), h0=to64(inp["h0"]),
        dh_final=to64(inp["dh_final"]), conv_w=to64(inp["conv_w"]))
    for k in GRADS:
        if k not in g1:
            continue
        r = ref[k]
        scale = 0.0 if k in ("dx", "ddelta", "dz", "dh0") else float(np.abs(r).mean())
        _close(k, to64(g1[k]), r, tol, scale)
