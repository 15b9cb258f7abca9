"""The backward pass of a scan too long for one launch (needs an MI355X).

The backward's first pass stores the state entering every 16-step block.  It
runs the forward scan kernel, whose buffer offsets are 32-bit: at D = 5120 in
bf16 the 900000-token sequence takes three launches of at most 419264 rows.
They start on block boundaries, so each launch leaves its final state in the
checkpoint of the next launch's first block, and the next launch starts from
there.  With the conv prologue the first rows of each later launch take their
conv history from the rows before the boundary.  The adjoint then walks all
56250 blocks back from their checkpoints ("Mamba: Linear-Time Sequence
Modeling with Selective State Spaces", sec. 4c: states recomputed in the
backward pass instead of stored).

The gradients must equal those of one uninterrupted recurrence.  The oracle
computes them on six sampled channels over every step: the per-channel ones
(dx, ddelta, dz, dh0 per element; dA and dDskip, sums over time, with the
backward tests' scaled bound).  dB and dC are sums over all 5120 channels and
are checked at normal sizes by the other backward tests.

About 100 GB of device memory (inputs, gradients and the workspace's 18 GB of
checkpoints and 12 GB of dB/dC partial sums); about 110 GB when the forward
writes the checkpoints (with its y) and the backward's workspace holds none.
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

B, L, D, N = 1, 900_000, 5120, 16
MAX_ROW_BYTES = 0xFFF00000


def _rows_per_launch(dim, es):
    r = MAX_ROW_BYTES // (dim * es) - 64
    return r - r % 32


def test_shape_needs_three_checkpoint_launches():
    r = _rows_per_launch(D, 2)
    assert r % 16 == 0 and 2 * r < L <= 3 * r


@pytest.fixture(scope="module")
def long_inputs():
    print("generating B=%d L=%d D=%d bf16 inputs" % (B, L, D), flush=True)
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=torch.bfloat16, seed=61, device=DEV,
                             delta_shift=3.0, conv_k=4, h0=True)
    g = torch.Generator(DEV).manual_seed(62)
    inp["dy"] = torch.randn((B, L, D), device=DEV, generator=g).to(torch.bfloat16)
    inp["dh_final"] = torch.randn((B, D, N), device=DEV, generator=g)
    torch.cuda.synchronize()
    yield inp
    del inp
    torch.cuda.empty_cache()


def _check(name, got, ref, tol, scale=0.0):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    err = np.abs(got - ref) / (1.0 + np.abs(ref) + scale)
    worst = float(err.max()) if err.size else 0.0
    print("  %-8s worst scaled error %.2e (tol %.0e)" % (name, worst, tol), flush=True)
    assert worst <= tol, (name, worst)


@pytest.mark.parametrize("conv,from_fwd", [(False, False), (True, False), (True, True)],
                         ids=["plain", "conv4", "conv4_forward_checkpoints"])
def test_chained_checkpoints_match_one_recurrence(long_inputs, conv, from_fwd):
    """from_fwd: the checkpoints come from the forward (three chained launches,
    each cut into sequence segments at this width) instead of the backward's
    own first pass."""
    inp = long_inputs
    conv_w = inp["conv_w"] if conv else None
    print("case conv=%s from_fwd=%s" % (conv, from_fwd), flush=True)
    ck = None
    if from_fwd:
        ck = torch.empty(ssm.checkpoint_shape(B, L, D), device=DEV)
        ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                               z=inp["z"], h0=inp["h0"], conv_w=conv_w, checkpoints=ck)
    g = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], inp["dy"],
                               Dskip=inp["Dskip"], z=inp["z"], h0=inp["h0"], dh_final=inp["dh_final"],
                               conv_w=conv_w, checkpoints=ck)
    torch.cuda.synchronize()
    del ck
    print("  backward done; oracle on sampled channels", flush=True)
    rng = np.random.default_rng(7 + int(conv))
    ds = rng.choice(D, 6, replace=False)
    ds[0], ds[-1] = 0, D - 1
    dsel = torch.tensor(ds, device=DEV)
    sel = lambda t: to64(t.index_select(2, dsel))
    ref = oracle.selective_scan_bwd(
        sel(inp["x"]), sel(inp["delta"]), to64(inp["A"].index_select(0, dsel)), to64(inp["Bm"]),
        to64(inp["Cm"]), sel(inp["dy"]), Dskip=to64(inp["Dskip"].index_select(0, dsel)), z=sel(inp["z"]),
        conv_w=None if conv_w is None else to64(conv_w.index_select(0, dsel)),
        h0=to64(inp["h0"].index_select(1, dsel)), dh_final=to64(inp["dh_final"].index_select(1, dsel)))
    tol = TOL[torch.bfloat16]
    for name in ("dx", "ddelta", "dz"):
        _check(name, sel(g[name]), ref[name], tol)
    _check("dh0", to64(g["dh0"].index_select(1, dsel)), ref["dh0"], tol)
    for name, got in (("dA", g["dA"].index_select(0, dsel)), ("dDskip", g["dDskip"].index_select(0, dsel))):
        r = ref[name]
        _check(name, to64(got), r, tol, scale=float(np.abs(r).mean()))
    del g
    torch.cuda.empty_cache()
