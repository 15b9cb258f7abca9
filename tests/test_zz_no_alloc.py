"""The no-allocation scan (ssm_selective_scan_fwd_noalloc) against the scan with a
caller workspace (needs an MI355X).

For callers that cannot allocate device memory the library runs the same scan
with its workspace in a fixed device array it owns.  Both entry points run the
same kernels on the same launch plan, so their outputs must agree bit for bit;
they are also held to the bf16 tolerance of the scan.  The array keeps the
last call's contents, so the calls run back to back with shapes that need a
workspace, the second smaller than the first, and again in the other order.
"""
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (B, L, D, conv_k): few channels over a long row, so the sequence is cut into
# segments whose records live in the workspace.
BIG = (1, 40000, 256, 4)
SMALL = (1, 9000, 64, 0)


def _inputs(B, L, D, K, seed):
    return W.make_scan_inputs(B, L, D, 16, io_dtype=torch.bfloat16, seed=seed, device=DEV,
                              conv_k=K, h0=True)


def _with_workspace(inp):
    return ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                  Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"],
                                  h0=inp["h0"], return_final_state=True)


def _no_alloc(inp):
    y = torch.empty_like(inp["x"])
    hf = torch.empty_like(inp["h0"])
    return ssm.selective_scan_fwd_noalloc(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                          Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"],
                                          h0=inp["h0"], y=y, h_final=hf)


def _compare(got, ref, what):
    for g, r, name in zip(got, ref, ("y", "h_final")):
        assert torch.equal(g, r), "%s %s differs from the scan with a workspace" % (what, name)
        assert_close(to64(g), to64(r), TOL[torch.bfloat16], "%s %s" % (what, name))


@pytest.mark.parametrize("order", [(BIG, SMALL), (SMALL, BIG)], ids=["big_then_small",
                                                                      "small_then_big"])
def test_no_alloc_scan_matches_scan_with_workspace(order):
    sets = [_inputs(*shape, seed=90 + i) for i, shape in enumerate(order)]
    for shape, inp in zip(order, sets):
        a, _, _ = ssm.selective_scan_args(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                          Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"],
                                          h0=inp["h0"])
        need = ssm.lib().ssm_selective_scan_workspace_size(a)
        print("shape", shape, "workspace bytes", need, flush=True)
        assert 0 < need <= ssm.NOALLOC_SCRATCH_BYTES
    refs = [_with_workspace(inp) for inp in sets]
    torch.cuda.synchronize()
    got = [_no_alloc(inp) for inp in sets]     # two calls in a row on one stream
    torch.cuda.synchronize()
    for shape, g, r in zip(order, got, refs):
        _compare(g, r, "B=%d L=%d D=%d K=%d" % shape)


def test_no_alloc_scan_without_a_workspace_need():
    """Sizes whose plan needs no workspace run the same way."""
    inp = _inputs(4, 300, 512, 0, seed=95)
    ref = _with_workspace(inp)
    got = _no_alloc(inp)
    torch.cuda.synchronize()
    _compare(got, ref, "no-workspace shape")


def test_no_alloc_scan_writes_the_same_checkpoints():
    """The forward's block checkpoints (an output the caller passes) through the
    no-allocation scan equal those of the scan with a workspace, on a segmented row."""
    B, L, D, K = BIG
    inp = _inputs(B, L, D, K, seed=97)
    shape = ssm.checkpoint_shape(B, L, D)
    ck_ref = torch.full(shape, float("nan"), device=DEV)
    ck = torch.full(shape, float("nan"), device=DEV)
    ref = ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                 Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"], h0=inp["h0"],
                                 return_final_state=True, checkpoints=ck_ref)
    y, hf = torch.empty_like(inp["x"]), torch.empty_like(inp["h0"])
    got = ssm.selective_scan_fwd_noalloc(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                         Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"],
                                         h0=inp["h0"], y=y, h_final=hf, checkpoints=ck)
    torch.cuda.synchronize()
    _compare(got, ref, "with checkpoints")
    assert torch.equal(ck, ck_ref)
