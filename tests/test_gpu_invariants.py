"""Invariants of the HIP path that hold at any size (needs an MI355X).

- resuming from a final state: scan[0,L) == scan[0,s) then scan[s,L) from h_final
- decode steps reproduce a scan over the same tokens
- the fused conv prologue equals the standalone conv kernel followed by the scan
- repeated runs are bit-identical (no order-dependent reductions)
"""
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def scan(inp, h0=None, sl=slice(None), final=True, conv=True):
    cut = lambda t: None if t is None else t[:, sl].contiguous()
    return ssm.selective_scan_fwd(cut(inp["x"]), cut(inp["delta"]), inp["A"], cut(inp["Bm"]),
                                  cut(inp["Cm"]), Dskip=inp["Dskip"], z=cut(inp["z"]),
                                  conv_w=inp["conv_w"] if conv else None, h0=h0,
                                  return_final_state=final)


@pytest.mark.parametrize("dt,split", [(torch.float32, 37), (torch.bfloat16, 1000)])
def test_resume_from_final_state(dt, split):
    inp = W.make_scan_inputs(2, 2100, 130, 16, io_dtype=dt, seed=21, device=DEV, h0=True)
    y, hf = scan(inp, h0=inp["h0"])
    y1, h1 = scan(inp, h0=inp["h0"], sl=slice(0, split))
    y2, h2 = scan(inp, h0=h1, sl=slice(split, None))
    torch.cuda.synchronize()
    tol = 1e-5 if dt == torch.float32 else 1e-2
    assert_close(to64(torch.cat([y1, y2], 1)), to64(y), tol, "y")
    assert_close(to64(h2), to64(hf), 1e-5, "h_final")


def test_decode_steps_equal_scan():
    B, L, D, N = 3, 64, 96, 16
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=torch.bfloat16, seed=22, device=DEV, h0=True)
    y, hf = scan(inp, h0=inp["h0"])
    st = inp["h0"].clone()
    for t in range(L):
        yt = ssm.state_update(st, inp["x"][:, t].contiguous(), inp["delta"][:, t].contiguous(),
                              inp["A"], inp["Bm"][:, t].contiguous(), inp["Cm"][:, t].contiguous(),
                              Dskip=inp["Dskip"], z=inp["z"][:, t].contiguous())
        assert_close(to64(yt), to64(y[:, t]), 1e-2, "y step %d" % t)
    torch.cuda.synchronize()
    assert_close(to64(st), to64(hf), 1e-4, "state")


def test_fused_conv_equals_conv_then_scan():
    inp = W.make_scan_inputs(2, 700, 150, 16, io_dtype=torch.float32, seed=23, device=DEV,
                             conv_k=4)
    y1, h1 = scan(inp)
    u = ssm.causal_conv1d_silu(inp["x"], inp["conv_w"])
    q = dict(inp)
    q["x"] = u
    y2, h2 = scan(q, conv=False)
    torch.cuda.synchronize()
    assert_close(to64(y1), to64(y2), 1e-5, "y")
    assert_close(to64(h1), to64(h2), 1e-5, "h_final")


def test_repeat_runs_are_bit_identical():
    inp = W.make_scan_inputs(2, 3000, 200, 16, io_dtype=torch.bfloat16, seed=24, device=DEV)
    y1, h1 = scan(inp)
    y2, h2 = scan(inp)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_outputs_outside_y_untouched():
    """Write y into the middle of a sentinel-filled buffer: bytes around it must stay."""
    inp = W.make_scan_inputs(1, 257, 65, 16, io_dtype=torch.bfloat16, seed=25, device=DEV)
    n = inp["x"].numel()
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = buf[2048:2048 + n].view(inp["x"].shape)
    ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                           Dskip=inp["Dskip"], z=inp["z"], y=y)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:2048].float()).all() and torch.isnan(buf[2048 + n:].float()).all()
    assert torch.isfinite(y.float()).all()


def test_concurrent_streams_use_separate_workspaces():
    """Two segmented scans (which need the workspace) launched on two streams at once give
    the results of the same calls run one after the other: each stream has its own scratch."""
    ins = [W.make_scan_inputs(1, 12000, 64, 16, io_dtype=torch.bfloat16, seed=60 + k, device=DEV, h0=True)
           for k in range(2)]

    def call(inp):
        return ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                      Dskip=inp["Dskip"], z=inp["z"], h0=inp["h0"], return_final_state=True)

    ref = [call(inp) for inp in ins]
    torch.cuda.synchronize()
    ref = [(y.clone(), h.clone()) for y, h in ref]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        for inp, s in zip(ins, streams):
            with torch.cuda.stream(s):
                outs.append(call(inp))
    torch.cuda.synchronize()
    for i, (y, h) in enumerate(outs):
        assert torch.equal(y, ref[i % 2][0]) and torch.equal(h, ref[i % 2][1]), i
