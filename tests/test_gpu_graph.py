"""The entry points under HIP graph capture (needs an MI355X).

A serving loop captures its launches once and replays them.  Every call here
is captured into a torch CUDA graph (on ROCm a HIP graph) after an eager
warm-up, then replayed several times with eager work and synchronisations in
between; each replay must give exactly the bits of the same call run eagerly.
The library issues no memsets, allocations or synchronisations inside its
calls, so its launches record as plain kernel nodes.  A workspace the binding
needs during a capture is a fresh tensor from the graph's own memory pool,
never the binding's cached one.
"""
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # eager warm-up on a side stream (library load, plan and GEMM set-up)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _scramble(*ts):
    for t in ts:
        t.fill_(float("nan")) if t.is_floating_point() else t.zero_()


@pytest.mark.parametrize("name,B,L,D,conv_k", [
    ("c2_like_small", 2, 300, 256, 0),
    ("segmented_long_conv", 1, 20000, 64, 4),   # workspace, three launches
])
def test_scan_replays_match_eager(name, B, L, D, conv_k):
    inp = W.make_scan_inputs(B, L, D, 16, io_dtype=torch.bfloat16, seed=41, device=DEV,
                             conv_k=conv_k, h0=True)
    y = torch.empty_like(inp["x"])
    hf = torch.empty(B, D, 16, device=DEV)

    def call():
        ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                               Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"], h0=inp["h0"],
                               y=y, h_final=hf)

    call()
    torch.cuda.synchronize()
    ref_y, ref_h = y.clone(), hf.clone()
    g = _capture(call)
    for _ in range(REPLAYS):
        _scramble(y, hf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(hf, ref_h), name


def test_decode_step_replays_advance_the_state_like_eager_steps():
    inp = W.make_decode_inputs(8, 300, 16, 1, io_dtype=torch.bfloat16, seed=42, device=DEV)
    st = inp["state0"].clone()
    y = torch.empty_like(inp["x"][0])
    args = (inp["x"][0], inp["delta"][0], inp["A"], inp["Bm"][0], inp["Cm"][0])

    def call(state, out):
        ssm.state_update(state, *args, Dskip=inp["Dskip"], z=inp["z"][0], y=out)

    g = _capture(lambda: call(st, y))   # the warm-up advances st one step; capture runs nothing
    ref = inp["state0"].clone()
    ref_y = torch.empty_like(y)
    call(ref, ref_y)
    torch.cuda.synchronize()
    assert torch.equal(st, ref)
    for _ in range(REPLAYS):
        call(ref, ref_y)                    # the eager twin of the next replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st, ref) and torch.equal(y, ref_y)


def test_ssd_step_replays_advance_the_state_like_eager_steps():
    inp = W.make_ssd_inputs(4, 1, 6, 64, 2, 128, seed=43, device=DEV, h0=True)
    one = lambda k: inp[k][:, 0].contiguous()
    x, dt, Bm, Cm, z = (one(k) for k in ("x", "delta", "Bm", "Cm", "z"))
    st = inp["h0"].clone()
    y = torch.empty_like(x)

    def call(state, out):
        ssm.ssd_step(state, x, dt, inp["A"], Bm, Cm, Dskip=inp["Dskip"], z=z, y=out)

    g = _capture(lambda: call(st, y))   # the warm-up advances st one step
    ref = inp["h0"].clone()
    ref_y = torch.empty_like(y)
    call(ref, ref_y)
    torch.cuda.synchronize()
    assert torch.equal(st, ref)
    for _ in range(REPLAYS):
        call(ref, ref_y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st, ref) and torch.equal(y, ref_y)


@pytest.mark.parametrize("name,B,L", [("one_pass", 2, 300), ("segmented", 1, 8192)])
def test_ssd_replays_match_eager(name, B, L):
    inp = W.make_ssd_inputs(B, L, 4, 64, 1, 128, seed=44, device=DEV, h0=True)
    y = torch.empty_like(inp["x"])
    hf = torch.empty_like(inp["h0"])

    def call():
        ssm.ssd_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                    z=inp["z"], h0=inp["h0"], y=y, h_final=hf)

    call()
    torch.cuda.synchronize()
    ref_y, ref_h = y.clone(), hf.clone()
    g = _capture(call)
    for _ in range(REPLAYS):
        _scramble(y, hf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(hf, ref_h), name


def test_backward_replays_match_eager():
    inp = W.make_scan_inputs(2, 200, 96, 16, io_dtype=torch.bfloat16, seed=45, device=DEV, h0=True)
    dy = torch.randn(inp["x"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(46))
    dy = dy.to(torch.bfloat16)
    out = {}

    def call():
        out["g"] = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy,
                                          Dskip=inp["Dskip"], z=inp["z"], h0=inp["h0"])

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out["g"].items() if v is not None}
    g = _capture(call)
    got = out["g"]  # the tensors the captured launches write
    for _ in range(REPLAYS):
        for v in got.values():
            if v is not None:
                _scramble(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(got[k], v), k


def test_block_replays_match_eager():
    """The Mamba block, hipBLASLt GEMMs included, with its plan and workspace made before the
    capture."""
    B, L, dm, D, N, R, K = 2, 100, 128, 256, 16, 8, 4
    inp = W.make_block_inputs(B, L, dm, D, N, R, K, seed=47, device=DEV)
    plan = ssm.BlockPlan(B, L, dm, D, N, R, K)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(inp["h"])
    names = ("norm_w", "w_in", "conv_w", "conv_b", "w_x", "w_dt", "dt_bias", "A", "Dskip", "w_out")

    def call():
        ssm.mamba_block_fwd(inp["h"], *(inp[k] for k in names), eps=1e-5, out=out, plan=plan,
                            workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(call)
    for _ in range(REPLAYS):
        _scramble(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    del g
    plan.close()
