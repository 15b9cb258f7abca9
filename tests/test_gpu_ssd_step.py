"""Parity of the SSD decode step (ssm_ssd_step) against the fp64 oracle (needs an MI355X).

A run of T decode steps on a state must equal the recurrent SSD layer over the
same T tokens started from that state: each step's y against the oracle's y at
that position (bf16 bound 1e-2 (1 + |ref|)), the state after T steps against
the oracle's final state (fp32 bound 1e-4 (1 + |ref|): the state never leaves
fp32 on the GPU).  A prefill by ssm_ssd_fwd followed by decode steps must
match the oracle over the whole sequence.
"""
import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16 = TOL[torch.bfloat16]
TOL_F32 = TOL[torch.float32]


def _steps(inp, state, softplus=False, bias=None, t0=0):
    """Decode tokens t0.. of `inp` one at a time on `state` (in place); returns y (B, T, H, P)."""
    T = inp["x"].shape[1]
    per_step = lambda t: None if t is None else t.transpose(0, 1).contiguous()
    xs, ds, bs, cs, zs = (per_step(inp[k]) for k in ("x", "delta", "Bm", "Cm", "z"))
    ys = []
    for t in range(t0, T):
        ys.append(ssm.ssd_step(state, xs[t], ds[t], inp["A"], bs[t], cs[t], Dskip=inp["Dskip"],
                               z=None if zs is None else zs[t], delta_bias=bias,
                               delta_softplus=softplus))
    torch.cuda.synchronize()
    return torch.stack(ys, 1)


def _oracle(inp, softplus=False, bias=None, b=slice(None)):
    sel = lambda k: None if inp[k] is None else to64(inp[k][b])
    return oracle.ssd(sel("x"), sel("delta"), to64(inp["A"]), sel("Bm"), sel("Cm"),
                      Dskip=to64(inp["Dskip"]), z=sel("z"), delta_bias=to64(bias),
                      delta_softplus=softplus, h0=sel("h0"))


CASES = [
    # name, B, T, H, P, G, N, extra
    ("n128_p64", 3, 6, 4, 64, 1, 128, {}),
    ("n16_groups", 2, 5, 6, 64, 3, 16, {}),
    ("n4_one_lane", 2, 4, 3, 16, 1, 4, {}),
    ("n256_full_wave", 1, 3, 2, 32, 2, 256, {}),
    ("ragged_p7_n8", 5, 4, 3, 7, 1, 8, {}),                    # a head is part of one tile
    ("p40_ragged_tile", 2, 3, 3, 40, 1, 128, {}),              # 16-channel tiles, last one ragged
    ("no_gate_no_skip", 2, 5, 2, 64, 1, 64, dict(gate=False, skip=False)),
    ("big_steps", 2, 6, 4, 64, 1, 32, dict(delta_shift=-1.0)),  # large dt: strong decay
]


@pytest.mark.parametrize("name,B,T,H,P,G,N,extra", CASES, ids=[c[0] for c in CASES])
def test_ssd_steps_match_oracle(name, B, T, H, P, G, N, extra):
    print("case", name, flush=True)
    inp = W.make_ssd_inputs(B, T, H, P, G, N, seed=900 + N + P, device=DEV, h0=True, **extra)
    state = inp["h0"].clone()
    y = _steps(inp, state)
    ry, rh = _oracle(inp)
    wy = assert_close(to64(y), ry, TOL_BF16, "y")
    wh = assert_close(to64(state), rh, TOL_F32, "state")
    print("  worst scaled error y %.2e state %.2e" % (wy, wh), flush=True)
    # the state moved: a step that left it alone would fail here
    assert float(np.abs(rh - to64(inp["h0"])).mean()) > 0.05


def test_ssd_step_softplus_bias():
    inp = W.make_ssd_inputs(2, 5, 4, 64, 2, 64, seed=950, device=DEV, h0=True)
    g = torch.Generator(DEV).manual_seed(951)
    # raw (pre-activation) steps and a per-head bias
    inp["delta"] = (torch.randn(inp["delta"].shape, device=DEV, generator=g) - 1.0).to(torch.bfloat16)
    bias = 0.5 * torch.randn(4, device=DEV, generator=g)
    state = inp["h0"].clone()
    y = _steps(inp, state, softplus=True, bias=bias)
    ry, rh = _oracle(inp, softplus=True, bias=bias)
    assert_close(to64(y), ry, TOL_BF16, "y")
    assert_close(to64(state), rh, TOL_F32, "state")


def test_prefill_then_decode_matches_whole_sequence():
    """ssm_ssd_fwd over the first 150 tokens (three chunks, ragged), then 5 decode steps on
    its final state: the oracle runs all 155 tokens in one pass."""
    inp = W.make_ssd_inputs(2, 155, 3, 64, 1, 128, seed=960, device=DEV, h0=True)
    pre = {k: (None if v is None or k in ("A", "Dskip", "h0") else v[:, :150].contiguous())
           for k, v in inp.items()}
    y_pre, h = ssm.ssd_fwd(pre["x"], pre["delta"], inp["A"], pre["Bm"], pre["Cm"],
                           Dskip=inp["Dskip"], z=pre["z"], h0=inp["h0"], return_final_state=True)
    y_dec = _steps(inp, h, t0=150)
    ry, rh = _oracle(inp)
    assert_close(to64(y_pre), ry[:, :150], TOL_BF16, "prefill y")
    assert_close(to64(y_dec), ry[:, 150:], TOL_BF16, "decode y")
    # the handed-over state went through the chunked kernel's bf16 products
    assert_close(to64(h), rh, TOL_BF16, "state")


def test_ssd_step_capped_grid():
    """More (batch, head) tiles than one launch grid holds (2^22 workgroups): each workgroup
    takes further tiles in turn."""
    B = (1 << 22) + 3
    inp = W.make_ssd_inputs(B, 2, 1, 1, 1, 4, seed=970, device=DEV, h0=True)
    state = inp["h0"].clone()
    y = _steps(inp, state)
    ry, rh = _oracle(inp)
    assert_close(to64(y), ry, TOL_BF16, "y")
    assert_close(to64(state), rh, TOL_F32, "state")


def test_ssd_step_empty_batch():
    st = torch.empty(0, 2, 64, 16, device=DEV)
    x = torch.empty(0, 2, 64, device=DEV, dtype=torch.bfloat16)
    y = ssm.ssd_step(st, x, torch.empty(0, 2, device=DEV, dtype=torch.bfloat16),
                     torch.full((2,), -1.0, device=DEV),
                     torch.empty(0, 1, 16, device=DEV, dtype=torch.bfloat16),
                     torch.empty(0, 1, 16, device=DEV, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert y.shape == (0, 2, 64)


def test_ssd_step_2p7b_decode_sampled_rows():
    """The 2.7B-like decode config (256 sequences, 80 heads x 64, N = 128) for its 16 steps
    in full on the GPU; the oracle checks sequences 0, 131 and 255."""
    cfg = W.S5_MAMBA2_DECODE
    print("config", cfg.name, flush=True)
    inp = W.make_ssd_config_inputs(cfg, device=DEV, h0=True)
    state = inp["h0"].clone()
    y = _steps(inp, state)
    for b in (0, 131, 255):
        ry, rh = _oracle(inp, b=slice(b, b + 1))
        wy = assert_close(to64(y[b:b + 1]), ry, TOL_BF16, "y seq %d" % b)
        wh = assert_close(to64(state[b:b + 1]), rh, TOL_F32, "state seq %d" % b)
        print("  seq %d worst scaled error y %.2e state %.2e" % (b, wy, wh), flush=True)
    del inp, state, y
    torch.cuda.empty_cache()
