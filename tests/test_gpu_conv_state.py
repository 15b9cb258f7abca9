"""Parity of the conv state carried between calls (needs an MI355X).

The prefill -> decode handoff of the conv window: a scan may enter with the
K-1 inputs before t = 0 and returns the last K-1 inputs; a decode step runs
the conv prologue on (window, x) and shifts the window in place.  Outputs are
compared with the fp64 oracle on the same input bits; the conv states are raw
copies of inputs and must match exactly.
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


def _inputs(B, L, D, N, K, dt, seed):
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=seed, device=DEV, conv_k=K, h0=True)
    g = torch.Generator(DEV).manual_seed(seed + 1)
    inp["conv_b"] = torch.randn(D, device=DEV, generator=g)
    inp["cs"] = torch.randn(B, K - 1, D, device=DEV, generator=g).to(dt)
    return inp


def _oracle(inp, cs_in):
    return oracle.selective_scan(
        to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]), to64(inp["Cm"]),
        Dskip=to64(inp["Dskip"]), z=to64(inp["z"]), conv_w=to64(inp["conv_w"]),
        conv_b=to64(inp["conv_b"]), h0=to64(inp["h0"]), conv_state_in=to64(cs_in),
        return_conv_state=True)


def _scan(inp, cs_in, cs_out=None):
    return ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                  Dskip=inp["Dskip"], z=inp["z"], conv_w=inp["conv_w"],
                                  conv_b=inp["conv_b"], h0=inp["h0"], return_final_state=True,
                                  conv_state_in=cs_in, conv_state_out=cs_out,
                                  return_conv_state=True)


SCAN_CASES = [
    # name, B, L, D, N, K, dtype
    ("vec_bf16", 2, 37, 130, 16, 4, torch.bfloat16),
    ("short_f32", 1, 2, 70, 16, 4, torch.float32),      # L < K-1: the window reaches back
    ("elem_n5_f32", 2, 50, 33, 5, 3, torch.float32),
    ("k2_bf16", 2, 1, 64, 16, 2, torch.bfloat16),
    ("segments_bf16", 1, 5000, 24, 16, 4, torch.bfloat16),
]


@pytest.mark.parametrize("name,B,L,D,N,K,dt", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_with_conv_state_matches_oracle(name, B, L, D, N, K, dt):
    print("case", name, flush=True)
    inp = _inputs(B, L, D, N, K, dt, seed=300 + L + D)
    for cs_in in (inp["cs"], None):
        y, hf, cs = _scan(inp, cs_in)
        torch.cuda.synchronize()
        yr, hr, csr = _oracle(inp, cs_in)
        assert_close(to64(y), yr, TOL[dt], "y")
        assert_close(to64(hf), hr, TOL[dt], "h_final")
        assert np.array_equal(to64(cs), csr), "conv_state_out"


def test_scan_conv_state_in_place():
    inp = _inputs(2, 20, 96, 16, 4, torch.bfloat16, seed=311)
    cs = inp["cs"].clone()
    y, hf, out = _scan(inp, cs, cs_out=cs)
    torch.cuda.synchronize()
    assert out.data_ptr() == cs.data_ptr()
    yr, hr, csr = _oracle(inp, inp["cs"])
    assert_close(to64(y), yr, TOL[torch.bfloat16], "y")
    assert np.array_equal(to64(cs), csr)


def test_scan_empty_sequence_passes_conv_state_on():
    inp = _inputs(2, 0, 40, 16, 4, torch.float32, seed=312)
    _, hf, cs = _scan(inp, inp["cs"])
    torch.cuda.synchronize()
    assert torch.equal(cs, inp["cs"]) and torch.equal(hf, inp["h0"])
    _, _, cs = _scan(inp, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(cs) == 0


def _decode_inputs(B, D, N, K, steps, dt, seed):
    inp = W.make_decode_inputs(B, D, N, steps, io_dtype=dt, seed=seed, device=DEV)
    g = torch.Generator(DEV).manual_seed(seed + 7)
    inp["conv_w"] = 0.5 * torch.randn(D, K, device=DEV, generator=g)
    inp["conv_b"] = torch.randn(D, device=DEV, generator=g)
    inp["cs0"] = torch.randn(B, K - 1, D, device=DEV, generator=g).to(dt)
    return inp


@pytest.mark.parametrize("B,D,N,K,dt", [(3, 70, 16, 4, torch.float32),
                                        (2, 64, 5, 4, torch.bfloat16),
                                        (2, 33, 16, 2, torch.bfloat16),
                                        (1, 5, 16, 1, torch.float32)])
def test_decode_with_conv_state_matches_oracle(B, D, N, K, dt):
    print("decode", B, D, N, K, dt, flush=True)
    steps = 8
    inp = _decode_inputs(B, D, N, K, steps, dt, seed=B + D + N + K)
    st, cs = inp["state0"].clone(), inp["cs0"].clone()
    ys = []
    for t in range(steps):
        ys.append(ssm.state_update(st, inp["x"][t], inp["delta"][t], inp["A"], inp["Bm"][t],
                                   inp["Cm"][t], Dskip=inp["Dskip"], z=inp["z"][t],
                                   conv_w=inp["conv_w"], conv_b=inp["conv_b"],
                                   conv_state=cs if K > 1 else None))
    torch.cuda.synchronize()
    ref, csr = inp["state0"].double().cpu().numpy(), to64(inp["cs0"])
    for t in range(steps):
        yr, ref, csr = oracle.state_update(ref, to64(inp["x"][t]), to64(inp["delta"][t]),
                                           to64(inp["A"]), to64(inp["Bm"][t]), to64(inp["Cm"][t]),
                                           Dskip=to64(inp["Dskip"]), z=to64(inp["z"][t]),
                                           conv_w=to64(inp["conv_w"]), conv_b=to64(inp["conv_b"]),
                                           conv_state=csr)
        assert_close(to64(ys[t]), yr, TOL[dt], "y step %d" % t)
    assert_close(to64(st), ref, TOL[dt], "state")
    assert np.array_equal(to64(cs), csr), "conv_state"


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_prefill_hands_over_to_decode(dt):
    """A prefill of L1 tokens returns (h, conv state); decoding the next tokens from
    them reproduces one scan over the whole sequence."""
    B, L1, T, D, N, K = 2, 37, 12, 130, 16, 4
    inp = _inputs(B, L1 + T, D, N, K, dt, seed=320)
    pre = {k: (v[:, :L1].contiguous() if k in ("x", "delta", "Bm", "Cm", "z") else v)
           for k, v in inp.items()}
    _, hf, cs = _scan(pre, inp["cs"])
    ys = []
    for t in range(T):
        s = L1 + t
        ys.append(ssm.state_update(hf, inp["x"][:, s].contiguous(), inp["delta"][:, s].contiguous(),
                                   inp["A"], inp["Bm"][:, s].contiguous(), inp["Cm"][:, s].contiguous(),
                                   Dskip=inp["Dskip"], z=inp["z"][:, s].contiguous(),
                                   conv_w=inp["conv_w"], conv_b=inp["conv_b"], conv_state=cs))
    torch.cuda.synchronize()
    yr, hr, csr = _oracle(inp, inp["cs"])
    for t in range(T):
        assert_close(to64(ys[t]), yr[:, L1 + t], TOL[dt], "y token %d" % (L1 + t))
    assert_close(to64(hf), hr, TOL[dt], "state")
    assert np.array_equal(to64(cs), csr)
