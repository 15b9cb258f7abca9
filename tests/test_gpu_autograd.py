"""The scan as a differentiable torch op (needs an MI355X).

selective_scan() runs the forward writing the block checkpoints and, under
backward(), the backward from them.  Its gradients must be those of
selective_scan_bwd called directly on the same inputs (bit for bit: the same
kernels; B and C gradients cast to their input dtype by autograd), and, in
fp32, those of the oracle within the backward's bound.
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
NAMES = ("x", "delta", "A", "Bm", "Cm", "Dskip", "z", "delta_bias", "h0", "conv_w")
GRAD_KEY = dict(x="dx", delta="ddelta", A="dA", Bm="dBm", Cm="dCm", Dskip="dDskip", z="dz",
                delta_bias="ddelta_bias", h0="dh0", conv_w="dconv_w")


def _case(dt, conv, softplus, seed):
    B, L, D, N = 2, 100, 32, 16
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=seed, device=DEV, conv_k=4 if conv else 0, h0=True)
    g = torch.Generator(DEV).manual_seed(seed + 1)
    inp["delta_bias"] = 0.1 * torch.randn(D, device=DEV, generator=g) if softplus else None
    dy = torch.randn(B, L, D, device=DEV, generator=g).to(dt)
    dhf = torch.randn(B, D, N, device=DEV, generator=g)
    return inp, dy, dhf


@pytest.mark.parametrize("dt,conv,softplus", [(torch.bfloat16, False, False), (torch.bfloat16, True, True),
                                              (torch.float32, True, False)],
                         ids=["bf16", "bf16_conv_softplus", "f32_conv"])
def test_autograd_matches_the_direct_backward(dt, conv, softplus):
    inp, dy, dhf = _case(dt, conv, softplus, seed=31)
    leaves = {k: inp[k].detach().clone().requires_grad_(True) for k in NAMES if inp.get(k) is not None}
    y, hf = ssm.selective_scan(leaves["x"], leaves["delta"], leaves["A"], leaves["Bm"], leaves["Cm"],
                               Dskip=leaves["Dskip"], z=leaves["z"], delta_bias=leaves.get("delta_bias"),
                               delta_softplus=softplus, h0=leaves["h0"], conv_w=leaves.get("conv_w"))
    torch.autograd.backward([y, hf], [dy, dhf])
    torch.cuda.synchronize()
    ref = ssm.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], dy, Dskip=inp["Dskip"],
                                 z=inp["z"], delta_bias=inp.get("delta_bias"), delta_softplus=softplus,
                                 h0=inp["h0"], dh_final=dhf, conv_w=inp.get("conv_w"))
    y2, hf2 = ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                                     z=inp["z"], delta_bias=inp.get("delta_bias"), delta_softplus=softplus,
                                     h0=inp["h0"], conv_w=inp.get("conv_w"), return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(hf, hf2)
    for k, leaf in leaves.items():
        want = ref[GRAD_KEY[k]].to(leaf.dtype)
        assert leaf.grad is not None, k
        assert torch.equal(leaf.grad, want), k


def test_autograd_fp32_against_the_oracle():
    inp, dy, dhf = _case(torch.float32, False, True, seed=37)
    leaves = {k: inp[k].detach().clone().requires_grad_(True) for k in NAMES if inp.get(k) is not None}
    y, hf = ssm.selective_scan(leaves["x"], leaves["delta"], leaves["A"], leaves["Bm"], leaves["Cm"],
                               Dskip=leaves["Dskip"], z=leaves["z"], delta_bias=leaves["delta_bias"],
                               delta_softplus=True, h0=leaves["h0"])
    torch.autograd.backward([y, hf], [dy, dhf])
    torch.cuda.synchronize()
    ref = oracle.selective_scan_bwd(
        to64(inp["x"]), to64(inp["delta"]), to64(inp["A"]), to64(inp["Bm"]), to64(inp["Cm"]), to64(dy),
        Dskip=to64(inp["Dskip"]), z=to64(inp["z"]), delta_bias=to64(inp["delta_bias"]), delta_softplus=True,
        h0=to64(inp["h0"]), dh_final=to64(dhf))
    tol = TOL[torch.float32]
    for k, leaf in leaves.items():
        r = ref[GRAD_KEY[k]]
        got = to64(leaf.grad)
        scale = 0.0 if k in ("x", "delta", "z", "h0") else float(np.abs(r).mean())
        err = np.abs(got - r) / (1.0 + np.abs(r) + scale)
        print("  %-10s worst scaled error %.2e" % (k, float(err.max())), flush=True)
        assert float(err.max()) <= tol, k
