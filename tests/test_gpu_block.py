"""Parity of the whole Mamba block (ssm_block_fwd) against the fp64 oracle (needs an MI355X).

Two checks per case, both on every element of h_out:

1. Against the block in float64 with no rounding at all, within the tolerance
   that `oracle.mamba_block_error_bound` derives for any implementation that
   stores the block's intermediates in bf16 and computes in fp32: lam = 10
   standard deviations of the first-order rounding error, propagated through
   the block under the probabilistic model of independent roundings, plus the
   bf16 rounding of h_out itself.  This holds whichever intermediates the GPU
   path keeps in bf16 and wherever it rounds them.
2. Against the block rounded to bf16 after each of its operations (the norm,
   in_proj, the conv with its SiLU, x_proj, the step dt = softplus(dt_proj +
   bias), the scan with its gate, out_proj with the residual), at the scan's
   bf16 tolerance |got - ref| <= 1e-2 (1 + |ref|).
"""
import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import ssm as binding
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16 = TOL[torch.bfloat16]
ARGS = ("norm_w", "w_in", "conv_w", "conv_b", "w_x", "w_dt", "dt_bias", "A", "Dskip", "w_out")


def _gpu(inp, out=None):
    return ssm.mamba_block_fwd(inp["h"], *(inp[k] for k in ARGS), eps=1e-5, out=out)


def _oracle(inp, rows=slice(None)):
    return oracle.mamba_block_fwd(to64(inp["h"][rows]), *(to64(inp[k]) for k in ARGS), eps=1e-5)


def _check(got, inp, rows=slice(None), what="h_out"):
    """Both checks of the module docstring; returns (worst |err|/tol against the
    unrounded block, worst scaled error against the rounded block)."""
    ref, tol, _ = oracle.mamba_block_error_bound(to64(inp["h"][rows]),
                                                 *(to64(inp[k]) for k in ARGS), eps=1e-5)
    err = np.abs(got - ref)
    ratio = float((err / tol).max())
    if ratio > 1.0:
        i = np.unravel_index(int((err / tol).argmax()), err.shape)
        raise AssertionError("%s: |err| %.3e > tol %.3e at %s (got %r, unrounded ref %r)"
                             % (what, err[i], tol[i], i, got[i], ref[i]))
    worst = assert_close(got, _oracle(inp, rows), TOL_BF16, what + " (bf16 per operation)")
    return ratio, worst


CASES = [
    # name, B, L, d_model, d_inner, N, R, K, unit_dt_proj
    ("small", 2, 37, 64, 128, 16, 8, 4, False),
    ("page_rank1_dt", 1, 100, 32, 64, 16, 1, 4, True),   # Linear_1 + Broadcast_D
    ("k3_n8_ragged", 3, 129, 48, 96, 8, 6, 3, False),
    ("l1", 2, 1, 64, 128, 16, 4, 4, False),
    ("long_two_tiles", 1, 700, 128, 256, 16, 8, 2, False),
    ("rank80_stepped", 1, 40, 64, 128, 16, 80, 4, False),   # rank > 64: operands per step
    ("rank70_narrow", 2, 33, 64, 136, 16, 70, 4, False),    # rank, row stride not multiples of 4
    ("wide_channels", 1, 20, 256, 1040, 16, 16, 4, False),  # channel blocks with a ragged last one
    ("many_rows", 1, 270000, 16, 16, 16, 2, 4, False),      # more rows than one norm grid covers
]


@pytest.mark.parametrize("name,B,L,dm,D,N,R,K,unit", CASES, ids=[c[0] for c in CASES])
def test_block_matches_oracle(name, B, L, dm, D, N, R, K, unit):
    print("case", name, flush=True)
    inp = W.make_block_inputs(B, L, dm, D, N, R, K, seed=700 + L + dm, device=DEV, unit_dt_proj=unit)
    out = _gpu(inp)
    torch.cuda.synchronize()
    ratio, worst = _check(to64(out), inp)
    # The block must change h (a zero update would pass a loose check trivially).
    upd = np.abs(to64(out) - to64(inp["h"])).mean()
    print("  worst |err|/tol %.3f (unrounded), worst scaled error %.2e (rounded), "
          "mean |update| %.3f" % (ratio, worst, upd), flush=True)
    assert upd > 0.05


def test_block_in_place_and_repeatable():
    inp = W.make_block_inputs(2, 50, 64, 128, 16, 4, 4, seed=790, device=DEV)
    first = _gpu(inp).clone()
    again = _gpu(inp)
    h = inp["h"].clone()
    inp2 = dict(inp, h=h)
    _gpu(inp2, out=h)
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    assert torch.equal(first, h)


def test_block_argument_errors_on_a_real_plan():
    inp = W.make_block_inputs(1, 16, 64, 128, 16, 4, 4, seed=791, device=DEV)
    plan = ssm.BlockPlan(1, 16, 64, 128, 16, 4, 4)
    L = binding.lib()
    wts = binding.BlockWeights(**{k: inp[k].data_ptr() for k in ARGS}, norm_eps=1e-5)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(inp["h"])
    h = inp["h"].data_ptr()

    def call(h_in=h, h_out=out.data_ptr(), w=ws.data_ptr(), nbytes=plan.workspace_bytes, weights=wts):
        return L.ssm_block_fwd(plan.handle, ctypes.byref(weights), h_in, h_out, w, nbytes, None)

    assert call(nbytes=plan.workspace_bytes - 1) == binding.SSM_ERR_WORKSPACE
    assert call(w=None) == binding.SSM_ERR_WORKSPACE
    assert call(h_out=h + 64) == binding.SSM_ERR_ALIAS             # overlaps h_in, not in place
    assert call(h_out=inp["w_in"].data_ptr()) == binding.SSM_ERR_ALIAS
    assert call(h_in=h + 2) == binding.SSM_ERR_ALIGN
    bad = binding.BlockWeights(**{k: inp[k].data_ptr() for k in ARGS}, norm_eps=0.0)
    assert call(weights=bad) == binding.SSM_ERR_BAD_SHAPE
    nul = binding.BlockWeights(**{k: inp[k].data_ptr() for k in ARGS}, norm_eps=1e-5)
    nul.w_dt = None
    assert call(weights=nul) == binding.SSM_ERR_NULL_ARG
    torch.cuda.synchronize()
    assert call() == binding.SSM_OK
    torch.cuda.synchronize()
    plan.close()


def test_block_130m_like_sampled_batch_row():
    """The 130M-like block (B=8, L=2048, d_model=768, D=1536, R=48, N=16, K=4) in full on the
    GPU, in the plan the benchmark times; the oracle checks batch rows 0 and 6 (the block
    treats batch rows independently)."""
    cfg = W.B2_130M
    print("config", cfg.name, flush=True)
    inp = W.make_block_config_inputs(cfg, device=DEV)
    out = _gpu(inp)
    torch.cuda.synchronize()
    for b in (0, 6):
        ratio, worst = _check(to64(out[b:b + 1]), inp, slice(b, b + 1), "h_out row %d" % b)
        print("  row %d worst |err|/tol %.3f (unrounded), worst scaled error %.2e (rounded)"
              % (b, ratio, worst), flush=True)
    del inp, out
    torch.cuda.empty_cache()
