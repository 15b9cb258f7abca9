"""Parity of the SSD (Mamba-2) layer (ssm_ssd_fwd) against the fp64 oracle (needs an MI355X).

Outputs y and the final state are compared element by element with the bf16
bound |got - ref| <= 1e-2 (1 + |ref|): the kernel rounds the masked decay
matrix, the weighted inputs and its copy of the state to bf16 before the
matrix products (fp32 accumulation), the oracle computes in fp64 on the same
input bits.  Each case also checks that the state-space part matters: y must
differ from the skip-and-gate term alone by far more than the tolerance.
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


def _run(inp, softplus=False, bias=None, rows=None):
    y, hf = ssm.ssd_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                        z=inp["z"], delta_bias=bias, delta_softplus=softplus, h0=inp["h0"],
                        return_final_state=True)
    torch.cuda.synchronize()
    return y, hf


def _oracle(inp, softplus=False, bias=None, b=slice(None), h=slice(None)):
    x = inp["x"][b][:, :, h]
    G = inp["Bm"].shape[2]
    assert G == 1 or h == slice(None)
    return oracle.ssd(to64(x), to64(inp["delta"][b][:, :, h]), to64(inp["A"][h]), to64(inp["Bm"][b]),
                      to64(inp["Cm"][b]), Dskip=to64(None if inp["Dskip"] is None else inp["Dskip"][h]),
                      z=to64(None if inp["z"] is None else inp["z"][b][:, :, h]),
                      delta_bias=to64(None if bias is None else bias[h]), delta_softplus=softplus,
                      h0=to64(None if inp["h0"] is None else inp["h0"][b][:, h]))


def _ssm_part_matters(y, inp):
    skip = to64(inp["x"]) * (0.0 if inp["Dskip"] is None else to64(inp["Dskip"])[None, None, :, None])
    if inp["z"] is not None:
        zz = to64(inp["z"])
        skip = skip * zz / (1.0 + np.exp(-zz))
    return float(np.mean(np.abs(to64(y) - skip)))


CASES = [
    # name, B, L, H, G, N, extra
    ("one_chunk_ragged_n16", 1, 37, 2, 1, 16, {}),
    ("chunks_ragged_n64_h0", 2, 200, 3, 1, 64, dict(h0=True)),
    ("groups_n32", 1, 130, 4, 2, 32, {}),
    ("n128_h0", 1, 257, 2, 1, 128, dict(h0=True)),
    ("no_gate_no_skip", 2, 64, 2, 1, 64, dict(gate=False, skip=False)),
    ("l1", 2, 1, 3, 1, 128, dict(h0=True)),
    ("long_n128", 1, 1000, 2, 1, 128, {}),
    # few (batch, head) pairs: the sequence runs as segments (end states, combine, outputs)
    ("segments_h0_n64", 1, 3000, 2, 1, 64, dict(h0=True)),
    ("segments_groups_n128", 1, 1100, 4, 2, 128, dict(h0=True)),
    ("segments_n16", 2, 2500, 1, 1, 16, {}),
]


@pytest.mark.parametrize("name,B,L,H,G,N,extra", CASES, ids=[c[0] for c in CASES])
def test_ssd_matches_oracle(name, B, L, H, G, N, extra):
    print("case", name, flush=True)
    inp = W.make_ssd_inputs(B, L, H, 64, G, N, seed=800 + L + N, device=DEV, **extra)
    y, hf = _run(inp)
    yr, hr = _oracle(inp)
    wy = assert_close(to64(y), yr, TOL_BF16, "y")
    wh = assert_close(to64(hf), hr, TOL_BF16, "h_final")
    print("  worst scaled error y %.2e, h_final %.2e" % (wy, wh), flush=True)
    assert _ssm_part_matters(y, inp) > 0.1


HEADDIM_CASES = [
    # name, B, L, H, P, G, N, extra
    ("p32_one_workgroup_per_head", 2, 150, 3, 32, 1, 64, dict(h0=True)),
    ("p96_three_workgroups", 1, 130, 2, 96, 1, 128, {}),
    ("p128_groups", 1, 200, 4, 128, 2, 32, dict(h0=True)),
    ("p32_segments", 1, 2600, 2, 32, 1, 16, dict(h0=True)),
    ("p256_segments_n128", 1, 1500, 1, 256, 1, 128, {}),
    # wide launches: hundreds of workgroups, a few chunks each
    ("wide_p32_n16_h0", 8, 70, 25, 32, 1, 16, dict(h0=True)),
    ("wide_p64_n128_groups", 4, 150, 26, 64, 2, 128, {}),
    ("wide_p96_n64_h0", 3, 100, 22, 96, 1, 64, dict(h0=True)),
    ("wide_n32_one_chunk", 6, 64, 17, 64, 1, 32, {}),
]


@pytest.mark.parametrize("name,B,L,H,P,G,N,extra", HEADDIM_CASES, ids=[c[0] for c in HEADDIM_CASES])
def test_ssd_head_dims(name, B, L, H, P, G, N, extra):
    """Head dims other than 64 (any multiple of 32: one workgroup per 32 channels of a
    head), whole sequences and segmented ones, against the oracle."""
    print("case", name, flush=True)
    inp = W.make_ssd_inputs(B, L, H, P, G, N, seed=820 + L + P, device=DEV, **extra)
    y, hf = _run(inp)
    yr, hr = _oracle(inp)
    wy = assert_close(to64(y), yr, TOL_BF16, "y")
    wh = assert_close(to64(hf), hr, TOL_BF16, "h_final")
    print("  worst scaled error y %.2e, h_final %.2e" % (wy, wh), flush=True)
    assert _ssm_part_matters(y, inp) > 0.1


F32_CASES = [
    # name, B, L, H, P, G, N, extra
    ("f32_n16_ragged", 2, 37, 3, 32, 1, 16, dict(h0=True)),
    ("f32_n128_groups", 1, 201, 4, 64, 2, 128, {}),
    ("f32_n64_l1", 3, 1, 2, 96, 1, 64, dict(h0=True)),
    ("f32_n32_no_gate_no_skip", 2, 130, 2, 64, 1, 32, dict(gate=False, skip=False)),
    ("f32_long_n128", 1, 3000, 2, 64, 1, 128, dict(h0=True)),
]


@pytest.mark.parametrize("name,B,L,H,P,G,N,extra", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_ssd_fp32_io(name, B, L, H, P, G, N, extra):
    """fp32 I/O: the recurrent form in fp32, held to the fp32 bound 1e-4 (1 + |ref|)."""
    print("case", name, flush=True)
    inp = W.make_ssd_inputs(B, L, H, P, G, N, seed=840 + L + N, device=DEV,
                            io_dtype=torch.float32, **extra)
    y, hf = _run(inp)
    yr, hr = _oracle(inp)
    tol = TOL[torch.float32]
    wy = assert_close(to64(y), yr, tol, "y")
    wh = assert_close(to64(hf), hr, tol, "h_final")
    print("  worst scaled error y %.2e, h_final %.2e" % (wy, wh), flush=True)
    assert _ssm_part_matters(y, inp) > 0.1


def test_ssd_fp32_softplus_bias_and_zero_A():
    """A = 0 (the weight's limit dt) and a small positive A.  A positive A makes the
    recurrence grow like exp(A sum(dt)), which amplifies every rounding by the same
    factor; A = 0.05 over these 150 steps grows the state about e^5, so the fp32 bound
    stays meaningful (at A = 0.3 the outputs reach 4e11 and no fp32 arithmetic holds a
    1e-4 relative bound)."""
    inp = W.make_ssd_inputs(2, 150, 3, 64, 1, 64, seed=851, device=DEV, io_dtype=torch.float32,
                            h0=True)
    g0 = torch.Generator(DEV).manual_seed(12)
    inp["delta"] = torch.randn(inp["delta"].shape, device=DEV, generator=g0) - 1.0
    inp["A"] = torch.tensor([0.0, -0.5, 0.05], device=DEV)
    bias = 0.3 * torch.randn(3, device=DEV, generator=g0)
    y, hf = _run(inp, softplus=True, bias=bias)
    yr, hr = _oracle(inp, softplus=True, bias=bias)
    tol = TOL[torch.float32]
    assert_close(to64(y), yr, tol, "y")
    assert_close(to64(hf), hr, tol, "h_final")


def test_ssd_fp32_matches_bf16_path_on_bf16_values():
    """The recurrent fp32 form and the chunked bf16 form compute the same map: on inputs
    that are bf16 values, the fp32 run (rounded to bf16) agrees with the bf16 run within
    the bf16 bound."""
    inp = W.make_ssd_inputs(2, 300, 4, 64, 2, 128, seed=852, device=DEV, h0=True)
    f32 = {k: (None if v is None else (v.float() if v.dtype == torch.bfloat16 else v))
           for k, v in inp.items()}
    y16, h16 = _run(inp)
    y32, h32 = _run(f32)
    assert_close(to64(y16), to64(y32), TOL_BF16, "y")
    assert_close(to64(h16), to64(h32), TOL_BF16, "h_final")


def test_ssd_softplus_bias_zero_and_positive_A():
    inp = W.make_ssd_inputs(1, 150, 4, 64, 1, 64, seed=851, device=DEV)
    g = torch.Generator(DEV).manual_seed(9)
    inp["delta"] = (torch.randn(1, 150, 4, device=DEV, generator=g) - 1.0).to(torch.bfloat16)
    bias = 0.5 * torch.randn(4, device=DEV, generator=g)
    inp["A"] = torch.tensor([-1.5, 0.0, 0.05, -8.0], device=DEV)
    y, hf = _run(inp, softplus=True, bias=bias)
    yr, hr = _oracle(inp, softplus=True, bias=bias)
    assert_close(to64(y), yr, TOL_BF16, "y")
    assert_close(to64(hf), hr, TOL_BF16, "h_final")


def test_ssd_segments_softplus_bias():
    """Segmented run with the softplus step and a bias (rows past the end of the last chunk
    must not move the state)."""
    inp = W.make_ssd_inputs(1, 2049, 2, 64, 1, 32, seed=854, device=DEV, h0=True)
    g = torch.Generator(DEV).manual_seed(10)
    inp["delta"] = (torch.randn(1, 2049, 2, device=DEV, generator=g) - 2.0).to(torch.bfloat16)
    bias = 0.5 * torch.randn(2, device=DEV, generator=g)
    y, hf = _run(inp, softplus=True, bias=bias)
    yr, hr = _oracle(inp, softplus=True, bias=bias)
    assert_close(to64(y), yr, TOL_BF16, "y")
    assert_close(to64(hf), hr, TOL_BF16, "h_final")


def test_ssd_empty_sequence_copies_h0():
    inp = W.make_ssd_inputs(2, 0, 3, 64, 1, 32, seed=852, device=DEV, h0=True)
    y, hf = _run(inp)
    assert torch.equal(hf, inp["h0"])
    inp["h0"] = None
    y, hf = _run(inp)
    assert torch.count_nonzero(hf) == 0


def test_ssd_state_handover_equals_one_pass():
    """Two calls with the final state handed over reproduce one call (the inter-chunk
    recurrence across a call boundary that is not a chunk boundary)."""
    inp = W.make_ssd_inputs(1, 230, 2, 64, 1, 64, seed=853, device=DEV, h0=True)
    y, hf = _run(inp)
    c = 101
    first = {k: (v[:, :c].contiguous() if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in inp.items()}
    second = {k: (v[:, c:].contiguous() if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in inp.items()}
    y1, h1 = _run(first)
    second["h0"] = h1
    y2, h2 = _run(second)
    yr, hr = _oracle(inp)
    assert_close(to64(torch.cat([y1, y2], 1)), yr, TOL_BF16, "y in two calls")
    assert_close(to64(h2), hr, TOL_BF16, "h_final in two calls")


def test_ssd_long_single_sequence_sampled_head():
    """One 65536-token sequence (24 heads, N = 128): the segmented schedule at full size;
    the oracle checks head 17 over the whole sequence."""
    cfg = W.S4_MAMBA2_LONG
    print("config", cfg.name, flush=True)
    inp = W.make_ssd_config_inputs(cfg, device=DEV)
    y, hf = _run(inp)
    h = 17
    yr, hr = _oracle(inp, b=slice(0, 1), h=slice(h, h + 1))
    wy = assert_close(to64(y[:, :, h:h + 1]), yr, TOL_BF16, "y head %d" % h)
    wh = assert_close(to64(hf[:, h:h + 1]), hr, TOL_BF16, "h_final head %d" % h)
    print("  head %d worst y %.2e, h_final %.2e" % (h, wy, wh), flush=True)
    del inp, y, hf
    torch.cuda.empty_cache()


def test_ssd_mamba2_130m_like_sampled_heads():
    """The Mamba-2 130M-like layer (B=8, L=2048, H=24, P=64, N=128) in full; the oracle checks
    3 (batch, head) pairs over the whole sequence, outputs and final states."""
    cfg = W.S2_MAMBA2_130M
    print("config", cfg.name, flush=True)
    inp = W.make_ssd_config_inputs(cfg, device=DEV)
    y, hf = _run(inp)
    for b, h in ((0, 0), (3, 11), (7, 23)):
        yr, hr = _oracle(inp, b=slice(b, b + 1), h=slice(h, h + 1))
        wy = assert_close(to64(y[b:b + 1, :, h:h + 1]), yr, TOL_BF16, "y (%d,%d)" % (b, h))
        wh = assert_close(to64(hf[b:b + 1, h:h + 1]), hr, TOL_BF16, "h_final (%d,%d)" % (b, h))
        print("  (b=%d, h=%d) worst y %.2e, h_final %.2e" % (b, h, wy, wh), flush=True)
    del inp, y, hf
    torch.cuda.empty_cache()
