"""Pins of the oracle's Mamba block forward (RMSNorm, projections, conv, S6, gate, residual).

The block of the paper summary page "Mamba: Linear-Time Sequence Modeling with
Selective State Spaces" (sec. 4a) has no printed values; it is pinned against
an independent plain torch fp64 implementation (F.rms_norm, F.linear,
F.conv1d, softplus and the recurrence written out), closed forms of the norm,
and special cases.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng


def _weights(rng, dm=12, D=24, N=4, R=3, K=4):
    return dict(
        norm_w=1.0 + 0.1 * rng.standard_normal(dm),
        w_in=rng.standard_normal((2 * D, dm)) / np.sqrt(dm),
        conv_w=0.5 * rng.standard_normal((D, K)),
        conv_b=0.1 * rng.standard_normal(D),
        w_x=rng.standard_normal((R + 2 * N, D)) / np.sqrt(D),
        w_dt=rng.standard_normal((D, R)) / np.sqrt(R),
        dt_bias=rng.uniform(-4.0, -2.0, D),
        A=-np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1)),
        Dskip=rng.standard_normal(D),
        w_out=rng.standard_normal((dm, D)) / np.sqrt(D),
    )


def _torch_block(h, w, eps=1e-5):
    t = {k: torch.tensor(v) for k, v in w.items()}
    h = torch.tensor(h)
    D = t["w_in"].shape[0] // 2
    N = t["A"].shape[1]
    R = t["w_dt"].shape[1]
    K = t["conv_w"].shape[1]
    L = h.shape[1]
    hn = torch.nn.functional.rms_norm(h, (h.shape[-1],), t["norm_w"], eps)
    xz = torch.nn.functional.linear(hn, t["w_in"])
    x, z = xz[..., :D], xz[..., D:]
    c = torch.nn.functional.conv1d(x.transpose(1, 2), t["conv_w"][:, None, :], t["conv_b"],
                                   padding=K - 1, groups=D)[..., :L]
    u = torch.nn.functional.silu(c).transpose(1, 2)
    xd = torch.nn.functional.linear(u, t["w_x"])
    dt_low, Bm, Cm = xd[..., :R], xd[..., R:R + N], xd[..., R + N:]
    dt = torch.nn.functional.softplus(torch.nn.functional.linear(dt_low, t["w_dt"]) + t["dt_bias"])
    hs = torch.zeros(h.shape[0], D, N, dtype=torch.float64)
    ys = []
    for s in range(L):
        e = torch.exp(dt[:, s, :, None] * t["A"])
        hs = e * hs + (e - 1.0) / t["A"] * Bm[:, s, None, :] * u[:, s, :, None]
        ys.append(((hs * Cm[:, s, None, :]).sum(-1) + t["Dskip"] * u[:, s]) *
                  torch.nn.functional.silu(z[:, s]))
    y = torch.stack(ys, 1)
    return (h + torch.nn.functional.linear(y, t["w_out"])).numpy()


def test_block_matches_independent_torch_implementation():
    rng = RNG(100)
    w = _weights(rng)
    h = rng.standard_normal((2, 17, 12))
    got = oracle.mamba_block_fwd(h, **w, bf16=False)
    np.testing.assert_allclose(got, _torch_block(h, w), rtol=1e-12, atol=1e-12)


def test_zero_out_projection_is_the_identity():
    rng = RNG(101)
    w = _weights(rng)
    w["w_out"][:] = 0.0
    h = oracle.round_bf16(rng.standard_normal((1, 9, 12)))
    assert np.array_equal(oracle.mamba_block_fwd(h, **w), h)


def test_rms_norm_closed_forms():
    """A constant row c normalises to sign(c) * weight (up to eps); scaling a row does
    not change its norm's output."""
    w = np.array([0.5, 2.0, -1.0, 3.0])
    h = np.array([[3.0, 3.0, 3.0, 3.0], [-0.25, -0.25, -0.25, -0.25]])
    out = oracle.rms_norm(h, w, eps=0.0)
    np.testing.assert_allclose(out, [w, -w], rtol=1e-15)
    rng = RNG(102)
    v = rng.standard_normal((3, 7))
    np.testing.assert_allclose(oracle.rms_norm(5.0 * v, np.ones(7), 0.0),
                               oracle.rms_norm(v, np.ones(7), 0.0), rtol=1e-14)


def test_round_bf16():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0, np.inf, np.nan])
    r = oracle.round_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2.0 ** -6 and r[3] == -2.5
    assert r[4] == 0.0 and r[5] == np.inf and np.isnan(r[6])
    t = torch.tensor(np.random.default_rng(3).standard_normal(1000), dtype=torch.float32)
    assert np.array_equal(oracle.round_bf16(t.numpy()), t.to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------------------
# The tolerance of the block: mamba_block_error_bound.  It must contain every
# outcome its error model admits (the block with bf16 storage, random roundings
# at every operation output) and must still reject plausible mistakes.
BOUND_CASES = [(32, 64, 16, 4, 4, 300), (48, 96, 8, 6, 3, 129)]


def _bound_case(dm, D, N, R, K, L):
    rng = RNG(dm)
    w = _weights(rng, dm=dm, D=D, N=N, R=R, K=K)
    h = oracle.round_bf16(rng.standard_normal((2, L, dm)))
    ref, tol, sigma = oracle.mamba_block_error_bound(h, **w)
    return w, h, ref, tol, sigma


def test_error_bound_reference_is_the_unrounded_block():
    w, h, ref, tol, sigma = _bound_case(*BOUND_CASES[0])
    np.testing.assert_allclose(ref, oracle.mamba_block_fwd(h, **w, bf16=False), rtol=1e-12,
                               atol=1e-12)
    assert np.all(sigma > 0) and np.all(tol > oracle.U_BF16 * np.abs(ref))


def test_bf16_unit_roundoff():
    """u = 2^-8: eight significant bits, so 1 + u is the midpoint between 1 and the next
    bf16 number, and no rounding moves a value by more than u of its size."""
    assert oracle.round_bf16(np.array([1.0 + oracle.U_BF16]))[0] == 1.0           # tie to even
    assert oracle.round_bf16(np.array([1.0 + 1.01 * oracle.U_BF16]))[0] == 1.0 + 2 * oracle.U_BF16
    v = RNG(7).standard_normal(100000) * 10.0 ** RNG(8).uniform(-3, 3, 100000)
    assert np.max(np.abs(oracle.round_bf16(v) - v) / np.abs(v)) <= oracle.U_BF16


@pytest.mark.parametrize("case", BOUND_CASES, ids=lambda c: "D%d_N%d" % (c[1], c[2]))
def test_error_bound_contains_bf16_storage(case):
    w, h, ref, tol, _ = _bound_case(*case)
    got = oracle.mamba_block_fwd(h, **w, bf16=True)
    assert np.max(np.abs(got - ref) / tol) < 0.8


@pytest.mark.parametrize("seed", range(4))
def test_error_bound_contains_random_roundings_everywhere(seed):
    """Every operation output, the conv output before its SiLU and the step before its
    softplus each perturbed by an independent relative error of at most u."""
    w, h, ref, tol, _ = _bound_case(*BOUND_CASES[seed % 2])
    g = RNG(200 + seed)
    pert = lambda v: v * (1.0 + oracle.U_BF16 * g.uniform(-1.0, 1.0, np.shape(v)))
    got = oracle.mamba_block_fwd(h, **w, bf16=False, perturb=pert)
    assert np.max(np.abs(got - ref) / tol) < 0.8
    # extreme roundings (every one at +u or -u) as well
    pert2 = lambda v: v * (1.0 + oracle.U_BF16 * g.choice([-1.0, 1.0], np.shape(v)))
    got2 = oracle.mamba_block_fwd(h, **w, bf16=False, perturb=pert2)
    assert np.max(np.abs(got2 - ref) / tol) < 1.0


@pytest.mark.parametrize("mistake", ["no_skip", "one_A_sign", "B_for_C", "gate_off",
                                     "conv_taps_reversed", "no_residual_norm_weight"])
def test_error_bound_rejects_plausible_mistakes(mistake):
    """Each of these mistakes moves most outputs outside the tolerance."""
    w, h, ref, tol, _ = _bound_case(*BOUND_CASES[0])
    w2 = {k: np.array(v, copy=True) for k, v in w.items()}
    D = w["w_in"].shape[0] // 2
    N = w["A"].shape[1]
    R = w["w_dt"].shape[1]
    if mistake == "no_skip":
        w2["Dskip"][:] = 0.0
    elif mistake == "one_A_sign":
        w2["A"][:, 0] *= -1.0
    elif mistake == "B_for_C":
        w2["w_x"][R + N:] = w["w_x"][R:R + N]
    elif mistake == "gate_off":                     # silu(z) replaced by a constant branch
        w2["w_in"][D:] = 0.0
    elif mistake == "conv_taps_reversed":
        w2["conv_w"] = w["conv_w"][:, ::-1].copy()
    elif mistake == "no_residual_norm_weight":
        w2["norm_w"][:] = 1.0
    got = oracle.mamba_block_fwd(h, **w2, bf16=False)
    assert np.mean(np.abs(got - ref) > tol) > 0.5
