"""Pins of the oracle's SSD (Mamba-2) layer.

"14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상", sec. 5.1 restricts the
state matrix to a scalar times the identity per step and states that the layer
is then a masked matrix product, Y = (L o (C B^T)) X with L the causal mask of
cumulative decays; sec. 5.2 runs it chunk by chunk, passing the state between
chunks.  The recurrence (``oracle.ssd``, C) is pinned to:
  * the already pinned S6 oracle, which it must equal when every state entry of
    a head shares one A and one step (a special case of Algorithm 2);
  * the page's quadratic (duality) form, written independently in numpy;
  * a hand-expanded two-step example;
  * state passing: scanning two halves with the state handed over equals one pass;
  * groups: heads of a group read that group's B and C.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng


def _problem(rng, B=2, L=11, H=4, P=3, G=1, N=5, a_sign=-1.0):
    return dict(
        x=rng.standard_normal((B, L, H, P)),
        delta=rng.uniform(0.01, 0.6, (B, L, H)),
        A=a_sign * rng.uniform(0.3, 2.0, H),
        Bm=rng.standard_normal((B, L, G, N)),
        Cm=rng.standard_normal((B, L, G, N)),
        Dskip=rng.standard_normal(H),
        z=rng.standard_normal((B, L, H, P)),
        h0=rng.standard_normal((B, H, P, N)),
    )


def test_ssd_equals_s6_with_one_scalar_per_head():
    rng = RNG(1)
    p = _problem(rng)
    B, L, H, P = p["x"].shape
    N = p["Bm"].shape[3]
    y, hf = oracle.ssd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"], z=p["z"],
                       h0=p["h0"])
    # S6 over D = H*P channels: channel (h, p) gets A[h] on every state entry and delta[h].
    D = H * P
    y6, h6 = oracle.selective_scan(
        p["x"].reshape(B, L, D), np.repeat(p["delta"], P, axis=2),
        np.repeat(p["A"], P)[:, None] * np.ones((1, N)), p["Bm"][:, :, 0], p["Cm"][:, :, 0],
        Dskip=np.repeat(p["Dskip"], P), z=p["z"].reshape(B, L, D), h0=p["h0"].reshape(B, D, N))
    np.testing.assert_allclose(y.reshape(B, L, D), y6, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hf.reshape(B, D, N), h6, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("a_sign,G", [(-1.0, 1), (-1.0, 2), (1.0, 1), (0.0, 4)])
def test_ssd_recurrence_equals_duality_form(a_sign, G):
    rng = RNG(2 + G)
    p = _problem(rng, B=2, L=17, H=4, P=3, G=G, N=6, a_sign=a_sign)
    y, hf = oracle.ssd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"], z=p["z"],
                       h0=p["h0"])
    yq, hq = oracle.ssd_quadratic(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"],
                                  z=p["z"], h0=p["h0"])
    np.testing.assert_allclose(y, yq, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hf, hq, rtol=1e-11, atol=1e-11)


def test_ssd_two_step_hand_expansion():
    """One head, P = N = 1: y_0 = C_0 w_0 B_0 x_0 and y_1 = C_1 (alpha_1 w_0 B_0 x_0 +
    w_1 B_1 x_1), alpha = e^{dt a}, w = (e^{dt a} - 1) / a."""
    a = -0.75
    dt = np.array([0.5, 0.25])
    xv, bv, cv = np.array([2.0, -1.0]), np.array([0.5, 3.0]), np.array([1.5, -2.0])
    al = np.exp(dt * a)
    w = (al - 1.0) / a
    s0 = w[0] * bv[0] * xv[0]
    s1 = al[1] * s0 + w[1] * bv[1] * xv[1]
    y, hf = oracle.ssd(xv.reshape(1, 2, 1, 1), dt.reshape(1, 2, 1), np.array([a]),
                       bv.reshape(1, 2, 1, 1), cv.reshape(1, 2, 1, 1))
    np.testing.assert_allclose(y.ravel(), [cv[0] * s0, cv[1] * s1], rtol=1e-15)
    np.testing.assert_allclose(hf.ravel(), [s1], rtol=1e-15)


def test_ssd_state_passing_between_chunks():
    rng = RNG(7)
    p = _problem(rng, B=1, L=20, H=2, P=4, N=3)
    y, hf = oracle.ssd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"], h0=p["h0"])
    c = 8
    y1, h1 = oracle.ssd(p["x"][:, :c], p["delta"][:, :c], p["A"], p["Bm"][:, :c], p["Cm"][:, :c],
                        Dskip=p["Dskip"], h0=p["h0"])
    y2, h2 = oracle.ssd(p["x"][:, c:], p["delta"][:, c:], p["A"], p["Bm"][:, c:], p["Cm"][:, c:],
                        Dskip=p["Dskip"], h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h2, hf, rtol=1e-13, atol=1e-13)


def test_ssd_groups_select_their_B_and_C():
    rng = RNG(9)
    p = _problem(rng, B=1, L=7, H=4, P=2, G=2, N=3)
    y, hf = oracle.ssd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"])
    for h in range(4):
        g = h // 2
        yh, hh = oracle.ssd(p["x"][:, :, h:h + 1], p["delta"][:, :, h:h + 1], p["A"][h:h + 1],
                            p["Bm"][:, :, g:g + 1], p["Cm"][:, :, g:g + 1])
        np.testing.assert_allclose(y[:, :, h:h + 1], yh, rtol=1e-15, atol=0)
        np.testing.assert_allclose(hf[:, h:h + 1], hh, rtol=1e-15, atol=0)


def test_ssd_softplus_step_and_bias():
    rng = RNG(11)
    p = _problem(rng, B=1, L=9, H=3, P=2, N=4)
    raw = rng.standard_normal((1, 9, 3)) - 1.0
    bias = rng.standard_normal(3)
    y, hf = oracle.ssd(p["x"], raw, p["A"], p["Bm"], p["Cm"], delta_bias=bias, delta_softplus=True)
    dt = torch.nn.functional.softplus(torch.tensor(raw + bias)).numpy()
    y2, h2 = oracle.ssd(p["x"], dt, p["A"], p["Bm"], p["Cm"])
    np.testing.assert_allclose(y, y2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(hf, h2, rtol=1e-14, atol=1e-14)


def test_ssd_rejects_bad_sizes():
    rng = RNG(12)
    p = _problem(rng, H=3, G=2)
    with pytest.raises(ValueError):
        oracle.ssd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"])
