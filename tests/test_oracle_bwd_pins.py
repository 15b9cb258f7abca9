"""Pins of the oracle's backward pass (gradients of the selective scan).

The pages describe the backward pass only as recomputing the states instead
of storing them ("Mamba: Linear-Time Sequence Modeling with Selective State
Spaces", sec. 4c), so the gradients have no printed values.  They are pinned
to the mathematics instead:
  * central finite differences of the oracle's own forward, for every input
    (including A = 0 entries, the conv prologue, the softplus bias and h0);
  * torch.autograd through an independent fp64 torch forward written here
    from eq. (4), (2a), (2b) and the block of sec. 4a.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng


def _problem(rng, B=2, L=6, D=3, N=3, K=3, zero_a=False):
    p = dict(
        x=rng.standard_normal((B, L, D)),
        delta=rng.standard_normal((B, L, D)) - 1.0,      # raw: softplus(delta + bias) in use
        A=-rng.uniform(0.3, 2.5, size=(D, N)),
        Bm=rng.standard_normal((B, L, N)),
        Cm=rng.standard_normal((B, L, N)),
        Dskip=rng.standard_normal(D),
        z=rng.standard_normal((B, L, D)),
        delta_bias=0.3 * rng.standard_normal(D),
        conv_w=0.5 * rng.standard_normal((D, K)),
        conv_b=0.5 * rng.standard_normal(D),
        h0=rng.standard_normal((B, D, N)),
    )
    if zero_a:
        p["A"][0, 1] = 0.0
        p["A"][2, 0] = 0.0
    return p


def _loss(p, W, V):
    y, hf = oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"],
                                  z=p["z"], delta_bias=p["delta_bias"], delta_softplus=True,
                                  conv_w=p["conv_w"], conv_b=p["conv_b"], h0=p["h0"], nthreads=1)
    return float(np.sum(y * W) + np.sum(hf * V))


GRAD_OF = dict(x="dx", delta="ddelta", A="dA", Bm="dBm", Cm="dCm", Dskip="dDskip", z="dz",
               delta_bias="ddelta_bias", conv_w="dconv_w", conv_b="dconv_b", h0="dh0")


@pytest.mark.parametrize("zero_a", [False, True])
def test_gradients_match_central_differences(zero_a):
    """Every gradient entry against a central difference of the oracle's forward
    (loss = sum(y * W) + sum(h_final * V)); fp64, step 1e-6."""
    rng = RNG(80 + int(zero_a))
    p = _problem(rng, zero_a=zero_a)
    W = rng.standard_normal(p["x"].shape)
    V = rng.standard_normal(p["h0"].shape)
    g = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], W,
                                  Dskip=p["Dskip"], z=p["z"], delta_bias=p["delta_bias"],
                                  delta_softplus=True, conv_w=p["conv_w"], conv_b=p["conv_b"],
                                  h0=p["h0"], dh_final=V, nthreads=1)
    for name, gname in GRAD_OF.items():
        arr = p[name]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            h = 1e-6 * max(1.0, abs(old))
            arr[idx] = old + h
            lp = _loss(p, W, V)
            arr[idx] = old - h
            lm = _loss(p, W, V)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-6, err_msg=name)


def _torch_forward(p, conv=True, gate=True):
    """An independent fp64 torch forward: causal conv + SiLU, softplus step, exact ZOH
    (e^{dt a} - 1)/a, the recurrence, C h + D u, SiLU gate."""
    x, delta, A, Bm, Cm = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"]
    Bsz, L, D = x.shape
    if conv:
        K = p["conv_w"].shape[1]
        xp = torch.nn.functional.pad(x.transpose(1, 2), (K - 1, 0))
        c = torch.nn.functional.conv1d(xp, p["conv_w"][:, None, :], p["conv_b"], groups=D)
        u = torch.nn.functional.silu(c).transpose(1, 2)
    else:
        u = x
    dt = torch.nn.functional.softplus(delta + p["delta_bias"])
    h = p["h0"]
    ys = []
    for t in range(L):
        e = torch.exp(dt[:, t, :, None] * A)
        bbar = (e - 1.0) / A * Bm[:, t, None, :]
        h = e * h + bbar * u[:, t, :, None]
        yt = (h * Cm[:, t, None, :]).sum(-1) + p["Dskip"] * u[:, t]
        if gate:
            yt = yt * torch.nn.functional.silu(p["z"][:, t])
        ys.append(yt)
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("conv,gate", [(True, True), (False, False)])
def test_gradients_match_torch_autograd(conv, gate):
    """torch.autograd through the independent torch forward, on a larger problem."""
    rng = RNG(90 + int(conv))
    p = _problem(rng, B=2, L=33, D=5, N=4, K=4)
    W = rng.standard_normal(p["x"].shape)
    V = rng.standard_normal(p["h0"].shape)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    y, hf = _torch_forward(tp, conv=conv, gate=gate)
    loss = (y * torch.tensor(W)).sum() + (hf * torch.tensor(V)).sum()
    keys = [k for k in GRAD_OF if (conv or not k.startswith("conv")) and (gate or k != "z")]
    grads = torch.autograd.grad(loss, [tp[k] for k in keys])
    g = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], W,
                                  Dskip=p["Dskip"], z=p["z"] if gate else None,
                                  delta_bias=p["delta_bias"], delta_softplus=True,
                                  conv_w=p["conv_w"] if conv else None,
                                  conv_b=p["conv_b"] if conv else None, h0=p["h0"], dh_final=V)
    for k, gt in zip(keys, grads):
        np.testing.assert_allclose(g[GRAD_OF[k]], gt.numpy(), rtol=1e-10, atol=1e-10, err_msg=k)


def test_gradient_of_zero_loss_is_zero_and_shapes():
    rng = RNG(95)
    p = _problem(rng)
    g = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"],
                                  np.zeros_like(p["x"]), h0=p["h0"])
    assert set(g) == {"dx", "ddelta", "dA", "dBm", "dCm", "dh0"}
    for v in g.values():
        assert not np.any(v)


# ---------------------------------------------------------------------------
# A conv state entering the sequence: the inputs before t = 0 that the conv
# prologue reads in place of zeros (the prefill -> decode handoff of the
# EulerStack tutorial's d_conv window, run backwards).
def _loss_cs(p, cs, W, V):
    y, hf = oracle.selective_scan(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], Dskip=p["Dskip"],
                                  z=p["z"], delta_bias=p["delta_bias"], delta_softplus=True,
                                  conv_w=p["conv_w"], conv_b=p["conv_b"], h0=p["h0"],
                                  conv_state_in=cs, nthreads=1)
    return float(np.sum(y * W) + np.sum(hf * V))


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv_state_gradient_matches_central_differences(K):
    """dconv_state_in and the gradients that the state changes (dconv_w, dx near t = 0)
    against central differences of the forward with the same conv state."""
    rng = RNG(120 + K)
    p = _problem(rng, B=2, L=5, D=3, N=2, K=K)
    cs = rng.standard_normal((2, K - 1, 3))
    W = rng.standard_normal(p["x"].shape)
    V = rng.standard_normal(p["h0"].shape)
    g = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], W,
                                  Dskip=p["Dskip"], z=p["z"], delta_bias=p["delta_bias"],
                                  delta_softplus=True, conv_w=p["conv_w"], conv_b=p["conv_b"],
                                  h0=p["h0"], dh_final=V, conv_state_in=cs, nthreads=1)
    targets = [("conv_state_in", cs, "dconv_state_in"), ("conv_w", p["conv_w"], "dconv_w"),
               ("x", p["x"], "dx"), ("conv_b", p["conv_b"], "dconv_b")]
    for name, arr, gname in targets:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            h = 1e-6 * max(1.0, abs(old))
            arr[idx] = old + h
            lp = _loss_cs(p, cs, W, V)
            arr[idx] = old - h
            lm = _loss_cs(p, cs, W, V)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-6, err_msg=name)


def test_conv_state_gradient_equals_gradient_of_the_concatenated_sequence():
    """The state is the K-1 inputs before the sequence: the gradients equal those of
    one pass over [state, x] (autograd through the independent torch forward), whose
    leading rows carry zero output weight and whose conv reads zeros before them."""
    rng = RNG(130)
    K = 4
    p = _problem(rng, B=2, L=20, D=4, N=3, K=K)
    cs = rng.standard_normal((2, K - 1, 4))
    W = rng.standard_normal(p["x"].shape)
    V = rng.standard_normal(p["h0"].shape)
    g = oracle.selective_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], W,
                                  Dskip=p["Dskip"], z=p["z"], delta_bias=p["delta_bias"],
                                  delta_softplus=True, conv_w=p["conv_w"], conv_b=p["conv_b"],
                                  h0=p["h0"], dh_final=V, conv_state_in=cs)
    # torch: conv over [cs, x] with zero left padding, keeping the last L outputs
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    tcs = torch.tensor(cs, requires_grad=True)
    xx = torch.cat([tcs, tp["x"]], 1)
    xp = torch.nn.functional.pad(xx.transpose(1, 2), (K - 1, 0))
    c = torch.nn.functional.conv1d(xp, tp["conv_w"][:, None, :], tp["conv_b"], groups=4)
    u = torch.nn.functional.silu(c).transpose(1, 2)[:, K - 1:]
    dt = torch.nn.functional.softplus(tp["delta"] + tp["delta_bias"])
    h = tp["h0"]
    ys = []
    for t in range(20):
        e = torch.exp(dt[:, t, :, None] * tp["A"])
        h = e * h + (e - 1.0) / tp["A"] * tp["Bm"][:, t, None, :] * u[:, t, :, None]
        ys.append(((h * tp["Cm"][:, t, None, :]).sum(-1) + tp["Dskip"] * u[:, t])
                  * torch.nn.functional.silu(tp["z"][:, t]))
    y = torch.stack(ys, 1)
    loss = (y * torch.tensor(W)).sum() + (h * torch.tensor(V)).sum()
    gcs, gx, gw = torch.autograd.grad(loss, [tcs, tp["x"], tp["conv_w"]])
    np.testing.assert_allclose(g["dconv_state_in"], gcs.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(g["dx"], gx.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(g["dconv_w"], gw.numpy(), rtol=1e-10, atol=1e-10)
