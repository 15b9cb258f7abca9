"""Shared helpers for the GPU tests: run the HIP path and the oracle on the
same input bits and compare element by element.

Tolerance (per element, on outputs and final states):
    |got - ref| <= tol * (1 + |ref|),  tol = 1e-4 for fp32 I/O, 1e-2 for bf16 I/O,
with fp32 state in the kernels and fp64 in the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def to64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    if worst > tol:
        idx = np.unravel_index(int(err.argmax()), err.shape)
        raise AssertionError("%s: max scaled error %.3e > %.1e at %s (got %r, ref %r)"
                             % (what, worst, tol, idx, got[idx], ref[idx]))
    return worst


def oracle_scan(inp, channels=None, delta_softplus=False, delta_bias=None):
    """Oracle on the exact device bits.  `channels` = optional (batch_idx, dim_idx)
    arrays selecting a subset of channels (full time range)."""
    x, delta, z = inp["x"], inp["delta"], inp.get("z")
    A, Bm, Cm = inp["A"], inp["Bm"], inp["Cm"]
    Dskip, conv_w, conv_b, h0 = inp.get("Dskip"), inp.get("conv_w"), inp.get("conv_b"), inp.get("h0")
    if channels is None:
        return oracle.selective_scan(to64(x), to64(delta), to64(A), to64(Bm), to64(Cm),
                                     Dskip=to64(Dskip), z=to64(z), delta_bias=to64(delta_bias),
                                     delta_softplus=delta_softplus, conv_w=to64(conv_w),
                                     conv_b=to64(conv_b), h0=to64(h0))
    bsel, dsel = channels
    ys, hs = [], []
    for b in sorted(set(int(v) for v in bsel)):
        ds = torch.tensor([int(d) for bb, d in zip(bsel, dsel) if int(bb) == b],
                          device=x.device, dtype=torch.long)
        sel = lambda t: None if t is None else t[b:b + 1].index_select(2, ds)
        y, hf = oracle.selective_scan(
            to64(sel(x)), to64(sel(delta)), to64(A.index_select(0, ds)), to64(Bm[b:b + 1]),
            to64(Cm[b:b + 1]), Dskip=None if Dskip is None else to64(Dskip.index_select(0, ds)),
            z=to64(sel(z)), delta_bias=None if delta_bias is None else to64(delta_bias.index_select(0, ds)),
            delta_softplus=delta_softplus,
            conv_w=None if conv_w is None else to64(conv_w.index_select(0, ds)),
            conv_b=None if conv_b is None else to64(conv_b.index_select(0, ds)),
            h0=None if h0 is None else to64(h0[b:b + 1].index_select(1, ds)))
        ys.append((b, ds.cpu().numpy(), y[0], hf[0]))
    return ys
