"""Seeded synthetic inputs for the selective scan and the decode step.

This module holds only the input recipe (shapes, distributions, seeds).  It
computes none of the scan's arithmetic, so the HIP path, the tests and the
benchmark can all draw the same inputs from it while the oracle stays an
independent implementation.

Shapes follow Algorithm 2 and the block table of sec. 4a on the paper summary
page "Mamba: Linear-Time Sequence Modeling with Selective State Spaces":
x, delta, z: (B, L, D); B, C: (B, L, N); A: (D, N); plus the D skip (D,),
conv1d weights (D, K) and states (B, D, N).  A uses the S4D-Real rule of that
page's sec. 4d, A[d, n] = -(n + 1), for every channel.

Recipe: every tensor is drawn in float32 from a torch.Generator seeded with
the config's seed, in a fixed order (x, delta, B, C, z, Dskip, conv_w, h0),
on the requested device, then rounded to the I/O dtype (round to nearest
even).  delta = softplus(N(0,1) - shift) is formed in float32 before the
rounding, so the kernels receive an already activated step size.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io_dtype: torch.dtype
    seed: int
    delta_shift: float = 2.0
    gate: bool = True
    skip: bool = True
    conv_k: int = 0
    conv_std: float = 0.5
    final_state: bool = True
    h0: bool = False
    description: str = ""

    @property
    def elems(self) -> int:
        return self.batch * self.seqlen * self.dim


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int
    io_dtype: torch.dtype
    seed: int
    delta_shift: float = 2.0
    gate: bool = True
    skip: bool = True
    description: str = ""


# The five workloads.  The first is small enough for the oracle to finish in
# well under a second; the others are full-size layer shapes.
C1_TINY = ScanConfig("c1_tiny_f32", 1, 64, 16, 4, torch.float32, seed=0,
                     description="tiny S6 scan, fp32 I/O, B=1 L=64 D=16 N=4")
C2_130M = ScanConfig("c2_mamba130m_layer", 8, 2048, 1536, 16, torch.bfloat16, seed=1,
                     description="Mamba-130M-like layer scan (d_model 768, expand 2), bf16 I/O")
C3_2P8B_CONV = ScanConfig("c3_mamba2p8b_conv", 4, 4096, 5120, 16, torch.bfloat16, seed=2,
                          conv_k=4, description="Mamba-2.8B-like layer, fused causal "
                          "conv1d(k=4)+SiLU prologue, bf16 I/O")
C4_DNA_1M = ScanConfig("c4_dna_1m", 1, 1 << 20, 1024, 16, torch.bfloat16, seed=3,
                       delta_shift=3.0, description="1M-token DNA-like scan, bf16 I/O, "
                       "final state")
C5_DECODE = DecodeConfig("c5_decode", 256, 5120, 16, 64, torch.bfloat16, seed=4,
                         description="decode state_update, fp32 state (256,5120,16), "
                         "64 single-token steps")

SCAN_CONFIGS = {c.name: c for c in (C1_TINY, C2_130M, C3_2P8B_CONV, C4_DNA_1M)}


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """Sizes of one Mamba block (pre-norm residual around in_proj, conv, S6, out_proj)."""
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    dstate: int
    dt_rank: int
    conv_k: int
    seed: int


# A 130M-like layer (d_model 768, E = 2, N = 16, dt_rank = d_model / 16, conv width 4)
# at the same batch and length as the 130M-like scan.
B2_130M = BlockConfig("b2_mamba130m_block", 8, 2048, 768, 1536, 16, 48, 4, seed=21)


@dataclasses.dataclass(frozen=True)
class SsdConfig:
    """Sizes of one SSD (Mamba-2) layer: H heads of P channels, N state entries."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    seed: int


# The 130M-like width (D = 1536 = 24 heads x 64) with the Mamba-2 state size N = 128,
# at the batch and length of the 130M-like scan.
S2_MAMBA2_130M = SsdConfig("s2_mamba2_130m_ssd", 8, 2048, 24, 64, 1, 128, seed=31)
# One long sequence at the same width: too few (batch, head) pairs to fill the GPU
# alone, so the layer runs as sequence segments.
S4_MAMBA2_LONG = SsdConfig("s4_mamba2_long_b1", 1, 65536, 24, 64, 1, 128, seed=32)
# Decode of a 2.7B-like Mamba-2 layer (d_model 2560, E = 2: 80 heads x 64, N = 128) for
# 256 sequences; seqlen is the number of decode steps drawn.
S5_MAMBA2_DECODE = SsdConfig("s5_mamba2_2p7b_decode", 256, 16, 80, 64, 1, 128, seed=33)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std: float = 1.0, shift: float = 0.0):
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if shift != 0.0:
        t.sub_(shift)
    return t


def s4d_real_A(dim: int, dstate: int, device="cpu") -> torch.Tensor:
    """A[d, n] = -(n + 1) for every channel (sec. 4d, S4D-Real)."""
    row = -torch.arange(1, dstate + 1, dtype=torch.float32, device=device)
    return row.expand(dim, dstate).contiguous()


def make_scan_inputs(batch: int, seqlen: int, dim: int, dstate: int,
                     io_dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                     device="cpu", delta_shift: float = 2.0, gate: bool = True,
                     skip: bool = True, conv_k: int = 0, conv_std: float = 0.5,
                     h0: bool = False, A: Optional[torch.Tensor] = None
                     ) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one scan input set.  Returns a dict keyed like the scan arguments."""
    g = _gen(device, seed)
    shp = (batch, seqlen, dim)
    x = _randn(shp, g, device).to(io_dtype)
    delta = F.softplus(_randn(shp, g, device, shift=delta_shift)).to(io_dtype)
    Bm = _randn((batch, seqlen, dstate), g, device).to(io_dtype)
    Cm = _randn((batch, seqlen, dstate), g, device).to(io_dtype)
    z = _randn(shp, g, device).to(io_dtype) if gate else None
    Dskip = _randn((dim,), g, device) if skip else None
    conv_w = _randn((dim, conv_k), g, device, std=conv_std) if conv_k else None
    hinit = _randn((batch, dim, dstate), g, device) if h0 else None
    if A is None:
        A = s4d_real_A(dim, dstate, device)
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=z,
                conv_w=conv_w, conv_b=None, h0=hinit)


def make_config_inputs(cfg: ScanConfig, device="cpu", **overrides):
    kw = dict(batch=cfg.batch, seqlen=cfg.seqlen, dim=cfg.dim, dstate=cfg.dstate,
              io_dtype=cfg.io_dtype, seed=cfg.seed, delta_shift=cfg.delta_shift,
              gate=cfg.gate, skip=cfg.skip, conv_k=cfg.conv_k, conv_std=cfg.conv_std,
              h0=cfg.h0)
    kw.update(overrides)
    return make_scan_inputs(device=device, **kw)


def make_decode_inputs(batch: int, dim: int, dstate: int, steps: int,
                       io_dtype: torch.dtype = torch.bfloat16, seed: int = 4,
                       device="cpu", delta_shift: float = 2.0, gate: bool = True,
                       skip: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Initial fp32 state ~ N(0,1) plus `steps` fresh single-token inputs.

    x, delta, z: (steps, B, D); Bm, Cm: (steps, B, N); state0: (B, D, N).
    """
    g = _gen(device, seed)
    state0 = _randn((batch, dim, dstate), g, device)
    shp = (steps, batch, dim)
    x = _randn(shp, g, device).to(io_dtype)
    delta = F.softplus(_randn(shp, g, device, shift=delta_shift)).to(io_dtype)
    Bm = _randn((steps, batch, dstate), g, device).to(io_dtype)
    Cm = _randn((steps, batch, dstate), g, device).to(io_dtype)
    z = _randn(shp, g, device).to(io_dtype) if gate else None
    Dskip = _randn((dim,), g, device) if skip else None
    A = s4d_real_A(dim, dstate, device)
    return dict(state0=state0, x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, z=z, Dskip=Dskip)


def make_decode_config_inputs(cfg: DecodeConfig, device="cpu", **overrides):
    kw = dict(batch=cfg.batch, dim=cfg.dim, dstate=cfg.dstate, steps=cfg.steps,
              io_dtype=cfg.io_dtype, seed=cfg.seed, delta_shift=cfg.delta_shift,
              gate=cfg.gate, skip=cfg.skip)
    kw.update(overrides)
    return make_decode_inputs(device=device, **kw)


def make_block_inputs(batch: int, seqlen: int, d_model: int, d_inner: int, dstate: int,
                      dt_rank: int, conv_k: int = 4, seed: int = 21, device="cpu",
                      unit_dt_proj: bool = False) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one block input set (bf16 activations and matrices, fp32 vectors).

    Order and laws: h ~ N(0,1); norm_w = 1 + 0.1 N(0,1); w_in ~ N(0, 1/d_model);
    conv_w ~ N(0, 0.25); conv_b ~ N(0, 0.01); w_x ~ N(0, 1/d_inner); w_dt ~ N(0, 1/dt_rank)
    (all ones with unit_dt_proj: the rank-1 broadcast form); dt_bias ~ U(-7, -2.3), so
    that softplus(dt_bias) spans about 1e-3 .. 0.1; A the S4D-Real rule; Dskip = 1 +
    0.1 N(0,1); w_out ~ N(0, 1/d_inner).  Matrices are drawn in fp32 and rounded to bf16.
    """
    g = _gen(device, seed)
    bf = torch.bfloat16
    D, R, N = d_inner, dt_rank, dstate
    h = _randn((batch, seqlen, d_model), g, device).to(bf)
    norm_w = _randn((d_model,), g, device, std=0.1, shift=-1.0)
    w_in = _randn((2 * D, d_model), g, device, std=d_model ** -0.5).to(bf)
    conv_w = _randn((D, conv_k), g, device, std=0.5)
    conv_b = _randn((D,), g, device, std=0.1)
    w_x = _randn((R + 2 * N, D), g, device, std=D ** -0.5).to(bf)
    if unit_dt_proj:
        w_dt = torch.ones((D, R), device=device, dtype=bf)
    else:
        w_dt = _randn((D, R), g, device, std=R ** -0.5).to(bf)
    dt_bias = torch.rand((D,), generator=g, device=device) * 4.7 - 7.0
    A = s4d_real_A(D, N, device)
    Dskip = _randn((D,), g, device, std=0.1, shift=-1.0)
    w_out = _randn((d_model, D), g, device, std=D ** -0.5).to(bf)
    return dict(h=h, norm_w=norm_w, w_in=w_in, conv_w=conv_w, conv_b=conv_b, w_x=w_x, w_dt=w_dt,
                dt_bias=dt_bias, A=A, Dskip=Dskip, w_out=w_out)


def make_block_config_inputs(cfg: BlockConfig, device="cpu", **overrides):
    kw = dict(batch=cfg.batch, seqlen=cfg.seqlen, d_model=cfg.d_model, d_inner=cfg.d_inner,
              dstate=cfg.dstate, dt_rank=cfg.dt_rank, conv_k=cfg.conv_k, seed=cfg.seed)
    kw.update(overrides)
    return make_block_inputs(device=device, **kw)


def make_ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, ngroups: int, dstate: int,
                    seed: int = 31, device="cpu", gate: bool = True, skip: bool = True,
                    h0: bool = False, delta_shift: float = 2.0,
                    io_dtype: torch.dtype = torch.bfloat16) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one SSD input set, in order: x ~ N(0,1); delta = softplus(N(0,1) - shift) (the
    step, already activated); B, C ~ N(0,1) (as for the scan); z ~ N(0,1);
    A = -(1 .. H) / H * 4 (one negative scalar per head, spread over (0, 4]); Dskip ~ N(0,1);
    h0 ~ N(0,1).  Activations in io_dtype (bf16 by default), the per-head vectors and the
    state in fp32."""
    g = _gen(device, seed)
    bf = io_dtype
    x = _randn((batch, seqlen, nheads, headdim), g, device).to(bf)
    delta = F.softplus(_randn((batch, seqlen, nheads), g, device, shift=delta_shift)).to(bf)
    Bm = _randn((batch, seqlen, ngroups, dstate), g, device).to(bf)
    Cm = _randn((batch, seqlen, ngroups, dstate), g, device).to(bf)
    z = _randn((batch, seqlen, nheads, headdim), g, device).to(bf) if gate else None
    A = -4.0 * torch.arange(1, nheads + 1, dtype=torch.float32, device=device) / nheads
    Dskip = _randn((nheads,), g, device) if skip else None
    hinit = _randn((batch, nheads, headdim, dstate), g, device) if h0 else None
    return dict(x=x, delta=delta, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=z, h0=hinit)


def make_ssd_config_inputs(cfg: SsdConfig, device="cpu", **overrides):
    kw = dict(batch=cfg.batch, seqlen=cfg.seqlen, nheads=cfg.nheads, headdim=cfg.headdim,
              ngroups=cfg.ngroups, dstate=cfg.dstate, seed=cfg.seed)
    kw.update(overrides)
    return make_ssd_inputs(device=device, **kw)
