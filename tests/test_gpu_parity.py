"""Parity of the HIP path against the fp64 oracle (needs an MI355X).

Small and medium shapes are compared on every output element; the full-size
workloads run in the same launch configuration the benchmark times and are
compared on sampled channels (all time steps of each sampled channel, plus
its final state), which the oracle can compute one channel at a time.
"""
import numpy as np
import pytest
import torch

import selective_state_space_59_amd as ssm
from selective_state_space_59_amd import workloads as W
from tests.gpu_helpers import TOL, assert_close, oracle_scan, to64

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_scan(inp, delta_softplus=False, delta_bias=None, final=True):
    return ssm.selective_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"],
                                  Dskip=inp.get("Dskip"), z=inp.get("z"),
                                  delta_bias=delta_bias, delta_softplus=delta_softplus,
                                  conv_w=inp.get("conv_w"), conv_b=inp.get("conv_b"),
                                  h0=inp.get("h0"), return_final_state=final)


def check_full(inp, tol, **kw):
    y, hf = run_scan(inp, **kw)
    torch.cuda.synchronize()
    yr, hr = oracle_scan(inp, **kw)
    e1 = assert_close(to64(y), yr, tol, "y")
    e2 = assert_close(to64(hf), hr, tol, "h_final")
    return max(e1, e2)


CASES = [
    # name, B, L, D, N, dtype, extra
    ("tiny_f32", 1, 64, 16, 4, torch.float32, {}),
    ("ragged_bf16", 2, 300, 200, 16, torch.bfloat16, {}),
    ("conv_bf16", 2, 257, 130, 16, torch.bfloat16, dict(conv_k=4)),
    ("long_bf16", 1, 5000, 70, 16, torch.bfloat16, dict(delta_shift=3.0)),
    ("h0_f32_n16", 3, 129, 65, 16, torch.float32, dict(h0=True)),
    ("n1_f32", 2, 63, 33, 1, torch.float32, dict(h0=True)),
    ("n3_f32", 1, 65, 64, 3, torch.float32, {}),
    ("n8_bf16", 2, 100, 100, 8, torch.bfloat16, dict(h0=True)),
    ("n15_f32", 1, 40, 129, 15, torch.float32, {}),
    ("L1_f32", 3, 1, 17, 16, torch.float32, dict(h0=True)),
    ("D1_bf16", 2, 500, 1, 16, torch.bfloat16, {}),
    ("nogate_noskip_f32", 2, 77, 90, 16, torch.float32, dict(gate=False, skip=False)),
    ("conv_k2_f32", 1, 50, 70, 16, torch.float32, dict(conv_k=2, h0=True)),
    ("conv_k1_f32", 1, 20, 10, 4, torch.float32, dict(conv_k=1)),
    ("conv_k3_bf16", 2, 33, 64, 16, torch.bfloat16, dict(conv_k=3)),
    ("L4097_bf16", 1, 4097, 64, 16, torch.bfloat16, {}),
    # shapes whose launch uses wide workgroups (several waves per tile)
    ("wide16_partial_bf16", 16, 33, 3000, 16, torch.bfloat16, {}),
    ("wide9_generic_bf16", 8, 40, 2050, 16, torch.bfloat16, dict(conv_k=4)),
    ("wide13_generic_f32", 6, 21, 4099, 16, torch.float32, dict(h0=True)),
    ("wide16_f32_conv", 24, 18, 2000, 16, torch.float32, dict(conv_k=4)),
    ("wide_n5_bf16", 32, 19, 1536, 5, torch.bfloat16, dict(h0=True)),
    # few channels and long sequences: scanned as concurrent segments
    ("seg4_bf16", 1, 8192, 64, 16, torch.bfloat16, dict(delta_shift=3.0)),
    ("seg2_f32_h0", 1, 6000, 40, 16, torch.float32, dict(h0=True)),
    ("seg2_conv_bf16", 2, 5000, 24, 16, torch.bfloat16, dict(conv_k=4)),
    ("seg2_n5_f32", 1, 4500, 30, 5, torch.float32, dict(h0=True)),
]


@pytest.mark.parametrize("name,B,L,D,N,dt,extra", CASES, ids=[c[0] for c in CASES])
def test_scan_matches_oracle(name, B, L, D, N, dt, extra):
    print("case", name, B, L, D, N, dt, extra, flush=True)
    inp = W.make_scan_inputs(B, L, D, N, io_dtype=dt, seed=1000 + L + D, device=DEV, **extra)
    check_full(inp, TOL[dt])


def test_c1_config_full():
    cfg = W.C1_TINY
    inp = W.make_config_inputs(cfg, device=DEV)
    check_full(inp, TOL[cfg.io_dtype])


def test_softplus_with_bias():
    inp = W.make_scan_inputs(2, 150, 96, 16, io_dtype=torch.float32, seed=7, device=DEV)
    raw = torch.randn(inp["delta"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(8))
    inp["delta"] = (2.0 * raw).contiguous()
    bias = torch.randn(96, device=DEV, generator=torch.Generator(DEV).manual_seed(9))
    check_full(inp, 1e-4, delta_softplus=True, delta_bias=bias)


def test_zero_and_positive_A():
    inp = W.make_scan_inputs(1, 120, 64, 16, io_dtype=torch.float32, seed=10, device=DEV, h0=True)
    A = inp["A"].clone()
    A[:, 0] = 0.0          # integrator channels: Bbar = dt * B
    A[5, :] = 0.0
    A[7, 3] = 0.05         # mildly unstable mode
    inp["A"] = A
    check_full(inp, 1e-4)


def test_segments_with_undecaying_entries():
    # A = 0 (and A > 0) entries never forget the entering state, so every
    # later segment is rescanned whole from its true entering state.
    inp = W.make_scan_inputs(1, 5000, 32, 16, io_dtype=torch.float32, seed=14, device=DEV, h0=True)
    A = inp["A"].clone()
    A[:, 0] = 0.0
    A[3, 5] = 1e-3
    inp["A"] = A
    check_full(inp, 1e-4)


def test_zero_step_holds_state():
    inp = W.make_scan_inputs(2, 40, 70, 16, io_dtype=torch.bfloat16, seed=11, device=DEV,
                             h0=True, gate=False)
    inp["delta"] = torch.zeros_like(inp["delta"])
    y, hf = run_scan(inp)
    torch.cuda.synchronize()
    # The state is carried as A h and divided by A on the way out: one
    # rounding at most, otherwise held exactly.
    assert torch.allclose(hf, inp["h0"], rtol=2.5e-7, atol=0.0)
    yr, _ = oracle_scan(inp)
    assert_close(to64(y), yr, 1e-2, "y")


def test_large_step_resets_state():
    inp = W.make_scan_inputs(1, 30, 64, 16, io_dtype=torch.float32, seed=12, device=DEV,
                             h0=True, gate=False, skip=False)
    inp["delta"] = torch.full_like(inp["delta"], 1e3)
    y, hf = run_scan(inp)
    torch.cuda.synchronize()
    ref = -(inp["Bm"][0, -1][None, :] * inp["x"][0, -1][:, None]) / inp["A"]
    assert_close(to64(hf[0]), to64(ref), 1e-6, "h_final")


def test_empty_sequence_copies_h0():
    inp = W.make_scan_inputs(2, 0, 32, 16, io_dtype=torch.float32, seed=13, device=DEV, h0=True)
    y, hf = run_scan(inp)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(hf, inp["h0"])
    inp["h0"] = None
    _, hf = run_scan(inp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hf) == 0


def _sampled(cfg, nsample, seed=0):
    g = np.random.default_rng(seed)
    b = g.integers(0, cfg.batch, nsample)
    d = g.choice(cfg.dim, nsample, replace=False)
    d[0], d[-1] = 0, cfg.dim - 1
    return b, d


@pytest.mark.parametrize("cfg", [W.C2_130M, W.C3_2P8B_CONV, W.C4_DNA_1M], ids=lambda c: c.name)
def test_full_size_config_sampled(cfg):
    print("config", cfg.name, flush=True)
    inp = W.make_config_inputs(cfg, device=DEV)
    y, hf = run_scan(inp, final=True)
    torch.cuda.synchronize()
    nsample = 6 if cfg.seqlen > 100000 else 12
    res = oracle_scan(inp, channels=_sampled(cfg, nsample))
    tol = TOL[cfg.io_dtype]
    for b, ds, yr, hr in res:
        dsel = torch.tensor(ds, device=DEV)
        assert_close(to64(y[b].index_select(1, dsel)), yr, tol, "%s y b=%d" % (cfg.name, b))
        assert_close(to64(hf[b].index_select(0, dsel)), hr, tol, "%s h b=%d" % (cfg.name, b))
    assert torch.isfinite(y.float()).all()
    del inp, y, hf
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- conv kernel
@pytest.mark.parametrize("B,L,D,K,dt", [(2, 100, 130, 4, torch.bfloat16),
                                        (1, 65, 64, 3, torch.float32),
                                        (3, 1, 7, 4, torch.float32),
                                        (1, 200, 33, 1, torch.bfloat16),
                                        # 16-byte channel groups (D a multiple of 8 / 4)
                                        (2, 100, 136, 4, torch.bfloat16),
                                        (1, 70, 64, 2, torch.bfloat16),
                                        (2, 37, 1536, 4, torch.bfloat16),
                                        (1, 40, 16, 1, torch.bfloat16),
                                        (2, 45, 20, 4, torch.float32)])
def test_conv1d_silu_matches_oracle(B, L, D, K, dt):
    g = torch.Generator(DEV).manual_seed(B * 1000 + L)
    x = torch.randn(B, L, D, device=DEV, generator=g).to(dt)
    w = 0.5 * torch.randn(D, K, device=DEV, generator=g)
    bias = torch.randn(D, device=DEV, generator=g)
    u = ssm.causal_conv1d_silu(x, w, bias)
    torch.cuda.synchronize()
    ref = oracle.causal_conv1d_silu(to64(x), to64(w), to64(bias))
    assert_close(to64(u), ref, TOL[dt], "u")


# ---------------------------------------------------------------- decode step
def _decode(inp, steps, y_dtype):
    st = inp["state0"].clone()
    ys = []
    for t in range(steps):
        ys.append(ssm.state_update(st, inp["x"][t], inp["delta"][t], inp["A"], inp["Bm"][t],
                                   inp["Cm"][t], Dskip=inp["Dskip"], z=inp["z"][t]))
    torch.cuda.synchronize()
    return torch.stack(ys), st


@pytest.mark.parametrize("B,D,N,dt", [(3, 70, 16, torch.float32), (4, 64, 5, torch.bfloat16),
                                      (2, 33, 16, torch.bfloat16), (1, 1, 1, torch.float32),
                                      (2, 300, 16, torch.bfloat16)])  # 128-channel tiles, ragged
def test_state_update_matches_oracle(B, D, N, dt):
    inp = W.make_decode_inputs(B, D, N, 8, io_dtype=dt, seed=B + D + N, device=DEV)
    ys, st = _decode(inp, 8, dt)
    ref = inp["state0"].double().cpu().numpy()
    for t in range(8):
        yr, ref = oracle.state_update(ref, to64(inp["x"][t]), to64(inp["delta"][t]), to64(inp["A"]),
                                      to64(inp["Bm"][t]), to64(inp["Cm"][t]),
                                      Dskip=to64(inp["Dskip"]), z=to64(inp["z"][t]))
        assert_close(to64(ys[t]), yr, TOL[dt], "y step %d" % t)
    assert_close(to64(st), ref, TOL[dt], "state")


def test_state_update_small_and_zero_A():
    # |A| < 1/16 anywhere in a wave switches it to the phi form (A = 0 included).
    inp = W.make_decode_inputs(3, 48, 16, 4, io_dtype=torch.float32, seed=21, device=DEV)
    A = inp["A"].clone()
    A[:, 0] = 0.0
    A[7, 3] = 0.01
    A[20, 9] = -0.03
    inp["A"] = A
    ys, st = _decode(inp, 4, torch.float32)
    ref = inp["state0"].double().cpu().numpy()
    for t in range(4):
        yr, ref = oracle.state_update(ref, to64(inp["x"][t]), to64(inp["delta"][t]), to64(A),
                                      to64(inp["Bm"][t]), to64(inp["Cm"][t]),
                                      Dskip=to64(inp["Dskip"]), z=to64(inp["z"][t]))
        assert_close(to64(ys[t]), yr, 1e-4, "y step %d" % t)
    assert_close(to64(st), ref, 1e-4, "state")


def test_state_update_capped_grid_sampled_rows():
    """More (batch row, channel run) tiles than one launch grid holds (2^22 workgroups):
    each workgroup takes further tiles in turn; the oracle checks three rows."""
    B = (1 << 22) + 2
    inp = W.make_decode_inputs(B, 8, 16, 2, io_dtype=torch.bfloat16, seed=77, device=DEV)
    ys, st = _decode(inp, 2, torch.bfloat16)
    rows = [0, 1 << 21, B - 1]
    ref = inp["state0"][rows].double().cpu().numpy()
    for t in range(2):
        yr, ref = oracle.state_update(ref, to64(inp["x"][t][rows]), to64(inp["delta"][t][rows]),
                                      to64(inp["A"]), to64(inp["Bm"][t][rows]),
                                      to64(inp["Cm"][t][rows]), Dskip=to64(inp["Dskip"]),
                                      z=to64(inp["z"][t][rows]))
        assert_close(to64(ys[t][rows]), yr, TOL[torch.bfloat16], "y step %d" % t)
    assert_close(to64(st[rows]), ref, TOL[torch.bfloat16], "state")
    del inp, ys, st
    torch.cuda.empty_cache()


def test_decode_config_sampled_rows():
    cfg = W.C5_DECODE
    inp = W.make_decode_config_inputs(cfg, device=DEV)
    ys, st = _decode(inp, cfg.steps, cfg.io_dtype)
    rows = [0, 97, cfg.batch - 1]
    ref = inp["state0"][rows].double().cpu().numpy()
    for t in range(cfg.steps):
        yr, ref = oracle.state_update(ref, to64(inp["x"][t][rows]), to64(inp["delta"][t][rows]),
                                      to64(inp["A"]), to64(inp["Bm"][t][rows]),
                                      to64(inp["Cm"][t][rows]), Dskip=to64(inp["Dskip"]),
                                      z=to64(inp["z"][t][rows]))
        assert_close(to64(ys[t][rows]), yr, TOL[cfg.io_dtype], "y step %d" % t)
    assert_close(to64(st[rows]), ref, TOL[cfg.io_dtype], "state")
