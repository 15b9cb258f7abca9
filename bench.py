"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]

A step is one selective-scan forward over one batch of the Mamba-130M-like
layer workload (B=8, L=2048, D=1536, N=16, bf16 I/O, fp32 state, SiLU gate,
D skip).  Three independent input sets (3 x 202 MB) rotate between steps, so
the 256 MB last-level cache cannot hold the next step's inputs.  Inputs are
resident in HBM before the timed region starts.

Prints ONE JSON line.  `value` is algorithmic HBM bytes per second (GB/s):
the minimum bytes a scan must move (each of x, delta, z read once, y written
once, the B/C rows read once, A and D once) divided by the time per step.
`roofline` relates the kernel to the MI355X HBM peak and to the vector-ALU
peak; `cpu_baseline` times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# Vector ALU: 256 CUs x 4 SIMDs x 16 fp32 lanes per clock x 2.4 GHz = 39.3 T lane-slots/s
# (one fp32 add, mul or fma per lane per slot; no packed-fp32 forms; exp2 takes two slots).
VALU_PEAK_LANE_SLOTS = 256 * 4 * 16 * 2.4e9
# Algorithmic VALU work of one state update (b, t, d, n) of the ZOH scan:
#   dt*A (1), exp (2), B*x (1), (Abar - 1) * Bx / A folded into one fma (1),
#   Abar*h + Bbar*x (1), C*h accumulated into y (1)  ->  7 lane-slots.
SLOTS_PER_UPDATE = 7


def scan_algorithmic_bytes(B, L, D, N, io_bytes, conv_k=0, final_state=False, h0=False,
                           gate=True, skip=True):
    """Minimum HBM bytes of one scan: x, delta, (z) read and y written once per element;
    B and C once per (b, t); A, D skip and conv weights once; states once if used."""
    elems = B * L * D
    per_elem = (3 + (1 if gate else 0)) * io_bytes
    total = elems * per_elem + 2 * B * L * N * io_bytes + 4 * D * N
    if skip:
        total += 4 * D
    if conv_k:
        total += 4 * D * conv_k
    if final_state:
        total += 4 * B * D * N
    if h0:
        total += 4 * B * D * N
    return total


def decode_algorithmic_bytes(B, D, N, io_bytes, gate=True, skip=True, conv_k=0):
    """One decode step: state read + written, x, delta, (z) read, y written, B/C rows, A, D;
    with a conv window also the window read + written and the conv weights and bias."""
    conv = (2 * (conv_k - 1) * io_bytes * B * D + 4 * D * conv_k + 4 * D) if conv_k else 0
    return (8 * B * D * N + (3 + (1 if gate else 0)) * io_bytes * B * D + 2 * B * N * io_bytes
            + 4 * D * N + (4 * D if skip else 0) + conv)


# The headline metric this benchmark reports.
METRIC = "selective-scan HBM GB/s and % of roofline; (B\u00b7L\u00b7D) elems/s; decode steps/s"


def _counter_traffic(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel source (matched by hash); else None."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except Exception:
        return None
    ent = rec.get(kernel_key)
    if not ent:
        return None
    from selective_state_space_59_amd import build as B
    if ent.get("source_hash") != B.source_hash(ent.get("sources")):
        return None
    return ent.get("bytes_per_launch")


def time_launches(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per launch


def bench_scan(cfg, steps, warmup, nsets=3, final_state=False):
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    sets = [W.make_config_inputs(cfg, device=dev, seed=cfg.seed + 100 * k) for k in range(nsets)]
    ys = [torch.empty_like(s["x"]) for s in sets]
    hfs = [torch.empty(cfg.batch, cfg.dim, cfg.dstate, device=dev) if final_state else None
           for _ in sets]

    def run(i):
        s = sets[i % nsets]
        ssm.selective_scan_fwd(s["x"], s["delta"], s["A"], s["Bm"], s["Cm"], Dskip=s["Dskip"],
                               z=s["z"], conv_w=s["conv_w"], y=ys[i % nsets],
                               h_final=hfs[i % nsets])

    ms = time_launches(run, steps, warmup)
    nbytes = scan_algorithmic_bytes(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate,
                                    2 if cfg.io_dtype == torch.bfloat16 else 4, cfg.conv_k,
                                    final_state, gate=cfg.gate, skip=cfg.skip)
    first = sets[0]
    del sets, ys, hfs
    torch.cuda.empty_cache()
    return ms, nbytes, first


def bwd_algorithmic_bytes(B, L, D, N, io_bytes, gate=True, skip=True, conv_k=0):
    """Backward pass: x, delta, (z), dy and B, C read once; dx, ddelta, (dz) written once;
    dB, dC written in fp32; A read and dA written; (Dskip read and dDskip written);
    (conv taps read and their gradients written)."""
    io = (3 + (1 if gate else 0)) * io_bytes * B * L * D      # x, delta, z, dy
    io += (2 + (1 if gate else 0)) * io_bytes * B * L * D     # dx, ddelta, dz
    bc = 2 * io_bytes * B * L * N + 2 * 4 * B * L * N
    conv = 2 * 4 * D * conv_k if conv_k else 0
    return io + bc + 2 * 4 * D * N + (2 * 4 * D if skip else 0) + conv


def bench_bwd(cfg, steps, warmup):
    """The backward pass of `cfg` (no conv prologue) on one seeded input set."""
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    s = W.make_config_inputs(cfg, device=dev)
    dy = torch.randn(s["x"].shape, device=dev,
                     generator=torch.Generator(dev).manual_seed(cfg.seed + 60)).to(cfg.io_dtype)

    def run(_):
        ssm.selective_scan_bwd(s["x"], s["delta"], s["A"], s["Bm"], s["Cm"], dy, Dskip=s["Dskip"],
                               z=s["z"], conv_w=s["conv_w"])

    ms = time_launches(run, steps, warmup)
    nbytes = bwd_algorithmic_bytes(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate,
                                   2 if cfg.io_dtype == torch.bfloat16 else 4,
                                   gate=cfg.gate, skip=cfg.skip, conv_k=cfg.conv_k)
    del s, dy
    torch.cuda.empty_cache()
    return ms, nbytes


def block_gemm_flops(cfg):
    """Multiply-adds x 2 of the block's projections per call: in_proj (2D x d_model),
    x_proj ((R + 2N) x D), dt_proj (D x R) and out_proj (d_model x D) over B*L rows."""
    M = cfg.batch * cfg.seqlen
    D, dm, R, N = cfg.d_inner, cfg.d_model, cfg.dt_rank, cfg.dstate
    return 2 * M * (2 * D * dm + (R + 2 * N) * D + D * R + dm * D)


def bench_block(cfg, steps, warmup):
    """The whole Mamba block forward of `cfg` (one plan, one workspace, output rotated
    between two buffers so no call writes what the previous one is still reading)."""
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    s = W.make_block_config_inputs(cfg, device=dev)
    plan = ssm.BlockPlan(cfg.batch, cfg.seqlen, cfg.d_model, cfg.d_inner, cfg.dstate, cfg.dt_rank,
                         cfg.conv_k)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s["h"]) for _ in range(2)]
    names = ("norm_w", "w_in", "conv_w", "conv_b", "w_x", "w_dt", "dt_bias", "A", "Dskip", "w_out")

    def run(i):
        ssm.mamba_block_fwd(s["h"], *(s[k] for k in names), out=outs[i % 2], plan=plan, workspace=ws)

    ms = time_launches(run, steps, warmup)
    del s, outs, ws
    plan.close()
    torch.cuda.empty_cache()
    return ms


def bench_decode(cfg, reps=3, conv_k=0):
    """Decode steps of `cfg`; with conv_k, each step also runs the conv prologue on
    its (B, conv_k-1, D) window and shifts it (weights N(0, 0.5), seeded)."""
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    inp = W.make_decode_config_inputs(cfg, device=dev)
    st = inp["state0"].clone()
    ys = torch.empty(cfg.steps, cfg.batch, cfg.dim, dtype=cfg.io_dtype, device=dev)
    conv = {}
    if conv_k:
        g = torch.Generator(dev).manual_seed(cfg.seed + 50)
        conv = dict(conv_w=0.5 * torch.randn(cfg.dim, conv_k, device=dev, generator=g),
                    conv_b=torch.randn(cfg.dim, device=dev, generator=g),
                    conv_state=torch.randn(cfg.batch, conv_k - 1, cfg.dim, device=dev,
                                           generator=g).to(cfg.io_dtype))

    # Each step's arguments are marshalled and checked once, up front; the timed
    # calls go straight to the C ABI.
    steps = [ssm.state_update_args(st, inp["x"][t], inp["delta"][t], inp["A"], inp["Bm"][t],
                                   inp["Cm"][t], Dskip=inp["Dskip"], z=inp["z"][t], y=ys[t],
                                   **conv)[0] for t in range(cfg.steps)]
    L = ssm.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def step(t):
        st_ = L.ssm_state_update(ctypes.byref(steps[t]), stream)
        if st_ != 0:
            raise RuntimeError("ssm_state_update: %s" % ssm.status_string(st_))

    def run_all(_):
        for t in range(cfg.steps):
            step(t)

    hot_ms = time_launches(run_all, reps, 1) / cfg.steps
    # Cold: evict the last-level cache (write 1 GiB) before each timed step.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    cold = []
    for t in range(cfg.steps):
        flush.fill_(float(t))
        start.record()
        step(t)
        stop.record()
        torch.cuda.synchronize()
        cold.append(start.elapsed_time(stop))
    cold.sort()
    cold_ms = cold[len(cold) // 2]
    nbytes = decode_algorithmic_bytes(cfg.batch, cfg.dim, cfg.dstate,
                                      2 if cfg.io_dtype == torch.bfloat16 else 4, conv_k=conv_k)
    del inp, st, ys, flush, conv, steps
    torch.cuda.empty_cache()
    return hot_ms, cold_ms, nbytes


def cpu_baseline(inp, cfg, min_seconds=10.0, max_passes=60):
    """The fp64 oracle as it stands, on the host cores, over the whole workload of one input
    set, repeated until about `min_seconds` of CPU work have run (the mean pass is reported)."""
    import oracle
    nthreads = oracle.default_threads()
    Lb = cfg.seqlen
    f = lambda t: None if t is None else t[:, :Lb].double().cpu().numpy()
    g = lambda t: None if t is None else t.double().cpu().numpy()
    args = (f(inp["x"]), f(inp["delta"]), g(inp["A"]), f(inp["Bm"]), f(inp["Cm"]))
    kw = dict(Dskip=g(inp["Dskip"]), z=f(inp["z"]), conv_w=g(inp["conv_w"]), nthreads=nthreads)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.selective_scan(*args, **kw)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds or passes >= max_passes:
            break
    total = time.perf_counter() - t0
    dt = total / passes
    elems = cfg.batch * Lb * cfg.dim
    nbytes = scan_algorithmic_bytes(cfg.batch, Lb, cfg.dim, cfg.dstate,
                                    2 if str(inp["x"].dtype).endswith("bfloat16") else 4,
                                    cfg.conv_k, gate=cfg.gate, skip=cfg.skip)
    return dict(value=round(nbytes / dt / 1e9, 4), unit="GB/s", cores=nthreads, kind="oracle",
                elems_per_s=round(elems / dt, 1), seconds_per_pass=round(dt, 3),
                seconds_total=round(total, 2), passes=passes,
                sample="%d full passes of the workload (B=%d, L=%d, D=%d, N=%d), fp64, "
                       "%d threads over independent channels; mean pass reported"
                       % (passes, cfg.batch, Lb, cfg.dim, cfg.dstate, nthreads))


def ssd_algorithmic(cfg, chunk=64):
    """HBM bytes and matrix FLOPs of one SSD layer call.  Bytes: x, z read and y written
    (bf16, B*L*H*P each), delta (B*L*H) and B, C (B*L*G*N each) read, h_final written (fp32).
    FLOPs of the chunked algorithm (2 per multiply-add), per (batch, head, chunk of Q): the
    causal half of C.B^T (Q(Q+1)/2 * N), its product with X (Q(Q+1)/2 * P), C H^T (Q N P) and
    the state update B^T X (Q N P)."""
    B, L, H, P, G, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    nbytes = 3 * 2 * B * L * H * P + 2 * B * L * H + 2 * 2 * B * L * G * N + 4 * B * H * P * N
    Q = chunk
    per_chunk = 2 * (Q * (Q + 1) // 2 * (N + P) + 2 * Q * N * P)
    flops = per_chunk * B * H * ((L + Q - 1) // Q)
    return nbytes, flops


def bench_ssd(cfg, steps, warmup):
    """The SSD (Mamba-2) layer of `cfg` on one seeded input set, with its final state."""
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    s = W.make_ssd_config_inputs(cfg, device=dev)
    y = torch.empty_like(s["x"])
    hf = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device=dev)

    def run(_):
        ssm.ssd_fwd(s["x"], s["delta"], s["A"], s["Bm"], s["Cm"], Dskip=s["Dskip"], z=s["z"],
                    y=y, h_final=hf)

    ms = time_launches(run, steps, warmup)
    del s, y, hf
    torch.cuda.empty_cache()
    return ms


def ssd_entry(cfg, steps, warmup):
    ms = bench_ssd(cfg, steps, warmup)
    nbytes, flops = ssd_algorithmic(cfg)
    tokens = cfg.batch * cfg.seqlen
    return dict(ms=round(ms, 4), tokens_per_s=round(tokens / (ms * 1e-3), 1),
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                algorithmic_bytes=nbytes, chunked_flops=flops,
                tflops=round(flops / (ms * 1e-3) / 1e12, 2),
                config=dict(batch=cfg.batch, seq_len=cfg.seqlen, nheads=cfg.nheads,
                            headdim=cfg.headdim, ngroups=cfg.ngroups, dstate=cfg.dstate,
                            io_dtype="bf16", chunk=64))


def ssd_step_algorithmic(cfg):
    """HBM bytes of one SSD decode step over the batch: the fp32 state read and written
    (B*H*P*N each), x, z read and y written (bf16, B*H*P each), delta (B*H) and B, C
    (B*G*N each) read, A and D (fp32, H each)."""
    B, H, P, G, N = cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    return 2 * 4 * B * H * P * N + 3 * 2 * B * H * P + 2 * B * H + 2 * 2 * B * G * N + 2 * 4 * H


def bench_ssd_step(cfg, reps=10):
    """`cfg.seqlen` decode steps of the SSD layer on a resident state: hot (steps back to
    back, per step) and cold (the last-level cache flushed before each timed step)."""
    import torch
    import selective_state_space_59_amd as ssm
    from selective_state_space_59_amd import workloads as W
    dev = "cuda:0"
    s = W.make_ssd_config_inputs(cfg, device=dev, h0=True)
    per_step = {k: s[k].transpose(0, 1).contiguous() for k in ("x", "delta", "Bm", "Cm", "z")}
    st = s["h0"]
    ys = torch.empty_like(per_step["x"])
    T = cfg.seqlen

    args = [ssm.ssd_step_args(st, per_step["x"][t], per_step["delta"][t], s["A"],
                              per_step["Bm"][t], per_step["Cm"][t], Dskip=s["Dskip"],
                              z=per_step["z"][t], y=ys[t])[0] for t in range(T)]
    L = ssm.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def step(t):
        st_ = L.ssm_ssd_step(ctypes.byref(args[t]), stream)
        if st_ != 0:
            raise RuntimeError("ssm_ssd_step: %s" % ssm.status_string(st_))

    def run_all(_):
        for t in range(T):
            step(t)

    hot_ms = time_launches(run_all, reps, 1) / T
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    cold = []
    for t in range(T):
        flush.fill_(float(t))
        start.record()
        step(t)
        stop.record()
        torch.cuda.synchronize()
        cold.append(start.elapsed_time(stop))
    cold.sort()
    cold_ms = cold[len(cold) // 2]
    del s, per_step, st, ys, flush, args
    torch.cuda.empty_cache()
    return hot_ms, cold_ms


def ssd_step_entry(cfg):
    hot, cold = bench_ssd_step(cfg)
    db = ssd_step_algorithmic(cfg)
    return dict(hot_ms_per_step=round(hot, 5), cold_ms_per_step=round(cold, 5),
                hot_tokens_per_s=round(cfg.batch * 1e3 / hot, 1),
                cold_gbs=round(db / (cold * 1e-3) / 1e9, 2),
                cold_frac_hbm=round(db / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                hot_gbs=round(db / (hot * 1e-3) / 1e9, 2), algorithmic_bytes_per_step=db,
                config=dict(batch=cfg.batch, nheads=cfg.nheads, headdim=cfg.headdim,
                            ngroups=cfg.ngroups, dstate=cfg.dstate, steps=cfg.seqlen,
                            io_dtype="bf16", state_dtype="f32"))


def block_entry(cfg, steps, warmup):
    ms = bench_block(cfg, steps, warmup)
    fl = block_gemm_flops(cfg)
    tokens = cfg.batch * cfg.seqlen
    return dict(ms=round(ms, 4), tokens_per_s=round(tokens / (ms * 1e-3), 1),
                gemm_flops=fl, gemm_tflops_over_block_time=round(fl / (ms * 1e-3) / 1e12, 2),
                config=dict(batch=cfg.batch, seq_len=cfg.seqlen, d_model=cfg.d_model,
                            d_inner=cfg.d_inner, dstate=cfg.dstate, dt_rank=cfg.dt_rank,
                            conv_k=cfg.conv_k, io_dtype="bf16"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("block", "ssd", "ssd_long", "ssd_decode"),
                    help="only time the 130M-like Mamba block forward, the Mamba-2 130M-like "
                         "SSD layer, that layer on one 65536-token sequence, or the 2.7B-like "
                         "SSD decode step, and print its numbers")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (fp32) five times; its "
                         "FETCH_SIZE / WRITE_SIZE counters scale the scan's traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the selective scan is benchmarked on a single "
              "MI355X (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_59_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = args.copy_calibration << 18
        src = torch.randn(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 5}))
        return

    if args.only == "block":
        print(json.dumps({W.B2_130M.name: block_entry(W.B2_130M, args.steps, args.warmup)}), flush=True)
        return
    if args.only in ("ssd", "ssd_long"):
        c = W.S2_MAMBA2_130M if args.only == "ssd" else W.S4_MAMBA2_LONG
        print(json.dumps({c.name: ssd_entry(c, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "ssd_decode":
        c = W.S5_MAMBA2_DECODE
        print(json.dumps({c.name: ssd_step_entry(c)}), flush=True)
        return

    cfg = W.C2_130M
    print("bench: %s, %d warmup + %d timed steps" % (cfg.name, args.warmup, args.steps),
          file=sys.stderr, flush=True)
    ms, nbytes, first = bench_scan(cfg, args.steps, args.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    elems = cfg.elems
    upd = elems * cfg.dstate
    traffic = _counter_traffic("scan_" + cfg.name)
    # The scan is bound by the vector ALU (7 lane-slots per update against
    # 8 bytes per 16 updates of HBM traffic); the HBM view is reported beside it.
    alu = SLOTS_PER_UPDATE * upd / (ms * 1e-3) / 1e12
    alu_peak = VALU_PEAK_LANE_SLOTS / 1e12
    roof = dict(bound="alu", achieved=round(alu, 3), peak=round(alu_peak, 2),
                unit="T VALU lane-slots/s", frac=round(alu / alu_peak, 4), traffic=traffic,
                algorithmic_slots_per_update=SLOTS_PER_UPDATE, state_updates_per_launch=upd,
                launch_ms=round(ms, 5), state_updates_per_s=round(upd / (ms * 1e-3), 1),
                hbm=dict(achieved=round(gbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), algorithmic_bytes_per_launch=nbytes))

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen,
                   "dim": cfg.dim, "dstate": cfg.dstate, "io_dtype": "bf16",
                   "gate": cfg.gate, "skip": cfg.skip, "input_sets_rotated": 3,
                   "parallelism": "single GPU"},
        "elems_per_s": round(elems / (ms * 1e-3), 1),
        "roofline": roof,
    }

    if not args.no_extras:
        extra = {}
        for c in (W.C3_2P8B_CONV, W.C4_DNA_1M):
            print("bench extra: %s" % c.name, file=sys.stderr, flush=True)
            reps, warm = (5, 2) if c.seqlen > 100000 else (30, 5)
            cms, cb, _ = bench_scan(c, reps, warm, nsets=1, final_state=c.final_state)
            extra[c.name] = dict(ms=round(cms, 4), gbs=round(cb / (cms * 1e-3) / 1e9, 2),
                                 frac_hbm=round(cb / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 elems_per_s=round(c.elems / (cms * 1e-3), 1),
                                 algorithmic_bytes=cb)
        # the backward pass (gradients of every input) of the 130M-like layer
        # and of the 2.8B-like layer with its conv prologue
        for c in (W.C2_130M, W.C3_2P8B_CONV):
            name = c.name + "_backward"
            print("bench extra: %s" % name, file=sys.stderr, flush=True)
            bms, bb = bench_bwd(c, 10, 2)
            extra[name] = dict(ms=round(bms, 4), gbs=round(bb / (bms * 1e-3) / 1e9, 2),
                               frac_hbm=round(bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               state_updates_per_s=round(c.elems * c.dstate / (bms * 1e-3), 1),
                               algorithmic_bytes=bb)
        # the decode config, and the same with the d_conv = 4 window of the
        # prefill -> decode handoff
        for name, k in ((W.C5_DECODE.name, 0), (W.C5_DECODE.name + "_conv4_window", 4)):
            print("bench extra: %s" % name, file=sys.stderr, flush=True)
            hot, cold, db = bench_decode(W.C5_DECODE, conv_k=k)
            extra[name] = dict(
                hot_ms_per_step=round(hot, 5), cold_ms_per_step=round(cold, 5),
                hot_steps_per_s=round(1e3 / hot, 1), cold_steps_per_s=round(1e3 / cold, 1),
                cold_gbs=round(db / (cold * 1e-3) / 1e9, 2),
                cold_frac_hbm=round(db / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                hot_gbs=round(db / (hot * 1e-3) / 1e9, 2), algorithmic_bytes_per_step=db)
        # the whole Mamba block around the scan (RMSNorm, projections, conv, scan, residual)
        print("bench extra: %s" % W.B2_130M.name, file=sys.stderr, flush=True)
        extra[W.B2_130M.name] = block_entry(W.B2_130M, 30, 5)
        # the SSD (Mamba-2) layer at the 130M-like width with N = 128
        print("bench extra: %s" % W.S2_MAMBA2_130M.name, file=sys.stderr, flush=True)
        extra[W.S2_MAMBA2_130M.name] = ssd_entry(W.S2_MAMBA2_130M, 30, 5)
        # one 65536-token sequence at that width: the segmented schedule
        print("bench extra: %s" % W.S4_MAMBA2_LONG.name, file=sys.stderr, flush=True)
        extra[W.S4_MAMBA2_LONG.name] = ssd_entry(W.S4_MAMBA2_LONG, 10, 2)
        # decode steps of a 2.7B-like Mamba-2 layer on its resident fp32 state
        print("bench extra: %s" % W.S5_MAMBA2_DECODE.name, file=sys.stderr, flush=True)
        extra[W.S5_MAMBA2_DECODE.name] = ssd_step_entry(W.S5_MAMBA2_DECODE)
        out["extra"] = extra

    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(first, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
