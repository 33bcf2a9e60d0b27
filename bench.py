"""Benchmark: selective-scan forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one selective_scan_fwd over one batch of the workload (softplus,
discretisation, chunked scan with carries, readout, D skip, SiLU gate, final
state), with every input already resident in HBM.  Default workload: the
2.8B-shaped layer (B=4, D=5120, N=16, L=2048, bf16 I/O, fp32 state).

Prints one JSON line: elements/s (B*L*D) of that workload, the roofline of
its scan kernel (ALU-bound: VALU issue slots per element, see algo_slots)
with the HBM bandwidth alongside, and the CPU fp64 oracle timed on this host
as baseline.  Also reported: the long-sequence scan (B=1, D=256, N=16,
L=2^20, fp32) under "long", the same layer prefilled as four scans resumed
from each other's state under "resume", the decode step (B=256, D=5120,
N=16, 128 steps) under "decode", flushed and back to back, and the causal
conv1d + SiLU ahead of the scan (sequence and decode step) under "conv1d",
the backward scan (selective_scan_bwd, all gradients) of the same layer
under "backward", the same layer in the Mamba-2 SSD form (80 heads of
64 channels, ssd_scan_fwd on the matrix cores) under "ssd", forward-scan
throughput against sequence length (8K to 1M steps at a fixed channel count)
under "l_sweep", and decode-step latency against the number of requests
under "decode" / "batch_sweep".
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
# VALU issue slots per second: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz (one fp32 lane-instruction each)
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def algo_slots(N: int, gate: bool = True, skip: bool = True, softplus: bool = True) -> int:
    """VALU issue slots per element (b, d, t) of the plain recurrence, counting v_exp / v_log /
    v_rcp as 2 slots (they issue at half rate and do not overlap FMAs on gfx950):
      Delta:   bias add + softplus (exp, add, log)            -> 2 + 2*2
      du = Delta*u                                             -> 1
      per n:   Delta*A, exp, du*B, fma(h), fma(C*h)            -> 4 + 2
      skip:    fma(D, u, y)                                    -> 1
      gate:    silu (exp, add, rcp, mul) and the product       -> 3 + 2*2
    """
    s = 1 + 1 + 6 * N
    if softplus:
        s += 1 + 4
    if skip:
        s += 1
    if gate:
        s += 3 + 4
    return s


# HBM traffic of the scan kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE counters, per launch, scaled by
# the same counters' reading for plain copies of known size (FETCH_SIZE x2, WRITE_SIZE x1); null until
# measured for the current kernel.  2: the 2.8B-shaped layer's one scan kernel; 3: the 2^20-step
# sequence's three kernels together (aggregate pass, segment carry, output pass).
TRAFFIC = {2: 359.8e6, 3: 8968.1e6}


def algo_slots_bwd(N: int) -> int:
    """VALU issue slots per element of the plain adjoint-method backward (exp/log/rcp = 2), with
    the forward states recomputed once and Abar kept from the forward half:
      per n, forward:  Delta*A, exp, du*B, fma(h), fma(C*h) for dz, ds*h and its channel sum  -> 8 + 2
      per n, adjoint:  fma(ds*C + lam), fma(lam*B), lam*du and its channel sum, Abar*lam,
                       q = (Abar lam) h, fma(q*A), fma(q*Delta)                               -> 8
      per element:     softplus 6, du = Delta*u 1, sigmoid(z) and silu 7, ds 1, dz 3, du 2,
                       dDelta 2, sigmoid(x) 5, ddelta 1, dD and ddt_bias sums 2                -> 30
    """
    return 18 * N + 30


def algo_bytes(B, D, N, L, es, gate=True, last_state=True):
    """HBM bytes of one scan: u, delta, (z) read, y written; B, C read; A, D, dt_bias; final state."""
    x = B * D * L * es * (3 + (1 if gate else 0))
    bc = 2 * B * N * L * es
    params = D * N * 4 + 2 * D * 4
    return x + bc + params + (B * D * N * 4 if last_state else 0)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[1, 2, 3])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-long", action="store_true", help="skip the long-sequence (L=2^20) scan figure")
    p.add_argument("--no-resume", action="store_true", help="skip the prefill-in-pieces figure")
    p.add_argument("--no-conv", action="store_true", help="skip the causal conv1d figures")
    p.add_argument("--no-bwd", action="store_true", help="skip the backward-scan figure")
    p.add_argument("--no-ssd", action="store_true", help="skip the SSD (Mamba-2 form) figure")
    p.add_argument("--no-sweeps", action="store_true", help="skip the sequence-length and decode-batch sweeps")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the scan, run 5 plain device copies of MIB MiB each (reference dispatches for "
                        "HBM byte counters)")
    return p.parse_args()


def time_scan(torch, gen, ssm, w, steps, warmup, x=None):
    """Time `steps` selective_scan_fwd calls on workload w (or on the inputs x, which carry their
    sizes); inputs resident in HBM.  Host-drawn inputs are copied to the device several times and
    consecutive steps rotate over the copies, enough to exceed the 256 MB last-level cache; inputs
    drawn on the device are used as they are (they are larger than that cache)."""
    import numpy as np
    x = gen.scan_inputs(w) if x is None else x
    B, D, N, L = x["batch"], x["dim"], x["dstate"], x["seqlen"]
    es = 2 if x["dtype"] == "bf16" else 4
    elems = B * D * L
    bytes_step = algo_bytes(B, D, N, L, es)
    copies = 1 if x["u"].is_cuda else max(1, min(4, int(np.ceil(1.0e9 / bytes_step))))
    ins = [{k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()} for _ in range(copies)]
    y = torch.empty_like(ins[0]["u"])
    last = torch.empty((B, D, N), dtype=torch.float32, device="cuda")

    def step(i):
        g = ins[i % copies]
        ssm.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["dt_bias"], True, y=y,
                     last_state=last)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # every launch of the call goes to torch's current stream (the binding passes it), so
    # events recorded on that stream bracket exactly the kernels of the timed steps
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    slots = algo_slots(N)
    tops = elems * slots / (ms * 1e-3) / 1e12
    gbs = bytes_step / (ms * 1e-3) / 1e9
    plan = ssm.scan_plan(B, D, N, L, torch.bfloat16 if x["dtype"] == "bf16" else torch.float32,
                         torch.cuda.get_device_properties(0).multi_processor_count)
    del ins, y, last
    return dict(ms=ms, value=elems / (ms * 1e-3), elems=elems, slots=slots, tops=tops, gbs=gbs,
                bytes_step=bytes_step, copies=copies, plan=plan, wall=t_wall)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs each call on "
              "one device and does not shard across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import selective_scan_02_amd as ssm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ssm.load()
    torch.cuda.set_device(0)
    w = gen.WORKLOADS[args.workload]
    x = gen.scan_inputs(w)
    r = time_scan(torch, gen, ssm, w, args.steps, args.warmup, x)
    B, D, N, L = w.batch, w.dim, w.dstate, w.seqlen
    out = {
        "metric": "selective-scan fwd elements/s (B*L*D_inner)",
        "value": r["value"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "d_inner": D, "d_state": N, "seqlen": L, "io_dtype": w.dtype,
                   "state_dtype": "f32", "parallelism": "single-gpu", "input_copies_rotated": r["copies"],
                   "launch_plan": r["plan"]},
        "roofline": {"bound": "alu", "achieved": r["tops"], "peak": PEAK_VALU_TOPS, "unit": "Tops/s",
                     "frac": r["tops"] / PEAK_VALU_TOPS, "traffic": TRAFFIC.get(args.workload),
                     "ops_per_element": r["slots"], "op": "fp32 VALU issue slot per lane (exp/log/rcp = 2)",
                     "kernel": "scan_chunked_kernel (the call's one launch: the interval plan keeps its ticket and hand-over "
                               "flags in the stream's control block, so nothing is cleared per call)"},
        "hbm": {"achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": r["gbs"] / PEAK_HBM_GBS,
                "bytes_per_step": r["bytes_step"]},
        "wall_s_timed": r["wall"],
    }
    if not args.no_long and args.workload != 3:
        wl = gen.WORKLOADS[3]
        rl = time_scan(torch, gen, ssm, wl, max(10, args.steps // 5), 3)
        out["long"] = {"workload": wl.name, "ms_per_step": rl["ms"], "value": rl["value"], "unit": "elements/s",
                       "roofline": {"bound": "alu", "achieved": rl["tops"], "peak": PEAK_VALU_TOPS, "unit": "Tops/s",
                                    "frac": rl["tops"] / PEAK_VALU_TOPS, "traffic": TRAFFIC.get(3),
                                    "ops_per_element": rl["slots"],
                                    "op": "fp32 VALU issue slot per lane (exp/log/rcp = 2)",
                                    "kernel": "the call's three kernels: aggregate pass, segment carry, output pass "
                                              "(elements counted once)"},
                       "hbm": {"achieved": rl["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": rl["gbs"] / PEAK_HBM_GBS, "bytes_per_step": rl["bytes_step"]},
                       "launch_plan": rl["plan"]}
    if not args.no_sweeps and args.workload == 2:
        out["l_sweep"] = bench_l_sweep(torch, gen, ssm)
    if not args.no_resume and args.workload == 2:
        out["resume"] = bench_resume(torch, gen, ssm, w, x, max(5, args.steps // 5))
    if not args.no_decode:
        out["decode"] = bench_decode(torch, gen, ssm, args)
        if not args.no_sweeps:
            out["decode"]["batch_sweep"] = bench_decode_sweep(torch, gen, ssm)
    if not args.no_conv:
        out["conv1d"] = bench_conv(torch, np, ssm, max(10, args.steps // 2))
        if args.workload == 2:
            out["conv1d"]["fused_scan"] = bench_conv_scan(torch, gen, ssm, w, max(10, args.steps // 2))
            out["conv1d"]["fused_scan_f32"] = bench_conv_scan(torch, gen, ssm, dataclasses.replace(w, dtype="f32"),
                                                              max(10, args.steps // 2))
    if not args.no_bwd and args.workload == 2:
        out["backward"] = bench_bwd(torch, ssm, w, x, max(5, args.steps // 5), r["ms"])
    if not args.no_ssd and args.workload == 2:
        out["ssd"] = bench_ssd(torch, gen, ssm, max(10, args.steps // 2), r["ms"])
    if args.copy_calibration:
        out["copy_calibration"] = copy_calibration(torch, args.copy_calibration)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, gen, x, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


L_SWEEP = (8192, 32768, 131072, 524288, 1 << 20)


def bench_l_sweep(torch, gen, ssm):
    """Forward-scan throughput against sequence length at a fixed channel count B*D: the
    2^20-step workload's shape (1 x 256 channels, fp32) and one sequence of a 1024-channel layer
    (bf16), L from 8K to 1M.  Inputs drawn on the device (same distributions).  The pages
    describe throughput that scales almost linearly from 8K to 1M tokens: elements/s flat in L."""
    res = []
    for B, D, dt in ((1, 256, "f32"), (1, 1024, "bf16")):
        for L in L_SWEEP:
            x = gen.device_scan_inputs(B, D, 16, L, seed=L % 1000 + D, device="cuda", dtype=dt)
            el = B * D * L
            steps = max(3, min(20, int(2e9 // el)))
            r = time_scan(torch, gen, ssm, None, steps, 2, x)
            res.append({"batch": B, "d_inner": D, "seqlen": L, "io_dtype": dt, "steps": steps,
                        "ms_per_step": r["ms"], "elements_per_s": r["value"],
                        "alu_frac": r["tops"] / PEAK_VALU_TOPS, "launch_plan": r["plan"]["mode"]})
            del x
    torch.cuda.empty_cache()
    return res


def bench_decode_sweep(torch, gen, ssm, batches=(1, 4, 16, 64, 256, 1024)):
    """Decode-step latency and throughput against the number of requests (2.8B-shaped layer:
    D = 5120, N = 16, bf16 inputs, fp32 state), back to back and with the cache flushed before each
    step.  Calls go through the C ABI with prepared arguments so that Python does not starve the
    GPU at small batches."""
    p = {k: v.cuda() for k, v in gen.decode_params(4).items()}
    D, N = 5120, 16
    lib = ssm.load()
    stream = torch.cuda.current_stream()
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(3)
    res = []
    for Bt in batches:
        state = torch.randn((Bt, D, N), generator=g, device="cuda")
        ins = []
        for _ in range(4):
            t = {k: (torch.randn((Bt, D), generator=g, device="cuda") * (0.1 if k == "delta" else 1.0)).to(
                torch.bfloat16) for k in ("u", "delta", "z")}
            t.update({k: torch.randn((Bt, N), generator=g, device="cuda").to(torch.bfloat16) for k in ("B", "C")})
            ins.append(t)
        y = torch.empty((Bt, D), dtype=torch.bfloat16, device="cuda")
        args = [(state.data_ptr(), t["u"].data_ptr(), t["delta"].data_ptr(), p["A"].data_ptr(), t["B"].data_ptr(),
                 t["C"].data_ptr(), p["D"].data_ptr(), t["z"].data_ptr(), p["dt_bias"].data_ptr(), y.data_ptr(), Bt,
                 D, N, 1, stream.cuda_stream) for t in ins]
        for i in range(4):
            assert lib.selective_state_update(*args[i]) == 0, ssm.last_error()
        torch.cuda.synchronize()
        n = 64
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            lib.selective_state_update(*args[i % 4])
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(16)]
        for i, (a, b) in enumerate(evs):
            torch.sum(flush, dim=0, out=sink)
            a.record(stream)
            lib.selective_state_update(*args[i % 4])
            b.record(stream)
        torch.cuda.synchronize()
        us_f = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
        by = Bt * D * (N * 8 + 8) + 2 * Bt * N * 2 + D * (N + 2) * 4
        res.append({"batch": Bt, "us_per_step": us, "us_per_step_flushed": us_f,
                    "tokens_per_s": Bt / (us * 1e-6), "tokens_per_s_flushed": Bt / (us_f * 1e-6),
                    "hbm_frac_flushed": by / (us_f * 1e-6) / 1e9 / PEAK_HBM_GBS, "bytes_per_step": by})
        del state, ins, y
    del flush
    return res


def bench_resume(torch, gen, ssm, w, x, steps, pieces=4):
    """Prefill in pieces: the same workload as `pieces` consecutive scans of L/pieces steps,
    each resumed in place from the state the previous one left (selective_scan_fwd_resume)."""
    B, D, N, L = w.batch, w.dim, w.dstate, w.seqlen
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    pl = L // pieces
    parts = [{k: g[k][..., i * pl:(i + 1) * pl].contiguous() for k in ("u", "delta", "z", "B", "C")}
             for i in range(pieces)]
    ys = [torch.empty_like(p["u"]) for p in parts]
    st = torch.zeros((B, D, N), dtype=torch.float32, device="cuda")

    def step():
        st.zero_()
        for p, y in zip(parts, ys):
            ssm.scan_fwd(p["u"], p["delta"], g["A"], p["B"], p["C"], g["D"], p["z"], g["dt_bias"], True, y=y,
                         last_state=st, initial_state=st)

    step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = B * D * L
    return {"workload": f"{w.name}, prefilled as {pieces} resumed pieces of {pl} steps", "steps": steps,
            "ms_per_step": ms, "value": el / (ms * 1e-3), "unit": "elements/s",
            "alu_frac": el * algo_slots(N) / (ms * 1e-3) / 1e12 / PEAK_VALU_TOPS,
            "note": "inputs resident (no rotation): the pieces' 337 MB exceed the last-level cache"}


def bench_bwd(torch, ssm, w, x, steps, fwd_ms):
    """Backward of the layer's scan: every gradient (du, ddelta, dz, dA, dB, dC, dD, ddt_bias) for a
    given dy, states recomputed.  Bound by VALU issue like the forward (algo_slots_bwd per element)."""
    B, D, N, L = w.batch, w.dim, w.dstate, w.seqlen
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    gen_ = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn(g["u"].shape, device="cuda", generator=gen_).to(g["u"].dtype)
    args = (g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["dt_bias"])
    for _ in range(2):
        ssm.scan_bwd(*args, dy=dy, need_dinitial_state=False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ssm.scan_bwd(*args, dy=dy, need_dinitial_state=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = B * D * L
    tops = el * algo_slots_bwd(N) / (ms * 1e-3) / 1e12
    return {"workload": w.name, "steps": steps, "ms_per_step": ms, "value": el / (ms * 1e-3),
            "unit": "elements/s", "alu": {"achieved": tops, "peak": PEAK_VALU_TOPS, "unit": "Tops/s",
                                           "frac": tops / PEAK_VALU_TOPS, "ops_per_element": algo_slots_bwd(N)},
            "vs_forward": ms / fwd_ms,
            "note": "checkpoint, adjoint-aggregate and main passes plus carries and deterministic reductions"}



def ssd_flops_per_element(N: int, Q: int = 64, P: int = 64) -> float:
    """Algorithmic flops per element of the chunked SSD form (chunk Q, head size P, state N): per
    chunk and head, the causal half of C B^T (Q(Q+1)/2 N MACs) and of M x (Q(Q+1)/2 P), C H_in
    (Q N P) and the chunk state B^T x (N Q P), over Q*P elements."""
    macs = Q * (Q + 1) // 2 * (N + P) + 2 * Q * N * P
    return 2.0 * macs / (Q * P)


def bench_ssd(torch, gen, ssm, steps, fwd_ms):
    """The 2.8B-shaped layer in the SSD form: 80 heads of 64 channels with one decay rate and step
    size per head, N = 16, bf16; two kernels (chunk states with state passing, chunk outputs)."""
    sp = gen.SSD_LAYER
    Bt, H, P, N, L = sp["batch"], sp["heads"], sp["headdim"], sp["dstate"], sp["seqlen"]
    x = gen.ssd_inputs(Bt, H, P, N, L, sp["dtype"], seed=2)
    copies = 3
    ins = [{k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()} for _ in range(copies)]
    y = torch.empty_like(ins[0]["x"])
    last = torch.empty((Bt, H * P, N), dtype=torch.float32, device="cuda")

    def step(i):
        g = ins[i % copies]
        ssm.ssd_fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["dt_bias"], True, y=y,
                    last_state=last)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = Bt * H * P * L
    by = el * 2 * 3 + Bt * H * L * 2 + 2 * Bt * N * L * 2 + H * P * 4 + 2 * H * 4 + Bt * H * P * N * 4
    gbs = by / (ms * 1e-3) / 1e9
    tf = el * ssd_flops_per_element(N) / (ms * 1e-3) / 1e12
    return {"workload": f"2.8B-shaped layer as SSD: B={Bt}, {H} heads x {P} channels, N={N}, L={L}, bf16",
            "steps": steps, "ms_per_step": ms, "value": el / (ms * 1e-3), "unit": "elements/s",
            "hbm": {"achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                    "bytes_per_step": by},
            "mfma": {"achieved": tf, "peak": 2500.0, "unit": "TFLOP/s", "frac": tf / 2500.0,
                     "flops_per_element": ssd_flops_per_element(N), "dtype": "bf16"},
            "vs_selective_scan": fwd_ms / ms, "inputs_rotated": copies,
            "note": "bound by HBM (about 6 bytes against 145 matrix-core flops per element)",
            "backward": bench_ssd_bwd(torch, ssm, ins, max(3, steps // 5), ms)}


def bench_ssd_bwd(torch, ssm, ins, steps, fwd_ms):
    """ssd_scan_bwd on the same layer: the backward scan's kernels on the step sizes broadcast to
    the channels, then the per-head sums.  ALU fraction against the backward scan's algorithmic
    count (algo_slots_bwd), elements counted once."""
    x0 = ins[0]
    Bt, dim, L = x0["x"].shape
    N = x0["B"].shape[1]
    dy = torch.randn(x0["x"].shape, generator=torch.Generator(device="cuda").manual_seed(5),
                     device="cuda").to(x0["x"].dtype)

    def step(i):
        g = ins[i % len(ins)]
        ssm.ssd_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["z"], g["dt_bias"], True, dy=dy,
                    headdim=dim // g["A"].shape[0], need_dinitial_state=False)

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    el = Bt * dim * L
    tops = el * algo_slots_bwd(N) / (ms * 1e-3) / 1e12
    return {"steps": steps, "ms_per_step": ms, "value": el / (ms * 1e-3), "unit": "elements/s",
            "alu": {"achieved": tops, "peak": PEAK_VALU_TOPS, "unit": "Tops/s", "frac": tops / PEAK_VALU_TOPS,
                    "ops_per_element": algo_slots_bwd(N)},
            "vs_ssd_forward": ms / fwd_ms}


def bench_conv(torch, np, ssm, steps, K=4):
    """Causal conv1d + SiLU (width 4) on the 2.8B-shaped layer's input [4, 5120, 2048] bf16, and its
    decode step on the 2.8B-shaped serving batch [256, 5120].  Both are HBM-bound: the sequence
    kernel moves 2 + 2 bytes per element (x in, out), the step 12 + 12 bytes of fp32 window state
    plus 2 + 2 bytes of x and out per row."""
    g = np.random.default_rng(0)
    B, D, L = 4, 5120, 2048
    xs = [torch.from_numpy(g.standard_normal((B, D, L), dtype=np.float32)).to(torch.bfloat16).cuda() for _ in range(3)]
    w = torch.from_numpy(g.standard_normal((D, K), dtype=np.float32) * 0.5).cuda()
    b = torch.from_numpy(g.standard_normal(D, dtype=np.float32) * 0.1).cuda()
    out = torch.empty_like(xs[0])
    st = torch.empty((B, D, K - 1), dtype=torch.float32, device="cuda")
    for i in range(3):
        ssm.conv1d_fwd(xs[i], w, b, True, None, out=out, state_out=st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        ssm.conv1d_fwd(xs[i % 3], w, b, True, None, out=out, state_out=st)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    by = B * D * L * 4 + B * D * (K - 1) * 4 + D * (K + 1) * 4
    gbs = by / (ms * 1e-3) / 1e9
    res = {"fwd": {"shape": [B, D, L], "width": K, "dtype": "bf16", "us_per_call": ms * 1e3,
                   "elements_per_s": B * D * L / (ms * 1e-3), "hbm_GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                   "bytes_per_call": by, "inputs_rotated": 3}}
    R, Dd = 256, 5120
    state = torch.from_numpy(g.standard_normal((R, Dd, K - 1), dtype=np.float32)).cuda()
    xt = [torch.from_numpy(g.standard_normal((R, Dd), dtype=np.float32)).to(torch.bfloat16).cuda() for _ in range(8)]
    yo = torch.empty((R, Dd), dtype=torch.bfloat16, device="cuda")
    for i in range(4):
        ssm.conv1d_update(state, xt[i], w, b, True, out=yo)
    torch.cuda.synchronize()
    # the step kernel is a few microseconds: call the C ABI with prepared arguments, so that
    # Python argument checking does not starve the GPU between steps
    lib = ssm.load()
    args = [(state.data_ptr(), x.data_ptr(), w.data_ptr(), b.data_ptr(), 1, yo.data_ptr(), R, Dd, K, 1,
             stream.cuda_stream) for x in xt]
    n = 128
    e0.record(stream)
    for i in range(n):
        lib.causal_conv1d_update(*args[i % 8])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    by = R * Dd * ((K - 1) * 8 + 4) + Dd * (K + 1) * 4
    gbs = by / (ms * 1e-3) / 1e9
    res["update"] = {"shape": [R, Dd], "width": K, "dtype": "bf16", "steps": n, "us_per_step": ms * 1e3,
                     "hbm_GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "bytes_per_step": by,
                     "note": "back to back: the 15.7 MB window state stays in the last-level cache"}
    return res


def bench_conv_scan(torch, gen, ssm, w, steps, K=4):
    """The causal conv1d + SiLU and the scan of the 2.8B-shaped layer, two ways: the one call
    (selective_scan_fwd_conv: for fp32 rows u is computed inside the scan kernels and never
    stored; for bf16 rows the call runs the convolution kernel into scratch and then the scan,
    the faster route there) and separate (causal_conv1d_fwd writing u, then selective_scan_fwd
    reading it).  Inputs rotated over three copies."""
    import numpy as np
    x = gen.scan_inputs(w)
    g = np.random.default_rng(5)
    cw = torch.from_numpy((g.standard_normal((w.dim, K)) * 0.5).astype(np.float32)).cuda()
    cb = torch.from_numpy((g.standard_normal(w.dim) * 0.1).astype(np.float32)).cuda()
    ins = [{k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in x.items()} for _ in range(3)]
    y = torch.empty_like(ins[0]["u"])
    u = torch.empty_like(ins[0]["u"])
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    cso = torch.empty((w.batch, w.dim, K - 1), dtype=torch.float32, device="cuda")

    def fused(i):
        a = ins[i % 3]
        ssm.scan_fwd_conv(a["u"], cw, a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], True,
                          conv_bias=cb, y=y, last_state=last, conv_state_out=cso)

    def separate(i):
        a = ins[i % 3]
        ssm.conv1d_fwd(a["u"], cw, cb, True, None, out=u, state_out=cso)
        ssm.scan_fwd(u, a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"], True,
                     y=y, last_state=last)

    stream = torch.cuda.current_stream()
    # the two routes alternate in rounds (the order flipping each round), so that a drift of the
    # clock over the run weighs on both alike
    for i in range(3):
        fused(i)
        separate(i)
    torch.cuda.synchronize()
    rounds = 4
    per = max(1, steps // rounds)
    ms = {"fused": 0.0, "separate": 0.0}
    for r in range(rounds):
        order = (("fused", fused), ("separate", separate)) if r % 2 == 0 else (("separate", separate), ("fused", fused))
        for name, fn in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(per):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms[name] += e0.elapsed_time(e1)
    res = {name + "_us_per_call": v / (rounds * per) * 1e3 for name, v in ms.items()}
    el = w.batch * w.dim * w.seqlen
    res.update({"workload": f"{w.name}, causal conv1d width {K} + SiLU ahead of the scan",
                "steps": rounds * per, "fused_elements_per_s": el / (res["fused_us_per_call"] * 1e-6),
                "fused_vs_separate": res["separate_us_per_call"] / res["fused_us_per_call"],
                "hbm_bytes_saved_per_call": 2 * el * 4 if w.dtype == "f32" else 0,
                "io_dtype": w.dtype,
                "note": "fused: selective_scan_fwd_conv (fp32 rows: u = silu(conv(x)) inside the scan kernels; bf16 "
                        "rows: the conv kernel into scratch, then the scan); separate: u written by the conv kernel "
                        "and read back by the scan"})
    del ins, y, u
    return res


def copy_calibration(torch, mib):
    """Plain device-to-device copies of a known size: what a byte counter reads for them
    gives the counter's scale (bytes counted per byte moved)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copies": 5, "bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4}


def bench_decode(torch, gen, ssm, args):
    """Decode steps of the 2.8B-shaped serving batch, 128 in a row on one state.
    Reported twice: back to back (the 84 MB state stays in the 256 MB last-level cache) and
    with the cache flushed before every step (a 1 GiB device read between steps, outside
    the per-step events), which is the HBM-bound figure."""
    w = gen.WORKLOADS[4]
    p = {k: v.cuda() for k, v in gen.decode_params(4).items()}
    state = gen.decode_state(4).cuda()
    steps_in = [{k: v.cuda() for k, v in gen.decode_step_inputs(4, s).items()} for s in range(8)]
    yb = torch.empty((w.batch, w.dim), dtype=torch.bfloat16, device="cuda")

    def one(s):
        st = steps_in[s % len(steps_in)]
        ssm.state_update(state, st["u"], st["delta"], p["A"], st["B"], st["C"], p["D"], st["z"], p["dt_bias"], y=yb)

    for s in range(4):
        one(s)
    torch.cuda.synchronize()
    n = w.seqlen
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(n):
        one(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s in range(n):
        torch.sum(flush, dim=0, out=sink)  # reads 1 GiB: evicts the state, leaves no dirty lines behind
        evs[s][0].record(stream)
        one(s)
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    ms_flushed = sum(a.elapsed_time(b) for a, b in evs) / n
    # a plain device copy of the state's bytes (read once, written once), timed the same way: what
    # one read and one write of 84 MB take on this device, as a practical roof for the step
    src, dst = torch.randn_like(state), torch.empty_like(state)
    for s in range(n):
        torch.sum(flush, dim=0, out=sink)
        evs[s][0].record(stream)
        dst.copy_(src)
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    ms_copy = sum(a.elapsed_time(b) for a, b in evs) / n
    del flush, src, dst
    rows = w.batch * w.dim
    bytes_step = rows * w.dstate * 4 * 2 + rows * 2 * 4 + 2 * w.batch * w.dstate * 2 + w.dim * (w.dstate + 2) * 4
    gbs = bytes_step / (ms * 1e-3) / 1e9
    gbs_f = bytes_step / (ms_flushed * 1e-3) / 1e9
    return {"workload": w.name, "steps": n, "bytes_per_step": bytes_step,
            "flushed": {"us_per_step": ms_flushed * 1e3, "rows_per_s": rows / (ms_flushed * 1e-3),
                        "hbm_achieved_GBs": gbs_f, "hbm_frac": gbs_f / PEAK_HBM_GBS,
                        "state_copy_us": ms_copy * 1e3,
                        "state_copy_GBs": 2 * state.numel() * 4 / (ms_copy * 1e-3) / 1e9,
                        "vs_state_copy": ms_copy / ms_flushed,
                        "note": "state_copy: a plain device copy of the 84 MB state (read + write), flushed "
                                "the same way"},
            "steady": {"us_per_step": ms * 1e3, "rows_per_s": rows / (ms * 1e-3), "hbm_achieved_GBs": gbs,
                       "hbm_frac": gbs / PEAK_HBM_GBS,
                       "note": "back to back: the state stays resident in the last-level cache"}}


def cpu_baseline(np, gen, x, w, target_s):
    """The fp64 CPU oracle on the same workload.  When the whole workload takes less than
    `target_s`, it is run repeatedly until `target_s` has elapsed; otherwise the first k
    channels, with k chosen from a timed probe, form the sample."""
    import oracle
    threads = oracle.max_threads()
    total = w.batch * w.dim
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], True)
    probe = np.arange(min(total, 256))
    t = time.perf_counter()
    oracle.scan(*args, chans=probe)
    dt = max(time.perf_counter() - t, 1e-6)
    k = int(min(total, max(len(probe), len(probe) * target_s / dt)))
    chans = None if k == total else np.arange(k)
    reps, sec = 0, 0.0
    t = time.perf_counter()
    while reps == 0 or sec < target_s:
        oracle.scan(*args, chans=chans)
        reps += 1
        sec = time.perf_counter() - t
    el = reps * k * w.seqlen
    what = (f"the whole workload ({total} (b, d) channels x L={w.seqlen}) run {reps} times" if k == total
            else f"the first {k} of {total} (b, d) channels, full length L={w.seqlen}")
    # the same oracle on one thread, over the first channels (about a third of the time budget)
    t = time.perf_counter()
    oracle.scan(*args, chans=np.arange(16), threads=1)
    dt1 = max(time.perf_counter() - t, 1e-6)
    k1 = int(min(total, max(16, 16 * (target_s / 3) / dt1)))
    t = time.perf_counter()
    oracle.scan(*args, chans=np.arange(k1), threads=1)
    sec1 = time.perf_counter() - t
    return {"value": el / sec, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: {el} elements in {sec:.1f} s, fp64, OpenMP over channels",
            "single_core": {"value": k1 * w.seqlen / sec1, "unit": "elements/s", "cores": 1,
                            "sample": f"the first {k1} (b, d) channels, full length L={w.seqlen}, one thread: "
                                      f"{k1 * w.seqlen} elements in {sec1:.1f} s"}}


if __name__ == "__main__":
    main()
