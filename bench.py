#!/usr/bin/env python3
"""Throughput of the M²RNN hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident
in HBM: gate precompute (m2rnn_gates) -> forward with state checkpoints every C
steps (m2rnn_fwd) -> reverse-time backward (m2rnn_bwd) with a synthetic
upstream gradient dy.  Default workload: B=4, T=16384, n_heads=16, K=V=64,
bf16 k/v/q, fp32 state, exp-softplus gate, checkpoints every C=4 steps: the
backward walks 4-step chunks at V=64, so every chunk start is a stored
checkpoint (4.3 GB of them at this workload) and no chunk start has to be
recomputed first; --C 64 measures the pre-pass variant.

Prints ONE JSON line.  Per-call durations come from HIP events recorded on the
stream the library launches on (torch's current stream); the roofline block
prices the dominant call (all kernels one library call launches) against the
fp32 MFMA peak with the algorithmic flop count (forward 2 K V^2, backward
4 K V^2 per token and head; the backward's recompute is not counted).  ``cpu_baseline`` times the float64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long_t16k_k64")
    ap.add_argument("--C", type=int, default=4, help="checkpoint interval")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the MFMA fraction of every workload and the decode-step, "
                         "block-kernel and Newton rates")
    ap.add_argument("--recompute", action="store_true",
                    help="the backward recomputes the states inside each checkpoint interval "
                         "instead of reading the per-step rc the forward stores")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the single-token step on the decoding workloads and "
                         "print those rates")
    ap.add_argument("--block-only", action="store_true",
                    help="only time the block prologue / epilogue kernels and print those rates")
    ap.add_argument("--newton-only", action="store_true",
                    help="only time the parallel-in-time Newton forward beside the sequential "
                         "one on the Newton workload and print those rates")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="first copy this many GiB twice with torch (a plain copy of known "
                         "size, to calibrate HBM byte counters)")
    return ap.parse_args()


# counter summaries of the backward call: states recomputed / stored rc read
TRAFFIC_FILES = {
    False: os.path.join(ROOT, "profiles", "m2rnn_bwd_long_t16k_k64_C4_hbm_traffic.md"),
    True: os.path.join(ROOT, "profiles", "m2rnn_bwd_long_t16k_k64_C4_stored_rc_hbm_traffic.md"),
}
BWD_SOURCES = ("m2rnn_bwd.hip", "m2rnn_device.h", "m2rnn_internal.h")


def measured_bwd_traffic(workload, C, stored_rc):
    """HBM bytes per m2rnn_bwd call from the committed counter summary, when it
    applies: same workload, C and mode, and the backward's sources unchanged
    since the counters were taken (their sha256 is recorded with the figure)."""
    import hashlib

    path = TRAFFIC_FILES[bool(stored_rc)]
    if workload != "long_t16k_k64" or C != 4 or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_call", "source_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in BWD_SOURCES:
        with open(os.path.join(ROOT, "matrix_state_nonlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_call" not in fields:
        return None
    return float(fields["traffic_bytes_per_call"])


def stream_bytes(wl):
    """Algorithmic bytes streamed per call, per the workload's dtypes: forward
    reads k, q (NQ heads), v, f and writes y; backward reads k, q, v, f, the
    gate logit and dy and writes dk, dq, dv and dlogit (fp32 gradients).
    Checkpoints, the optional per-step rc, W and per-head sums are not counted."""
    in_b = 2 if wl.bf16 else 4
    tok = wl.B * wl.T
    kq = 2 * tok * wl.qk_heads * wl.K
    vv = tok * wl.N * wl.V
    g = tok * wl.N
    fwd = (kq + vv) * in_b + 4 * g + 4 * vv
    bwd = (kq + vv) * in_b + 8 * g + 4 * vv + 4 * (kq + vv + g)
    return fwd, bwd


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def per_config_fractions(reps=3):
    """Achieved fraction of the fp32 MFMA peak of every workload: the forward
    call alone (no checkpoints) and, for the workloads that define a
    checkpoint interval, the backward call from checkpoints at that interval,
    recomputing the states and reading the forward's stored rc.
    Flops are the algorithmic ones (forward 2 K V^2, backward 4 K V^2 per token
    and head)."""
    import torch

    from m2rnn_inputs import WORKLOADS, make_inputs, to_device
    from matrix_state_nonlinear_amd import m2rnn_bwd, m2rnn_fwd, m2rnn_gates

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    rows = []
    for wl in WORKLOADS.values():
        inp = make_inputs(wl, with_dy=wl.C > 0)
        d = to_device(inp, "float32")
        f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
        th = wl.B * wl.T * wl.N
        fb, bb = stream_bytes(wl)
        ms = timed(lambda: m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], None, 0))
        tf = 2.0 * th * wl.K * wl.V * wl.V / (ms * 1e-3) / 1e12
        row = {"workload": wl.name, "B": wl.B, "T": wl.T, "n_heads": wl.N,
               "qk_heads": wl.qk_heads, "K": wl.K, "V": wl.V,
               "fwd_ms": ms, "fwd_tflops": tf, "fwd_mfma_frac": tf / MFMA_F32_PEAK_TFLOPS,
               "fwd_stream_bytes": fb, "fwd_stream_gbs": fb / (ms * 1e-3) / 1e9}
        if wl.C > 0:
            rc = torch.empty((wl.B, wl.N, wl.T, wl.K, wl.V), dtype=torch.float32, device="cuda")
            _, _, ck = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], None, wl.C,
                                 rc_out=rc)
            bw = lambda r: m2rnn_bwd(d["k"], d["v"], d["q"], wl.gate, d["logit"],  # noqa: E731
                                     d["alpha"], d["beta"], f, d["W"], d["w_r"], None, ck, wl.C,
                                     d["dy"], rc=r)
            ms = timed(lambda: bw(None))
            ms_rc = timed(lambda: bw(rc))
            fl = 4.0 * th * wl.K * wl.V * wl.V
            tf = fl / (ms * 1e-3) / 1e12
            rcb = th * wl.K * wl.V * 4
            row.update({"C": wl.C, "bwd_ms": ms, "bwd_tflops": tf,
                        "bwd_mfma_frac": tf / MFMA_F32_PEAK_TFLOPS, "bwd_stream_bytes": bb,
                        "bwd_stream_gbs": bb / (ms * 1e-3) / 1e9, "bwd_stored_rc_ms": ms_rc,
                        "bwd_stored_rc_mfma_frac": fl / (ms_rc * 1e-3) / 1e12
                        / MFMA_F32_PEAK_TFLOPS,
                        "bwd_stored_rc_stream_gbs": (bb + rcb) / (ms_rc * 1e-3) / 1e9})
            del rc, ck
        rows.append(row)
        del d, f, inp
        torch.cuda.empty_cache()
    return rows


def decode_rates(reps=50):
    """The single-token step (m2rnn_step) on the decoding workloads: one token
    for each of B sequences, the state updated in place.  HBM-bound by design:
    the algorithmic bytes per (sequence, head) are the state read and written
    (2 K V 4 B) plus v, f, y and the shared k, q; the rate is priced against
    the 8 TB/s HBM peak."""
    import torch

    from m2rnn_inputs import DECODE_WORKLOADS, make_inputs, to_device
    from matrix_state_nonlinear_amd import m2rnn_gates, m2rnn_step

    rows = []
    for wl in DECODE_WORKLOADS.values():
        inp = make_inputs(wl)
        d = to_device(inp, "float32")
        f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])[:, 0].contiguous()
        H = torch.empty((wl.B, wl.N, wl.K, wl.V), device="cuda").uniform_(-0.5, 0.5)
        k, v, q = (d[x][:, 0].contiguous() for x in ("k", "v", "q"))
        y = torch.empty((wl.B, wl.N, wl.V), device="cuda")
        stream = torch.cuda.current_stream()
        for _ in range(3):
            m2rnn_step(H, k, v, q, f, d["W"], d["w_r"], out=y)
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            m2rnn_step(H, k, v, q, f, d["W"], d["w_r"], out=y)
        e1.record(stream)
        stream.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        th = wl.B * wl.N
        in_b = 2 if wl.bf16 else 4
        nbytes = (th * (2 * wl.K * wl.V * 4 + wl.V * in_b + 4 + wl.V * 4)
                  + wl.B * wl.qk_heads * 2 * wl.K * in_b)
        gbs = nbytes / us / 1e3
        rows.append({"workload": wl.name, "B": wl.B, "n_heads": wl.N, "qk_heads": wl.qk_heads,
                     "K": wl.K, "V": wl.V, "us_per_step": us,
                     "tokens_heads_per_s": th / us * 1e6, "bytes_per_step": nbytes,
                     "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "mfma_frac": 2.0 * th * wl.K * wl.V * wl.V / us / 1e6 / MFMA_F32_PEAK_TFLOPS})
        del d, f, H, k, v, q, y, inp
        torch.cuda.empty_cache()
    return rows


def newton_rates(reps=5, iters=3):
    """The parallel-in-time Newton forward (m2rnn_newton_fwd, three iterations)
    beside the sequential forward kernel on the Newton workload (one sequence,
    four value heads of K = 64, V = 16, shared q/k, contractive W) and on one
    head of it.  Rates are tokens x heads per second of the whole call; the
    dominant kernel, the chunk maps, does 2 V^3 flops per (unit, row, step) and
    iteration on the fp32 MFMA units (V times the sequential forward's 2 K V^2
    per token and head); its share of the fp32 MFMA peak is given over the whole
    call."""
    import torch

    from m2rnn_inputs import NEWTON_WORKLOADS, make_inputs, to_device
    from matrix_state_nonlinear_amd import (m2rnn_fwd, m2rnn_gates, m2rnn_newton_fwd,
                                            m2rnn_newton_workspace_bytes)

    base = NEWTON_WORKLOADS["newton_k64_v16"]
    rows = []
    for wl in (base, base.replace(name="newton_k64_v16_one_head", N=1)):
        inp = make_inputs(wl)
        d = to_device(inp, "float32")
        f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
        ws = torch.empty(m2rnn_newton_workspace_bytes(wl.B, wl.T, wl.N, wl.K, wl.V, False),
                         dtype=torch.uint8, device="cuda")
        y = torch.empty((wl.B, wl.T, wl.N, wl.V), device="cuda")
        stream = torch.cuda.current_stream()

        def timed(fn):
            fn()
            stream.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            stream.synchronize()
            return e0.elapsed_time(e1) / reps

        ms_seq = timed(lambda: m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"],
                                         want_ht=False, out=(y, None, None)))
        ms_newton = timed(lambda: m2rnn_newton_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"],
                                                   iters=iters, want_ht=False, workspace=ws,
                                                   out=(y, None, None, None)))
        _, _, _, res = m2rnn_newton_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], iters=iters,
                                        want_residual=True, workspace=ws)
        stream.synchronize()
        th = wl.B * wl.T * wl.N
        maps_flops = iters * 2.0 * wl.V ** 3 * wl.K * wl.T * wl.B * wl.N
        rows.append({"workload": wl.name, "B": wl.B, "T": wl.T, "n_heads": wl.N,
                     "qk_heads": wl.qk_heads, "K": wl.K, "V": wl.V, "iters": iters,
                     "ms": ms_newton, "tokens_heads_per_s": th / ms_newton * 1e3,
                     "sequential_ms": ms_seq, "sequential_tokens_heads_per_s": th / ms_seq * 1e3,
                     "speedup": ms_seq / ms_newton, "residual": [float(r) for r in res.tolist()],
                     "maps_flops": maps_flops,
                     "maps_mfma_frac_whole_call": maps_flops / (ms_newton * 1e-3) / 1e12
                     / MFMA_F32_PEAK_TFLOPS})
        del d, f, ws, y, inp
        torch.cuda.empty_cache()
    return rows

def block_rates(reps=20):
    """The block around the recurrence at the long-context workload's sizes:
    the causal conv + SiLU prologue on one projected tensor [4, 16384, 1024]
    (bf16, e.g. v of 16 heads x 64) and the gate + RMSNorm epilogue on the
    readout [65536, 1024], forward and backward.  HBM-bound; algorithmic bytes
    per element: conv forward 2 s_in (read x, write out), conv backward s_in + 8
    (x, dout, dx), epilogue forward 4 + 2 s_in (y, g_pre, out), backward 16 + s_in
    (y, g_pre, dout, dy, dg_pre); parameter partials are not counted."""
    import numpy as np
    import torch

    from m2rnn_inputs import make_conv_inputs, make_norm_inputs
    from matrix_state_nonlinear_amd import (m2rnn_conv_silu, m2rnn_conv_silu_bwd,
                                            m2rnn_gate_rmsnorm, m2rnn_gate_rmsnorm_bwd)
    from matrix_state_nonlinear_amd._lib import lib

    B, T, C = 4, 16384, 1024
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(3):
            fn()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        stream.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    bf = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    ci = make_conv_inputs(B, T, C, seed=1)
    x, w, b, dout = bf(ci.x_bits), f32(ci.w), f32(ci.bias), f32(ci.dout)
    ws = torch.empty(int(lib().m2rnn_block_workspace_bytes(0, B, T, C, 0)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(x)
    E = B * T * C
    rows = []
    us = timed(lambda: m2rnn_conv_silu(x, w, b, out=out))
    rows.append(("conv_silu", us, E * 4))
    us = timed(lambda: m2rnn_conv_silu_bwd(x, w, b, dout, workspace=ws))
    rows.append(("conv_silu_bwd", us, E * 10))
    del x, w, b, dout, ws, out, ci
    ni = make_norm_inputs(B * T, C, seed=2)
    y, g, gamma, nd = f32(ni.y), bf(ni.g_bits), f32(ni.gamma), f32(ni.dout)
    ws = torch.empty(int(lib().m2rnn_block_workspace_bytes(1, B * T, 1, C, 0)),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(g)
    us = timed(lambda: m2rnn_gate_rmsnorm(y, g, gamma, 1e-6, out=o))
    rows.append(("gate_rmsnorm", us, E * 8))
    us = timed(lambda: m2rnn_gate_rmsnorm_bwd(y, g, gamma, nd, 1e-6, workspace=ws))
    rows.append(("gate_rmsnorm_bwd", us, E * 18))
    del y, g, gamma, nd, ws, o, ni
    torch.cuda.empty_cache()
    return [{"op": op, "shape": [B, T, C], "us": us, "bytes": nb, "hbm_gbs": nb / us / 1e3,
             "hbm_frac": nb / us / 1e3 / HBM_PEAK_GBS} for op, us, nb in rows]


def oracle_baseline(wl, target_s):
    """float64 oracle (forward + backward) on the first Ts steps of every unit."""
    import numpy as np

    import oracle
    from m2rnn_inputs import make_inputs

    def run(T):
        w = wl.replace(T=T)
        inp = make_inputs(w, with_dy=True)
        t0 = time.perf_counter()
        f = oracle.gates(w.gate, inp.logit, inp.alpha, inp.beta)
        oracle.forward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r)
        oracle.backward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, inp.dy, gate_kind=w.gate,
                        logit=inp.logit, alpha=inp.alpha, beta=inp.beta)
        return time.perf_counter() - t0

    probe_T = 32
    per_step = run(probe_T) / probe_T
    Ts = int(max(probe_T, min(wl.T, target_s / max(per_step, 1e-9))))
    el = run(Ts)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 0) for p in threadpool_info()), default=None)
    except Exception:  # noqa: BLE001
        pass
    cores = threads or len(os.sched_getaffinity(0))
    return {"value": wl.B * Ts * wl.N / el, "unit": "tokens*heads/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"float64 numpy oracle, gates+forward+backward (forward rerun inside the "
                      f"backward), all {wl.B * wl.N} (b,n) units, first {Ts} of {wl.T} steps, "
                      f"{el:.1f} s; {len(os.sched_getaffinity(0))} host cpus visible, "
                      f"{np.__version__=}"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from m2rnn_inputs import WORKLOADS, make_inputs, to_device
    from matrix_state_nonlinear_amd import m2rnn_bwd, m2rnn_fwd, m2rnn_gates
    from matrix_state_nonlinear_amd.ops import m2rnn_workspace_bytes

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 28))
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if args.decode_only or args.block_only or args.newton_only:
        torch.cuda.set_device(0)
        if args.decode_only:
            print(json.dumps({"decode": decode_rates()}), flush=True)
        elif args.block_only:
            print(json.dumps({"block": block_rates()}), flush=True)
        else:
            print(json.dumps({"newton": newton_rates()}), flush=True)
        return

    wl = WORKLOADS[args.workload]
    C = args.C
    B, T, N, K, V = wl.B, wl.T, wl.N, wl.K, wl.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, with_dy=True)
    d = to_device(inp, "float32", dev)
    f = torch.empty((B, T, N), dtype=torch.float32, device=dev)
    y = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
    HT = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
    ckpt = torch.empty((B, N, (T + C - 1) // C, K, V), dtype=torch.float32, device=dev)
    NQ = wl.qk_heads
    wsf = torch.empty(max(1, m2rnn_workspace_bytes(False, B, T, N, NQ, K, V, C)),
                      dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, m2rnn_workspace_bytes(True, B, T, N, NQ, K, V, C)),
                      dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    # every step's rc = 1 / (1 + e^{2A}) from the forward, read by the backward in
    # place of its recomputation (K V 4 bytes per token and head: 17 GB here)
    rc = None if args.recompute else torch.empty((B, N, T, K, V), dtype=torch.float32, device=dev)

    names = ("gates", "fwd", "bwd")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"], out=f)
        if ev is not None:
            ev[1].record(stream)
        m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], None, C, out=(y, HT, ckpt),
                  workspace=wsf, rc_out=rc)
        if ev is not None:
            ev[2].record(stream)
        g = m2rnn_bwd(d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f,
                      d["W"], d["w_r"], None, ckpt, C, d["dy"], workspace=wsb, rc=rc)
        if ev is not None:
            ev[3].record(stream)
        return g

    def recompute_step_ms(reps=3):
        # the whole step without the per-step rc: the forward stores only the
        # checkpoints and the backward recomputes the states from them
        def run(ev=None):
            if ev is not None:
                ev[0].record(stream)
            m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"], out=f)
            m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], None, C, out=(y, HT, ckpt),
                      workspace=wsf)
            if ev is not None:
                ev[1].record(stream)
            m2rnn_bwd(d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f,
                      d["W"], d["w_r"], None, ckpt, C, d["dy"], workspace=wsb)
            if ev is not None:
                ev[2].record(stream)
        run()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ev in evs:
            run(ev)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / reps
        fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        return wall, fwd, bwd

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per_call[n].append(ev[j].elapsed_time(ev[j + 1]))
    avg_ms = {n: float(np.mean(v)) for n, v in per_call.items()}
    ms_step = wall * 1e3 / args.steps
    th = B * T * N
    flops = {"fwd": 2.0 * th * K * V * V, "bwd": 4.0 * th * K * V * V}
    kernels = {}
    for n in names:
        ms = avg_ms[n]
        entry = {"avg_ms": ms}
        if n in flops:
            tf = flops[n] / (ms * 1e-3) / 1e12
            entry.update({"bound": "mfma", "achieved_tflops": tf,
                          "frac": tf / MFMA_F32_PEAK_TFLOPS, "tokens_heads_per_s": th / (ms * 1e-3)})
        else:
            gbs = th * 8 / (ms * 1e-3) / 1e9   # read logit, write f (fp32)
            entry.update({"bound": "hbm", "achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS})
        kernels[n] = entry
    # streamed bytes of each call (stream_bytes), plus the per-step rc written by
    # the forward and read by the backward when it is stored
    fb, bb = stream_bytes(wl)
    rcb = th * K * V * 4 if rc is not None else 0
    kernels["fwd"]["stream_bytes"] = fb + rcb
    kernels["fwd"]["stream_gbs"] = (fb + rcb) / (avg_ms["fwd"] * 1e-3) / 1e9
    kernels["bwd"]["stream_bytes"] = bb + rcb
    kernels["bwd"]["stream_gbs"] = (bb + rcb) / (avg_ms["bwd"] * 1e-3) / 1e9
    dom = max(("fwd", "bwd"), key=lambda n: avg_ms[n])
    dom_tf = kernels[dom]["achieved_tflops"]
    out = {
        "metric": "M2RNN fwd+bwd tokens*heads/s at T=16K, K=V=64 (gates + forward with "
                  "checkpoints + backward)",
        "value": th / (ms_step * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "n_heads": N, "qk_heads": NQ, "K": K, "V": V,
                   "C": C, "kvq_dtype": "bf16" if wl.bf16 else "f32", "state_dtype": "f32",
                   "gate": "exp_softplus" if wl.gate == 1 else "sigmoid",
                   "backward_states": "recomputed" if rc is None else "stored rc",
                   "ckpt_bytes": int(ckpt.numel() * 4),
                   "rc_bytes": 0 if rc is None else int(rc.numel() * 4),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": f"m2rnn_{dom} (whole call)", "achieved": dom_tf,
                     "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": dom_tf / MFMA_F32_PEAK_TFLOPS,
                     "traffic": (measured_bwd_traffic(wl.name, C, rc is not None)
                                 if dom == "bwd" else None)},
        "fwd_only": {"checkpoint_interval": C,
                     "tokens_heads_per_s": kernels["fwd"]["tokens_heads_per_s"],
                     "ms": avg_ms["fwd"], "mfma_frac": kernels["fwd"]["frac"],
                     "achieved_tflops": kernels["fwd"]["achieved_tflops"]},
        "kernels": kernels,
    }
    if rc is not None:
        # the same step with no per-step rc (checkpoints only, states recomputed)
        wall, fms, bms = recompute_step_ms()
        out["recompute_step"] = {
            "ms_per_step": wall, "tokens_heads_per_s": th / (wall * 1e-3),
            "fwd_ms": fms, "bwd_ms": bms,
            "fwd_mfma_frac": flops["fwd"] / (fms * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS,
            "bwd_mfma_frac": flops["bwd"] / (bms * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS,
            "ckpt_bytes": int(ckpt.numel() * 4), "rc_bytes": 0}
        out["bwd_recompute"] = {"ms": bms, "mfma_frac": out["recompute_step"]["bwd_mfma_frac"]}
    if not args.no_per_config:
        out["per_config"] = per_config_fractions()
        out["decode"] = decode_rates()
        out["block"] = block_rates()
        out["newton"] = newton_rates()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = oracle_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
