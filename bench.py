#!/usr/bin/env python3
"""KDA benchmark on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  * kda_chunk_fwd over the prefill workload (B=4, T=4096, H=16, d_k=d_v=128, bf16 q/k/v,
    fp32 gate/beta/state, chunk 64 as the workload names it, initial state given, final state
    written; the library's default chunk, 32, is timed beside it), and
  * kda_decode_step over the decode workload (256 sequences x 32 heads, fp32 state
    128x128 updated in place).
The long-prefill (1 x 131,072 tokens x 32 heads) and packed-varlen (64 sequences, lengths
U[1, 8192], 32 heads) workloads are timed as their own legs (`long_prefill`, `varlen`), each with
its CPU-oracle rate on a sample of heads.
The prologue (kda_prologue: short convolution + Swish, q/k L2 norm, gate and beta activations)
and the output epilogue (kda_norm_gate: per-head RMSNorm and output gate) are timed on their
own over the prefill shapes and reported next to the step, and so is the backward (kda_chunk_bwd:
the gradients for a synthetic output gradient and final-state gradient on the prefill tensors).
The decode step with the epilogue fused in (kda_decode_step_gated) is timed on the decode
workload next to the two-kernel composition (kda_decode_step, then kda_norm_gate), and the
forward on raw projections with the prologue fused in (kda_chunk_fwd_prologue) on the prefill
shape next to kda_prologue followed by kda_chunk_fwd.
`value` is prefill tokens/s (B*T tokens per chunk_fwd launch); the decode step is
reported in GB/s next to it.  Inputs are resident in HBM before the timed region.
Timing uses HIP events recorded on the stream the kernels are launched on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--algo auto|fused|two_pass] [--dv-tile T]
                       [--no-cpu-baseline] [--no-tune] [--no-compare] [--no-workloads] [--dplr-sweep]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode-step GB/s + % HBM peak"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """SHA-256 over the kernel sources and the ABI header (file names and contents)."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "include", "kda.h")]
    csrc = os.path.join(ROOT, "gated_delta_rule_45_amd", "csrc")
    files += sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch recorded from rocprofv3 counters under profiles/, keyed by
    the kernel-source hash they were taken at; {} when the sources have changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_4x4096x16_decode_256x32.txt")
    if not os.path.exists(path):
        return {}
    vals = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = v
    if vals.get("source_sha256") != kernel_source_hash():
        return {}
    return {k: float(v) for k, v in vals.items() if k.endswith("_bytes")}


def time_launches(fn, n, stream):
    """Average duration of one call of fn (ms), from HIP events around n back-to-back calls.

    One call is queued before the start event so the stream is already busy when the event
    fires: the measured span then holds the n calls' GPU time, not the host's launch delay."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def time_each(fn, n, stream):
    """Median and minimum duration (ms) of n calls, each bracketed by its own pair of HIP events
    on the launch stream (the calls still run back to back)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    fn()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    ev[-1][1].synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp):
    import oracle
    import kda_inputs as ki
    a = [ki.to_numpy_io(x) for x in (inp.q, inp.k, inp.v)]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.fwd(*a, inp.g.numpy(), inp.beta.numpy(), initial_state=inp.s0.numpy(), threads=threads)
    dt = time.perf_counter() - t0
    B, T = inp.q.shape[0], inp.q.shape[1]
    # decode leg: 10 steps of the decode workload through the same oracle
    dinp = ki.workload_inputs("decode")
    sq = lambda x: x[:, 0].contiguous()
    dq, dk, dv = (ki.to_numpy_io(sq(x)) for x in (dinp.q, dinp.k, dinp.v))
    dg, db, st = sq(dinp.g).numpy(), sq(dinp.beta).numpy(), dinp.s0.numpy()
    t1 = time.perf_counter()
    for _ in range(10):
        _, st = oracle.decode(dq, dk, dv, dg, db, st.astype(np.float32), threads=threads)
    ddt = (time.perf_counter() - t1) / 10
    return {"value": B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the whole prefill batch (B={B}, T={T}, H={inp.q.shape[2]}), fp64 token recurrence, "
                      f"{dt:.2f} s wall; decode leg: 10 steps of the decode workload",
            "decode_ms_per_step": round(ddt * 1e3, 2)}


def workload_leg(name, kda, ki, torch, dev, stream, steps, cpu_heads, want_cpu):
    """kda_chunk_fwd over one of the other full-size chunked workloads (long prefill, packed varlen),
    inputs drawn on the GPU with the workload's recipe and seed (kda_inputs.workload_inputs_on),
    at the workload's chunk with the library's other defaults, and again with the library's
    default chunk (`default_chunk`); initial state given and final state written.  The CPU oracle
    is timed on `cpu_heads` of its heads (all sequences, all tokens of those heads)."""
    w = ki.WORKLOADS[name]
    inp = ki.workload_inputs_on(name, dev)
    B, T, H = inp.q.shape[0], inp.q.shape[1], inp.q.shape[2]
    n = inp.num_seqs
    varlen = inp.cu_seqlens is not None
    out = torch.empty_like(inp.v)
    fin = torch.empty((n, H, w.dk, w.dv), dtype=torch.float32, device=dev)
    cu_host = inp.cu_seqlens.cpu() if varlen else None
    reps = max(3, steps // 4)

    def timed(chunk):
        q = kda.query(B, T, H, w.dk, w.dv, w.io, num_seqs=n if varlen else 0, chunk_size=chunk, device=True)
        ws = torch.empty(max(q["workspace_bytes"], 1), dtype=torch.uint8, device=dev)

        def call():
            kda.chunk_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0, inp.cu_seqlens, cu_seqlens_host=cu_host,
                          chunk_size=chunk, workspace=ws, out=out, final_state=fin)

        for _ in range(2):
            call()
        torch.cuda.synchronize()
        ms = time_launches(call, reps, stream)
        del ws
        return q, ms

    tokens = B * T
    qd, msd = timed(0)
    q, ms = timed(w.chunk)
    gbps = q["hbm_bytes"] / (ms * 1e-3) / 1e9
    leg = {"workload": f"{name}: " + (f"{n} packed sequences, {T} tokens" if varlen else f"B={B} T={T}") +
                       f", H={H}, d_k=d_v={w.dk}, {w.io} q/k/v, fp32 gate/beta/state",
           "chunk": q["chunk_size"], "dv_tile": q["dv_tile"], "algo": ["auto", "fused", "two_pass"][q["algo"]],
           "calls_timed": reps, "ms": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
           "bytes_per_launch": q["hbm_bytes"], "gb_per_s": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
           "tflops": round(q["flops"] / (ms * 1e-3) / 1e12, 2),
           "default_chunk": {"chunk": qd["chunk_size"], "dv_tile": qd["dv_tile"], "ms": round(msd, 4),
                             "tokens_per_s": round(tokens / (msd * 1e-3), 1),
                             "hbm_frac": round(qd["hbm_bytes"] / (msd * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
           "data": "synthetic, drawn on the GPU with the workload's recipe and seed"}
    log(f"{name}: {leg['ms']} ms per call, {leg['tokens_per_s'] / 1e6:.1f} M tokens/s, hbm_frac {leg['hbm_frac']}")
    if want_cpu:
        import oracle
        sel = list(range(min(cpu_heads, H)))
        host = lambda x: x[:, :, sel].contiguous().cpu()
        a = [ki.to_numpy_io(host(x)) for x in (inp.q, inp.k, inp.v)]
        g, beta = host(inp.g).numpy(), host(inp.beta).numpy()
        s0 = inp.s0[:, sel].contiguous().cpu().numpy()
        threads = oracle.default_threads()
        t0 = time.perf_counter()
        oracle.fwd(*a, g, beta, initial_state=s0, cu_seqlens=None if cu_host is None else cu_host.numpy(),
                   threads=threads)
        dt = time.perf_counter() - t0
        # tokens/s of the whole workload at the sample's rate (the oracle's cost is linear in heads)
        leg["cpu_baseline"] = {"value": round(tokens * len(sel) / H / dt, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{len(sel)} of {H} heads, every sequence and token, fp64 token recurrence, "
                                         f"{dt:.2f} s wall, scaled to the whole workload"}
        log(f"{name}: CPU oracle on {len(sel)} heads took {dt:.1f} s")
    del inp, out, fin
    torch.cuda.empty_cache()
    return leg


def dplr_sweep(kda, ki, torch, dev, stream, steps):
    """KDA (fused and two-pass) against the general-DPLR comparator over sequence lengths,
    4 sequences x 16 heads, d = 128, chunk 64, bf16."""
    rows = []
    for T in (1024, 4096, 16384):
        inp = ki.make_inputs(4, T, 16, 128, 128, "bf16", seed=11)
        t = {k: x.to(dev) for k, x in dict(q=inp.q, k=inp.k, v=inp.v, g=inp.g, beta=inp.beta, s0=inp.s0).items()}
        a, b, kw = (x.to(dev) for x in ki.dplr_inputs(inp, 9))
        o = torch.empty_like(t["v"])
        f = torch.empty_like(t["s0"])
        ws = torch.empty(max(kda.query(4, T, 16, 128, 128, "bf16", chunk_size=64)["workspace_bytes"], 1),
                         dtype=torch.uint8, device=dev)
        calls = {
            "dplr_fused": lambda: kda.dplr_chunk_fwd(t["q"], kw, t["v"], a, b, t["g"], t["s0"], chunk_size=64,
                                                     dv_tile=32, out=o, final_state=f),
            "kda_fused": lambda: kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk_size=64,
                                               dv_tile=32, algo="fused", out=o, final_state=f),
            "kda_two_pass": lambda: kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["s0"], chunk_size=64,
                                                  algo="two_pass", workspace=ws, out=o, final_state=f),
        }
        row = {"T": T}
        for name, fn in calls.items():
            fn()
            row[name + "_ms"] = round(time_launches(fn, max(3, steps // 4), stream), 4)
        row["kda_speedup_same_design"] = round(row["dplr_fused_ms"] / row["kda_fused_ms"], 3)
        row["kda_speedup_vs_default"] = round(row["dplr_fused_ms"] / row["kda_two_pass_ms"], 3)
        log(f"dplr sweep T={T}: {row}")
        rows.append(row)
        del t, a, b, kw, o, f, ws
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--dv-tile", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=64,
                    help="forward chunk of the prefill step (the workload's 64; 0: the library's default)")
    ap.add_argument("--bwd-chunk", type=int, default=64, help="backward chunk")
    ap.add_argument("--algo", default="auto", choices=["auto", "fused", "two_pass"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the long-prefill and packed-varlen legs (profiling runs of the prefill shape)")
    ap.add_argument("--dplr-sweep", action="store_true",
                    help="also time the general-DPLR comparator against KDA over sequence lengths 1K..16K")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the general-DPLR comparison (profiling runs: its fused-KDA timing launches the same "
                         "kernel instantiation as the backward's forward pass)")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the autotuning sweep (profiling runs: it launches the same fused kernel "
                         "instantiation as the backward's forward pass)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA path has no multi-GPU mode (heads and sequences are "
              "independent, so more GPUs would each take a share of them). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_45_amd as kda
    import kda_inputs as ki

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------------------------------------------------------- prefill
    w = ki.WORKLOADS["prefill"]
    inp = ki.workload_inputs("prefill")
    d = {k: (None if x is None else x.to(dev)) for k, x in
         dict(q=inp.q, k=inp.k, v=inp.v, g=inp.g, beta=inp.beta, s0=inp.s0).items()}
    B, T, H = w.B, w.T, w.H
    out = torch.empty((B, T, H, w.dv), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, H, w.dk, w.dv), dtype=torch.float32, device=dev)
    q = kda.query(B, T, H, w.dk, w.dv, "bf16", chunk_size=args.chunk, dv_tile=args.dv_tile, algo=args.algo,
                  device=True)
    ws = torch.empty(max(q["workspace_bytes"], 1), dtype=torch.uint8, device=dev)

    def prefill():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk_size=args.chunk,
                      dv_tile=args.dv_tile, algo=args.algo, workspace=ws, out=out, final_state=fin)

    # the same call with the library's default chunk, reported beside the step
    qdef = kda.query(B, T, H, w.dk, w.dv, "bf16", device=True)
    ws_def = torch.empty(max(qdef["workspace_bytes"], 1), dtype=torch.uint8, device=dev)

    def prefill_default():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], workspace=ws_def, out=out,
                      final_state=fin)

    # ----------------------------------------------------------------- decode
    wd = ki.WORKLOADS["decode"]
    dinp = ki.workload_inputs("decode")
    sq = lambda x: x[:, 0].contiguous().to(dev)
    dq, dk_, dv_, dg, db = (sq(x) for x in (dinp.q, dinp.k, dinp.v, dinp.g, dinp.beta))
    dstate = dinp.s0.to(dev)
    dout = torch.empty((wd.B, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)

    def decode():
        kda.decode_step(dq, dk_, dv_, dg, db, dstate, out=dout)

    # decode step with the output epilogue: fused (one kernel) and composed (decode, then norm_gate)
    _, dgate, dnw = (x.to(dev) for x in ki.epilogue_inputs((wd.B, wd.H, wd.dv), "bf16", seed=15))
    dgout = torch.empty_like(dout)

    def decode_gated():
        kda.decode_step_gated(dq, dk_, dv_, dg, db, dstate, dgate, dnw, eps=1e-6, out=dgout)

    def decode_then_norm_gate():
        kda.decode_step(dq, dk_, dv_, dg, db, dstate, out=dout)
        kda.norm_gate(dout, dgate, dnw, eps=1e-6, out=dgout)

    # ------------------------------------------- prologue (raw projections of the prefill shape)
    pin = ki.prologue_inputs(B, T, H, w.dk, w.dv, 4, "bf16", seed=6)
    pd = {k: (None if x is None else x.to(dev)) for k, x in pin.items()}

    def prologue():
        kda.prologue(pd["q_raw"], pd["k_raw"], pd["v_raw"], pd["conv_q"], pd["conv_k"], pd["conv_v"], pd["g_raw"],
                     pd["beta_raw"])

    # the forward on raw projections: prologue fused into the two-pass kernels, and composed
    # (kda_prologue, then kda_chunk_fwd)
    def forward_raw_fused():
        kda.chunk_fwd_prologue(pd["q_raw"], pd["k_raw"], pd["v_raw"], pd["conv_q"], pd["conv_k"], pd["conv_v"],
                               pd["g_raw"], pd["beta_raw"], d["s0"], chunk_size=args.chunk, workspace=ws, out=out,
                               final_state=fin)

    def forward_raw_composed():
        pq, pk, pv, pg, pb = kda.prologue(pd["q_raw"], pd["k_raw"], pd["v_raw"], pd["conv_q"], pd["conv_k"],
                                          pd["conv_v"], pd["g_raw"], pd["beta_raw"])
        kda.chunk_fwd(pq, pk, pv, pg, pb, d["s0"], chunk_size=args.chunk, algo="two_pass", workspace=ws, out=out,
                      final_state=fin)

    # ------------------------------------------- output epilogue (prefill output shape)
    eo, ez, ew = (x.to(dev) for x in ki.epilogue_inputs((B, T, H, w.dv), "bf16", seed=5))
    eout = torch.empty_like(eo)

    def epilogue():
        kda.norm_gate(eo, ez, ew, eps=1e-6, out=eout)

    # ------------------------------------------- backward (training) on the prefill tensors
    d_out_b, dsf_b = (None if x is None else x.to(dev) for x in ki.grad_inputs(inp, 8))
    bp, _ = kda._problem_from(d["q"], d["v"], None, args.bwd_chunk, 1.0, 0, 0)
    bws = torch.empty(kda.bwd_workspace_bytes(bp), dtype=torch.uint8, device=dev)
    bout = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_out_b, initial_state=d["s0"],
                         d_final_state=dsf_b, chunk_size=args.bwd_chunk, workspace=bws)

    def backward():
        kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_out_b, initial_state=d["s0"], d_final_state=dsf_b,
                      chunk_size=args.bwd_chunk, workspace=bws, out=bout)

    # ------------------------------------------- general-DPLR comparator on the prefill tensors
    a_d, b_d, kw_d = (x.to(dev) for x in ki.dplr_inputs(inp, 9))
    cmp_out, cmp_fin = torch.empty_like(out), torch.empty_like(fin)

    def dplr_fused():
        kda.dplr_chunk_fwd(d["q"], kw_d, d["v"], a_d, b_d, d["g"], d["s0"], chunk_size=64, dv_tile=32, out=cmp_out,
                           final_state=cmp_fin)

    def kda_fused():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], chunk_size=64, dv_tile=32, algo="fused",
                      out=cmp_out, final_state=cmp_fin)

    # the comparator's long fused kernels are warmed right before their own timing, so that they do not
    # set the clock and power state the step itself is timed in
    for _ in range(args.warmup):
        backward()
        prefill()
        decode()
        decode_gated()
        decode_then_norm_gate()
        epilogue()
        prologue()
        forward_raw_fused()
        forward_raw_composed()
        prefill_default()
    torch.cuda.synchronize()

    # timed region: K steps, each = one prefill launch + one decode launch
    t_pre = time_launches(prefill, args.steps, stream)
    t_dec = time_launches(decode, args.steps, stream)
    t_epi = time_launches(epilogue, args.steps, stream)
    pre_med, pre_min = time_each(prefill, args.steps, stream)
    t_pre_def = time_launches(prefill_default, args.steps, stream)
    dec_med, dec_min = time_each(decode, args.steps, stream)
    t_decg = time_launches(decode_gated, args.steps, stream)
    t_decc = time_launches(decode_then_norm_gate, args.steps, stream)
    t_pro = time_launches(prologue, args.steps, stream)
    t_rawf = time_launches(forward_raw_fused, args.steps, stream)
    t_rawc = time_launches(forward_raw_composed, args.steps, stream)
    t_bwd = time_launches(backward, args.steps, stream)
    t_dplr = t_kfused = None
    if not args.no_compare:
        for _ in range(args.warmup):
            dplr_fused()
            kda_fused()
        t_dplr = time_launches(dplr_fused, args.steps, stream)
        t_kfused = time_launches(kda_fused, args.steps, stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    decode()
    start.record(stream)
    for _ in range(args.steps):
        prefill()
        decode()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    # autotuning over (chunk, d_v tile, algorithm) on the prefill tensors, reported alongside
    tuned = None if args.no_tune else kda.tune(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                                final_state=torch.empty_like(fin))
    traffic = measured_traffic()
    tokens = B * T
    pre_tps = tokens / (t_pre * 1e-3)
    pre_bytes = q["hbm_bytes"]
    pre_gbps = pre_bytes / (t_pre * 1e-3) / 1e9
    pre_tflops = q["flops"] / (t_pre * 1e-3) / 1e12
    dec_bytes = (wd.B * wd.H * (2 * 4 * wd.dk * wd.dv + (2 * wd.dk + 2 * wd.dv) * 2 + 4 * wd.dk + 4))
    dec_gbps = dec_bytes / (t_dec * 1e-3) / 1e9
    decg_bytes = dec_bytes + wd.B * wd.H * wd.dv * 2 + wd.dv * 4  # + gate (bf16) and the norm weight
    decg_gbps = decg_bytes / (t_decg * 1e-3) / 1e9
    epi_rows = B * T * H
    epi_bytes = epi_rows * w.dv * 2 * 3 + w.dv * 4  # o and gate read, out written (bf16), weight
    epi_gbps = epi_bytes / (t_epi * 1e-3) / 1e9
    # prologue per (token, head): raw q, k, v (bf16) + g_raw + beta_raw read, the same written
    pro_bytes = B * T * H * 2 * ((2 * w.dk + w.dv) * 2 + 4 * w.dk + 4) + 4 * H * (2 * w.dk + w.dv) * 4
    pro_gbps = pro_bytes / (t_pro * 1e-3) / 1e9
    # backward per (token, head): q, k, v, dO (bf16), g (fp32), beta read; dq, dk, dv (bf16), dg (fp32),
    # dbeta written; per (sequence, head): initial state and final-state gradient read, d(initial state) written
    bwd_bytes = B * T * H * 2 * ((2 * w.dk + w.dv) * 2 + 4 * w.dk + 4) + B * T * H * w.dv * 2 + \
        3 * B * H * w.dk * w.dv * 4
    bwd_gbps = bwd_bytes / (t_bwd * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(pre_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill B={B} T={T} H={H} d_k=d_v={w.dk} chunk={q['chunk_size']} bf16 q/k/v, "
                               f"fp32 gate/beta/state + decode {wd.B} seqs x {wd.H} heads, d=128",
                   "dv_tile": q["dv_tile"], "algo": ["auto", "fused", "two_pass"][q["algo"]],
                   "workspace_bytes": q["workspace_bytes"], "device": q["arch"], "compute_units": q["compute_units"]},
        "roofline": {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(pre_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic.get("prefill_bytes") if q["algo"] == 2 else None,
                     "frac_measured": None if q["algo"] != 2 or traffic.get("prefill_bytes") is None else
                     round(traffic["prefill_bytes"] / (t_pre * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "kernel": "kda_chunk_fwd (" + ["auto", "fused", "two_pass"][q["algo"]] + ")",
                     "launch_ms": round(t_pre, 4),
                     "bytes_per_launch": pre_bytes},
        "decode_roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic.get("decode_bytes"),
                            "kernel": "kda_decode_step", "launch_ms": round(t_dec, 4),
                            "bytes_per_launch": dec_bytes},
        "prefill": {"ms": round(t_pre, 4), "ms_median": round(pre_med, 4), "ms_min": round(pre_min, 4),
                    "tokens_per_s": round(pre_tps, 1), "gb_per_s": round(pre_gbps, 1),
                    "hbm_frac": round(pre_gbps / PEAK_HBM_GBPS, 4), "tflops": round(pre_tflops, 2),
                    "mfma_frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4), "flops_per_launch": q["flops"],
                    "flops_count": "per head-token 2C(d_k+d_v) + C^2/3 + 6 d_k d_v: the products this algorithm "
                                   "runs (A, P, T(V - K~S), PD, K~S, Q~S, K-^T D); forming W = T K~ as well, which "
                                   "it never does, would add C d_k",
                    "mfma_frac_with_w": round(pre_tflops * (1 + tokens * H * q["chunk_size"] * w.dk / q["flops"])
                                              / PEAK_BF16_TFLOPS, 4)},
        "prefill_default_chunk": {"chunk": qdef["chunk_size"], "dv_tile": qdef["dv_tile"], "ms": round(t_pre_def, 4),
                                  "tokens_per_s": round(tokens / (t_pre_def * 1e-3), 1),
                                  "hbm_frac": round(pre_bytes / (t_pre_def * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                  "tflops": round(qdef["flops"] / (t_pre_def * 1e-3) / 1e12, 2),
                                  "traffic": traffic.get("prefill_default_chunk_bytes")},
        "decode": {"ms": round(t_dec, 4), "ms_median": round(dec_med, 4), "ms_min": round(dec_min, 4),
                   "gb_per_s": round(dec_gbps, 1), "hbm_frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                   "bytes_per_launch": dec_bytes},
        "decode_gated": {"kernel": "kda_decode_step_gated", "ms": round(t_decg, 4), "gb_per_s": round(decg_gbps, 1),
                         "hbm_frac": round(decg_gbps / PEAK_HBM_GBPS, 4), "bytes_per_launch": decg_bytes,
                         "composed_ms": round(t_decc, 4), "composed": "kda_decode_step + kda_norm_gate",
                         "speedup_vs_composed": round(t_decc / t_decg, 3),
                         "traffic": traffic.get("decode_gated_bytes")},
        "tuned": None if tuned is None else {"chunk": tuned["chunk_size"], "dv_tile": tuned["dv_tile"],
                                             "algo": ["auto", "fused", "two_pass"][tuned["algo"]],
                                             "ms": round(tuned["tuned_ms"], 4)},
        "backward": {"kernel": "kda_chunk_bwd", "chunk": args.bwd_chunk, "ms": round(t_bwd, 4),
                     "tokens_per_s": round(tokens / (t_bwd * 1e-3), 1), "gb_per_s": round(bwd_gbps, 1),
                     "hbm_frac": round(bwd_gbps / PEAK_HBM_GBPS, 4), "bytes_per_launch": bwd_bytes,
                     "traffic": traffic.get("backward_bytes")},
        "dplr_comparator": None if t_dplr is None else {
            "shape": "prefill", "chunk": 64, "dv_tile": 32, "dplr_fused_ms": round(t_dplr, 4),
            "kda_fused_ms": round(t_kfused, 4), "kda_two_pass_ms": round(t_pre, 4),
            "kda_speedup_same_design": round(t_dplr / t_kfused, 3), "kda_speedup_vs_default": round(t_dplr / t_pre, 3)},
        "prologue": {"kernel": "kda_prologue", "conv_width": 4, "ms": round(t_pro, 4),
                     "gb_per_s": round(pro_gbps, 1), "hbm_frac": round(pro_gbps / PEAK_HBM_GBPS, 4),
                     "bytes_per_launch": pro_bytes, "traffic": traffic.get("prologue_bytes")},
        "forward_raw": {"kernel": "kda_chunk_fwd_prologue", "conv_width": 4, "ms": round(t_rawf, 4),
                        "tokens_per_s": round(tokens / (t_rawf * 1e-3), 1), "composed_ms": round(t_rawc, 4),
                        "composed": "kda_prologue + kda_chunk_fwd (two-pass)",
                        "speedup_vs_composed": round(t_rawc / t_rawf, 3),
                        "traffic": traffic.get("forward_raw_bytes")},
        "epilogue": {"kernel": "kda_norm_gate", "rows": epi_rows, "d": w.dv, "ms": round(t_epi, 4),
                     "gb_per_s": round(epi_gbps, 1), "hbm_frac": round(epi_gbps / PEAK_HBM_GBPS, 4),
                     "bytes_per_launch": epi_bytes, "traffic": traffic.get("epilogue_bytes")},
    }
    if not args.no_workloads:
        del d, d_out_b, dsf_b, bws, bout, a_d, b_d, kw_d, cmp_out, cmp_fin, ws, pd, eo, ez, ew, eout
        torch.cuda.empty_cache()
        res["long_prefill"] = workload_leg("long_prefill", kda, ki, torch, dev, stream, args.steps, 16,
                                           not args.no_cpu_baseline)
        res["varlen"] = workload_leg("varlen", kda, ki, torch, dev, stream, args.steps, 8, not args.no_cpu_baseline)
    if args.dplr_sweep:
        res["dplr_sweep"] = dplr_sweep(kda, ki, torch, dev, stream, args.steps)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the prefill batch ...")
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
