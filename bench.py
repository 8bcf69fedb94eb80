"""Benchmark of the GDN-2 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunk-parallel forward (gdn2_chunk_fwd) over the training-shape
workload B=8, T=4096, H=16, dk=dv=128 (bf16 q,k,v,b,w, fp32 log alpha, zero
initial state, fp32 final state; o in fp32 unless --out-bf16), inputs resident
in HBM before timing.  The decode workload (N=256 sequences x H=16, 128x128 fp32
state, one token per step, 1024 steps) is timed in the same run and reported
under "decode"; the long-context workload (B=1, T=32768) under "long_context";
a sweep of T at B*T = 32768 under "t_sweep".

Prints one JSON line.  `value` is tokens/s (B*T tokens per step).  `roofline`
gives the chunk kernel's algorithmic HBM bytes per launch (2,048 B per
head-token: q, k, b, v, w in bf16, log alpha fp32, o counted as bf16, plus the
fp32 final state) over its average launch time, measured with HIP events on the
stream the kernel runs on; the extra bytes of an fp32 o are listed beside it.
`cpu_baseline` is the fp64 oracle timed on the same workload on this host's
cores.
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

METRIC = "GDN-2 chunked fwd tokens/s (T=4K,H=16,d=128); decode state GB/s vs peak"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def chunk_bytes(B, T, H, dk, dv, in_bytes=2, with_s0=False):
    """Algorithmic HBM bytes of one forward: q, k, b, v, w read once in the input dtype, log
    alpha fp32, o written once in the input dtype (2,048 B per head-token at d = 128 in bf16),
    plus the fp32 final state (and the initial state when one is given)."""
    per_head_token = 3 * dk * in_bytes + 2 * dv * in_bytes + dk * 4 + dv * in_bytes
    state = B * H * dk * dv * 4 * (2 if with_s0 else 1)
    return B * T * H * per_head_token + state


def logits_chunk_bytes(B, T, H, dk, dv, in_bytes=2):
    """The same for the forward from gate logits: the decay logits are read in the input dtype
    instead of an fp32 log alpha (1,792 B per head-token at d = 128 in bf16)."""
    per_head_token = 4 * dk * in_bytes + 2 * dv * in_bytes + dv * in_bytes
    return B * T * H * per_head_token + B * H * dk * dv * 4


def fp32_o_extra_bytes(B, T, H, dv, in_bytes=2):
    """Bytes an fp32 o writes beyond the input-dtype o that chunk_bytes counts."""
    return B * T * H * dv * (4 - in_bytes)


def chunk_flops(B, T, H, dk, dv, C=64):
    """Algorithmic matrix flops of the chunk form per launch (2 per multiply-add), counting the
    causal (triangular) parts only: per chunk A (C(C-1)/2 dk), P (C(C+1)/2 dk), W = T(b.k.Gamma)
    (C(C+1)/2 dk), U0 = T(w.v) and P U (C(C+1)/2 dv each), the triangular inverse (C^3/6) and the
    state products W S, (q.Gamma) S, (k.Gamma')^T U (3 C dk dv)."""
    nchunks = B * H * ((T + C - 1) // C)
    tri_lo, tri = C * (C - 1) // 2, C * (C + 1) // 2
    mac = tri_lo * dk + tri * dk + tri * dk + 2 * tri * dv + C ** 3 / 6 + 3 * C * dk * dv
    return int(nchunks * 2 * mac)


def host_info():
    """CPU model and logical CPU count of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count()}


def decode_bytes(N, H, dk, dv, in_bytes=2, out_bytes=4):
    """Algorithmic HBM bytes of one decode step: state read + written, token vectors, o."""
    return N * H * (2 * dk * dv * 4 + 3 * dk * in_bytes + 2 * dv * in_bytes + dk * 4 + dv * out_bytes)


def recorded_traffic(profile, sources):
    """HBM bytes per launch from a committed counter summary, or None.

    The summary's `traffic-record:` line holds FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy of known size, and a hash of the kernel sources that were
    profiled; the figure is reported only while the sources still hash to it."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "gated_delta_rule_gdn2_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(path) as fh:
        m = re.search(r"^traffic-record: kernel=.* sources=([0-9a-f]+) bytes=(\d+)$", fh.read(), re.M)
    if m is None or m.group(1) != h.hexdigest()[:len(m.group(1))]:
        return None
    return int(m.group(2))


CHUNK_PROFILE = ("chunk_fwd_train_B8_T4096_H16_d128.md", ("gdn2_chunk_bf16.hip", "gdn2_bf16_ops.h", "gdn2_device.h"))
DECODE_PROFILE = ("decode_step_N256_H16_d128.md", ("gdn2_decode.hip", "gdn2_device.h"))
PREFILL_PROFILE = ("prefill_varlen_N64_H16_d128.md", ("gdn2_chunk_bf16.hip", "gdn2_bf16_ops.h", "gdn2_device.h"))


def spin_up(fn, torch, seconds=0.3):
    """Run fn untimed for about `seconds` of GPU time: the GPU's clocks ramp up over the first
    tenths of a second of work, and a short warm-up alone times a cold GPU."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds or n < 2:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


SPIN_UP = True  # --no-spin-up clears it (counter runs, where every dispatch is collected)


def time_launches(fn, steps, warmup, torch, spin=True):
    if spin and SPIN_UP:
        spin_up(fn, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per launch


def cpu_baseline(wl, torch):
    """The oracle as it stands, on the same workload (all 128 sequences, all 4096 tokens)."""
    import oracle
    import workloads as W

    Bs, Ts = wl.B, wl.T
    inp = W.make_inputs(wl, B=Bs, T=Ts)
    threads = min(oracle.default_threads(), Bs * wl.H)
    t0 = time.perf_counter()
    oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["s0"],
               nthreads=threads)
    dt = time.perf_counter() - t0
    out = {"value": Bs * Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "fp64 oracle on the whole workload: B=%d T=%d H=%d d=%d (%d of %d sequences, "
                     "%d tokens each), %.2f s wall on %d threads" % (Bs, Ts, wl.H, wl.dk, Bs * wl.H,
                                                                    wl.B * wl.H, Ts, dt, threads)}
    out.update(host_info())
    return out


def cpu_baseline_decode(steps=8):
    """The oracle's decode step on the decode workload (all 256 sequences x 16 heads), a bounded
    number of steps: steps/s and the fp64 state bytes it streams (read + written) per second."""
    import oracle
    import workloads as W

    wl = W.DECODE
    pool = W.make_decode_pool(wl)
    state = pool["state"].double().numpy()
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    for s in range(steps):
        p = s % wl.pool
        _, state = oracle.decode(pool["q"][p], pool["k"][p], pool["v"][p], pool["log_alpha"][p],
                                 pool["b"][p], pool["w"][p], state, nthreads=threads)
    dt = (time.perf_counter() - t0) / steps
    state_bytes = 2 * wl.B * wl.H * wl.dk * wl.dv * 8
    return {"us_per_step": dt * 1e6, "state_GBps_fp64": state_bytes / dt / 1e9, "cores": threads,
            "kind": "oracle", "sample": "%d steps of N=%d x H=%d, d=%d (fp64 state %d MB)" % (
                steps, wl.B, wl.H, wl.dk, state_bytes // 2 // 1000000)}


def run_chunk(args, torch, gdn2, W, dev, out_dtype, keep=False):
    """Chunk forward on the training-shape workload; returns (ms per launch, workload, bytes,
    device inputs if keep)."""
    wl = W.TRAIN_4K
    inp = W.make_inputs(wl)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    del inp
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=out_dtype, device=dev)
    sT = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn2.chunk_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, split=True) + 256,
                     dtype=torch.uint8, device=dev)

    def step(fused=None):
        gdn2.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["s0"], o=o,
                       final_state=sT, out_dtype=out_dtype, workspace=ws, fused=fused)

    ms = time_launches(step, args.steps, args.warmup, torch)
    forms = {"fused": time_launches(lambda: step(True), args.steps, args.warmup, torch),
             "split": time_launches(lambda: step(False), args.steps, args.warmup, torch)}
    nbytes = chunk_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    del o, sT, ws
    if not keep:
        del d
        d = None
    torch.cuda.empty_cache()
    return ms, wl, nbytes, d, forms


def run_long(args, torch, gdn2, W, dev, out_dtype):
    """The long-context workload: one sequence of 32,768 tokens, 16 heads (half with strong
    decay), the same kernel and byte count per head-token as the training shape."""
    wl = W.LONG_32K
    inp = W.make_inputs(wl)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    del inp
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=out_dtype, device=dev)
    sT = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn2.chunk_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, split=True) + 256,
                     dtype=torch.uint8, device=dev)

    def step(fused=None):
        gdn2.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["s0"], o=o,
                       final_state=sT, out_dtype=out_dtype, workspace=ws, fused=fused)

    ms = time_launches(step, max(3, args.steps // 4), 2, torch)
    ms_fused = time_launches(lambda: step(True), 3, 1, torch)
    ms_split = time_launches(lambda: step(False), 3, 1, torch, spin=False)
    nbytes = chunk_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    gbps = nbytes / (ms * 1e-3) / 1e9
    del d, o, sT, ws
    torch.cuda.empty_cache()
    return {"workload": wl.name, "us_per_launch": ms * 1e3, "tokens_per_s": wl.B * wl.T / (ms * 1e-3),
            "GBps": gbps, "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": nbytes, "fused_us": ms_fused * 1e3, "split_us": ms_split * 1e3,
            "form": "split" if gdn2.chunk_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv) else "fused",
            "note": "B*H = 16 (sequence, head) chains of 512 chunks each"}


def run_sweep(args, torch, gdn2, d, dev, out_dtype, H=16, dk=128, dv=128, total=32768):
    """Tokens/s against sequence length at a fixed B*T = 32,768 tokens: the training-shape inputs
    (already on the device) viewed as B = 32768 / T sequences of T tokens each."""
    out = []
    for T in (512, 1024, 2048, 4096, 8192, 16384, 32768):
        B = total // T
        v = {n: x.view(B, T, *x.shape[2:]) for n, x in d.items() if x is not None}
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
        sT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        ws = torch.empty(gdn2.chunk_fwd_workspace_bytes(B, T, H, dk, dv, split=True) + 256, dtype=torch.uint8,
                         device=dev)

        def step(fused=None):
            gdn2.chunk_fwd(v["q"], v["k"], v["v"], v["log_alpha"], v["b"], v["w"], None, o=o, final_state=sT,
                           out_dtype=out_dtype, workspace=ws, fused=fused)

        ms = time_launches(step, max(3, args.steps // 4), 2, torch)
        ms_fused = time_launches(lambda: step(True), 3, 1, torch, spin=False)
        ms_split = time_launches(lambda: step(False), 3, 1, torch, spin=False)
        nbytes = chunk_bytes(B, T, H, dk, dv)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out.append({"T": T, "B": B, "us_per_launch": ms * 1e3, "tokens_per_s": total / (ms * 1e-3),
                    "frac": gbps / HBM_PEAK_GBPS, "fused_us": ms_fused * 1e3, "split_us": ms_split * 1e3,
                    "form": "split" if gdn2.chunk_fwd_workspace_bytes(B, T, H, dk, dv) else "fused"})
        del o, sT, ws
    torch.cuda.empty_cache()
    return out


def run_prefill(args, torch, gdn2, W, dev, out_dtype):
    """Serving prefill: 64 prompts of a seeded length mix packed along one token axis, with
    continuation states, through the packed-sequence forward."""
    wl = W.SERVE_PREFILL
    lengths = W.make_lengths(wl.B, wl.seed)
    inp = W.make_packed_inputs(wl, lengths)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    del inp
    total = sum(lengths)
    o = torch.empty((total, wl.H, wl.dv), dtype=out_dtype, device=dev)
    sT = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)

    def step():
        gdn2.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["cu_seqlens"],
                              d["s0"], o=o, final_state=sT, out_dtype=out_dtype)

    ms = time_launches(step, args.steps, args.warmup, torch)
    per_tok = 3 * wl.dk * 2 + 2 * wl.dv * 2 + wl.dk * 4 + wl.dv * 2  # o counted in the input dtype
    nbytes = total * wl.H * per_tok + 2 * wl.B * wl.H * wl.dk * wl.dv * 4 + (wl.B + 1) * 8
    extra = fp32_o_extra_bytes(1, total, wl.H, wl.dv) if out_dtype == torch.float32 else 0
    gbps = nbytes / (ms * 1e-3) / 1e9
    del d, o, sT
    torch.cuda.empty_cache()
    return {"workload": wl.name, "sequences": wl.B, "tokens": total,
            "lengths": "log-normal around 512 (sigma 1), clipped to [1, 4096], seed %d" % wl.seed,
            "us_per_launch": ms * 1e3, "tokens_per_s": total / (ms * 1e-3), "GBps": gbps,
            "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS,
            "traffic": recorded_traffic(*PREFILL_PROFILE) if out_dtype == torch.float32 else None,
            "algorithmic_bytes_per_launch": nbytes, "fp32_o_extra_bytes_per_launch": extra}


def bwd_bytes(B, T, H, dk, dv, in_bytes=2, s0=True):
    """Algorithmic HBM bytes of one backward call: the inputs (q, k, b, v, w in the input
    dtype, log alpha fp32), the upstream gradient d_o (fp32) and S_0, and the gradients written
    (dq, dk, db, dlog alpha, dv, dw fp32, dS_0).  The workspace round trips (states entering
    every chunk, their gradients, U, dR, T and P) are the implementation's, not the method's."""
    ht = B * T * H
    per_tok = (3 * dk + 2 * dv) * in_bytes + dk * 4 + dv * 4 + (4 * dk + 2 * dv) * 4
    return ht * per_tok + (2 if s0 else 1) * B * H * dk * dv * 4


def run_bwd(args, torch, gdn2, W, dev):
    """Backward pass on the fwd+bwd workload: gradients of every input from d_o ~ N(0,1),
    with S_0 ~ N(0, 0.02^2) and no upstream state gradient."""
    wl = W.FWD_BWD_4K
    inp = W.make_inputs(wl)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    d_o = W.make_upstream_grad(wl).to(dev)
    del inp
    ws = torch.empty(gdn2.chunk_bwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv), dtype=torch.uint8,
                     device=dev)
    grads = gdn2.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d_o, d["s0"], workspace=ws)

    def step():
        gdn2.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d_o, d["s0"], workspace=ws,
                       grads=grads)

    ms = time_launches(step, args.steps, args.warmup, torch)
    nbytes = bwd_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    gbps = nbytes / (ms * 1e-3) / 1e9
    tokens = wl.B * wl.T
    out = {"workload": wl.name, "us_per_call": ms * 1e3, "tokens_per_s": tokens / (ms * 1e-3), "GBps": gbps,
           "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_call": nbytes,
           "workspace_bytes": ws.numel(),
           "kernels": "bwd_local_kernel (chunk-local quantities), bwd_fwd_kernel (forward re-run), "
                      "bwd_state_kernel (reverse pass), bwd_chunk_kernel (per-chunk gradients)"}
    del d, d_o, ws, grads
    torch.cuda.empty_cache()
    return out


def mixer_bytes(B, T, H, dk, dv, in_bytes=2, o_bytes=4):
    """Algorithmic HBM bytes of the two fused mixer passes.  prep: the six projection outputs
    read, q, k, v, b, w (input dtype) and log alpha (fp32) written, and the taps; out: o and z
    read, y written, and gamma."""
    ht = B * T * H
    prep = ht * ((4 * dk + 2 * dv) * in_bytes + (3 * dk + 2 * dv) * in_bytes + dk * 4) + H * (2 * dk + dv) * 16
    out = ht * (dv * o_bytes + 2 * dv * in_bytes) + dv * 4
    return prep, out


def run_mixer(args, torch, gdn2, W, dev):
    """The mixer's fused passes on the training shape: prep (projection outputs to the
    recurrence's inputs) and out (RMS norm and SiLU gate of an fp32 recurrence output)."""
    wl = W.TRAIN_4K
    x = {n: t.to(dev) for n, t in W.make_mixer_inputs(wl).items()}
    names = ("xq", "xk", "xv", "xb", "xw", "xa", "conv_q", "conv_k", "conv_v")
    res = gdn2.mixer_prep(*[x[n] for n in names])
    o = torch.randn((wl.B, wl.T, wl.H, wl.dv), dtype=torch.float32, device=dev)
    y = gdn2.mixer_out(o, x["z"], x["gamma"])
    ms_p = time_launches(lambda: gdn2.mixer_prep(*[x[n] for n in names], out=res), args.steps, args.warmup, torch)
    ms_o = time_launches(lambda: gdn2.mixer_out(o, x["z"], x["gamma"], y=y), args.steps, args.warmup, torch)
    bp, bo = mixer_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    gp, go = bp / (ms_p * 1e-3) / 1e9, bo / (ms_o * 1e-3) / 1e9
    del x, res, o, y
    torch.cuda.empty_cache()
    return {"workload": wl.name,
            "prep": {"kernel": "prep_kernel", "us_per_launch": ms_p * 1e3, "GBps": gp, "peak": HBM_PEAK_GBPS,
                     "frac": gp / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": bp},
            "out": {"kernel": "out_kernel", "us_per_launch": ms_o * 1e3, "GBps": go, "peak": HBM_PEAK_GBPS,
                    "frac": go / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": bo}}


def run_logits(args, torch, gdn2, W, dev, out_dtype):
    """Gate activations inside the recurrence kernels, on the training shape: the forward from
    gate logits alone, and the layer's two passes both ways -- prep forming every input
    (q, k, v, b, w, log alpha) then the forward, against prep forming q, k, v only then the
    forward from logits.  Inputs are the mixer workload's projection outputs."""
    wl = W.TRAIN_4K
    x = {n: t.to(dev) for n, t in W.make_mixer_inputs(wl).items()}
    names = ("xq", "xk", "xv", "xb", "xw", "xa", "conv_q", "conv_k", "conv_v")
    full = gdn2.mixer_prep(*[x[n] for n in names])
    part = gdn2.mixer_prep(*[x[n] for n in names], gates=False)
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=out_dtype, device=dev)
    sT = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)

    def fwd_logits():
        gdn2.chunk_fwd_logits(part["q"], part["k"], part["v"], x["xa"], x["xb"], x["xw"], None, o=o,
                              final_state=sT, out_dtype=out_dtype)

    def layer_activated():
        gdn2.mixer_prep(*[x[n] for n in names], out=full)
        gdn2.chunk_fwd(full["q"], full["k"], full["v"], full["log_alpha"], full["b"], full["w"], None, o=o,
                       final_state=sT, out_dtype=out_dtype)

    def layer_logits():
        gdn2.mixer_prep(*[x[n] for n in names], out=part, gates=False)
        fwd_logits()

    ms = time_launches(fwd_logits, args.steps, args.warmup, torch)
    ms_la = time_launches(layer_activated, args.steps, args.warmup, torch)
    ms_ll = time_launches(layer_logits, args.steps, args.warmup, torch)
    nbytes = logits_chunk_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    gbps = nbytes / (ms * 1e-3) / 1e9
    del x, full, part, o, sT
    torch.cuda.empty_cache()
    return {"workload": wl.name + " (gate logits)", "us_per_launch": ms * 1e3,
            "tokens_per_s": wl.B * wl.T / (ms * 1e-3), "GBps": gbps, "peak": HBM_PEAK_GBPS,
            "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": nbytes,
            "bytes_per_head_token": 4 * wl.dk * 2 + 3 * wl.dv * 2,
            "prep_then_forward_us": {"activated_gates": ms_la * 1e3, "gates_in_kernel": ms_ll * 1e3},
            "activations_not_stored_bytes": wl.B * wl.T * wl.H * (wl.dk * 4 + wl.dk * 2 + wl.dv * 2),
            "note": "alpha, b, w = sigmoid of bf16 logits, formed on load; no activated copy is written"}


def run_decode(args, torch, gdn2, W, dev, out_dtype):
    """Decode workload: N=256 sequences x H=16, one token per step, state updated in place.  The
    whole loop of --decode-steps steps (1024, the workload's length) is timed as one event pair
    (per-step time includes the host launch gaps), then the same loop captured once in a HIP
    graph (kernel nodes only) and replayed, timed the same way."""
    dwl = W.DECODE
    pool = W.make_decode_pool(dwl)
    state = pool["state"].to(dev)
    dp = {n: pool[n].to(dev) for n in ("q", "k", "v", "log_alpha", "b", "w")}
    del pool
    o_dec = torch.empty((dwl.B, dwl.H, dwl.dv), dtype=out_dtype, device=dev)
    nsteps = args.decode_steps
    toks = [{n: dp[n][s % dwl.pool] for n in dp} for s in range(dwl.pool)]

    def loop():
        for s in range(nsteps):
            t = toks[s % dwl.pool]
            gdn2.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], state, o=o_dec,
                             out_dtype=out_dtype)

    loop()  # warm-up pass over the whole loop
    dms = time_launches(loop, 1, 0, torch, spin=False) / nsteps
    dbytes = decode_bytes(dwl.B, dwl.H, dwl.dk, dwl.dv, out_bytes=out_dtype.itemsize)
    dgbps = dbytes / (dms * 1e-3) / 1e9
    graph = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                loop()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()  # first replay uploads the graph
        gms = time_launches(g.replay, 1, 0, torch, spin=False) / nsteps
        ggbps = dbytes / (gms * 1e-3) / 1e9
        graph = {"us_per_step": gms * 1e3, "state_GBps": ggbps, "frac": ggbps / HBM_PEAK_GBPS,
                 "steps": nsteps}
        del g
    except RuntimeError as e:  # report, do not hide, a capture failure
        graph = {"error": str(e)[:200]}
    del state, dp, o_dec, toks
    torch.cuda.empty_cache()
    return {"workload": dwl.name, "us_per_step": dms * 1e3, "state_GBps": dgbps,
            "peak": HBM_PEAK_GBPS, "frac": dgbps / HBM_PEAK_GBPS,
            "traffic": recorded_traffic(*DECODE_PROFILE) if out_dtype == torch.float32 else None,
            "algorithmic_bytes_per_step": dbytes, "steps": nsteps,
            "timing": "the whole loop as one event pair, launch gaps included", "graph": graph}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-spin-up", action="store_true",
                    help="skip the untimed clock spin-up before each timing (counter runs: fewer dispatches)")
    ap.add_argument("--out-bf16", action="store_true", help="write o in bf16 instead of fp32")
    ap.add_argument("--only", choices=("chunk", "decode", "prefill", "bwd", "mixer", "long", "sweep", "logits"),
                    default=None, help="time one workload only (profiler runs); prints its figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain device-to-device copy of MIB MiB (--steps times): "
                         "the reference point that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    global SPIN_UP
    SPIN_UP = not args.no_spin_up
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the GDN-2 recurrence shards over independent "
              "(sequence, head) pairs with no exchange, so more GPUs only replicate this "
              "measurement; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_gdn2_amd as gdn2
    import workloads as W

    gdn2._load()
    dev = torch.device("cuda:0")
    out_dtype = torch.bfloat16 if args.out_bf16 else torch.float32

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = time_launches(lambda: dst.copy_(src), args.steps, args.warmup, torch)
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "avg_launch_us": ms * 1e3,
                          "GBps": 2 * n / (ms * 1e-3) / 1e9}))
        return
    only = {"decode": lambda: {"decode": run_decode(args, torch, gdn2, W, dev, out_dtype)},
            "prefill": lambda: {"prefill_varlen": run_prefill(args, torch, gdn2, W, dev, out_dtype)},
            "bwd": lambda: {"backward": run_bwd(args, torch, gdn2, W, dev)},
            "mixer": lambda: {"mixer": run_mixer(args, torch, gdn2, W, dev)},
            "long": lambda: {"long_context": run_long(args, torch, gdn2, W, dev, out_dtype)},
            "logits": lambda: {"gates_in_kernel": run_logits(args, torch, gdn2, W, dev, out_dtype)}}
    if args.only in only:
        print(json.dumps(only[args.only]()), flush=True)
        return
    ms, wl, nbytes, d, forms = run_chunk(args, torch, gdn2, W, dev, out_dtype, keep=True)
    tokens = wl.B * wl.T
    achieved = nbytes / (ms * 1e-3) / 1e9
    if args.only == "chunk":
        print(json.dumps({"workload": wl.name, "avg_launch_us": ms * 1e3,
                          "forms_us": {f: t * 1e3 for f, t in forms.items()},
                          "tokens_per_s": tokens / (ms * 1e-3), "achieved_GBps": achieved}), flush=True)
        return
    sweep = run_sweep(args, torch, gdn2, d, dev, out_dtype)
    del d
    torch.cuda.empty_cache()
    if args.only == "sweep":
        print(json.dumps({"t_sweep": sweep}), flush=True)
        return
    print("chunk forward %.1f us; sweep done" % (ms * 1e3), file=sys.stderr, flush=True)
    long_ctx = run_long(args, torch, gdn2, W, dev, out_dtype)
    dec = run_decode(args, torch, gdn2, W, dev, out_dtype)
    print("decode done", file=sys.stderr, flush=True)
    pre = run_prefill(args, torch, gdn2, W, dev, out_dtype)
    bwd = run_bwd(args, torch, gdn2, W, dev)
    mixer = run_mixer(args, torch, gdn2, W, dev)
    mixer["gates_in_kernel"] = run_logits(args, torch, gdn2, W, dev, out_dtype)
    print("prefill, backward, mixer done", file=sys.stderr, flush=True)
    flops = chunk_flops(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    extra = fp32_o_extra_bytes(wl.B, wl.T, wl.H, wl.dv) if out_dtype == torch.float32 else 0

    result = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, distributions of the training-shape workload)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "dk": wl.dk, "dv": wl.dv,
                   "chunk": 64, "inputs": "bf16 q,k,v,b,w; fp32 log_alpha",
                   "o_dtype": "bf16" if args.out_bf16 else "f32", "initial_state": "zeros"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(*CHUNK_PROFILE) if not args.out_bf16 else None,
                     "kernel": "chunk_bf16_kernel" if not gdn2.chunk_fwd_workspace_bytes(
                         wl.B, wl.T, wl.H, wl.dk, wl.dv) else "local_kernel + state_kernel",
                     "algorithmic_bytes_per_launch": nbytes,
                     "forms_us": {f: t * 1e3 for f, t in forms.items()},
                     "bytes_per_head_token": 3 * wl.dk * 2 + 2 * wl.dv * 2 + wl.dk * 4 + wl.dv * 2,
                     "fp32_o_extra_bytes_per_launch": extra,
                     "frac_with_fp32_o_bytes": (nbytes + extra) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "avg_launch_us": ms * 1e3,
                     "mfma_context": {"algorithmic_flops_per_launch": flops,
                                      "count": "causal (triangular) multiply-adds x 2",
                                      "TFLOPs": flops / (ms * 1e-3) / 1e12,
                                      "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}},
        "long_context": long_ctx,
        "t_sweep": sweep,
        "decode": dec,
        "prefill_varlen": pre,
        "backward": bwd,
        "mixer": mixer,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, torch)
        result["decode"]["cpu_baseline"] = cpu_baseline_decode()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
