"""Benchmark of the GDN-2 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunk-parallel forward (gdn2_chunk_fwd) over the training-shape
workload B=8, T=4096, H=16, dk=dv=128 (bf16 q,k,v,b,w, fp32 log alpha, zero
initial state, fp32 o and final state), inputs resident in HBM before timing.
The decode workload (N=256 sequences x H=16, 128x128 fp32 state, one token per
step) is timed in the same run and reported under "decode".

Prints one JSON line.  `value` is tokens/s (B*T tokens per step); `roofline`
gives the chunk kernel's algorithmic HBM bytes per launch over its average
launch time, measured with HIP events on the stream the kernel runs on;
`cpu_baseline` is the fp64 oracle timed on a bounded sample of the same
workload on this host's cores.
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


def chunk_bytes(B, T, H, dk, dv, in_bytes=2, out_bytes=4, with_s0=False):
    """Algorithmic HBM bytes of one forward: every input read once, o and S_T written once."""
    per_head_token = 3 * dk * in_bytes + 2 * dv * in_bytes + dk * 4 + dv * out_bytes
    state = B * H * dk * dv * 4 * (2 if with_s0 else 1)
    return B * T * H * per_head_token + state


def chunk_flops(B, T, H, dk, dv, C=64):
    """Algorithmic matrix flops of the chunk form per launch (2 per multiply-add): per chunk the
    C x C products A and P (2 x C*C*dk), W = T(b.k.Gamma) and U = T(w.v) (C*C*(dk+dv)), the
    triangular inverse (C^3/3), and the state products W S, (q.Gamma) S, k'^T U (3 x C*dk*dv) and
    P U (C*C*dv)."""
    nchunks = B * H * ((T + C - 1) // C)
    per_chunk = 2 * (2 * C * C * dk + C * C * (dk + dv) + C ** 3 // 3 + 3 * C * dk * dv + C * C * dv)
    return nchunks * per_chunk


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


CHUNK_PROFILE = ("chunk_fwd_train_B8_T4096_H16_d128.md", ("gdn2_chunk_bf16.hip", "gdn2_device.h"))
DECODE_PROFILE = ("decode_step_N256_H16_d128.md", ("gdn2_decode.hip", "gdn2_device.h"))
PREFILL_PROFILE = ("prefill_varlen_N64_H16_d128.md", ("gdn2_chunk_bf16.hip", "gdn2_device.h"))


def time_launches(fn, steps, warmup, torch):
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
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["s0"],
               nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": Bs * Ts / dt, "unit": "tokens/s", "cores": min(threads, Bs * wl.H),
            "kind": "oracle",
            "sample": "fp64 oracle on the whole workload: B=%d T=%d H=%d d=%d (%d of %d sequences, "
                      "%d tokens each), %.2f s wall" % (Bs, Ts, wl.H, wl.dk, Bs * wl.H, wl.B * wl.H,
                                                        Ts, dt)}


def run_chunk(args, torch, gdn2, W, dev, out_dtype):
    """Chunk forward on the training-shape workload; returns (ms per launch, workload, bytes)."""
    wl = W.TRAIN_4K
    inp = W.make_inputs(wl)
    d = {n: (None if x is None else x.to(dev)) for n, x in inp.items()}
    del inp
    o = torch.empty((wl.B, wl.T, wl.H, wl.dv), dtype=out_dtype, device=dev)
    sT = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)

    def step():
        gdn2.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["s0"], o=o,
                       final_state=sT, out_dtype=out_dtype)

    ms = time_launches(step, args.steps, args.warmup, torch)
    nbytes = chunk_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, out_bytes=out_dtype.itemsize)
    del d, o, sT
    torch.cuda.empty_cache()
    return ms, wl, nbytes


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
    per_tok = 3 * wl.dk * 2 + 2 * wl.dv * 2 + wl.dk * 4 + wl.dv * out_dtype.itemsize
    nbytes = total * wl.H * per_tok + 2 * wl.B * wl.H * wl.dk * wl.dv * 4 + (wl.B + 1) * 8
    gbps = nbytes / (ms * 1e-3) / 1e9
    del d, o, sT
    torch.cuda.empty_cache()
    return {"workload": wl.name, "sequences": wl.B, "tokens": total,
            "lengths": "log-normal around 512 (sigma 1), clipped to [1, 4096], seed %d" % wl.seed,
            "us_per_launch": ms * 1e3, "tokens_per_s": total / (ms * 1e-3), "GBps": gbps,
            "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS,
            "traffic": recorded_traffic(*PREFILL_PROFILE) if out_dtype == torch.float32 else None,
            "algorithmic_bytes_per_launch": nbytes}


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


def run_decode(args, torch, gdn2, W, dev, out_dtype):
    """Decode workload: N=256 sequences x H=16, one token per step, state updated in place."""
    dwl = W.DECODE
    pool = W.make_decode_pool(dwl)
    state = pool["state"].to(dev)
    dp = {n: pool[n].to(dev) for n in ("q", "k", "v", "log_alpha", "b", "w")}
    del pool
    o_dec = torch.empty((dwl.B, dwl.H, dwl.dv), dtype=out_dtype, device=dev)
    it = [0]

    def dstep():
        p = it[0] % dwl.pool
        it[0] += 1
        gdn2.decode_step(dp["q"][p], dp["k"][p], dp["v"][p], dp["log_alpha"][p], dp["b"][p],
                         dp["w"][p], state, o=o_dec, out_dtype=out_dtype)

    dms = time_launches(dstep, args.decode_steps, 5, torch)
    dbytes = decode_bytes(dwl.B, dwl.H, dwl.dk, dwl.dv, out_bytes=out_dtype.itemsize)
    dgbps = dbytes / (dms * 1e-3) / 1e9
    del state, dp, o_dec
    torch.cuda.empty_cache()
    return {"workload": dwl.name, "us_per_step": dms * 1e3, "state_GBps": dgbps,
            "peak": HBM_PEAK_GBPS, "frac": dgbps / HBM_PEAK_GBPS,
            "traffic": recorded_traffic(*DECODE_PROFILE) if out_dtype == torch.float32 else None,
            "algorithmic_bytes_per_step": dbytes, "steps": args.decode_steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out-bf16", action="store_true", help="write o in bf16 instead of fp32")
    ap.add_argument("--only", choices=("chunk", "decode", "prefill", "bwd", "mixer"), default=None,
                    help="time one workload only (profiler runs); prints its figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain device-to-device copy of MIB MiB (--steps times): "
                         "the reference point that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
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
    if args.only == "decode":
        print(json.dumps({"decode": run_decode(args, torch, gdn2, W, dev, out_dtype)}))
        return
    if args.only == "prefill":
        print(json.dumps({"prefill_varlen": run_prefill(args, torch, gdn2, W, dev, out_dtype)}))
        return
    if args.only == "bwd":
        print(json.dumps({"backward": run_bwd(args, torch, gdn2, W, dev)}))
        return
    if args.only == "mixer":
        print(json.dumps({"mixer": run_mixer(args, torch, gdn2, W, dev)}))
        return
    ms, wl, nbytes = run_chunk(args, torch, gdn2, W, dev, out_dtype)
    tokens = wl.B * wl.T
    achieved = nbytes / (ms * 1e-3) / 1e9
    if args.only == "chunk":
        print(json.dumps({"workload": wl.name, "avg_launch_us": ms * 1e3,
                          "tokens_per_s": tokens / (ms * 1e-3), "achieved_GBps": achieved}))
        return
    dec = run_decode(args, torch, gdn2, W, dev, out_dtype)
    pre = run_prefill(args, torch, gdn2, W, dev, out_dtype)
    bwd = run_bwd(args, torch, gdn2, W, dev)
    mixer = run_mixer(args, torch, gdn2, W, dev)
    flops = chunk_flops(wl.B, wl.T, wl.H, wl.dk, wl.dv)

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
                     "kernel": "chunk_bf16_kernel", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": ms * 1e3,
                     "mfma_context": {"algorithmic_flops_per_launch": flops,
                                      "TFLOPs": flops / (ms * 1e-3) / 1e12,
                                      "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}},
        "decode": dec,
        "prefill_varlen": pre,
        "backward": bwd,
        "mixer": mixer,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, torch)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
