"""Seeded synthetic workloads for the GDN-2 recurrence.

This module is shared by the oracle side and the HIP side and therefore holds
none of the recurrence's arithmetic: it only draws inputs.  All draws come from
``torch.Generator('cpu')`` so that a seed gives the same tensors on every host,
in a fixed order: q, k, v, log_alpha, b, w, initial state, then extras.

Distributions follow the workloads the pages describe (key/query paths end in an
L2 normalisation and the two gates are sigmoid projections: page "Why NVIDIA
Gated DeltaNet-2 separates erase and write gates", sections "Gated Delta Rule-2"
and "implications for practitioners"; training shape of sequence 4K and a 0.5M
token global batch with a 262,144-float recurrent state per layer: same page,
section "1.3B parameters and 100B-token training spec"):

* q, k ~ N(0,1), L2-normalised over the key dimension per (b, t, h)
* v ~ N(0,1)
* log_alpha ~ U[lo, hi] per key channel per token (fp32 always)
* b, w = sigmoid(2 * N(0,1)) per channel
* optional initial state ~ N(0, std^2) (fp32 always)

Values are drawn in fp32 and then cast to the workload's dtype; the oracle is
handed exactly the cast values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    seed: int
    g_lo: float = -0.2
    g_hi: float = -0.001
    # heads [0, strong_heads) take log_alpha ~ U[strong_lo, strong_hi]
    strong_heads: int = 0
    strong_lo: float = -5.0
    strong_hi: float = -1.0
    weak_lo: Optional[float] = None
    weak_hi: Optional[float] = None
    s0_std: Optional[float] = None  # None = zero initial state
    steps: int = 0  # decode workloads: number of steps
    pool: int = 0  # decode workloads: distinct token sets, used cyclically

    @property
    def dtype_name(self) -> str:
        return {torch.float32: "f32", torch.bfloat16: "bf16"}[self.dtype]


# The five workloads.  Index i uses seed i.
TINY_FP32 = Workload("tiny_fp32_B1_T256_H2_d64", B=1, T=256, H=2, dk=64, dv=64,
                     dtype=torch.float32, seed=0)
TRAIN_4K = Workload("train_bf16_B8_T4096_H16_d128", B=8, T=4096, H=16, dk=128, dv=128,
                    dtype=torch.bfloat16, seed=1)
DECODE = Workload("decode_bf16_N256_H16_d128_x1024", B=256, T=1, H=16, dk=128, dv=128,
                  dtype=torch.bfloat16, seed=2, s0_std=0.02, steps=1024, pool=16)
LONG_32K = Workload("long_bf16_B1_T32768_H16_d128", B=1, T=32768, H=16, dk=128, dv=128,
                    dtype=torch.bfloat16, seed=3, strong_heads=8, strong_lo=-5.0,
                    strong_hi=-1.0, weak_lo=-0.05, weak_hi=-0.0001)
FWD_BWD_4K = Workload("fwdbwd_bf16_B4_T4096_H16_d128", B=4, T=4096, H=16, dk=128, dv=128,
                      dtype=torch.bfloat16, seed=4, s0_std=0.02)

# Serving prefill: a batch of prompts of mixed lengths packed along one token axis, with
# per-sequence initial states (a continuation), followed by decode steps from the final states.
SERVE_PREFILL = Workload("serve_prefill_bf16_N64_H16_d128", B=64, T=0, H=16, dk=128, dv=128,
                         dtype=torch.bfloat16, seed=5, s0_std=0.02)

ALL = (TINY_FP32, TRAIN_4K, DECODE, LONG_32K, FWD_BWD_4K)


def _uniform(gen, shape, lo, hi):
    return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def _unit_normal_rows(gen, shape):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _gate(gen, shape):
    return torch.sigmoid(2.0 * torch.randn(shape, generator=gen, dtype=torch.float32))


def make_inputs(wl: Workload, seed: Optional[int] = None, B: Optional[int] = None,
                T: Optional[int] = None):
    """Draw (q, k, v, log_alpha, b, w, s0) for a forward workload on the CPU.

    ``B``/``T`` override the workload's sizes (same distributions), so that a
    smaller case of the same recipe can be drawn.  Returns a dict of CPU
    tensors; q,k,v,b,w in ``wl.dtype``, log_alpha and s0 in fp32 (s0 may be
    None)."""
    seed = wl.seed if seed is None else seed
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    H, dk, dv = wl.H, wl.dk, wl.dv
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _unit_normal_rows(gen, (B, T, H, dk))
    k = _unit_normal_rows(gen, (B, T, H, dk))
    v = torch.randn((B, T, H, dv), generator=gen, dtype=torch.float32)
    if wl.strong_heads:
        g = torch.empty((B, T, H, dk), dtype=torch.float32)
        hs = wl.strong_heads
        g[:, :, :hs] = _uniform(gen, (B, T, hs, dk), wl.strong_lo, wl.strong_hi)
        g[:, :, hs:] = _uniform(gen, (B, T, H - hs, dk), wl.weak_lo, wl.weak_hi)
    else:
        g = _uniform(gen, (B, T, H, dk), wl.g_lo, wl.g_hi)
    b = _gate(gen, (B, T, H, dk))
    w = _gate(gen, (B, T, H, dv))
    s0 = None
    if wl.s0_std is not None:
        s0 = torch.randn((B, H, dk, dv), generator=gen, dtype=torch.float32) * wl.s0_std
    dt = wl.dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=g, b=b.to(dt), w=w.to(dt), s0=s0)


def make_upstream_grad(wl: Workload, seed: Optional[int] = None, B=None, T=None):
    """do ~ N(0,1) of the output's shape, drawn after the forward inputs."""
    seed = (wl.seed if seed is None else seed) + 1_000_003
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    gen = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((B, T, wl.H, wl.dv), generator=gen, dtype=torch.float32)


def make_upstream_state_grad(wl: Workload, seed: Optional[int] = None, B=None):
    """dS_T ~ N(0,1) of the final state's shape [B,H,dk,dv], from its own stream."""
    seed = (wl.seed if seed is None else seed) + 2_000_029
    B = wl.B if B is None else B
    gen = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((B, wl.H, wl.dk, wl.dv), generator=gen, dtype=torch.float32)


def make_mixer_inputs(wl: Workload, seed: Optional[int] = None, B=None, T=None):
    """The mixer's inputs for a workload's shape, from their own stream: projection outputs
    xq, xk, xv ~ N(0,1); gate logits xb, xw ~ N(0, 2^2); decay logits xa ~ U[2, 7] (so that
    log sigmoid(xa) lies in [-0.13, -0.001], the range of the workloads' log alpha); causal
    taps ~ U[-0.5, 0.5] with the current-token tap U[0.5, 1.5]; output-gate logits
    z ~ N(0,1); norm weight gamma ~ U[0.5, 1.5].  Projection outputs, gate logits and z in
    the workload's dtype; taps and gamma fp32."""
    seed = (wl.seed if seed is None else seed) + 3_000_041
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    H, dk, dv, dt = wl.H, wl.dk, wl.dv, wl.dtype
    gen = torch.Generator("cpu").manual_seed(seed)
    out = {}
    for name, d in (("xq", dk), ("xk", dk), ("xv", dv)):
        out[name] = torch.randn((B, T, H, d), generator=gen, dtype=torch.float32).to(dt)
    for name, d in (("xb", dk), ("xw", dv)):
        out[name] = (2.0 * torch.randn((B, T, H, d), generator=gen, dtype=torch.float32)).to(dt)
    out["xa"] = _uniform(gen, (B, T, H, dk), 2.0, 7.0).to(dt)
    for name, d in (("conv_q", dk), ("conv_k", dk), ("conv_v", dv)):
        taps = _uniform(gen, (H * d, 4), -0.5, 0.5)
        taps[:, 3] = _uniform(gen, (H * d,), 0.5, 1.5)
        out[name] = taps.contiguous()
    out["z"] = torch.randn((B, T, H, dv), generator=gen, dtype=torch.float32).to(dt)
    out["gamma"] = _uniform(gen, (dv,), 0.5, 1.5)
    return out


def make_logit_inputs(wl: Workload, seed: Optional[int] = None, B: Optional[int] = None,
                      T: Optional[int] = None, a_lo: float = 2.0, a_hi: float = 7.0):
    """Inputs of the forward that activates its gates in the kernel: q, k, v and s0 as
    make_inputs draws them for the same seed, then from their own stream the decay logits
    xa ~ U[a_lo, a_hi] per key channel per token (the default puts log sigmoid(xa) in
    [-0.13, -0.001], the range of the workloads' log alpha; U[-6, -1] gives strong decay) and
    the gate logits xb [.., dk], xw [.., dv] ~ N(0, 2^2), all three in the workload's dtype."""
    base = make_inputs(wl, seed=seed, B=B, T=T)
    seed = (wl.seed if seed is None else seed) + 4_000_037
    B, T, H = base["q"].shape[0], base["q"].shape[1], wl.H
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = wl.dtype
    xa = _uniform(gen, (B, T, H, wl.dk), a_lo, a_hi).to(dt)
    xb = (2.0 * torch.randn((B, T, H, wl.dk), generator=gen, dtype=torch.float32)).to(dt)
    xw = (2.0 * torch.randn((B, T, H, wl.dv), generator=gen, dtype=torch.float32)).to(dt)
    return dict(q=base["q"], k=base["k"], v=base["v"], xa=xa, xb=xb, xw=xw, s0=base["s0"])


def make_decode_pool(wl: Workload, seed: Optional[int] = None, N: Optional[int] = None):
    """Decode workload: initial state [N,H,dk,dv] fp32 ~ N(0, s0_std^2) and a pool
    of ``wl.pool`` token sets (q,k,v,log_alpha,b,w each [P,N,H,d]); step s uses
    pool entry s mod P."""
    seed = wl.seed if seed is None else seed
    N = wl.B if N is None else N
    H, dk, dv, P = wl.H, wl.dk, wl.dv, wl.pool
    gen = torch.Generator("cpu").manual_seed(seed)
    state = torch.randn((N, H, dk, dv), generator=gen, dtype=torch.float32) * wl.s0_std
    q = _unit_normal_rows(gen, (P, N, H, dk))
    k = _unit_normal_rows(gen, (P, N, H, dk))
    v = torch.randn((P, N, H, dv), generator=gen, dtype=torch.float32)
    g = _uniform(gen, (P, N, H, dk), wl.g_lo, wl.g_hi)
    b = _gate(gen, (P, N, H, dk))
    w = _gate(gen, (P, N, H, dv))
    dt = wl.dtype
    return dict(state=state, q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=g, b=b.to(dt),
                w=w.to(dt))


def make_lengths(n: int, seed: int, median: int = 512, lo: int = 1, hi: int = 4096):
    """Seeded prompt lengths for a serving batch: log-normal around ``median``
    (sigma 1), clipped to [lo, hi].  Returns a list of ints."""
    gen = torch.Generator("cpu").manual_seed(seed + 7_000_001)
    z = torch.randn((n,), generator=gen, dtype=torch.float64)
    x = torch.exp(z + float(torch.log(torch.tensor(float(median)))))
    return [int(min(max(round(float(t)), lo), hi)) for t in x]


def make_packed_inputs(wl: Workload, lengths, seed: Optional[int] = None):
    """Packed sequences: q, k, v, log_alpha, b, w as [total_T, H, d] (the recipe of
    ``make_inputs`` over one axis of sum(lengths) tokens), cu_seqlens int64 [N+1], and
    initial states [N, H, dk, dv] (~ N(0, s0_std^2), or None)."""
    seed = wl.seed if seed is None else seed
    total = int(sum(lengths))
    d = make_inputs(wl, seed=seed, B=1, T=max(total, 1))
    out = {n: d[n][0, :total] for n in ("q", "k", "v", "log_alpha", "b", "w")}
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int64)
    s0 = None
    if wl.s0_std is not None:
        gen = torch.Generator("cpu").manual_seed(seed + 3_000_017)
        s0 = torch.randn((len(lengths), wl.H, wl.dk, wl.dv), generator=gen,
                         dtype=torch.float32) * wl.s0_std
    out["s0"] = s0
    return out
