"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars (max |x - x_ref| / RMS(x_ref) per output tensor, no non-finite value):
1e-4 for fp32 inputs, 3e-2 for bf16 inputs with fp32 accumulation.  The oracle
sees exactly the values the GPU sees (bf16 inputs upcast exactly).

Small cases span several chunks and a ragged last chunk and run the oracle on
everything; the full-size workloads run exactly the launch the benchmark times
and check sampled (sequence, head) pairs one by one, plus properties on all
outputs (finiteness)."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import oracle
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, rel_max_err, say, take_sequences, to_dev, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn2._load()  # fail loudly if the library is missing


def run_gpu(inp, **kw):
    d = to_dev(inp)
    o, s = gdn2.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["s0"], **kw)
    torch.cuda.synchronize()
    return o, s


def run_oracle(inp):
    return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["s0"])


def check(o, s, o_ref, s_ref, tol, label):
    eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
    say("  %-40s o err %.3e   S_T err %.3e   (bar %.0e)" % (label, eo, es, tol))
    assert eo <= tol and es <= tol, (label, eo, es)
    return eo, es


# ----------------------------------------------------------------- small ----

def test_tiny_fp32_workload():
    wl = W.TINY_FP32
    say("case: %s seed %d" % (wl.name, wl.seed))
    inp = W.make_inputs(wl)
    o, s = run_gpu(inp)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, TOL_F32, wl.name)


SMALL = [
    # dtype, dk, B, T, H, initial state, seed
    (torch.float32, 64, 2, 200, 3, True, 101),
    (torch.float32, 64, 1, 1, 2, True, 102),
    (torch.float32, 64, 1, 64, 1, False, 103),
    (torch.float32, 64, 3, 129, 5, False, 104),
    (torch.bfloat16, 128, 2, 200, 3, True, 105),
    (torch.bfloat16, 128, 1, 333, 4, False, 106),
    (torch.bfloat16, 128, 1, 1, 2, True, 107),
    (torch.bfloat16, 128, 1, 64, 1, True, 108),
    (torch.bfloat16, 64, 2, 257, 3, True, 109),
    (torch.bfloat16, 64, 5, 31, 7, False, 110),
    (torch.bfloat16, 128, 9, 130, 19, True, 111),  # B*H not a multiple of 8
]


@pytest.mark.parametrize("dtype,dk,B,T,H,with_s0,seed", SMALL)
def test_small_cases(dtype, dk, B, T, H, with_s0, seed):
    wl = dataclasses.replace(W.TRAIN_4K, name="small", dtype=dtype, dk=dk, dv=dk, H=H,
                             s0_std=0.05 if with_s0 else None)
    say("case: %s dk=%d B=%d T=%d H=%d s0=%s seed=%d" % (dtype, dk, B, T, H, with_s0, seed))
    inp = W.make_inputs(wl, seed=seed, B=B, T=T)
    o, s = run_gpu(inp)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, tol_for(dtype), "small")


@pytest.mark.parametrize("dtype,dk", [(torch.float32, 64), (torch.bfloat16, 128), (torch.bfloat16, 64)])
@pytest.mark.parametrize("g_lo,g_hi", [(-5.0, -1.0), (-60.0, -20.0), (-3.0, 0.0)])
def test_strong_and_extreme_decay(dtype, dk, g_lo, g_hi):
    """Chunk decays far below fp32 range take the boundary-pivoted path; must stay exact."""
    wl = dataclasses.replace(W.TRAIN_4K, name="decay", dtype=dtype, dk=dk, dv=dk, H=4,
                             g_lo=g_lo, g_hi=g_hi, s0_std=0.05)
    say("case: decay U[%g,%g] %s dk=%d" % (g_lo, g_hi, dtype, dk))
    inp = W.make_inputs(wl, seed=7, B=2, T=300)
    o, s = run_gpu(inp)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, tol_for(dtype), "decay U[%g,%g]" % (g_lo, g_hi))


def test_mixed_decay_heads_small():
    """The long-context recipe (strong heads 0-7, weak 8-15) at T = 1024: per-head bar."""
    wl = W.LONG_32K
    say("case: %s at T=1024" % wl.name)
    inp = W.make_inputs(wl, T=1024)
    o, s = run_gpu(inp)
    o_ref, s_ref = run_oracle(inp)
    for h in range(wl.H):
        eo = rel_max_err(o[:, :, h], o_ref[:, :, h])
        es = rel_max_err(s[:, h], s_ref[:, h])
        say("  head %2d  o %.3e  S %.3e" % (h, eo, es))
        assert eo <= TOL_BF16 and es <= TOL_BF16, (h, eo, es)


# ----------------------------------------------------------- full sizes ----

def _sampled(wl, pairs):
    say("case: %s (full size), sampled (b,h) = %s" % (wl.name, pairs))
    inp = W.make_inputs(wl)
    o, s = run_gpu(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    sub = take_sequences(inp, pairs)
    o_ref, s_ref = run_oracle(sub)
    tol = tol_for(wl.dtype)
    for n, (b, h) in enumerate(pairs):
        eo = rel_max_err(o[b, :, h], o_ref[n, :, 0])
        es = rel_max_err(s[b, h], s_ref[n, 0])
        say("  (b=%d,h=%2d)  o %.3e  S %.3e" % (b, h, eo, es))
        assert eo <= tol and es <= tol, (b, h, eo, es)


def test_train_4k_full_size_sampled():
    _sampled(W.TRAIN_4K, [(0, 0), (3, 7), (5, 12), (7, 15)])


def test_long_32k_full_size_sampled():
    _sampled(W.LONG_32K, [(0, 0), (0, 7), (0, 8), (0, 15)])


def test_fwdbwd_4k_forward_full_size_sampled():
    _sampled(W.FWD_BWD_4K, [(0, 0), (1, 5), (3, 15)])


# --------------------------------------------------------------- decode ----

def test_decode_workload_sampled():
    """1024 steps over N=256 sequences; every step's o and the final state of
    two sequences (all heads) are checked against the oracle's replay."""
    wl = W.DECODE
    say("case: %s" % wl.name)
    pool = W.make_decode_pool(wl)
    dpool = to_dev({k: v for k, v in pool.items() if k != "state"})
    state = pool["state"].cuda().contiguous()
    seqs = [0, 201]
    o_hist = []
    for s in range(wl.steps):
        p = s % wl.pool
        o = gdn2.decode_step(dpool["q"][p], dpool["k"][p], dpool["v"][p], dpool["log_alpha"][p],
                             dpool["b"][p], dpool["w"][p], state)
        o_hist.append(o[seqs].float().cpu())
    torch.cuda.synchronize()
    ref_state = pool["state"][seqs].double().numpy()
    worst_o = 0.0
    for s in range(wl.steps):
        p = s % wl.pool
        tok = {n: pool[n][p][seqs] for n in ("q", "k", "v", "log_alpha", "b", "w")}
        o_ref, ref_state = oracle.decode(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["b"],
                                         tok["w"], ref_state)
        e = rel_max_err(o_hist[s], o_ref)
        worst_o = max(worst_o, e)
        assert e <= TOL_BF16, (s, e)
    es = rel_max_err(state[seqs], ref_state)
    say("  worst o err over %d steps %.3e   final state err %.3e" % (wl.steps, worst_o, es))
    assert es <= TOL_BF16
    assert torch.isfinite(state).all()


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.float32, 128), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128)])
def test_decode_steps_match_oracle_and_chunk(dtype, d):
    wl = dataclasses.replace(W.TRAIN_4K, name="dec", dtype=dtype, dk=d, dv=d, H=3, s0_std=0.05)
    say("case: decode vs chunk %s d=%d" % (dtype, d))
    inp = W.make_inputs(wl, seed=31, B=3, T=70)
    dd = to_dev(inp)
    state = dd["s0"].clone()
    outs = []
    for t in range(70):
        outs.append(gdn2.decode_step(dd["q"][:, t].contiguous(), dd["k"][:, t].contiguous(),
                                     dd["v"][:, t].contiguous(), dd["log_alpha"][:, t].contiguous(),
                                     dd["b"][:, t].contiguous(), dd["w"][:, t].contiguous(), state))
    o_dec = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(inp)
    check(o_dec, state, o_ref, s_ref, tol_for(dtype), "decode steps")
    if gdn2.supported("chunk_fwd", d, d, dtype):
        o_c, s_c = run_gpu(inp)
        check(o_c, s_c, o_ref, s_ref, tol_for(dtype), "chunk")


# ------------------------------------------------------ semantics checks ----

@pytest.mark.parametrize("split", [64, 100, 1])
def test_resume_equals_one_call(split):
    wl = dataclasses.replace(W.TRAIN_4K, name="resume", H=2, s0_std=0.05)
    say("case: resume split %d" % split)
    inp = W.make_inputs(wl, seed=41, B=2, T=257)
    d = to_dev(inp)
    a = {n: x[:, :split].contiguous() for n, x in d.items() if n != "s0"}
    o1, s1 = gdn2.chunk_fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["b"], a["w"], d["s0"])
    b2 = {n: x[:, split:].contiguous() for n, x in d.items() if n != "s0"}
    o2, s2 = gdn2.chunk_fwd(b2["q"], b2["k"], b2["v"], b2["log_alpha"], b2["b"], b2["w"], s1)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(inp)
    check(torch.cat([o1, o2], dim=1), s2, o_ref, s_ref, TOL_BF16, "resume")


def test_in_place_state_update():
    wl = dataclasses.replace(W.TRAIN_4K, name="inplace", H=2, s0_std=0.05)
    inp = W.make_inputs(wl, seed=42, B=1, T=150)
    say("case: in-place final state")
    d = to_dev(inp)
    st = d["s0"].clone()
    o, s = gdn2.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], st, final_state=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    o_ref, s_ref = run_oracle(inp)
    check(o, st, o_ref, s_ref, TOL_BF16, "in place")


def test_no_final_state_requested():
    inp = W.make_inputs(W.TRAIN_4K, seed=43, B=1, T=70)
    say("case: no final state")
    o, s = run_gpu(inp, output_final_state=False)
    assert s is None
    o_ref, _ = run_oracle(inp)
    assert rel_max_err(o, o_ref) <= TOL_BF16


def test_run_twice_bitwise_identical():
    inp = W.make_inputs(W.TRAIN_4K, seed=44, B=4, T=512)
    say("case: determinism")
    o1, s1 = run_gpu(inp)
    o2, s2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_nan_in_one_head_stays_isolated():
    inp = W.make_inputs(W.TRAIN_4K, seed=45, B=2, T=200)
    say("case: NaN isolation")
    o_clean, s_clean = run_gpu(inp)
    bad = {n: (x.clone() if x is not None else None) for n, x in inp.items()}
    bad["v"][1, 150, 5, 3] = float("nan")
    o_bad, s_bad = run_gpu(bad)
    mask = torch.ones(2, 16, dtype=torch.bool)
    mask[1, 5] = False
    for b in range(2):
        for h in range(16):
            if mask[b, h]:
                assert torch.equal(o_bad[b, :, h], o_clean[b, :, h]), (b, h)
                assert torch.equal(s_bad[b, h], s_clean[b, h]), (b, h)
    # the poisoned head is untouched before the NaN's chunk
    assert torch.equal(o_bad[1, :128, 5], o_clean[1, :128, 5])


def test_exact_retrieval_property_full_shape():
    """q = k (unit up to bf16 rounding), b = 1  =>  o_t = w_t . v_t at every token."""
    inp = W.make_inputs(W.TRAIN_4K, seed=46)
    say("case: retrieval property at B=8 T=4096 H=16 d=128")
    inp["q"] = inp["k"].clone()
    inp["b"] = torch.ones_like(inp["b"])
    o, _ = run_gpu(inp)
    target = (inp["w"].double() * inp["v"].double()).numpy()
    e = rel_max_err(o, target)
    say("  o vs w.v: %.3e" % e)
    assert e <= TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_output_is_fp32_output_rounded_once(d):
    """The bf16-output build differs from the fp32-output one only in the store."""
    wl = dataclasses.replace(W.TRAIN_4K, name="outdt", dk=d, dv=d, H=3, s0_std=0.05)
    inp = W.make_inputs(wl, seed=47, B=2, T=190)
    say("case: bf16 output vs fp32 output, d=%d" % d)
    o32, s32 = run_gpu(inp)
    o16, s16 = run_gpu(inp, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(s16, s32)


def test_decode_bf16_output_is_fp32_output_rounded_once():
    wl = dataclasses.replace(W.DECODE, B=8)
    pool = W.make_decode_pool(wl, N=8)
    say("case: decode bf16 output vs fp32 output")
    d = to_dev({k: v[0] for k, v in pool.items() if k != "state"})
    st1 = pool["state"].cuda()
    st2 = st1.clone()
    o32 = gdn2.decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], st1)
    o16 = gdn2.decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], st2,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(st1, st2)


@pytest.mark.parametrize("dtype,dk", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_caller_outputs_are_fully_written(dtype, dk):
    """Output buffers passed in, filled with NaN first, come back bit for bit equal to the
    outputs of a call that allocates its own: every element of o and S_T is written, with a
    ragged last chunk."""
    wl = dataclasses.replace(W.TRAIN_4K, name="outs", dtype=dtype, dk=dk, dv=dk, H=3, s0_std=0.05)
    say("case: caller outputs %s dk=%d B=2 T=300 H=3" % (dtype, dk))
    inp = W.make_inputs(wl, seed=17, B=2, T=300)
    o_ref, s_ref = run_gpu(inp)
    o_buf, s_buf = torch.full_like(o_ref, float("nan")), torch.full_like(s_ref, float("nan"))
    o, s = run_gpu(inp, o=o_buf, final_state=s_buf)
    assert o is o_buf and s is s_buf
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
