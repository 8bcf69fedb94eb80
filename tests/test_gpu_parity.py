"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars (max |x - x_ref| / RMS(x_ref) per output tensor, no non-finite value):
1e-4 for fp32 inputs, 3e-2 for bf16 inputs with fp32 accumulation.  The oracle
sees exactly the values the GPU sees (bf16 inputs upcast exactly).

Small cases span several chunks and a ragged last chunk; the full-size workloads
run exactly the launch the benchmark times.  Every case runs the oracle on every
(sequence, head) and takes the metric over the whole output tensors."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import oracle
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, ErrAccum, rel_max_err, say, to_dev, tol_for

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


# fused: the single-kernel forward (no workspace); otherwise bf16 runs the two-kernel form
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,dk,B,T,H,with_s0,seed", SMALL)
def test_small_cases(dtype, dk, B, T, H, with_s0, seed, fused):
    if fused and dtype == torch.float32:
        pytest.skip("fp32 inputs always run the fused kernel")
    wl = dataclasses.replace(W.TRAIN_4K, name="small", dtype=dtype, dk=dk, dv=dk, H=H,
                             s0_std=0.05 if with_s0 else None)
    say("case: %s dk=%d B=%d T=%d H=%d s0=%s seed=%d fused=%s" % (dtype, dk, B, T, H, with_s0, seed, fused))
    inp = W.make_inputs(wl, seed=seed, B=B, T=T)
    o, s = run_gpu(inp, fused=fused)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, tol_for(dtype), "small")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,dk", [(torch.float32, 64), (torch.bfloat16, 128), (torch.bfloat16, 64)])
@pytest.mark.parametrize("g_lo,g_hi", [(-5.0, -1.0), (-60.0, -20.0), (-3.0, 0.0)])
def test_strong_and_extreme_decay(dtype, dk, g_lo, g_hi, fused):
    """Chunk decays far below fp32 range take the boundary-pivoted path; must stay exact."""
    if fused and dtype == torch.float32:
        pytest.skip("fp32 inputs always run the fused kernel")
    wl = dataclasses.replace(W.TRAIN_4K, name="decay", dtype=dtype, dk=dk, dv=dk, H=4,
                             g_lo=g_lo, g_hi=g_hi, s0_std=0.05)
    say("case: decay U[%g,%g] %s dk=%d fused=%s" % (g_lo, g_hi, dtype, dk, fused))
    inp = W.make_inputs(wl, seed=7, B=2, T=300)
    o, s = run_gpu(inp, fused=fused)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, tol_for(dtype), "decay U[%g,%g]" % (g_lo, g_hi))


def _split_final_state_case(B, T, H, d, with_s0, final, label, g_lo=None, g_hi=None):
    wl = dataclasses.replace(W.TRAIN_4K, name=label, dk=d, dv=d, H=H, s0_std=0.05 if with_s0 else None)
    if g_lo is not None:
        wl = dataclasses.replace(wl, g_lo=g_lo, g_hi=g_hi)
    say("case: %s B=%d T=%d H=%d d=%d s0=%s final=%s decay=%s (workspace %d bytes)"
        % (label, B, T, H, d, with_s0, final, (g_lo, g_hi), gdn2.chunk_fwd_workspace_bytes(B, T, H, d, d, split=True)))
    inp = W.make_inputs(wl, seed=61, B=B, T=T)
    x = to_dev(inp)
    if final == "inplace":
        st = x["s0"].clone()
        o, s = gdn2.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], st, final_state=st,
                              fused=False)
        assert s.data_ptr() == st.data_ptr()
    else:
        o, s = gdn2.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["s0"],
                              output_final_state=final == "new", fused=False)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(inp)
    if final == "none":
        assert s is None
        eo = rel_max_err(o, o_ref)
        say("  o err %.3e" % eo)
        assert eo <= TOL_BF16
    else:
        check(o, s, o_ref, s_ref, TOL_BF16, label)


# Sizes whose chunk-heads exceed one batch of the two-kernel form (about 1024), with chains
# enough (more than half the compute units) or too few chunks to cut, so that it runs in batches,
# ragged tails: the state is carried between batches, through final_state or the workspace.
@pytest.mark.parametrize("B,T,H,d,with_s0,final", [
    (3, 2100, 48, 128, True, "new"),      # 33 chunks x 144 heads: batches of 7 chunks
    (9, 1500, 16, 128, False, "none"),    # no final state: carried in the workspace
    (3, 1500, 16, 128, True, "inplace"),  # final state written over the initial state
])
def test_split_across_batches(B, T, H, d, with_s0, final):
    _split_final_state_case(B, T, H, d, with_s0, final, "across batches")


# Few chains: each sequence is cut into segments walked in parallel, joined by their transitions
# (3 or 4 segments here, ragged or whole last chunks, strong decay in one case).
@pytest.mark.parametrize("B,T,H,d,with_s0,final,g_lo,g_hi", [
    (1, 5000, 3, 64, True, "new", None, None),        # 4 segments of 20 chunks, the last partial
    (2, 3200, 16, 128, True, "inplace", None, None),  # 3 segments of 17, 17 and 16 chunks
    (1, 4196, 4, 128, False, "none", None, None),     # 4 segments, no final state
    (1, 3840, 2, 128, True, "new", None, None),       # 3 segments of 20 whole chunks
    (1, 3100, 2, 128, True, "new", -60.0, -20.0),     # strong decay: every chunk pivots
    (1, 3072, 2, 128, True, "new", None, None),       # the fewest chunks cut: 3 segments of 16
    (1, 3073, 2, 128, True, "new", None, None),       # 49 chunks, the last of one token
])
def test_split_segments(B, T, H, d, with_s0, final, g_lo, g_hi):
    _split_final_state_case(B, T, H, d, with_s0, final, "segments", g_lo, g_hi)


# The fused kernel's value-column slice follows B * H (16, 32 or 64 columns, so that the
# workgroups fill the compute units), and with it the number of waves that hold state columns
# (one per 16 columns).  One case per width and head size, ragged last chunk, initial state.
@pytest.mark.parametrize("d,B,H,dvs", [
    (128, 4, 16, 32),   # B H = 64: two state waves of four
    (128, 1, 5, 16),    # B H = 5: one state wave
    (64, 8, 16, 32),    # B H = 128 at d = 64
    (64, 16, 16, 64),   # B H = 256 at d = 64: every state wave
])
def test_fused_slice_widths(d, B, H, dvs):
    wl = dataclasses.replace(W.TRAIN_4K, name="slices", dk=d, dv=d, H=H, s0_std=0.05)
    say("case: fused d=%d B=%d H=%d (slices of %d columns)" % (d, B, H, dvs))
    inp = W.make_inputs(wl, seed=71, B=B, T=200)
    o, s = run_gpu(inp, fused=True, output_final_state=True)
    o_ref, s_ref = run_oracle(inp)
    check(o, s, o_ref, s_ref, TOL_BF16, "fused, %d-column slices" % dvs)


def test_split_and_fused_agree():
    """The two forms compute the same function: on the same inputs their outputs differ by no
    more than the bar allows each of them against the oracle."""
    inp = W.make_inputs(W.TRAIN_4K, seed=62, B=2, T=700)
    o1, s1 = run_gpu(inp, fused=False)
    o2, s2 = run_gpu(inp, fused=True)
    o_ref, s_ref = run_oracle(inp)
    say("  split vs fused: o %.3e  S %.3e" % (rel_max_err(o1, o2.double().cpu().numpy()),
                                             rel_max_err(s1, s2.double().cpu().numpy())))
    check(o1, s1, o_ref, s_ref, TOL_BF16, "split")
    check(o2, s2, o_ref, s_ref, TOL_BF16, "fused")


@pytest.mark.parametrize("fused", [False, True])
def test_mixed_decay_heads_small(fused):
    """The long-context recipe (strong heads 0-7, weak 8-15) at T = 1024: per-head bar."""
    wl = W.LONG_32K
    say("case: %s at T=1024 fused=%s" % (wl.name, fused))
    inp = W.make_inputs(wl, T=1024)
    o, s = run_gpu(inp, fused=fused)
    o_ref, s_ref = run_oracle(inp)
    for h in range(wl.H):
        eo = rel_max_err(o[:, :, h], o_ref[:, :, h])
        es = rel_max_err(s[:, h], s_ref[:, h])
        say("  head %2d  o %.3e  S %.3e" % (h, eo, es))
        assert eo <= TOL_BF16 and es <= TOL_BF16, (h, eo, es)


# ----------------------------------------------------------- full sizes ----
# Every (sequence, head) of each full-size workload, in the launch the benchmark times, against
# the oracle run on the whole workload: the metric is taken over the whole o and S_T tensors,
# and per head so that the weak heads' RMS cannot hide a strong head's error.

def _whole(wl, report_bf16_o=False, fused=False):
    say("case: %s (full size, whole tensors) fused=%s" % (wl.name, fused))
    inp = W.make_inputs(wl)
    o, s = run_gpu(inp, fused=fused)
    o_ref, s_ref = run_oracle(inp)
    tol = tol_for(wl.dtype)
    eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
    say("  whole tensors: o err %.3e   S_T err %.3e   (bar %.0e)" % (eo, es, tol))
    worst = (0.0, 0.0)
    for h in range(wl.H):
        eoh, esh = rel_max_err(o[:, :, h], o_ref[:, :, h]), rel_max_err(s[:, h], s_ref[:, h])
        worst = (max(worst[0], eoh), max(worst[1], esh))
        if wl.H <= 16:
            say("  head %2d  o %.3e  S %.3e" % (h, eoh, esh))
    say("  worst head: o %.3e  S %.3e" % worst)
    if report_bf16_o:
        o16, _ = run_gpu(inp, out_dtype=torch.bfloat16, output_final_state=False, fused=fused)
        say("  bf16 o (rounded once on the store): o err %.3e (informational)" % rel_max_err(o16, o_ref))
        del o16
    assert eo <= tol and es <= tol, (wl.name, eo, es)
    assert worst[0] <= tol and worst[1] <= tol, (wl.name, worst)


@pytest.mark.parametrize("fused", [False, True])
def test_train_4k_full_size_whole_tensor(fused):
    _whole(W.TRAIN_4K, report_bf16_o=True, fused=fused)


@pytest.mark.parametrize("fused", [False, True])
def test_long_32k_full_size_whole_tensor(fused):
    _whole(W.LONG_32K, report_bf16_o=True, fused=fused)


def test_fwdbwd_4k_forward_full_size_whole_tensor():
    _whole(W.FWD_BWD_4K)


# --------------------------------------------------------------- decode ----

def test_decode_workload_whole():
    """All 1024 steps over all N=256 sequences: o of every step and the final state against
    the oracle.  The oracle runs the 1024 tokens of each (sequence, head) as one sequence
    (decode steps equal the forward over the same tokens: a pinned property of the oracle),
    in batches of sequences."""
    wl = W.DECODE
    say("case: %s (all sequences, all steps)" % wl.name)
    pool = W.make_decode_pool(wl)
    dpool = to_dev({k: v for k, v in pool.items() if k != "state"})
    state = pool["state"].cuda().contiguous()
    o_all = torch.empty((wl.steps, wl.B, wl.H, wl.dv), dtype=torch.float32)
    for s in range(wl.steps):
        p = s % wl.pool
        o = gdn2.decode_step(dpool["q"][p], dpool["k"][p], dpool["v"][p], dpool["log_alpha"][p],
                             dpool["b"][p], dpool["w"][p], state)
        o_all[s].copy_(o, non_blocking=False)
    torch.cuda.synchronize()
    state_gpu = state.cpu()
    del dpool, state
    idx = torch.arange(wl.steps) % wl.pool
    acc_o, acc_s = ErrAccum(), ErrAccum()
    nb = 32
    for n0 in range(0, wl.B, nb):
        seq = {n: pool[n][idx, n0:n0 + nb].transpose(0, 1).contiguous()
               for n in ("q", "k", "v", "log_alpha", "b", "w")}
        o_ref, s_ref = oracle.fwd(seq["q"], seq["k"], seq["v"], seq["log_alpha"], seq["b"], seq["w"],
                                  pool["state"][n0:n0 + nb])
        acc_o.add(o_all[:, n0:n0 + nb].transpose(0, 1), o_ref)
        acc_s.add(state_gpu[n0:n0 + nb], s_ref)
        say("  sequences %3d-%3d checked" % (n0, n0 + nb - 1))
    eo, es = acc_o.value(), acc_s.value()
    say("  o over all %d steps and %d sequences: err %.3e   final state err %.3e   (bar %.0e)"
        % (wl.steps, wl.B, eo, es, TOL_BF16))
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


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


@pytest.mark.parametrize("fused", [False, True])
def test_run_twice_bitwise_identical(fused):
    inp = W.make_inputs(W.TRAIN_4K, seed=44, B=4, T=512)
    say("case: determinism fused=%s" % fused)
    o1, s1 = run_gpu(inp, fused=fused)
    o2, s2 = run_gpu(inp, fused=fused)
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


@pytest.mark.parametrize("d,T,fused", [(64, 190, True), (128, 190, True), (128, 190, False),
                                        (128, 2100, False)])  # the last in 2 segments
def test_bf16_output_is_fp32_output_rounded_once(d, T, fused):
    """The bf16-output build differs from the fp32-output one only in the store."""
    wl = dataclasses.replace(W.TRAIN_4K, name="outdt", dk=d, dv=d, H=3, s0_std=0.05)
    inp = W.make_inputs(wl, seed=47, B=1 if T > 1000 else 2, T=T)
    say("case: bf16 output vs fp32 output, d=%d T=%d fused=%s" % (d, T, fused))
    o32, s32 = run_gpu(inp, fused=fused)
    o16, s16 = run_gpu(inp, out_dtype=torch.bfloat16, fused=fused)
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
