"""GPU parity of the packed-sequence forward (serving prefill) and its hand-off to decode.

Every sequence of a packed batch is checked against the fp64 oracle run on that
sequence alone, with the same bars as the fixed-length forward (max |x - x_ref| /
RMS(x_ref): 1e-4 for fp32 inputs, 3e-2 for bf16 inputs).  Lengths mix empty, single
token, one token short of, exactly and one past a chunk, and several chunks with a
ragged tail."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import oracle
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, rel_max_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn2._load()


def packed_case(dtype, d, H, lengths, seed, s0_std=0.05, g_lo=-0.2, g_hi=-0.001):
    wl = dataclasses.replace(W.SERVE_PREFILL, name="varlen", dtype=dtype, dk=d, dv=d, H=H,
                             s0_std=s0_std, g_lo=g_lo, g_hi=g_hi)
    return W.make_packed_inputs(wl, lengths, seed=seed)


def run_varlen(inp, **kw):
    d = to_dev(inp)
    o, s = gdn2.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                                 d["cu_seqlens"], d["s0"], **kw)
    torch.cuda.synchronize()
    return o, s


def oracle_sequence(inp, n):
    """The oracle on sequence n alone: returns o [L, H, dv] and S_T [H, dk, dv]."""
    cu = inp["cu_seqlens"].tolist()
    a, e = cu[n], cu[n + 1]
    H, dk = inp["q"].shape[1], inp["q"].shape[2]
    dv = inp["v"].shape[2]
    s0 = None if inp["s0"] is None else inp["s0"][n:n + 1]
    if e == a:
        st = np.zeros((H, dk, dv)) if s0 is None else s0[0].double().numpy()
        return np.zeros((0, H, dv)), st
    x = {nm: inp[nm][a:e][None] for nm in ("q", "k", "v", "log_alpha", "b", "w")}
    o, s = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], s0)
    return o[0], s[0]


def check_all(inp, o, s, tol, label):
    N = inp["cu_seqlens"].numel() - 1
    refs = [oracle_sequence(inp, n) for n in range(N)]
    o_ref = np.concatenate([r[0] for r in refs], axis=0)
    s_ref = np.stack([r[1] for r in refs])
    eo, es = rel_max_err(o, o_ref), rel_max_err(s, s_ref)
    say("  %-44s o err %.3e   S_T err %.3e   (bar %.0e)" % (label, eo, es, tol))
    assert eo <= tol and es <= tol, (label, eo, es)


MIX = [0, 1, 63, 64, 65, 200, 7, 130]

CASES = [
    # dtype, d, H, seed
    (torch.bfloat16, 128, 3, 201),
    (torch.bfloat16, 64, 5, 202),
    (torch.float32, 64, 2, 203),
]


@pytest.mark.parametrize("dtype,d,H,seed", CASES)
def test_packed_mix_matches_oracle_per_sequence(dtype, d, H, seed):
    say("case: varlen %s d%d H%d seed %d lengths %s" % (dtype, d, H, seed, MIX))
    inp = packed_case(dtype, d, H, MIX, seed)
    o, s = run_varlen(inp)
    check_all(inp, o, s, TOL_F32 if dtype == torch.float32 else TOL_BF16, "packed mix")


def test_packed_strong_decay():
    say("case: varlen strong decay bf16 d128")
    inp = packed_case(torch.bfloat16, 128, 2, [70, 1, 150, 64], 204, g_lo=-5.0, g_hi=-1.0)
    o, s = run_varlen(inp)
    check_all(inp, o, s, TOL_BF16, "packed strong decay")


def test_equal_lengths_match_fixed_length_call_exactly():
    """Packed sequences run the fused kernel: with equal lengths they are bit-identical to the
    fixed-length call in its fused form."""
    say("case: varlen == fixed length, bf16 d128, 4 x 130 tokens")
    L, N, H = 130, 4, 3
    inp = packed_case(torch.bfloat16, 128, H, [L] * N, 205)
    o, s = run_varlen(inp)
    d = to_dev(inp)
    shp = lambda x: x.reshape(N, L, H, x.shape[-1])
    o2, s2 = gdn2.chunk_fwd(shp(d["q"]), shp(d["k"]), shp(d["v"]), shp(d["log_alpha"]), shp(d["b"]),
                            shp(d["w"]), d["s0"], fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(N, L, H, -1), o2)
    assert torch.equal(s, s2)


def test_empty_sequences_pass_their_state_through():
    say("case: varlen with empty sequences")
    inp = packed_case(torch.bfloat16, 128, 2, [0, 5, 0, 0], 206)
    o, s = run_varlen(inp)
    s0 = inp["s0"].cuda()
    for n in (0, 2, 3):
        assert torch.equal(s[n], s0[n]), n
    check_all(inp, o, s, TOL_BF16, "empty sequences")


def test_tokens_outside_every_sequence_are_untouched():
    say("case: varlen offsets covering part of the token axis")
    inp = packed_case(torch.bfloat16, 64, 2, [40, 30], 207)
    d = to_dev(inp)
    d["cu_seqlens"] = torch.tensor([5, 45, 60], dtype=torch.int64, device="cuda")  # tokens 0-4, 60-69 unused
    o = torch.full((70, 2, 64), 7.0, device="cuda")
    gdn2.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["cu_seqlens"],
                          d["s0"], o=o)
    torch.cuda.synchronize()
    assert torch.all(o[:5] == 7.0) and torch.all(o[60:] == 7.0)
    assert torch.isfinite(o[5:60]).all()


def test_prefill_then_decode_continues_the_sequences():
    """Prefill N prompts (packed, with initial states), then decode 8 tokens per sequence
    from the prefill's final states; compare every decode output and the final state with
    the oracle run over prompt + decoded tokens."""
    say("case: varlen prefill -> decode hand-off, bf16 d128")
    lengths, H, d, steps = [33, 64, 1, 97], 2, 128, 8
    N = len(lengths)
    inp = packed_case(torch.bfloat16, d, H, lengths, 208)
    _, s = run_varlen(inp)
    dec = packed_case(torch.bfloat16, d, H, [steps] * N, 209, s0_std=None)  # decode tokens
    dd = to_dev(dec)
    state = s.clone()
    outs = []
    for t in range(steps):
        idx = torch.arange(N, device="cuda") * steps + t
        x = {nm: dd[nm][idx].contiguous() for nm in ("q", "k", "v", "log_alpha", "b", "w")}
        outs.append(gdn2.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], state))
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    worst = 0.0
    for n in range(N):
        cat = {nm: torch.cat([inp[nm][cu[n]:cu[n + 1]], dec[nm][n * steps:(n + 1) * steps]])[None]
               for nm in ("q", "k", "v", "log_alpha", "b", "w")}
        o_ref, s_ref = oracle.fwd(cat["q"], cat["k"], cat["v"], cat["log_alpha"], cat["b"], cat["w"],
                                  inp["s0"][n:n + 1])
        o_dec = torch.stack([outs[t][n] for t in range(steps)])
        eo = rel_max_err(o_dec, o_ref[0, lengths[n]:])
        es = rel_max_err(state[n], s_ref[0])
        worst = max(worst, eo, es)
        assert eo <= TOL_BF16 and es <= TOL_BF16, (n, eo, es)
    say("  prefill -> decode, worst err %.3e (bar %.0e)" % (worst, TOL_BF16))


def test_serving_prefill_workload_whole():
    """The serving prefill workload at full size (64 prompts, seeded length mix, H=16,
    d=128, continuation states), in the launch the benchmark times; every sequence against
    the oracle run on it alone, the metric over the whole o and S_T tensors."""
    wl = W.SERVE_PREFILL
    lengths = W.make_lengths(wl.B, wl.seed)
    say("case: %s total %d tokens" % (wl.name, sum(lengths)))
    inp = W.make_packed_inputs(wl, lengths)
    o, s = run_varlen(inp)
    check_all(inp, o, s, TOL_BF16, "serving prefill, all 64 sequences")


def test_multi_token_steps_in_place_continue_the_sequences():
    """Decode several tokens per sequence per call: the fixed-length forward with T = 3 and
    the state passed as both initial and final state, three calls in a row after a packed
    prefill; every output and the final states against the oracle over prompt + steps."""
    say("case: multi-token steps in place after prefill, bf16 d128")
    lengths, H, d, per, calls = [20, 64, 90], 2, 128, 3, 3
    N = len(lengths)
    inp = packed_case(torch.bfloat16, d, H, lengths, 210)
    _, state = run_varlen(inp)
    steps = per * calls
    dec = packed_case(torch.bfloat16, d, H, [steps] * N, 211, s0_std=None)
    dd = {nm: dec[nm].reshape(N, steps, H, -1).cuda() for nm in ("q", "k", "v", "log_alpha", "b", "w")}
    outs = []
    for c in range(calls):
        x = {nm: dd[nm][:, c * per:(c + 1) * per].contiguous() for nm in dd}
        o, s = gdn2.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], state,
                              final_state=state)
        assert s.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    o_all = torch.cat(outs, dim=1)  # [N, steps, H, dv]
    cu = inp["cu_seqlens"].tolist()
    for n in range(N):
        cat = {nm: torch.cat([inp[nm][cu[n]:cu[n + 1]], dec[nm][n * steps:(n + 1) * steps]])[None]
               for nm in ("q", "k", "v", "log_alpha", "b", "w")}
        o_ref, s_ref = oracle.fwd(cat["q"], cat["k"], cat["v"], cat["log_alpha"], cat["b"], cat["w"],
                                  inp["s0"][n:n + 1])
        eo = rel_max_err(o_all[n], o_ref[0, lengths[n]:])
        es = rel_max_err(state[n], s_ref[0])
        say("  sequence %d: o err %.3e   S err %.3e" % (n, eo, es))
        assert eo <= TOL_BF16 and es <= TOL_BF16, (n, eo, es)


def test_sequence_order_does_not_change_results():
    """Workgroups take the packed sequences longest first; every sequence's o and S_T are
    bit-identical when the same sequences are packed in the reverse order."""
    say("case: varlen order independence, bf16 d128")
    lengths, H = [300, 5, 130, 64, 1, 257], 2
    inp = packed_case(torch.bfloat16, 128, H, lengths, 210)
    o, s = run_varlen(inp)
    cu = inp["cu_seqlens"].tolist()
    N = len(lengths)
    rev = {}
    for nm in ("q", "k", "v", "log_alpha", "b", "w"):
        rev[nm] = torch.cat([inp[nm][cu[n]:cu[n + 1]] for n in reversed(range(N))])
    rev["s0"] = inp["s0"].flip(0).contiguous()
    rcu = [0]
    for n in reversed(range(N)):
        rcu.append(rcu[-1] + lengths[n])
    rev["cu_seqlens"] = torch.tensor(rcu, dtype=torch.int64)
    o2, s2 = run_varlen(rev)
    for n in range(N):
        m = N - 1 - n
        assert torch.equal(o[cu[n]:cu[n + 1]], o2[rcu[m]:rcu[m + 1]]), n
        assert torch.equal(s[n], s2[m]), n


def _split(inp, lo, hi):
    """Sequences lo..hi-1 of a packed batch as a packed batch of their own."""
    cu = inp["cu_seqlens"].tolist()
    out = {nm: inp[nm][cu[lo]:cu[hi]] for nm in ("q", "k", "v", "log_alpha", "b", "w")}
    out["cu_seqlens"] = torch.tensor([c - cu[lo] for c in cu[lo:hi + 1]], dtype=torch.int64)
    out["s0"] = None if inp["s0"] is None else inp["s0"][lo:hi].contiguous()
    return out


def test_more_sequences_than_the_sorted_range():
    """600 packed sequences (past the 512 the longest-first order sorts; they go in index
    order), lengths 0-70.  bf16: bit-identical to the same sequences in two calls of 300
    (sorted order).  fp32: against the oracle per sequence."""
    gen = torch.Generator("cpu").manual_seed(211)
    lengths = torch.randint(0, 71, (600,), generator=gen).tolist()
    say("case: varlen 600 sequences bf16 d64, one call vs two")
    inp = packed_case(torch.bfloat16, 64, 1, lengths, 211)
    o, s = run_varlen(inp)
    cu = inp["cu_seqlens"].tolist()
    for lo, hi in ((0, 300), (300, 600)):
        o2, s2 = run_varlen(_split(inp, lo, hi))
        assert torch.equal(o[cu[lo]:cu[hi]], o2), (lo, hi)
        assert torch.equal(s[lo:hi], s2), (lo, hi)
    say("case: varlen 600 sequences fp32 d64 vs oracle")
    inp = packed_case(torch.float32, 64, 1, lengths, 212)
    o, s = run_varlen(inp)
    check_all(inp, o, s, TOL_F32, "600 sequences fp32")


def test_caller_outputs_are_fully_written():
    """o and S_T buffers passed in, filled with NaN first, come back bit for bit equal to those
    of a call that allocates its own, for packed lengths with an empty sequence, a one-token
    sequence and ragged last chunks."""
    inp = packed_case(torch.bfloat16, 128, 2, [70, 0, 150, 1, 64], 216)
    o_ref, s_ref = run_varlen(inp)
    o_buf, s_buf = torch.full_like(o_ref, float("nan")), torch.full_like(s_ref, float("nan"))
    o, s = run_varlen(inp, o=o_buf, final_state=s_buf)
    assert o is o_buf and s is s_buf
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
