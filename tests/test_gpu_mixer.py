"""GPU parity of the mixer's fused passes (gdn2_mixer_prep, gdn2_mixer_out) against the fp64
mixer oracle, and of a whole layer: prep -> chunk forward -> output.

Bars.  These passes are elementwise (plus row reductions), so the bound follows from the
arithmetic: an fp32 result must be within 1e-4 of the oracle in max |x - x_ref| / RMS(x_ref);
a bf16 result is the fp32 result rounded once, so every element must lie within half a bf16
unit in the last place plus the fp32 arithmetic before it,
|x - x_ref| <= (2^-8 + 4e-6) |x_ref| + 1e-6 (the max/RMS measure is reported beside it: on
heavy-tailed outputs one correct rounding of the largest element already exceeds 3e-2).
The recurrence inside the layer test keeps its own bar (3e-2 for bf16 inputs).  Cases: several 64-token blocks with a
ragged tail, sequences shorter than the convolution, saturated gate and decay logits, zero
rows, and the whole training shape."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import oracle
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, rel_max_err, say

pytestmark = pytest.mark.gpu

PREP_OUT = ("q", "k", "v", "b", "w", "log_alpha")
X_IN = ("xq", "xk", "xv", "xb", "xw", "xa", "conv_q", "conv_k", "conv_v")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn2._load()


def mixer_case(dtype, d, B, T, H, seed):
    wl = dataclasses.replace(W.TRAIN_4K, name="mixer", dtype=dtype, dk=d, dv=d, B=B, T=T, H=H)
    return W.make_mixer_inputs(wl, seed=seed)


def run_prep(x):
    d = {n: x[n].cuda() for n in X_IN}
    out = gdn2.mixer_prep(*[d[n] for n in X_IN])
    torch.cuda.synchronize()
    return out


def oracle_prep(x):
    return oracle.mixer_prep(*[x[n] for n in X_IN])


def check_close(got, ref, dtype, label):
    err = rel_max_err(got, ref)
    if got.dtype == torch.bfloat16:
        g = got.detach().cpu().double().numpy()
        step = np.abs(g - ref) / ((2.0 ** -8 + 4e-6) * np.abs(ref) + 1e-6)
        ok = bool(np.all(step <= 1.0))
        say("  %-12s max/RMS %.2e; worst element %.2f bf16 steps%s" % (label, err, step.max(), "" if ok else "  FAIL"))
    else:
        ok = err <= TOL_F32
        say("  %-12s err %.2e (bar %.0e)%s" % (label, err, TOL_F32, "" if ok else "  FAIL"))
    return ok


PREP_CASES = [
    (torch.bfloat16, 128, 2, 200, 3, 401),
    (torch.bfloat16, 64, 1, 130, 2, 402),
    (torch.float32, 64, 2, 100, 2, 403),
    (torch.float32, 128, 1, 65, 2, 404),
    (torch.bfloat16, 128, 3, 2, 2, 405),   # shorter than the convolution
    (torch.float32, 64, 1, 1, 1, 406),
]


@pytest.mark.parametrize("dtype,d,B,T,H,seed", PREP_CASES)
def test_prep_matches_oracle(dtype, d, B, T, H, seed):
    say("case: mixer prep %s d%d B%d T%d H%d seed %d" % (dtype, d, B, T, H, seed))
    x = mixer_case(dtype, d, B, T, H, seed)
    got, ref = run_prep(x), oracle_prep(x)
    assert all([check_close(got[n], ref[n], dtype, n) for n in PREP_OUT])
    assert got["log_alpha"].dtype == torch.float32 and (got["log_alpha"] <= 0).all()


def test_prep_saturated_logits():
    """Gate and decay logits far in both tails: sigmoid 0 or 1, log sigmoid finite."""
    x = mixer_case(torch.float32, 64, 1, 70, 2, 407)
    sign = torch.where(torch.arange(64) % 2 == 0, 1.0, -1.0)
    x["xb"] = 100.0 * sign.expand_as(x["xb"]).contiguous()
    x["xw"] = -100.0 * sign.expand_as(x["xw"]).contiguous()
    x["xa"] = (80.0 * sign).expand_as(x["xa"]).contiguous()
    got, ref = run_prep(x), oracle_prep(x)
    for n in PREP_OUT:
        assert torch.isfinite(got[n]).all(), n
        assert check_close(got[n], ref[n], torch.float32, n)
    assert set(got["b"].unique().tolist()) <= {0.0, 1.0}


def test_out_matches_oracle():
    for dtype, o_dtype, d, seed in ((torch.bfloat16, torch.float32, 128, 411), (torch.bfloat16, torch.bfloat16, 64, 412),
                                    (torch.float32, torch.float32, 64, 413), (torch.float32, torch.float32, 128, 414)):
        say("case: mixer out %s o %s d%d" % (dtype, o_dtype, d))
        x = mixer_case(dtype, d, 2, 150, 3, seed)
        gen = torch.Generator("cpu").manual_seed(seed)
        o = (3.0 * torch.randn((2, 150, 3, d), generator=gen)).to(o_dtype)
        o[0, 5] = 0.0  # zero rows stay zero
        y = gdn2.mixer_out(o.cuda(), x["z"].cuda(), x["gamma"].cuda())
        torch.cuda.synchronize()
        ref = oracle.mixer_out(o, x["z"], x["gamma"])
        assert check_close(y, ref, dtype, "y")
        assert torch.all(y[0, 5] == 0)


def test_layer_prep_forward_out():
    """A whole mixer layer on the GPU (prep, chunk forward, output) against the oracle run on
    the values each GPU stage consumed: prep and output against the mixer oracle, the
    recurrence against the recurrence oracle on the GPU's prep outputs."""
    dtype, d, B, T, H = torch.bfloat16, 128, 2, 200, 2
    say("case: mixer layer bf16 d128 B2 T200 H2")
    x = mixer_case(dtype, d, B, T, H, 421)
    ins = run_prep(x)
    o, s = gdn2.chunk_fwd(ins["q"], ins["k"], ins["v"], ins["log_alpha"], ins["b"], ins["w"])
    y = gdn2.mixer_out(o, x["z"].cuda(), x["gamma"].cuda())
    torch.cuda.synchronize()
    assert all([check_close(ins[n], oracle_prep(x)[n], dtype, n) for n in PREP_OUT])
    cpu = {n: t.cpu() for n, t in ins.items()}
    o_ref, _ = oracle.fwd(cpu["q"], cpu["k"], cpu["v"], cpu["log_alpha"], cpu["b"], cpu["w"])
    eo = rel_max_err(o, o_ref)
    say("  layer recurrence: o err %.2e (bar %.0e)" % (eo, TOL_BF16))
    assert eo <= TOL_BF16
    assert check_close(y, oracle.mixer_out(o.cpu(), x["z"], x["gamma"]), dtype, "y")


def test_prep_training_shape_whole():
    """The training shape (B=8, T=4096, H=16, d=128, bf16) through the fused prep; every
    output of every (sequence, head) against the oracle run on the whole input."""
    wl = W.TRAIN_4K
    say("case: mixer prep %s whole" % wl.name)
    x = W.make_mixer_inputs(wl)
    got = run_prep(x)
    ref = oracle_prep(x)
    for n in PREP_OUT:
        assert check_close(got[n], ref[n], wl.dtype, n)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_caller_outputs_are_fully_written(dtype, d):
    """Output buffers of both passes, filled with NaN first, come back bit for bit equal to the
    outputs of calls that allocate their own."""
    x = mixer_case(dtype, d, 2, 150, 3, 415)
    ref = run_prep(x)
    dx = {n: x[n].cuda() for n in X_IN}
    bufs = {n: torch.full_like(t, float("nan")) for n, t in ref.items()}
    got = gdn2.mixer_prep(*[dx[n] for n in X_IN], out=bufs)
    gen = torch.Generator("cpu").manual_seed(415)
    o = (3.0 * torch.randn((2, 150, 3, d), generator=gen)).cuda()
    z, gamma = x["z"].cuda(), x["gamma"].cuda()
    y_ref = gdn2.mixer_out(o, z, gamma)
    y_buf = torch.full_like(y_ref, float("nan"))
    y = gdn2.mixer_out(o, z, gamma, y=y_buf)
    torch.cuda.synchronize()
    for n in ref:
        assert got[n] is bufs[n] and torch.equal(got[n], ref[n]), n
    assert y is y_buf and torch.equal(y, y_ref)
