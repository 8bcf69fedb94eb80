"""GPU parity of the backward pass (gdn2_chunk_bwd) against the fp64 oracle's reverse sweep.

Every gradient (q, k, v, log alpha, b, w and the initial state) is compared with the oracle
VJP on the same inputs, upstream gradients d_o and d_final_state included, with the
forward's bars: max |x - x_ref| / RMS(x_ref) <= 1e-4 for fp32 inputs, 3e-2 for bf16 inputs.
The cases span several chunks with a ragged tail, a single token, chunks whose decay takes
the element-by-element path (whole-chunk decay below e^-40), a mix of both kinds, and the
full fwd+bwd workload compared as whole tensors."""
import dataclasses

import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import oracle
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, rel_max_err, say, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn2._load()


def make_case(dtype, d, B, T, H, seed, s0_std=0.05, g_lo=-0.2, g_hi=-0.001, with_dsT=True):
    wl = dataclasses.replace(W.FWD_BWD_4K, name="bwd", dtype=dtype, dk=d, dv=d, B=B, T=T, H=H,
                             s0_std=s0_std, g_lo=g_lo, g_hi=g_hi)
    inp = W.make_inputs(wl, seed=seed)
    inp["do"] = W.make_upstream_grad(wl, seed=seed)
    inp["dsT"] = W.make_upstream_state_grad(wl, seed=seed) if with_dsT else None
    return inp


def run_bwd(inp, **kw):
    d = to_dev(inp)
    g = gdn2.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["do"], d["s0"], d["dsT"], **kw)
    torch.cuda.synchronize()
    return g


def oracle_vjp(inp):
    return oracle.vjp(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["do"],
                      inp["s0"], inp["dsT"])


def check(g, ref, tol, label, with_s0=True):
    errs = {n: rel_max_err(g[n], ref[n]) for n in GRADS}
    if with_s0 and g.get("d_initial_state") is not None:
        errs["d_initial_state"] = rel_max_err(g["d_initial_state"], ref["ds0"])
    say("  %-34s %s  (bar %.0e)" % (label, "  ".join("%s %.2e" % (n, e) for n, e in errs.items()), tol))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, (label, bad)


CASES = [
    # dtype, d, B, T, H, seed, s0_std, with_dsT
    (torch.float32, 64, 1, 150, 2, 301, 0.05, True),
    (torch.float32, 64, 2, 64, 1, 302, None, False),
    (torch.bfloat16, 64, 2, 128, 3, 303, None, False),
    (torch.bfloat16, 64, 1, 100, 2, 304, 0.05, True),
    (torch.bfloat16, 128, 1, 200, 2, 305, 0.05, True),
    (torch.bfloat16, 128, 2, 64, 1, 306, None, True),
]


@pytest.mark.parametrize("dtype,d,B,T,H,seed,s0_std,with_dsT", CASES)
def test_bwd_matches_oracle(dtype, d, B, T, H, seed, s0_std, with_dsT):
    say("case: bwd %s d%d B%d T%d H%d seed %d s0 %s dS_T %s" % (dtype, d, B, T, H, seed, s0_std, with_dsT))
    inp = make_case(dtype, d, B, T, H, seed, s0_std=s0_std, with_dsT=with_dsT)
    g = run_bwd(inp)
    check(g, oracle_vjp(inp), TOL_F32 if dtype == torch.float32 else TOL_BF16, "bwd", with_s0=True)


def test_bwd_single_token():
    say("case: bwd T=1, fp32 d64")
    inp = make_case(torch.float32, 64, 3, 1, 2, 307)
    check(run_bwd(inp), oracle_vjp(inp), TOL_F32, "T=1")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_bwd_strong_decay_chunks(dtype, d):
    """log alpha in [-5, -1]: every chunk's decay is far below e^-40, so the per-chunk gradient
    kernel takes its element-by-element path."""
    say("case: bwd strong decay %s d%d" % (dtype, d))
    inp = make_case(dtype, d, 1, 130, 2, 308, g_lo=-5.0, g_hi=-1.0)
    check(run_bwd(inp), oracle_vjp(inp), TOL_F32 if dtype == torch.float32 else TOL_BF16, "strong decay")


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_mixed_chunk_kinds(d):
    """Chunks 1, 3 and 5 of each sequence take log alpha in [-3, -1] (whole-chunk decay far below
    e^-40, element-by-element path), the others the default [-0.2, -0.001] (pivoted path)."""
    say("case: bwd mixed chunk kinds bf16 d%d" % d)
    inp = make_case(torch.bfloat16, d, 1, 512, 2, 309)
    gen = torch.Generator("cpu").manual_seed(309)
    for n in (1, 3, 5):
        inp["log_alpha"][:, n * 64:(n + 1) * 64] = -1.0 - 2.0 * torch.rand((1, 64, 2, d), generator=gen)
    G = inp["log_alpha"].double().reshape(1, 8, 64, 2, d).sum(2)  # whole-chunk log decays
    kinds = (G.min(-1).values >= -40.0)
    assert kinds.any() and (~kinds).any(), "expected both chunk kinds"
    check(run_bwd(inp), oracle_vjp(inp), TOL_BF16, "mixed chunks")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_bwd_chunk_runs_with_partial_tail(dtype, d):
    """Enough chunks that the chunk-local and per-chunk gradient kernels walk runs of several
    consecutive chunks per workgroup (8 heads x 72 chunks over the compute units), the last run
    ending in a partial chunk (T = 71 x 64 + 10), with element-by-element chunks (log alpha in
    [-3, -1]) inside runs and as the partial chunk; every gradient of every head against the
    oracle."""
    B, T, H = 1, 71 * 64 + 10, 8
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nch = (T + 63) // 64
    nper = (B * H * nch + cus - 1) // cus
    say("case: bwd chunk runs %s d%d B%d T%d H%d (%d chunks per run on %d CUs)" % (dtype, d, B, T, H, nper, cus))
    inp = make_case(dtype, d, B, T, H, 313)
    gen = torch.Generator("cpu").manual_seed(313)
    for n in (2, 5, 40, 70, 71):
        t1 = min(T, (n + 1) * 64)
        inp["log_alpha"][:, n * 64:t1] = -1.0 - 2.0 * torch.rand((B, t1 - n * 64, H, d), generator=gen)
    check(run_bwd(inp), oracle_vjp(inp), TOL_F32 if dtype == torch.float32 else TOL_BF16,
          "chunk runs, partial tail")


def test_bwd_without_initial_state_grad():
    inp = make_case(torch.bfloat16, 64, 1, 96, 2, 310)
    g_all = run_bwd(inp)
    g_no = run_bwd(inp, want_initial_state_grad=False)
    assert g_no["d_initial_state"] is None
    for n in GRADS:
        assert torch.equal(g_all[n], g_no[n]), n


def test_bwd_state_gradient_only():
    """d_o = 0: only dS_T drives the gradients; the oracle agrees, and dq is exactly zero
    (q reaches nothing but o)."""
    inp = make_case(torch.bfloat16, 128, 1, 96, 2, 311)
    inp["do"] = torch.zeros_like(inp["do"])
    g = run_bwd(inp)
    assert torch.count_nonzero(g["dq"]) == 0
    check(g, oracle_vjp(inp), TOL_BF16, "dS_T only")


def test_bwd_deterministic():
    inp = make_case(torch.bfloat16, 128, 1, 200, 2, 312)
    a, b = run_bwd(inp), run_bwd(inp)
    for n in GRADS + ("d_initial_state",):
        assert torch.equal(a[n], b[n]), n


def test_fwdbwd_workload_whole_tensor():
    """The fwd+bwd workload at full size (B=4, T=4096, H=16, d=128, bf16, S_0 ~ N(0, 0.02^2),
    d_o ~ N(0,1)) in the launch the benchmark times; the oracle's reverse sweep over every
    (sequence, head), every gradient compared as a whole tensor and per head."""
    wl = W.FWD_BWD_4K
    say("case: %s (full size, whole tensors)" % wl.name)
    inp = W.make_inputs(wl)
    inp["do"] = W.make_upstream_grad(wl)
    inp["dsT"] = None
    g = run_bwd(inp)
    ref = oracle_vjp(inp)
    check(g, ref, TOL_BF16, "fwdbwd whole tensors")
    worst = {}
    for n in GRADS:
        worst[n] = max(rel_max_err(g[n][:, :, h], ref[n][:, :, h]) for h in range(wl.H))
    worst["d_initial_state"] = max(rel_max_err(g["d_initial_state"][:, h], ref["ds0"][:, h]) for h in range(wl.H))
    say("  worst head: %s" % "  ".join("%s %.2e" % (n, e) for n, e in worst.items()))
    assert all(e <= TOL_BF16 for e in worst.values()), worst


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_bwd_caller_workspace_and_outputs(dtype, d):
    """A caller's workspace and gradient buffers, filled with NaN bytes first and reused by a
    smaller second call, give bit for bit the gradients of calls that allocate their own:
    nothing reads a workspace slot it has not written, and every output element is written."""
    cases = [make_case(dtype, d, 2, 300, 2, 314), make_case(dtype, d, 1, 70, 3, 315)]
    need = max(gdn2.chunk_bwd_workspace_bytes(*c["q"].shape[:3], d, d) for c in cases)
    say("case: bwd caller workspace %s d%d (%d bytes, NaN-filled)" % (dtype, d, need))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    names = GRADS + ("d_initial_state",)
    for inp in cases:
        ref = run_bwd(inp)
        x = to_dev(inp)
        grads = {n: torch.full_like(ref[n], float("nan")) for n in names}
        g = gdn2.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["do"], x["s0"], x["dsT"],
                           workspace=ws, grads=grads)
        torch.cuda.synchronize()
        for n in names:
            assert g[n] is grads[n], n
            assert torch.equal(g[n], ref[n]), n
