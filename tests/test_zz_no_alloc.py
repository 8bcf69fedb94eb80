"""The allocation-free backward (gdn2_chunk_bwd_noalloc) against gdn2_chunk_bwd.

Both entry points run the same kernels; the allocation-free one takes its workspace from the
library's fixed device array.  Two calls in a row, the second smaller, each with gradient
buffers filled with NaN first, must give exactly the gradients of gdn2_chunk_bwd with a
workspace of its own: every output element is written, and nothing the second call reads
comes from the first call's contents of the shared array."""
import dataclasses

import pytest
import torch

import gated_delta_rule_gdn2_amd as gdn2
import workloads as W
from tests.parity_util import TOL_BF16, TOL_F32, rel_max_err, say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "d_initial_state")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn2._load()


def case(dtype, d, B, T, H, seed):
    wl = dataclasses.replace(W.FWD_BWD_4K, name="noalloc", dtype=dtype, dk=d, dv=d, B=B, T=T, H=H, s0_std=0.05)
    inp = W.make_inputs(wl, seed=seed)
    inp["do"] = W.make_upstream_grad(wl, seed=seed)
    inp["dsT"] = W.make_upstream_state_grad(wl, seed=seed)
    return to_dev(inp)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_noalloc_matches_chunk_bwd_twice(dtype, d):
    shapes = [(1, 576, 16), (2, 130, 3)] if d == 128 else [(3, 700, 8), (1, 65, 2)]
    for i, (B, T, H) in enumerate(shapes):
        need = gdn2.chunk_bwd_workspace_bytes(B, T, H, d, d)
        assert need <= gdn2.SCRATCH_BYTES
        say("case: noalloc call %d %s d=%d B=%d T=%d H=%d (workspace %d bytes)" % (i, dtype, d, B, T, H, need))
        x = case(dtype, d, B, T, H, 900 + i)
        ref = gdn2.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["do"], x["s0"], x["dsT"])
        grads = {n: torch.full_like(ref[n], float("nan")) for n in NAMES}
        got = gdn2.chunk_bwd_noalloc(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["do"], x["s0"],
                                     x["dsT"], grads=grads)
        torch.cuda.synchronize()
        tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
        for n in NAMES:
            assert got[n] is grads[n], n
            e = rel_max_err(got[n], ref[n].double().cpu().numpy())
            assert e <= tol, (n, e)
            assert torch.equal(got[n], ref[n]), n
        say("  all seven gradients bit-identical to gdn2_chunk_bwd")


def test_noalloc_rejects_sizes_beyond_the_array():
    x = case(torch.bfloat16, 128, 1, 640, 16, 910)
    assert gdn2.chunk_bwd_workspace_bytes(1, 640, 16, 128, 128) > gdn2.SCRATCH_BYTES
    with pytest.raises(gdn2.Gdn2Error) as ei:
        gdn2.chunk_bwd_noalloc(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["do"], x["s0"], x["dsT"],
                               grads=None)
    assert ei.value.status == 6  # GDN2_ERR_WORKSPACE
