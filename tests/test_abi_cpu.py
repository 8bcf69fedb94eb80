"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid calls before touching the HIP runtime.

The pointers used here are host addresses that are never dereferenced: every
call below fails validation, which happens before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_gdn2_amd as gdn2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP = range(8)
BF16, F32 = 1, 0


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn2.library_path()):
        pytest.skip("libgdn2.so not built")
    return gdn2._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for name in ("gdn2_chunk_fwd", "gdn2_chunk_fwd_logits", "gdn2_chunk_fwd_workspace_bytes", "gdn2_chunk_fwd_varlen",
                 "gdn2_chunk_bwd",
                 "gdn2_chunk_bwd_workspace_bytes", "gdn2_decode_step", "gdn2_mixer_prep", "gdn2_mixer_out",
                 "gdn2_status_string", "gdn2_version"):
        assert name in names, name


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for s in range(8):
        assert lib.gdn2_status_string(s)
    assert lib.gdn2_status_string(ERR_WORKSPACE) != lib.gdn2_status_string(99)
    assert gdn2.version().startswith("gdn2-gfx950")


def test_supported_table(lib):
    assert lib.gdn2_supported(0, 128, 128, BF16) == 1
    assert lib.gdn2_supported(0, 64, 64, BF16) == 1
    assert lib.gdn2_supported(0, 64, 64, F32) == 1
    assert lib.gdn2_supported(0, 128, 128, F32) == 0
    assert lib.gdn2_supported(0, 96, 96, BF16) == 0
    assert lib.gdn2_supported(1, 128, 128, F32) == 1
    assert lib.gdn2_supported(1, 32, 32, BF16) == 0
    assert lib.gdn2_supported(2, 128, 128, BF16) == 1
    assert lib.gdn2_supported(2, 64, 64, F32) == 1
    assert lib.gdn2_supported(2, 128, 128, F32) == 0
    assert lib.gdn2_supported(3, 128, 128, BF16) == 1
    assert lib.gdn2_supported(3, 128, 128, F32) == 1
    assert lib.gdn2_supported(3, 96, 96, BF16) == 0
    assert lib.gdn2_supported(4, 128, 128, BF16) == 0


# --- validation paths (no HIP call is reached) ---------------------------------

class Fake:
    """Distinct, 16-byte aligned, never-dereferenced addresses."""

    def __init__(self, nbytes=1 << 20, slots=12):
        self.buf = ctypes.create_string_buffer(nbytes * slots + 64)
        base = (ctypes.addressof(self.buf) + 15) & ~15
        self.nbytes = nbytes
        self.base = base

    def p(self, i, offset=0):
        return ctypes.c_void_p(self.base + i * self.nbytes + offset)


def chunk(lib, f, B=1, T=64, H=1, dk=64, dv=64, dtype=BF16, odt=F32, **over):
    args = dict(q=f.p(0), k=f.p(1), v=f.p(2), g=f.p(3), b=f.p(4), w=f.p(5), s0=None, o=f.p(7),
                sT=None)
    args.update(over)
    return lib.gdn2_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["b"], args["w"],
                              args["s0"], args["o"], args["sT"], B, T, H, dk, dv, dtype, odt,
                              args.get("ws"), args.get("ws_bytes", 0), None)


def chunk_logits(lib, f, B=1, T=64, H=1, dk=64, dv=64, dtype=BF16, odt=F32, **over):
    args = dict(q=f.p(0), k=f.p(1), v=f.p(2), a=f.p(3), b=f.p(4), w=f.p(5), s0=None, o=f.p(7),
                sT=None)
    args.update(over)
    return lib.gdn2_chunk_fwd_logits(args["q"], args["k"], args["v"], args["a"], args["b"], args["w"],
                                     args["s0"], args["o"], args["sT"], B, T, H, dk, dv, dtype, odt,
                                     args.get("ws"), args.get("ws_bytes", 0), None)


def decode(lib, f, N=1, H=1, dk=64, dv=64, dtype=BF16, odt=F32, **over):
    args = dict(q=f.p(0), k=f.p(1), v=f.p(2), g=f.p(3), b=f.p(4), w=f.p(5), s=f.p(6), o=f.p(7))
    args.update(over)
    return lib.gdn2_decode_step(args["q"], args["k"], args["v"], args["g"], args["b"], args["w"],
                                args["s"], args["o"], N, H, dk, dv, dtype, odt, None)


def test_chunk_null_pointers(lib):
    f = Fake()
    for name in ("q", "k", "v", "g", "b", "w", "o"):
        assert chunk(lib, f, **{name: None}) == ERR_NULL, name


def test_chunk_bad_shapes(lib):
    f = Fake()
    assert chunk(lib, f, B=0) == ERR_SHAPE
    assert chunk(lib, f, T=0) == ERR_SHAPE
    assert chunk(lib, f, H=-1) == ERR_SHAPE
    assert chunk(lib, f, B=1 << 40, T=1 << 40) == ERR_SHAPE
    # token stride H * d must stay below 2^22 elements
    assert chunk(lib, f, H=1 << 15, dk=128, dv=128) == ERR_SHAPE
    assert chunk(lib, f, H=1 << 16, dk=64, dv=64) == ERR_SHAPE


def test_chunk_unsupported(lib):
    f = Fake()
    assert chunk(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    assert chunk(lib, f, dk=128, dv=128, dtype=F32) == ERR_UNSUPPORTED
    assert chunk(lib, f, dtype=7) == ERR_UNSUPPORTED
    assert chunk(lib, f, dtype=F32, dk=64, dv=64, odt=BF16) == ERR_UNSUPPORTED
    assert chunk(lib, f, odt=9) == ERR_UNSUPPORTED


def test_chunk_misaligned(lib):
    f = Fake()
    assert chunk(lib, f, q=f.p(0, 2)) == ERR_MISALIGNED
    assert chunk(lib, f, sT=f.p(8, 4)) == ERR_MISALIGNED


def test_chunk_aliasing(lib):
    f = Fake()
    # o on top of v
    assert chunk(lib, f, o=f.p(2, 64)) == ERR_ALIAS
    # final state overlapping k
    assert chunk(lib, f, sT=f.p(1, 16)) == ERR_ALIAS
    # final state partially overlapping the initial state
    assert chunk(lib, f, s0=f.p(8), sT=f.p(8, 16)) == ERR_ALIAS


def test_decode_validation(lib):
    f = Fake()
    for name in ("q", "k", "v", "g", "b", "w", "s", "o"):
        assert decode(lib, f, **{name: None}) == ERR_NULL, name
    assert decode(lib, f, N=0) == ERR_SHAPE
    assert decode(lib, f, dk=32, dv=32) == ERR_UNSUPPORTED
    assert decode(lib, f, dtype=F32, odt=BF16) == ERR_UNSUPPORTED
    assert decode(lib, f, s=f.p(6, 8)) == ERR_MISALIGNED
    assert decode(lib, f, o=f.p(6)) == ERR_ALIAS
    assert decode(lib, f, s=f.p(0)) == ERR_ALIAS


def test_python_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        gdn2.chunk_fwd(x, x, x, g, x, x)


def varlen(lib, f, N=2, total=64, H=1, dk=64, dv=64, dtype=BF16, odt=F32, **over):
    args = dict(q=f.p(0), k=f.p(1), v=f.p(2), g=f.p(3), b=f.p(4), w=f.p(5), s0=None, o=f.p(7),
                sT=None, cu=f.p(9))
    args.update(over)
    return lib.gdn2_chunk_fwd_varlen(args["q"], args["k"], args["v"], args["g"], args["b"], args["w"],
                                     args["s0"], args["o"], args["sT"], args["cu"], N, total, H, dk,
                                     dv, dtype, odt, None)


def test_varlen_validation(lib):
    f = Fake()
    assert varlen(lib, f, cu=None) == ERR_NULL
    for name in ("q", "k", "v", "g", "b", "w", "o"):
        assert varlen(lib, f, **{name: None}) == ERR_NULL, name
    assert varlen(lib, f, N=0) == ERR_SHAPE
    assert varlen(lib, f, total=-1) == ERR_SHAPE
    assert varlen(lib, f, cu=f.p(9, 4)) == ERR_MISALIGNED
    assert varlen(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    # offsets inside o, final state overlapping the offsets
    assert varlen(lib, f, cu=f.p(7, 8)) == ERR_ALIAS
    assert varlen(lib, f, sT=f.p(9)) == ERR_ALIAS


def test_status_values_follow_the_boundary_table(lib):
    """GDN2_ERR_WORKSPACE is 6 and GDN2_ERR_HIP is 7; the strings name them."""
    assert b"workspace" in lib.gdn2_status_string(ERR_WORKSPACE)
    assert b"HIP" in lib.gdn2_status_string(ERR_HIP)
    assert (ERR_WORKSPACE, ERR_HIP) == (6, 7)


def split_segments(B, T, H, d, cus=256):
    """Segments of the few-chains form, by the library's cost model: each (sequence, head) is a
    chain; g segments of L chunks cost (transition rounds + forward rounds) * L + 2 (g - 1) chunk
    steps (two workgroups per chain for the transitions of all segments but the last), batches
    ceil(chains / cus) * nchunks; the cheapest wins (1: batches)."""
    nc, chains = (T + 63) // 64, B * H
    rounds = lambda wg: -(-wg // cus)
    best_g, best = 1, rounds(chains) * nc
    for g in range(2, min(nc // 16, 64) + 1):
        ln = -(-nc // g)
        gg = -(-nc // ln)
        cost = (rounds(2 * (gg - 1) * chains) + rounds(gg * chains)) * ln + 2 * (gg - 1)
        if cost < best:
            best, best_g = cost, gg
    return best_g


def split_ws_bytes(B, T, H, d):
    """Records of one batch (about 1024 chunk-heads) plus one fp32 state; with segments, every
    chunk's record, the transitions ([d][2 d]) of segments 0 .. g - 2 and every segment's start
    state."""
    part_a = 2 * 64 * d * 2                                   # QG, BG
    part_b = d * 64 * 2 + 3 * (32 * 32 + 32 * 64) * 2 + d * 4  # KG^T; T; P hi, lo; Gamma_C
    rec = part_a + (part_b + 1023) // 1024 * 1024
    nc = (T + 63) // 64
    g = split_segments(B, T, H, d)
    if g > 1:
        return B * H * nc * rec + (g - 1) * B * H * d * 2 * d * 4 + g * B * H * d * d * 4
    bc = min(max(1024 // (B * H), 1), nc)
    return B * H * bc * rec + B * H * d * d * 4


def test_fwd_workspace_bytes(lib):
    """bf16 with d = 64 or 128 has the two-kernel form: its workspace is the records of one
    batch of chunks plus a state; fp32 and other sizes take none."""
    assert split_ws_bytes(1, 64, 1, 128) - 128 * 128 * 4 == 68608
    assert split_ws_bytes(1, 64, 1, 64) - 64 * 64 * 4 == 44032
    assert [split_segments(*x) for x in ((1, 32768, 16, 128), (8, 4096, 16, 128), (1, 5000, 3, 64),
                                         (2, 2100, 16, 128), (1, 1000, 1, 64), (4, 8192, 16, 128),
                                         (2, 16384, 16, 128))] == [16, 1, 4, 1, 1, 3, 8]
    for (B, T, H, d) in ((1, 1, 1, 64), (8, 4096, 16, 128), (1, 32768, 16, 128), (3, 1000, 5, 64),
                         (1, 5000, 3, 64), (2, 2100, 16, 128)):
        assert lib.gdn2_chunk_fwd_split_workspace_bytes(B, T, H, d, d, BF16) == split_ws_bytes(B, T, H, d)
        assert lib.gdn2_chunk_fwd_split_workspace_bytes(B, T, H, d, d, F32) == 0
    assert lib.gdn2_chunk_fwd_split_workspace_bytes(1, 64, 1, 96, 96, BF16) == 0
    assert lib.gdn2_chunk_fwd_split_workspace_bytes(0, 64, 1, 128, 128, BF16) == 0
    assert gdn2.chunk_fwd_workspace_bytes(8, 4096, 16, 128, 128, split=True) == split_ws_bytes(8, 4096, 16, 128)
    # the faster form: the two-kernel form only when the fused kernel's chains, one per
    # (sequence, head, 64 columns), are fewer than the compute units (256 here: no GPU)
    assert lib.gdn2_chunk_fwd_workspace_bytes(1, 32768, 16, 128, 128, BF16) == split_ws_bytes(1, 32768, 16, 128)
    assert lib.gdn2_chunk_fwd_workspace_bytes(8, 4096, 16, 128, 128, BF16) == 0
    assert lib.gdn2_chunk_fwd_workspace_bytes(1, 32768, 16, 128, 128, F32) == 0


def test_fwd_workspace_validation(lib):
    """No workspace selects the fused kernel; a workspace must be large enough, 256-byte aligned,
    overlap nothing, and only where the two-kernel form exists (all before any HIP call)."""
    f = Fake(nbytes=1 << 22, slots=12)
    need = lib.gdn2_chunk_fwd_split_workspace_bytes(1, 64, 1, 64, 64, BF16)
    a256 = lambda slot: f.p(slot, (-f.p(slot).value) % 256)
    ws = a256(10)
    assert chunk(lib, f, q=f.p(0, 2), ws=None, ws_bytes=0) == ERR_MISALIGNED  # fused path, fails later
    assert chunk(lib, f, ws=ws, ws_bytes=need - 1) == ERR_WORKSPACE
    assert chunk(lib, f, ws=None, ws_bytes=need) == ERR_WORKSPACE
    assert chunk(lib, f, ws=ctypes.c_void_p(ws.value + 16), ws_bytes=need) == ERR_MISALIGNED
    assert chunk(lib, f, ws=a256(2), ws_bytes=need) == ERR_ALIAS              # overlaps v
    assert chunk(lib, f, dtype=F32, odt=F32, ws=ws, ws_bytes=need) == ERR_WORKSPACE


def test_bwd_workspace_bytes(lib):
    # 4 bytes x (2 B H NC dk dv + 2 B T H dv + B H NC R), parts rounded to 256 bytes, with R the
    # floats of a chunk record: 2*64*64 + 5*64*dk + 64*dv + dk rounded up to 64
    B, T, H, d = 2, 130, 3, 64
    nc = 3
    rec = (2 * 64 * 64 + 5 * 64 * d + 64 * d + d + 63) // 64 * 64
    parts = [B * H * nc * d * d * 4] * 2 + [B * T * H * d * 4] * 2 + [B * H * nc * rec * 4]
    assert lib.gdn2_chunk_bwd_workspace_bytes(B, T, H, d, d) == sum((x + 255) // 256 * 256 for x in parts)
    assert gdn2.chunk_bwd_workspace_bytes(B, T, H, d, d) == lib.gdn2_chunk_bwd_workspace_bytes(B, T, H, d, d)
    assert lib.gdn2_chunk_bwd_workspace_bytes(1 << 40, 1 << 40, 1, 64, 64) == 0
    assert lib.gdn2_chunk_bwd_workspace_bytes(1, 64, 1, 1 << 21, 64) == 0


def bwd(lib, f, B=1, T=64, H=1, dk=64, dv=64, dtype=BF16, ws_bytes=None, **over):
    names = ("q k v g b w s0 do dsT gq gk gv gg gb gw gs0 ws").split()
    args = {n: f.p(i) for i, n in enumerate(names)}
    args["s0"] = args["dsT"] = args["gs0"] = None
    args.update(over)
    if ws_bytes is None:
        ws_bytes = lib.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv)
    return lib.gdn2_chunk_bwd(*[args[n] for n in names], ws_bytes, B, T, H, dk, dv, dtype, None)


def test_bwd_validation(lib):
    f = Fake(slots=18)
    for name in ("q", "k", "v", "g", "b", "w", "do", "gq", "gk", "gv", "gg", "gb", "gw"):
        assert bwd(lib, f, **{name: None}) == ERR_NULL, name
    assert bwd(lib, f, B=0) == ERR_SHAPE
    assert bwd(lib, f, T=0) == ERR_SHAPE
    assert bwd(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    assert bwd(lib, f, dk=128, dv=128, dtype=F32) == ERR_UNSUPPORTED
    assert bwd(lib, f, dtype=5) == ERR_UNSUPPORTED
    assert bwd(lib, f, H=1 << 17, dk=128, dv=128) == ERR_SHAPE
    assert bwd(lib, f, gq=f.p(9, 4)) == ERR_MISALIGNED
    assert bwd(lib, f, ws=None) == ERR_WORKSPACE
    need = lib.gdn2_chunk_bwd_workspace_bytes(1, 64, 1, 64, 64)
    assert bwd(lib, f, ws_bytes=need - 1) == ERR_WORKSPACE
    assert bwd(lib, f, ws=f.p(16, 8)) == ERR_MISALIGNED
    # an output on an input, two outputs on each other, the workspace on an input or output
    assert bwd(lib, f, gq=f.p(0)) == ERR_ALIAS
    assert bwd(lib, f, gk=f.p(9, 64)) == ERR_ALIAS
    assert bwd(lib, f, gs0=f.p(14, 16)) == ERR_ALIAS
    assert bwd(lib, f, ws=f.p(7)) == ERR_ALIAS
    assert bwd(lib, f, ws=f.p(14, 256)) == ERR_ALIAS
    assert bwd(lib, f, s0=f.p(6), gs0=f.p(6, 32)) == ERR_ALIAS


def prep(lib, f, B=1, T=64, H=1, dk=64, dv=64, eps=1e-6, dtype=BF16, **over):
    names = "xq xk xv xb xw xa cq ck cv q k v b w g".split()
    args = {n: f.p(i) for i, n in enumerate(names)}
    args.update(over)
    return lib.gdn2_mixer_prep(*[args[n] for n in names], B, T, H, dk, dv, eps, dtype, None)


def mout(lib, f, B=1, T=64, H=1, dv=64, eps=1e-6, dtype=BF16, odt=F32, **over):
    args = dict(o=f.p(0), z=f.p(1), gamma=f.p(2), y=f.p(3))
    args.update(over)
    return lib.gdn2_mixer_out(args["o"], args["z"], args["gamma"], args["y"], B, T, H, dv, eps, dtype, odt, None)


def test_mixer_validation(lib):
    f = Fake(slots=16)
    for name in "xq xk xv xb xw xa cq ck cv q k v b w g".split():
        assert prep(lib, f, **{name: None}) == ERR_NULL, name
    assert prep(lib, f, T=0) == ERR_SHAPE
    assert prep(lib, f, eps=-1.0) == ERR_SHAPE
    assert prep(lib, f, eps=float("nan")) == ERR_SHAPE
    assert prep(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    assert prep(lib, f, dk=64, dv=128) == ERR_UNSUPPORTED
    assert prep(lib, f, dtype=3) == ERR_UNSUPPORTED
    assert prep(lib, f, q=f.p(9, 2)) == ERR_MISALIGNED
    assert prep(lib, f, q=f.p(0)) == ERR_ALIAS
    assert prep(lib, f, v=f.p(9, 64)) == ERR_ALIAS
    assert prep(lib, f, g=f.p(6)) == ERR_ALIAS
    for name in ("o", "z", "gamma", "y"):
        assert mout(lib, f, **{name: None}) == ERR_NULL, name
    assert mout(lib, f, H=0) == ERR_SHAPE
    assert mout(lib, f, dv=32) == ERR_UNSUPPORTED
    assert mout(lib, f, dtype=F32, odt=BF16) == ERR_UNSUPPORTED
    assert mout(lib, f, y=f.p(3, 4)) == ERR_MISALIGNED
    assert mout(lib, f, y=f.p(0, 64)) == ERR_ALIAS
    assert mout(lib, f, y=f.p(2)) == ERR_ALIAS


def bwd_noalloc(lib, f, B=1, T=64, H=1, dk=64, dv=64, dtype=BF16, **over):
    names = ("q k v g b w s0 do dsT gq gk gv gg gb gw gs0").split()
    args = {n: f.p(i) for i, n in enumerate(names)}
    args["s0"] = args["dsT"] = args["gs0"] = None
    args.update(over)
    return lib.gdn2_chunk_bwd_noalloc(*[args[n] for n in names], B, T, H, dk, dv, dtype, None)


def test_bwd_noalloc_validation(lib):
    """The allocation-free backward validates like gdn2_chunk_bwd, and a size whose workspace
    exceeds the library's array (64 MiB) is GDN2_ERR_WORKSPACE, all before any HIP call."""
    f = Fake(slots=18)
    assert bwd_noalloc(lib, f, q=None) == ERR_NULL
    assert bwd_noalloc(lib, f, B=0) == ERR_SHAPE
    assert bwd_noalloc(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    assert bwd_noalloc(lib, f, gq=f.p(9, 4)) == ERR_MISALIGNED
    assert gdn2.SCRATCH_BYTES == 64 << 20
    assert lib.gdn2_chunk_bwd_workspace_bytes(1, 640, 16, 128, 128) > gdn2.SCRATCH_BYTES
    assert lib.gdn2_chunk_bwd_workspace_bytes(1, 576, 16, 128, 128) <= gdn2.SCRATCH_BYTES
    assert bwd_noalloc(lib, f, T=640, H=16, dk=128, dv=128) == ERR_WORKSPACE


def test_chunk_logits_validation(lib):
    """The logits forward validates like gdn2_chunk_fwd, with bf16 inputs only and its decay
    logits counted in the input dtype (2 bytes an element) for the overlap checks."""
    f = Fake()
    for name in ("q", "k", "v", "a", "b", "w", "o"):
        assert chunk_logits(lib, f, **{name: None}) == ERR_NULL, name
    assert chunk_logits(lib, f, B=0) == ERR_SHAPE
    assert chunk_logits(lib, f, T=0) == ERR_SHAPE
    assert chunk_logits(lib, f, dtype=F32) == ERR_UNSUPPORTED
    assert chunk_logits(lib, f, dk=128, dv=128, dtype=F32) == ERR_UNSUPPORTED
    assert chunk_logits(lib, f, dk=96, dv=96) == ERR_UNSUPPORTED
    assert chunk_logits(lib, f, a=f.p(3, 2)) == ERR_MISALIGNED
    # decay logits [1,64,1,64] bf16 span 8,192 bytes: o at +4,096 overlaps them; o at +8,192
    # passes the overlap checks and then fails the workspace check (a short workspace), which
    # comes after them -- so no call here reaches the HIP runtime
    assert chunk_logits(lib, f, a=f.p(3), o=f.p(3, 4096)) == ERR_ALIAS
    assert chunk_logits(lib, f, a=f.p(3), o=f.p(3, 8192), ws=f.p(9), ws_bytes=16) == ERR_WORKSPACE


def test_mixer_prep_gate_pointers(lib):
    """Gates all absent (b, w, log_alpha NULL) is a valid request; some but not all absent is
    GDN2_ERR_NULL.  Checked on calls that fail validation (a misaligned q, or a NULL), so none
    reaches the HIP runtime."""
    f = Fake()
    P = f.p

    def prep(b, w, g, xb=P(3), xw=P(4), xa=P(5), q=P(9)):
        return lib.gdn2_mixer_prep(P(0), P(1), P(2), xb, xw, xa, P(6), P(7), P(8), q, P(10), P(11), b, w, g,
                                   1, 64, 1, 64, 64, ctypes.c_float(1e-6), BF16, None)

    assert prep(P(12), None, P(14)) == ERR_NULL
    assert prep(None, P(13), None) == ERR_NULL
    assert prep(P(12), P(13), P(14), xb=None) == ERR_NULL
    # all gates absent: xb, xw, xa are not needed; a misaligned q is still caught
    assert prep(None, None, None, xb=None, xw=None, xa=None, q=P(9, 2)) == ERR_MISALIGNED
    assert prep(None, None, None, q=P(9, 2)) == ERR_MISALIGNED
