"""fp64 CPU oracle of the Gated DeltaNet-2 recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library (``gated_delta_rule_gdn2_amd``)
and never imports it.

The arithmetic lives in ``gdn2_oracle.c`` (plain C, fp64, built with gcc, no
fast-math); this module only builds it, marshals numpy arrays and calls it.

What is computed is the recurrence of the page "Why NVIDIA Gated DeltaNet-2
separates erase and write gates" (axbrief.com), section "Gated Delta Rule-2:
channel-wise separation of erase and write", written as a sequential loop in
the residual form that the same section describes, with the read-out taken
after the update.

Layouts: q, k, b, log_alpha [B,T,H,dk]; v, w, o [B,T,H,dv]; state [B,H,dk,dv].

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (dense transition products, the KDA and Gated
DeltaNet reductions, exact retrieval, closed-form decay, gated linear attention,
linearity, resume, decode equivalence, finite differences for the VJP).  The
pages print no worked numerical example, so no pin is a value quoted from them.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB = os.path.join(_HERE, "libgdn2_oracle.so")
_lock = threading.Lock()
_lib = None
_override = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into ``oracle/libgdn2_oracle.so``.

    ``src``/``out`` let the tests build a deliberately altered copy of the
    source elsewhere (to show that the pins catch planted mistakes)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.gdn2_oracle_fwd.argtypes = [P] * 9 + [I64] * 5 + [ctypes.c_int]
    lib.gdn2_oracle_fwd.restype = ctypes.c_int
    lib.gdn2_oracle_decode.argtypes = [P] * 8 + [I64] * 4 + [ctypes.c_int]
    lib.gdn2_oracle_decode.restype = ctypes.c_int
    lib.gdn2_oracle_vjp.argtypes = [P] * 16 + [I64] * 5 + [ctypes.c_int]
    lib.gdn2_oracle_vjp.restype = ctypes.c_int
    lib.gdn2_oracle_version.restype = ctypes.c_char_p
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


@contextlib.contextmanager
def use_build(path: str):
    """Route the functions below to another build of the oracle (tests only)."""
    global _override
    prev = _override
    _override = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _override = prev


def _active():
    return _override if _override is not None else _load()


def default_threads() -> int:
    """Host threads for the pool: OMP_NUM_THREADS when set, else the CPU count, at most 64."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(os.cpu_count() or 1, 64))


def _f64(x, name):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU): exact upcast
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, log_alpha, b, w, initial_state=None, nthreads=None):
    """Sequential fp64 forward.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv])."""
    q, k, v, g, b, w = (_f64(x, n) for x, n in
                        zip((q, k, v, log_alpha, b, w), "q k v g b w".split()))
    s0 = _f64(initial_state, "s0")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for x, shp in ((k, (B, T, H, dk)), (b, (B, T, H, dk)), (g, (B, T, H, dk)),
                   (v, (B, T, H, dv)), (w, (B, T, H, dv))):
        if x.shape != shp:
            raise ValueError("oracle.fwd: shape mismatch %s vs %s" % (x.shape, shp))
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("oracle.fwd: initial_state shape %s" % (s0.shape,))
    o = np.zeros((B, T, H, dv))
    sT = np.zeros((B, H, dk, dv))
    rc = _active().gdn2_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(s0),
                                 _ptr(o), _ptr(sT), B, T, H, dk, dv,
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("gdn2_oracle_fwd failed: %d" % rc)
    return o, sT


def decode(q, k, v, log_alpha, b, w, state, nthreads=None):
    """One recurrent step for N sequences.  Returns (o [N,H,dv], new state)."""
    q, k, v, g, b, w = (_f64(x, n) for x, n in
                        zip((q, k, v, log_alpha, b, w), "q k v g b w".split()))
    st = _f64(state, "state").copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if st.shape != (N, H, dk, dv):
        raise ValueError("oracle.decode: state shape %s" % (st.shape,))
    o = np.zeros((N, H, dv))
    rc = _active().gdn2_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                    _ptr(st), _ptr(o), N, H, dk, dv,
                                    nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("gdn2_oracle_decode failed: %d" % rc)
    return o, st


def vjp(q, k, v, log_alpha, b, w, d_o, initial_state=None, d_final_state=None, nthreads=None):
    """Gradients of sum(d_o*o) + sum(d_final_state*S_T).

    Returns dict with dq, dk, dv, dlog_alpha, db, dw, ds0."""
    q, k, v, g, b, w, do = (_f64(x, n) for x, n in
                            zip((q, k, v, log_alpha, b, w, d_o), "q k v g b w do".split()))
    s0 = _f64(initial_state, "s0")
    dsT = _f64(d_final_state, "dsT")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {n: np.zeros(x.shape) for n, x in
           (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", g), ("db", b), ("dw", w))}
    out["ds0"] = np.zeros((B, H, dk, dv))
    rc = _active().gdn2_oracle_vjp(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(s0),
                                 _ptr(do), _ptr(dsT), _ptr(out["dq"]), _ptr(out["dk"]),
                                 _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]),
                                 _ptr(out["dw"]), _ptr(out["ds0"]), B, T, H, dk, dv,
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("gdn2_oracle_vjp failed: %d" % rc)
    return out


def version() -> str:
    return _active().gdn2_oracle_version().decode()


# the mixer around the recurrence (numpy, fp64): see oracle/mixer.py
from .mixer import mixer_out, mixer_prep  # noqa: E402,F401
