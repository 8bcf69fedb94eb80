"""Gated DeltaNet-2 recurrence on AMD MI355X (gfx950): Python binding.

This module only marshals arguments to the C ABI of ``libgdn2.so``
(``include/gdn2.h``): it checks tensor dtypes, shapes, devices and contiguity,
allocates outputs with PyTorch (device memory and streams are all PyTorch is
used for) and passes raw pointers plus the current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.

    o, S_T = chunk_fwd(q, k, v, log_alpha, b, w, initial_state=None)
    o, S_T = chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens)  # packed sequences
    o      = decode_step(q, k, v, log_alpha, b, w, state)   # state updated in place
    grads  = chunk_bwd(q, k, v, log_alpha, b, w, d_o, initial_state=None, d_final_state=None)
    ins    = mixer_prep(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v)  # q, k, v, b, w, log_alpha
    y      = mixer_out(o, z, gamma)                            # RMS norm and SiLU output gate

Layouts: q, k, b, log_alpha [B,T,H,dk]; v, w, o [B,T,H,dv]; state [B,H,dk,dv]
(packed: [total_T,H,d] with int64 offsets cu_seqlens [N+1] and states [N,H,dk,dv];
decode: [N,H,d] and the same states).  q, k, v, b, w are bf16 or fp32 (all the same);
log_alpha and the state are fp32.  o is fp32 by default (the fp32 accumulation
carried to the output); ``out_dtype=`` the input dtype rounds it on the store.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["chunk_fwd", "chunk_fwd_logits", "chunk_fwd_workspace_bytes", "chunk_fwd_varlen", "chunk_bwd", "chunk_bwd_workspace_bytes",
           "chunk_bwd_noalloc", "SCRATCH_BYTES", "decode_step", "mixer_prep",
           "mixer_out", "supported", "version", "library_path", "Gdn2Error", "CHUNK"]

CHUNK = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn2.so")
_lock = threading.Lock()
_lib = None

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_STATUS = {0: "GDN2_OK", 1: "GDN2_ERR_NULL", 2: "GDN2_ERR_SHAPE", 3: "GDN2_ERR_UNSUPPORTED",
           4: "GDN2_ERR_MISALIGNED", 5: "GDN2_ERR_ALIAS", 6: "GDN2_ERR_WORKSPACE", 7: "GDN2_ERR_HIP"}


class Gdn2Error(RuntimeError):
    def __init__(self, call, status, message):
        super().__init__("%s failed: %s (%s)" % (call, _STATUS.get(status, status), message))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                "libgdn2.so is not built (expected at %s); run "
                "`python -m gated_delta_rule_gdn2_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.gdn2_chunk_fwd.argtypes = [P] * 9 + [I64] * 5 + [I32, I32, P, ctypes.c_size_t, P]
        lib.gdn2_chunk_fwd.restype = I32
        lib.gdn2_chunk_fwd_logits.argtypes = [P] * 9 + [I64] * 5 + [I32, I32, P, ctypes.c_size_t, P]
        lib.gdn2_chunk_fwd_logits.restype = I32
        lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [I64] * 5 + [I32]
        lib.gdn2_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_fwd_split_workspace_bytes.argtypes = [I64] * 5 + [I32]
        lib.gdn2_chunk_fwd_split_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_fwd_varlen.argtypes = [P] * 10 + [I64] * 5 + [I32, I32, P]
        lib.gdn2_chunk_fwd_varlen.restype = I32
        lib.gdn2_decode_step.argtypes = [P] * 8 + [I64] * 4 + [I32, I32, P]
        lib.gdn2_decode_step.restype = I32
        lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [I64] * 5
        lib.gdn2_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_bwd.argtypes = [P] * 17 + [ctypes.c_size_t] + [I64] * 5 + [I32, P]
        lib.gdn2_chunk_bwd.restype = I32
        lib.gdn2_chunk_bwd_noalloc.argtypes = [P] * 16 + [I64] * 5 + [I32, P]
        lib.gdn2_chunk_bwd_noalloc.restype = I32
        lib.gdn2_mixer_prep.argtypes = [P] * 15 + [I64] * 5 + [ctypes.c_float, I32, P]
        lib.gdn2_mixer_prep.restype = I32
        lib.gdn2_mixer_out.argtypes = [P] * 4 + [I64] * 4 + [ctypes.c_float, I32, I32, P]
        lib.gdn2_mixer_out.restype = I32
        lib.gdn2_supported.argtypes = [I32, I64, I64, I32]
        lib.gdn2_supported.restype = I32
        lib.gdn2_status_string.argtypes = [I32]
        lib.gdn2_status_string.restype = ctypes.c_char_p
        lib.gdn2_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def version() -> str:
    return _load().gdn2_version().decode()


def supported(which: str, dk: int, dv: int, dtype: torch.dtype) -> bool:
    w = {"chunk_fwd": 0, "decode_step": 1, "chunk_bwd": 2, "mixer": 3}[which]
    return bool(_load().gdn2_supported(w, dk, dv, _DTYPES[dtype]))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd(q, k, v, log_alpha, b, w, initial_state=None, *, o=None, final_state=None,
              output_final_state=True, out_dtype=torch.float32, workspace=None, fused=None):
    """Chunk-parallel forward.  Returns (o, S_T); S_T is None when
    ``output_final_state`` is False.  ``final_state`` may be passed (and may be
    ``initial_state`` itself, for an in-place update).  ``fused=None`` runs the
    form the library reports faster for the shape (chunk_fwd_workspace_bytes);
    ``fused=True`` the single fused kernel; ``fused=False`` the two-kernel form
    where it exists (bf16, d = 64 or 128).  The two-kernel form's workspace is
    allocated here unless ``workspace`` (uint8) is passed."""
    return _chunk_fwd_call("gdn2_chunk_fwd", q, k, v, log_alpha, torch.float32, b, w, initial_state, o,
                           final_state, output_final_state, out_dtype, workspace, fused)


def chunk_fwd_logits(q, k, v, a_logit, b_logit, w_logit, initial_state=None, *, o=None, final_state=None,
                     output_final_state=True, out_dtype=torch.float32, workspace=None, fused=None):
    """chunk_fwd from the projections' outputs: the kernels form alpha = sigmoid(a_logit),
    b = sigmoid(b_logit) and w = sigmoid(w_logit) on load.  a_logit, b_logit [B,T,H,dk] and
    w_logit [B,T,H,dv] in the inputs' dtype (bf16 only).  Everything else as chunk_fwd."""
    return _chunk_fwd_call("gdn2_chunk_fwd_logits", q, k, v, a_logit, q.dtype, b_logit, w_logit, initial_state,
                           o, final_state, output_final_state, out_dtype, workspace, fused)


def _chunk_fwd_call(fn, q, k, v, decay, decay_dtype, b, w, initial_state, o, final_state,
                    output_final_state, out_dtype, workspace, fused):
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("%s runs on the GPU; got tensors on %s" % (fn, dev))
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q dtype must be float32 or bfloat16")
    decay_name = "log_alpha" if fn == "gdn2_chunk_fwd" else "a_logit"
    for name, t, shp, tdt in (("k", k, (B, T, H, dk), dt), ("v", v, (B, T, H, dv), dt),
                              (decay_name, decay, (B, T, H, dk), decay_dtype),
                              ("b", b, (B, T, H, dk), dt), ("w", w, (B, T, H, dv), dt),
                              ("q", q, (B, T, H, dk), dt)):
        _check(name, t, shp, tdt, dev)
    if initial_state is not None:
        _check("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    if out_dtype not in (torch.float32, dt):
        raise TypeError("out_dtype must be float32 or the input dtype")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _check("o", o, (B, T, H, dv), out_dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check("final_state", final_state, (B, H, dk, dv), torch.float32, dev)
    if fused is None:
        ws_bytes = _load().gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, _DTYPES[dt])
    else:
        ws_bytes = 0 if fused else _load().gdn2_chunk_fwd_split_workspace_bytes(B, T, H, dk, dv, _DTYPES[dt])
    ws = None
    if ws_bytes:
        if workspace is None:
            workspace = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
        elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
        off = (-workspace.data_ptr()) % 256  # 256-byte alignment
        ws = workspace[off:]
        if ws.numel() < ws_bytes:
            raise ValueError("workspace holds %d bytes, %d needed" % (ws.numel(), ws_bytes))
    st = getattr(_load(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(b), _ptr(w),
                              _ptr(initial_state), _ptr(o), _ptr(final_state), B, T, H, dk, dv,
                              _DTYPES[dt], _DTYPES[out_dtype], _ptr(ws), ws.numel() if ws is not None else 0,
                              _stream_handle(dev))
    if st != 0:
        raise Gdn2Error(fn, st, _load().gdn2_status_string(st).decode())
    return o, final_state


def chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, initial_state=None, *, o=None,
                     final_state=None, output_final_state=True, out_dtype=torch.float32):
    """Forward over N sequences packed along the token axis: q, k, b, log_alpha
    [total_T,H,dk], v, w [total_T,H,dv], cu_seqlens int64 [N+1] on the device
    (sequence n is tokens cu_seqlens[n]:cu_seqlens[n+1]).  Returns (o, S_T) with
    S_T [N,H,dk,dv], the layout decode_step continues from."""
    if q.dim() != 3:
        raise ValueError("q must be [total_T,H,dk]")
    total_T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_varlen runs on the GPU; got tensors on %s" % dev)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q dtype must be float32 or bfloat16")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    for name, t, shp, tdt in (("k", k, (total_T, H, dk), dt), ("v", v, (total_T, H, dv), dt),
                              ("log_alpha", log_alpha, (total_T, H, dk), torch.float32),
                              ("b", b, (total_T, H, dk), dt), ("w", w, (total_T, H, dv), dt),
                              ("q", q, (total_T, H, dk), dt),
                              ("cu_seqlens", cu_seqlens, (N + 1,), torch.int64)):
        _check(name, t, shp, tdt, dev)
    if initial_state is not None:
        _check("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if out_dtype not in (torch.float32, dt):
        raise TypeError("out_dtype must be float32 or the input dtype")
    if o is None:
        o = torch.empty((total_T, H, dv), dtype=out_dtype, device=dev)
    else:
        _check("o", o, (total_T, H, dv), out_dtype, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    st = _load().gdn2_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                       _ptr(initial_state), _ptr(o), _ptr(final_state),
                                       _ptr(cu_seqlens), N, total_T, H, dk, dv, _DTYPES[dt],
                                       _DTYPES[out_dtype], _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd_varlen", st, _load().gdn2_status_string(st).decode())
    return o, final_state


def decode_step(q, k, v, log_alpha, b, w, state, *, o=None, out_dtype=torch.float32):
    """One recurrent step; ``state`` [N,H,dk,dv] fp32 is updated in place.  Returns o."""
    if q.dim() != 3:
        raise ValueError("q must be [N,H,dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step runs on the GPU; got tensors on %s" % dev)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q dtype must be float32 or bfloat16")
    for name, t, shp, tdt in (("k", k, (N, H, dk), dt), ("v", v, (N, H, dv), dt),
                              ("log_alpha", log_alpha, (N, H, dk), torch.float32),
                              ("b", b, (N, H, dk), dt), ("w", w, (N, H, dv), dt),
                              ("state", state, (N, H, dk, dv), torch.float32),
                              ("q", q, (N, H, dk), dt)):
        _check(name, t, shp, tdt, dev)
    if out_dtype not in (torch.float32, dt):
        raise TypeError("out_dtype must be float32 or the input dtype")
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _check("o", o, (N, H, dv), out_dtype, dev)
    st = _load().gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                  _ptr(state), _ptr(o), N, H, dk, dv, _DTYPES[dt],
                                  _DTYPES[out_dtype], _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_decode_step", st, _load().gdn2_status_string(st).decode())
    return o


def chunk_fwd_workspace_bytes(B, T, H, dk, dv, dtype=torch.bfloat16, split=False) -> int:
    """Device workspace (bytes) of chunk_fwd's faster form for these sizes (0: the fused kernel);
    with ``split=True``, that of the two-kernel form whichever is faster (0 where it does not exist)."""
    f = _load().gdn2_chunk_fwd_split_workspace_bytes if split else _load().gdn2_chunk_fwd_workspace_bytes
    return int(f(B, T, H, dk, dv, _DTYPES[dtype]))


def chunk_bwd_workspace_bytes(B, T, H, dk, dv) -> int:
    """Device workspace (bytes) that chunk_bwd needs for these sizes."""
    return int(_load().gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv))


def _bwd_outputs(q, k, v, log_alpha, b, w, d_o, initial_state, d_final_state, grads,
                 want_initial_state_grad, name):
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("%s runs on the GPU; got tensors on %s" % (name, dev))
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError("q dtype must be float32 or bfloat16")
    for nm, t, shp, tdt in (("k", k, (B, T, H, dk), dt), ("v", v, (B, T, H, dv), dt),
                            ("log_alpha", log_alpha, (B, T, H, dk), torch.float32),
                            ("b", b, (B, T, H, dk), dt), ("w", w, (B, T, H, dv), dt),
                            ("q", q, (B, T, H, dk), dt), ("d_o", d_o, (B, T, H, dv), torch.float32)):
        _check(nm, t, shp, tdt, dev)
    for nm, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(nm, t, (B, H, dk, dv), torch.float32, dev)
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dlog_alpha": (B, T, H, dk),
              "db": (B, T, H, dk), "dw": (B, T, H, dv), "d_initial_state": (B, H, dk, dv)}
    out = dict(grads) if grads is not None else {}
    for nm, shp in shapes.items():
        if nm == "d_initial_state" and not want_initial_state_grad:
            out[nm] = None
            continue
        if out.get(nm) is None:
            out[nm] = torch.empty(shp, dtype=torch.float32, device=dev)
        else:
            _check(nm, out[nm], shp, torch.float32, dev)
    return (B, T, H, dk, dv, dev, dt), out


def _bwd_ptrs(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, out):
    return [_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(initial_state), _ptr(d_o),
            _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
            _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["d_initial_state"])]


def chunk_bwd(q, k, v, log_alpha, b, w, d_o, initial_state=None, d_final_state=None, *, workspace=None,
              grads=None, want_initial_state_grad=True):
    """Gradients of sum(d_o * o) + sum(d_final_state * S_T) for the forward chunk_fwd(q, k, v,
    log_alpha, b, w, initial_state).  d_o [B,T,H,dv] and d_final_state [B,H,dk,dv] are fp32.
    Returns a dict of fp32 tensors dq, dk, dv, dlog_alpha, db, dw and d_initial_state (None
    when not requested).  ``workspace`` (uint8, at least chunk_bwd_workspace_bytes) and
    ``grads`` (a dict of preallocated outputs) may be passed to avoid allocations."""
    (B, T, H, dk, dv, dev, dt), out = _bwd_outputs(q, k, v, log_alpha, b, w, d_o, initial_state, d_final_state,
                                                   grads, want_initial_state_grad, "chunk_bwd")
    need = chunk_bwd_workspace_bytes(B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    st = _load().gdn2_chunk_bwd(*_bwd_ptrs(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, out),
                                _ptr(workspace), workspace.numel(), B, T, H, dk, dv, _DTYPES[dt],
                                _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_bwd", st, _load().gdn2_status_string(st).decode())
    return out


SCRATCH_BYTES = 64 << 20  # GDN2_SCRATCH_BYTES of include/gdn2.h


def chunk_bwd_noalloc(q, k, v, log_alpha, b, w, d_o, initial_state=None, d_final_state=None, *, grads,
                      want_initial_state_grad=True):
    """chunk_bwd through gdn2_chunk_bwd_noalloc: the library's fixed device array serves as the
    workspace, so with ``grads`` preallocated nothing is allocated (for capture into a HIP
    graph, say).  Sizes whose workspace exceeds SCRATCH_BYTES raise Gdn2Error
    (GDN2_ERR_WORKSPACE).  Calls that may overlap on one GPU race on the array."""
    (B, T, H, dk, dv, dev, dt), out = _bwd_outputs(q, k, v, log_alpha, b, w, d_o, initial_state, d_final_state,
                                                   grads, want_initial_state_grad, "chunk_bwd_noalloc")
    st = _load().gdn2_chunk_bwd_noalloc(*_bwd_ptrs(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state,
                                                   out), B, T, H, dk, dv, _DTYPES[dt], _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_bwd_noalloc", st, _load().gdn2_status_string(st).decode())
    return out


def mixer_prep(xq, xk, xv, xb, xw, xa, conv_q, conv_k, conv_v, eps=1e-6, *, out=None, gates=True):
    """The recurrence's inputs from the layer's projection outputs, in one pass:
    q, k = L2(SiLU(conv(xq, xk))), v = SiLU(conv(xv)), b, w = sigmoid(xb, xw),
    log_alpha = log sigmoid(xa).  x* [B,T,H,d] in one dtype (bf16 or fp32); conv_* [H*d, 4]
    fp32 causal depthwise taps.  Returns a dict q, k, v, b, w (input dtype) and log_alpha
    (fp32); ``out`` may hold preallocated outputs.  ``gates=False`` forms q, k and v only
    (xb, xw, xa may be None): for chunk_fwd_logits, which activates the gates itself."""
    if xq.dim() != 4:
        raise ValueError("xq must be [B,T,H,dk]")
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    dev = xq.device
    if dev.type != "cuda":
        raise ValueError("mixer_prep runs on the GPU; got tensors on %s" % dev)
    dt = xq.dtype
    if dt not in _DTYPES:
        raise TypeError("xq dtype must be float32 or bfloat16")
    checks = [("xk", xk, (B, T, H, dk), dt), ("xv", xv, (B, T, H, dv), dt), ("xq", xq, (B, T, H, dk), dt),
              ("conv_q", conv_q, (H * dk, 4), torch.float32), ("conv_k", conv_k, (H * dk, 4), torch.float32),
              ("conv_v", conv_v, (H * dv, 4), torch.float32)]
    if gates:
        checks += [("xb", xb, (B, T, H, dk), dt), ("xw", xw, (B, T, H, dv), dt), ("xa", xa, (B, T, H, dk), dt)]
    else:
        xb = xw = xa = None
    for name, t, shp, tdt in checks:
        _check(name, t, shp, tdt, dev)
    shapes = {"q": ((B, T, H, dk), dt), "k": ((B, T, H, dk), dt), "v": ((B, T, H, dv), dt)}
    if gates:
        shapes.update({"b": ((B, T, H, dk), dt), "w": ((B, T, H, dv), dt),
                       "log_alpha": ((B, T, H, dk), torch.float32)})
    res = {n: t for n, t in (dict(out) if out is not None else {}).items() if n in shapes}
    for name, (shp, tdt) in shapes.items():
        if res.get(name) is None:
            res[name] = torch.empty(shp, dtype=tdt, device=dev)
        else:
            _check(name, res[name], shp, tdt, dev)
    st = _load().gdn2_mixer_prep(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(xb), _ptr(xw), _ptr(xa), _ptr(conv_q),
                                 _ptr(conv_k), _ptr(conv_v), _ptr(res["q"]), _ptr(res["k"]), _ptr(res["v"]),
                                 _ptr(res.get("b")), _ptr(res.get("w")), _ptr(res.get("log_alpha")), B, T, H,
                                 dk, dv, float(eps), _DTYPES[dt], _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_mixer_prep", st, _load().gdn2_status_string(st).decode())
    return res


def mixer_out(o, z, gamma, eps=1e-6, *, y=None):
    """Layer output y = o / sqrt(mean(o^2) + eps) * gamma * SiLU(z) (mean over dv), in one
    pass.  o [B,T,H,dv] fp32 or z's dtype; z [B,T,H,dv] bf16 or fp32; gamma [dv] fp32.
    Returns y in z's dtype."""
    if o.dim() != 4:
        raise ValueError("o must be [B,T,H,dv]")
    B, T, H, dv = o.shape
    dev = o.device
    if dev.type != "cuda":
        raise ValueError("mixer_out runs on the GPU; got tensors on %s" % dev)
    dt = z.dtype
    if dt not in _DTYPES:
        raise TypeError("z dtype must be float32 or bfloat16")
    if o.dtype not in (torch.float32, dt):
        raise TypeError("o must be float32 or z's dtype")
    _check("o", o, (B, T, H, dv), o.dtype, dev)
    _check("z", z, (B, T, H, dv), dt, dev)
    _check("gamma", gamma, (dv,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check("y", y, (B, T, H, dv), dt, dev)
    st = _load().gdn2_mixer_out(_ptr(o), _ptr(z), _ptr(gamma), _ptr(y), B, T, H, dv, float(eps), _DTYPES[dt],
                                _DTYPES[o.dtype], _stream_handle(dev))
    if st != 0:
        raise Gdn2Error("gdn2_mixer_out", st, _load().gdn2_status_string(st).decode())
    return y
