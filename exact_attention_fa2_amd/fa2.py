"""ctypes binding of libfa2.so (include/fa2.h).

Marshalling only: tensors are turned into device pointers and the current
torch stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")
POLYEXP_LIB_PATH = os.path.join(_PKG, "libfa2_polyexp.so")  # measurement build (polynomial exp2)

FA2_F32, FA2_F16, FA2_BF16 = 0, 1, 2
STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "unsupported configuration",
          4: "pointer not 16-byte aligned", 5: "kernel launch failed",
          6: "no usable gfx950 device"}

EXPORTS = ("attn_fwd", "attn_fwd_ws", "attn_fwd_noalloc", "attn_fwd_workspace_size", "attn_bwd",
           "attn_decode_split", "attn_decode_combine", "attn_decode_default_splits",
           "fa2_time_next_launch", "fa2_status_string")
NOALLOC_SCRATCH_BYTES = 32 << 20  # FA2_NOALLOC_SCRATCH_BYTES in include/fa2.h

_lib = None


class FA2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, STATUS.get(status, "?"), status))


def lib():
    """Load libfa2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path):
    """A ctypes handle on one build of the library (libfa2.so, or a
    measurement build beside it such as libfa2_polyexp.so), with the
    signatures of include/fa2.h.  Raises if it has not been built."""
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (%s); run `python -m exact_attention_fa2_amd.build`"
                           % (os.path.basename(path), path))
    # torch first: it brings its own HIP runtime and asks for it by another
    # file name than the library does, so a library loaded before torch would
    # pull in the system runtime as a second copy, whose device state the
    # tensors' runtime does not share (hipGetDevice then reports no device).
    # Loaded after torch, the library binds to torch's runtime by its soname.
    _torch()
    L = ctypes.CDLL(path)
    vp, fp, i, f = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_ws.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
    L.attn_fwd_ws.restype = i
    L.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_noalloc.restype = i
    L.attn_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    L.attn_fwd_workspace_size.restype = ctypes.c_size_t
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, fp, vp, vp, vp, fp, i, i, i, i, i, f, i, i, vp]
    L.attn_bwd.restype = i
    L.attn_decode_split.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, f, i, i, vp]
    L.attn_decode_split.restype = i
    L.attn_decode_combine.argtypes = [fp, fp, fp, vp, i, i, i, i, i, vp]
    L.attn_decode_combine.restype = i
    L.attn_decode_default_splits.argtypes = [i, i, i, i]
    L.attn_decode_default_splits.restype = i
    L.fa2_time_next_launch.argtypes = [vp, vp]
    L.fa2_time_next_launch.restype = i
    L.fa2_status_string.argtypes = [i]
    L.fa2_status_string.restype = ctypes.c_char_p
    return L


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: FA2_F32, torch.float16: FA2_F16, torch.bfloat16: FA2_BF16}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _alloc(stream, *args, like=None, **kw):
    """A tensor the binding allocates for a call on ``stream``.  torch's
    caching allocator ties a new tensor to the current stream; when the
    kernels run on another stream, the tensor is also recorded on that one,
    so its memory is not handed out again before the kernels are done with
    it (this matters for the ones dropped at the end of the call)."""
    torch = _torch()
    t = torch.empty_like(like) if like is not None else torch.empty(*args, **kw)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _check(fn, status):
    if status != 0:
        raise FA2Error(fn, status)


def _validate(ref, specs):
    """Every tensor the library reads or writes through a raw pointer: the
    exact shape and dtype, contiguous, and on the same GPU as ``ref`` (the
    library cannot see buffer sizes, so a short buffer would be overrun).
    ``specs`` holds (tensor, name, shape, dtype); shape None checks only the
    rest (a byte workspace)."""
    # (cheap attribute checks first: these run on every call)
    for t, name, shape, dtype in specs:
        if shape is not None and t.shape != shape:
            raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
        if dtype is not None and t.dtype != dtype:
            raise TypeError("%s must be %s, not %s" % (name, dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    dev = ref.get_device()  # -1 on the host
    if dev < 0:
        raise ValueError("tensors must be on a GPU, not %s" % ref.device)
    for t, name, _, _ in specs:
        if t.get_device() != dev:
            raise ValueError("%s must be on %s, not %s" % (name, ref.device, t.device))


def _dims(t, n, name):
    if t.dim() != n:
        raise ValueError("%s must have %d dimensions, not %d" % (name, n, t.dim()))
    return tuple(t.shape)


def workspace_size(B, H, Nq, Nk, D, causal, dtype_code_) -> int:
    return int(lib().attn_fwd_workspace_size(B, H, Nq, Nk, D, int(bool(causal)), dtype_code_))


def attn_fwd(q, k, v, scale=None, causal=False, return_lse=False, out=None, lse=None,
             stream=None, workspace=None, use_workspace=True):
    """Exact attention forward.  q [B,H,Nq,D], k/v [B,H,Nk,D] (same dtype).

    When the library asks for a workspace for this shape (few query tiles: it
    then splits the keys across workgroups), one is taken from ``workspace``
    if given and large enough, else allocated with torch for this call.
    ``use_workspace=False`` calls the plain attn_fwd entry point instead.
    Returns o (and lse [B,H,Nq] float32 when ``return_lse``)."""
    torch = _torch()
    B, H, Nq, D = _dims(q, 4, "q")
    Nk = _dims(k, 4, "k")[2]
    # buffers the binding allocates below are right by construction; the
    # caller's are checked with the inputs
    specs = [(q, "q", None, None), (k, "k", (B, H, Nk, D), q.dtype), (v, "v", (B, H, Nk, D), q.dtype)]
    if out is not None:
        specs.append((out, "out", q.shape, q.dtype))
    if return_lse and lse is not None:
        specs.append((lse, "lse", (B, H, Nq), torch.float32))
    _validate(q, specs)
    dc = dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = _alloc(stream, like=q)
    if return_lse and lse is None:
        lse = _alloc(stream, (B, H, Nq), dtype=torch.float32, device=q.device)
    if not use_workspace:
        st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                            _ptr(lse if return_lse else None), B, H, Nq, Nk, D, float(scale),
                            int(bool(causal)), dc, _stream(stream))
        _check("attn_fwd", st)
        return (out, lse) if return_lse else out
    need = workspace_size(B, H, Nq, Nk, D, causal, dc)
    if need and workspace is not None:
        _validate(q, [(workspace, "workspace", None, None)])
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _alloc(stream, need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    st = lib().attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse if return_lse else None),
                           B, H, Nq, Nk, D, float(scale), int(bool(causal)), dc, ws_ptr, ws_bytes,
                           _stream(stream))
    _check("attn_fwd", st)
    return (out, lse) if return_lse else out


def attn_fwd_noalloc(q, k, v, out, scale=None, causal=False, lse=None, stream=None):
    """attn_fwd through the entry point that allocates nothing (its key-split
    workspace is the library's own device array).  The caller passes ``out``
    [B,H,Nq,D] and, to get the LSE, ``lse`` [B,H,Nq] float32; nothing is
    allocated here either.  Calls that overlap in time on one device race on
    that array.  Returns ``out`` (and ``lse`` when given)."""
    torch = _torch()
    B, H, Nq, D = _dims(q, 4, "q")
    Nk = _dims(k, 4, "k")[2]
    specs = [(q, "q", None, None), (k, "k", (B, H, Nk, D), q.dtype), (v, "v", (B, H, Nk, D), q.dtype),
             (out, "out", q.shape, q.dtype)]
    if lse is not None:
        specs.append((lse, "lse", (B, H, Nq), torch.float32))
    _validate(q, specs)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = lib().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D,
                                float(scale), int(bool(causal)), dtype_code(q), _stream(stream))
    _check("attn_fwd_noalloc", st)
    return out if lse is None else (out, lse)


def attn_bwd(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
             delta=None, stream=None):
    """Exact attention backward.  q/o/dout [B,H,Nq,D], k/v [B,H,Nk,D] (same
    dtype), lse [B,H,Nq] float32 from attn_fwd.  Returns (dq, dk, dv, delta)
    with delta [B,H,Nq] float32 = rowsum(dout * o)."""
    torch = _torch()
    B, H, Nq, D = _dims(q, 4, "q")
    Nk = _dims(k, 4, "k")[2]
    qs, ks, f32 = (B, H, Nq, D), (B, H, Nk, D), torch.float32
    specs = [(q, "q", None, None), (k, "k", ks, q.dtype), (v, "v", ks, q.dtype),
             (o, "o", qs, q.dtype), (dout, "dout", qs, q.dtype), (lse, "lse", (B, H, Nq), f32)]
    for t, name, shape, dtype in ((dq, "dq", qs, q.dtype), (dk, "dk", ks, q.dtype),
                                  (dv, "dv", ks, q.dtype), (delta, "delta", (B, H, Nq), f32)):
        if t is not None:
            specs.append((t, name, shape, dtype))
    _validate(q, specs)
    dc = dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = _alloc(stream, like=q) if dq is None else dq
    dk = _alloc(stream, like=k) if dk is None else dk
    dv = _alloc(stream, like=v) if dv is None else dv
    if delta is None:
        delta = _alloc(stream, (B, H, Nq), dtype=f32, device=q.device)
    st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(delta), B, H, Nq, Nk, D, float(scale),
                        int(bool(causal)), dc, _stream(stream))
    _check("attn_bwd", st)
    return dq, dk, dv, delta


def attn_decode_split(q, k, v, scale, n_splits, o_part=None, m_part=None, l_part=None,
                      stream=None):
    """Flash-decoding partials.  q [B,H,D], k/v [B,H,N,D]."""
    torch = _torch()
    B, H, D = _dims(q, 3, "q")
    N = _dims(k, 4, "k")[2]
    n_splits = int(n_splits)
    if n_splits < 1:
        raise ValueError("n_splits must be at least 1")
    f32 = torch.float32
    specs = [(q, "q", None, None), (k, "k", (B, H, N, D), q.dtype), (v, "v", (B, H, N, D), q.dtype)]
    for t, name, shape in ((o_part, "o_part", (B, H, n_splits, D)),
                           (m_part, "m_part", (B, H, n_splits)), (l_part, "l_part", (B, H, n_splits))):
        if t is not None:
            specs.append((t, name, shape, f32))
    _validate(q, specs)
    dc = dtype_code(q)
    if o_part is None:
        o_part = _alloc(stream, (B, H, n_splits, D), dtype=torch.float32, device=q.device)
    if m_part is None:
        m_part = _alloc(stream, (B, H, n_splits), dtype=torch.float32, device=q.device)
    if l_part is None:
        l_part = _alloc(stream, (B, H, n_splits), dtype=torch.float32, device=q.device)
    st = lib().attn_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(m_part),
                                 _ptr(l_part), B, H, N, D, float(scale), n_splits, dc,
                                 _stream(stream))
    _check("attn_decode_split", st)
    return o_part, m_part, l_part


def attn_decode_combine(o_part, m_part, l_part, dtype, out=None, stream=None):
    """Merge partials into o [B,H,D] of ``dtype``."""
    torch = _torch()
    B, H, S, D = _dims(o_part, 4, "o_part")
    f32 = torch.float32
    specs = [(o_part, "o_part", None, f32), (m_part, "m_part", (B, H, S), f32),
             (l_part, "l_part", (B, H, S), f32)]
    if out is not None:
        specs.append((out, "out", (B, H, D), dtype))
    _validate(o_part, specs)
    if out is None:
        out = _alloc(stream, (B, H, D), dtype=dtype, device=o_part.device)
    st = lib().attn_decode_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(out), B, H,
                                   D, S, dtype_code(out), _stream(stream))
    _check("attn_decode_combine", st)
    return out


def default_splits(B, H, N, D) -> int:
    return int(lib().attn_decode_default_splits(B, H, N, D))


def attn_decode(q, k, v, scale=None, n_splits=None, stream=None):
    """Split + combine.  q [B,H,D], k/v [B,H,N,D]; returns o [B,H,D]."""
    B, H, D = _dims(q, 3, "q")
    N = _dims(k, 4, "k")[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if n_splits is None:
        n_splits = default_splits(B, H, N, D)
    parts = attn_decode_split(q, k, v, scale, n_splits, stream=stream)
    return attn_decode_combine(*parts, dtype=q.dtype, stream=stream)


def time_next_launch(start, stop):
    """The next kernel this thread enqueues through the library records the
    torch.cuda.Event ``start`` and ``stop`` (enable_timing=True) from its own
    dispatch: ``start.elapsed_time(stop)`` is then that kernel's execution
    alone.  Either may be None."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:  # torch creates the event on its first record
            ev.record()
        return ctypes.c_void_p(ev.cuda_event)
    _check("fa2_time_next_launch", lib().fa2_time_next_launch(handle(start), handle(stop)))


def status_string(code: int) -> str:
    return lib().fa2_status_string(int(code)).decode()
