"""fp64 CPU oracle for exact attention and flash-decoding -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library in
``exact_attention_fa2_amd`` and never imports it; the two meet only through the
seeded inputs of ``exact_attention_fa2_amd.inputs`` (which hold none of the
method's arithmetic).

Contents
  * ``attn_rows`` / ``attn``   -- the plain definition O = softmax(scale Q K^T) V
    and LSE = m + ln l, in fp64 C loops (``oracle.c``).  Source: "Flash
    attention, f32" (opening paragraph); "Flash Attention", Definition 1,
    Proposition 1 and section FlashAttention 2 (log-sum-exp statistic);
    "06: Fused attention", attn_fwd (causal keeps key j <= query i).
  * ``decode_split`` / ``decode_combine`` -- flash-decoding partials and their
    merge, "Flash decoding", Overview of the algorithm (split and combine
    equations), with the scale inside the score as the page's split kernel has it.
  * ``attn_bwd`` -- the gradients dQ, dK, dV of O = softmax(scale Q K^T) V for an
    upstream dO, and D = rowsum(dO o O), from the plain chain rule in fp64
    ("Flash Attention", section IO complexity, the backward pass: D_i and
    dS = P o (dP - D_i); "06: Fused attention", the backward kernels).
  * ``brute`` -- a pure-Python brute force for tiny inputs (no max subtraction).
  * ``recurrence`` -- the tiled online-softmax recurrence in fp64, used only to
    show that the recurrence equals the batched definition.

Pins (tests/test_oracle.py, ``-m "not gpu"``): brute force, closed forms
(V = I rows sum to 1, K = 0 gives the mean of V, one key gives V_0), shift
invariance with shifts far past exp's f32 overflow, key-permutation invariance,
convex-hull bounds, the tiled recurrence for many block sizes, the (m, l) monoid
under random groupings, split-then-combine = unsplit, hand-derived golden cases
in tests/golden/, and torch's CPU float64 attention as a library cross-check.
Backward: central finite differences of the forward definition, closed forms
(constant V rows give dQ = dK = 0; K = 0 gives dV = column means of dO), and
torch's CPU float64 autograd.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with the host compiler (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes view of one build of ``oracle.c`` (the default one, or a copy
    that a test compiled with a planted mistake)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        llp = ctypes.POINTER(ctypes.c_longlong)
        lib.oracle_attn_rows.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         ctypes.c_int, llp, ctypes.c_longlong, dp, dp,
                                         ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_decode_split.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                            dp, dp, dp]
        lib.oracle_decode_split.restype = ctypes.c_int
        lib.oracle_decode_combine.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, dp]
        lib.oracle_decode_combine.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                        llp, ctypes.c_longlong, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        self.lib = lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = Oracle(_LIB).lib
    return _lib


def compile_variant(source_text: str, out_path: str) -> "Oracle":
    """Compile an edited copy of oracle.c (used by the mutation pins only)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", out_path, src, "-lm"])
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float64:
        raise TypeError("oracle inputs must already be promoted to float64, got %s" % a.dtype)
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def attn_rows(q, k, v, scale: float, causal: bool = False, rows=None, nthreads: int = 0,
              lib=None):
    """Exact attention for selected rows.

    q [B,H,Nq,D], k/v [B,H,Nk,D] float64.  ``rows`` holds flat row ids
    r = (b*H + h)*Nq + i (``None`` = every row).  Returns (o [n,D], lse [n]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, D) or v.shape != (B, H, Nk, D):
        raise ValueError("shape mismatch")
    if rows is None:
        n = B * H * Nq
        rp = None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.size
        rp = _ptr(rows, ctypes.c_longlong)
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, H, Nq, Nk, D, float(scale),
                                  int(bool(causal)), rp, n, _ptr(o), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return o, lse


def attn(q, k, v, scale: float, causal: bool = False, nthreads: int = 0, lib=None):
    """Exact attention for every row; returns (o [B,H,Nq,D], lse [B,H,Nq])."""
    B, H, Nq, D = np.shape(q)
    o, lse = attn_rows(q, k, v, scale, causal, None, nthreads, lib)
    return o.reshape(B, H, Nq, D), lse.reshape(B, H, Nq)


def decode_split(q, k, v, scale: float, n_splits: int, lib=None):
    """Flash-decoding partials.  q [B,H,D], k/v [B,H,N,D] float64.

    Returns (o_part [B,H,n_splits,D], m_part [B,H,n_splits], l_part [B,H,n_splits]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, D = q.shape
    N = k.shape[2]
    if k.shape != (B, H, N, D) or v.shape != (B, H, N, D):
        raise ValueError("shape mismatch")
    o_part = np.empty((B, H, n_splits, D), dtype=np.float64)
    m_part = np.empty((B, H, n_splits), dtype=np.float64)
    l_part = np.empty((B, H, n_splits), dtype=np.float64)
    rc = (lib or _load()).oracle_decode_split(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, float(scale),
                                     int(n_splits), _ptr(o_part), _ptr(m_part), _ptr(l_part))
    if rc != 0:
        raise ValueError("oracle_decode_split rejected its arguments")
    return o_part, m_part, l_part


def decode_combine(o_part, m_part, l_part, lib=None):
    """Merge flash-decoding partials; returns o [B,H,D] float64."""
    o_part, m_part, l_part = _f64(o_part), _f64(m_part), _f64(l_part)
    B, H, S, D = o_part.shape
    if m_part.shape != (B, H, S) or l_part.shape != (B, H, S):
        raise ValueError("shape mismatch")
    o = np.empty((B, H, D), dtype=np.float64)
    rc = (lib or _load()).oracle_decode_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), B, H, D, S,
                                       _ptr(o))
    if rc != 0:
        raise ValueError("oracle_decode_combine rejected its arguments")
    return o


def attn_bwd(q, k, v, dout, scale: float, causal: bool = False, heads=None, nthreads: int = 0,
             lib=None):
    """Gradients of O = softmax(scale Q K^T) V (masked keys left out).

    q, dout [B,H,Nq,D], k/v [B,H,Nk,D] float64.  ``heads`` holds flat head ids
    b*H + h (``None`` = every head).  Returns (dq [n,Nq,D], dk [n,Nk,D],
    dv [n,Nk,D], delta [n,Nq]) for the n selected heads.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, D) or v.shape != (B, H, Nk, D) or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    if heads is None:
        n = B * H
        hp = None
    else:
        heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        n = heads.size
        hp = _ptr(heads, ctypes.c_longlong)
    dq = np.empty((n, Nq, D), dtype=np.float64)
    dk = np.empty((n, Nk, D), dtype=np.float64)
    dv = np.empty((n, Nk, D), dtype=np.float64)
    delta = np.empty((n, Nq), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, Nq, Nk, D,
                                          float(scale), int(bool(causal)), hp, n, _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(delta), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dv, delta
