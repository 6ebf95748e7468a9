"""fp64 CPU oracle for the affine associative scan family.

TEST INFRASTRUCTURE ONLY: the plain, sequential definition that the GPU
library (``associative_scan_amd``) is checked against. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it; the GPU library never does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, time-sequential per
(row, segment), built with ``-ffp-contract=off``); this module only builds it,
marshals numpy arrays and reshapes results. Each function cites the passage it
follows in ``oracle.c``'s comments.

Array conventions: the last axis of scalar inputs is time T and every leading
axis is an independent row; matrix inputs are [..., T, k, k] (transition) and
[..., T, k, v] (injection / state). ``h0`` is [nseg, rows] (scalar) or
[nseg, rows, k, v] (matrix); with a single segment it may also be given in the
shape of the leading axes. ``cu_seqlens`` follows the flash-attn convention.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exact-rational regrouping, brute force, library special cases,
adjoint identities and hand-derived fixtures under ``tests/golden/``).
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

__all__ = ["build", "scan_fwd", "scan_bwd", "scan_log_fwd", "scan_log_bwd", "gate", "gate_grad",
           "scan_fwd_gated", "scan_bwd_gated", "scan_log_fwd_gated", "scan_log_bwd_gated", "matrix_affine_scan_fwd",
           "matrix_affine_scan_bwd", "num_threads"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction, OpenMP)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.oracle_scan_fwd.argtypes = [i64, i64, i64, p, i32, i32, p, p, p, p]
        lib.oracle_scan_bwd.argtypes = [i64, i64, i64, p, i32, i32, p, p, p, p, p, p, p]
        lib.oracle_scan_log_fwd.argtypes = [i64, i64, i64, p, i32, i32, p, p, p, p]
        lib.oracle_scan_log_bwd.argtypes = [i64, i64, i64, p, i32, i32, p, p, p, p, p, p, p, p]
        lib.oracle_gate.argtypes = [i32, i64, p, p]
        lib.oracle_gate_grad.argtypes = [i32, i64, p, p, p]
        lib.oracle_matrix_fwd.argtypes = [i64, i64, i64, p, i32, i32, i32, i32, p, p, p, p]
        lib.oracle_matrix_bwd.argtypes = [i64, i64, i64, p, i32, i32, i32, i32, p, p, p, p, p, p, p]
        for f in (lib.oracle_scan_fwd, lib.oracle_scan_bwd, lib.oracle_scan_log_fwd,
                  lib.oracle_matrix_fwd, lib.oracle_matrix_bwd):
            f.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _segments(cu_seqlens, T):
    if cu_seqlens is None:
        return None, 1
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be nondecreasing with cu[0]=0 and cu[-1]=T")
    return cu, cu.size - 1


def _h0(h0, nseg, rows, tail=()):
    if h0 is None:
        return None
    h0 = _f64(h0)
    if h0.size != nseg * rows * int(np.prod(tail, dtype=np.int64)):
        raise ValueError("h0 must hold nseg*rows initial states")
    return h0.reshape((nseg, rows) + tuple(tail))


def scan_fwd(g, x, h0=None, cu_seqlens=None, reverse=False):
    """h_t = g_t*h_{t-1} + x_t per (row, segment); see oracle_scan_fwd in oracle.c."""
    g, x = _f64(g), _f64(x)
    assert g.shape == x.shape
    T = g.shape[-1]
    rows = int(np.prod(g.shape[:-1], dtype=np.int64))
    cu, nseg = _segments(cu_seqlens, T)
    h0 = _h0(h0, nseg, rows)
    h = np.zeros_like(g)
    _load().oracle_scan_fwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), _ptr(g), _ptr(x), _ptr(h0), _ptr(h))
    return h


def scan_bwd(g, h, dy, h0=None, cu_seqlens=None, reverse=False):
    """Adjoint of scan_fwd: returns (dx, dg, dh0[nseg, rows]); see oracle_scan_bwd."""
    g, h, dy = _f64(g), _f64(h), _f64(dy)
    assert g.shape == h.shape == dy.shape
    T = g.shape[-1]
    rows = int(np.prod(g.shape[:-1], dtype=np.int64))
    cu, nseg = _segments(cu_seqlens, T)
    h0 = _h0(h0, nseg, rows)
    dx, dg = np.zeros_like(g), np.zeros_like(g)
    dh0 = np.zeros((nseg, rows))
    _load().oracle_scan_bwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), _ptr(g), _ptr(h), _ptr(dy),
                            _ptr(h0), _ptr(dx), _ptr(dg), _ptr(dh0))
    return dx, dg, dh0


def scan_log_fwd(log_a, log_b, log_h0=None, cu_seqlens=None, reverse=False):
    """h = exp(A_t + LSE(log_b - A)) with A the running sum of log_a; see oracle_scan_log_fwd."""
    la, lb = _f64(log_a), _f64(log_b)
    assert la.shape == lb.shape
    T = la.shape[-1]
    rows = int(np.prod(la.shape[:-1], dtype=np.int64))
    cu, nseg = _segments(cu_seqlens, T)
    lh0 = _h0(log_h0, nseg, rows)
    h = np.zeros_like(la)
    _load().oracle_scan_log_fwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), _ptr(la), _ptr(lb), _ptr(lh0), _ptr(h))
    return h


def scan_log_bwd(log_a, log_b, h, dy, log_h0=None, cu_seqlens=None, reverse=False):
    """Adjoint of scan_log_fwd for L = <dy, h>: returns (dlog_a, dlog_b, dlog_h0[nseg, rows]);
    see oracle_scan_log_bwd."""
    la, lb, h, dy = _f64(log_a), _f64(log_b), _f64(h), _f64(dy)
    assert la.shape == lb.shape == h.shape == dy.shape
    T = la.shape[-1]
    rows = int(np.prod(la.shape[:-1], dtype=np.int64))
    cu, nseg = _segments(cu_seqlens, T)
    lh0 = _h0(log_h0, nseg, rows)
    dla, dlb = np.zeros_like(la), np.zeros_like(la)
    dlh0 = np.zeros((nseg, rows))
    _load().oracle_scan_log_bwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), _ptr(la), _ptr(lb), _ptr(h),
                                _ptr(dy), _ptr(lh0), _ptr(dla), _ptr(dlb), _ptr(dlh0))
    return dla, dlb, dlh0


SIGMOID, NEG_SOFTPLUS = 1, 2


def gate(kind, z):
    """f(z): sigmoid (kind 1) or -softplus (kind 2); see oracle_gate."""
    z = _f64(z)
    out = np.zeros_like(z)
    _load().oracle_gate(int(kind), z.size, _ptr(z), _ptr(out))
    return out


def gate_grad(kind, z, dact):
    """dz = dact * f'(z); see oracle_gate_grad."""
    z, dact = _f64(z), _f64(dact)
    assert z.shape == dact.shape
    dz = np.zeros_like(z)
    _load().oracle_gate_grad(int(kind), z.size, _ptr(z), _ptr(dact), _ptr(dz))
    return dz


def scan_fwd_gated(z, x, h0=None, cu_seqlens=None, reverse=False):
    """Scalar scan with gates g = sigmoid(z): the activation, then the scan."""
    return scan_fwd(gate(SIGMOID, z), x, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse)


def scan_bwd_gated(z, h, dy, h0=None, cu_seqlens=None, reverse=False):
    """Adjoint of scan_fwd_gated: (dx, dz, dh0), dz = dg * g (1 - g) by the chain rule."""
    g = gate(SIGMOID, z)
    dx, dg, dh0 = scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse)
    return dx, gate_grad(SIGMOID, z, dg), dh0


def scan_log_fwd_gated(z, log_b, log_h0=None, cu_seqlens=None, reverse=False):
    """Log-space scan with log_a = -softplus(z): the activation, then the scan."""
    return scan_log_fwd(gate(NEG_SOFTPLUS, z), log_b, log_h0=log_h0, cu_seqlens=cu_seqlens, reverse=reverse)


def scan_log_bwd_gated(z, log_b, h, dy, log_h0=None, cu_seqlens=None, reverse=False):
    """Adjoint of scan_log_fwd_gated: (dz, dlog_b, dlog_h0), dz = dlog_a * (-sigmoid(z))."""
    la = gate(NEG_SOFTPLUS, z)
    dla, dlb, dlh0 = scan_log_bwd(la, log_b, h, dy, log_h0=log_h0, cu_seqlens=cu_seqlens, reverse=reverse)
    return gate_grad(NEG_SOFTPLUS, z, dla), dlb, dlh0


def _mat_shapes(A, B_or_h):
    k = A.shape[-1]
    v = B_or_h.shape[-1]
    assert A.shape[-2] == k and B_or_h.shape[-2] == k and A.shape[:-2] == B_or_h.shape[:-2]
    T = A.shape[-3]
    rows = int(np.prod(A.shape[:-3], dtype=np.int64))
    return rows, T, k, v


def matrix_affine_scan_fwd(A, B, h0=None, cu_seqlens=None, reverse=False):
    """h_t = A_t h_{t-1} + B_t, A [...,T,k,k], B [...,T,k,v]; see oracle_matrix_fwd."""
    A, B = _f64(A), _f64(B)
    rows, T, k, v = _mat_shapes(A, B)
    if k * v > 256:
        raise ValueError("k*v > 256 not supported by the oracle")
    cu, nseg = _segments(cu_seqlens, T)
    h0 = _h0(h0, nseg, rows, (k, v))
    h = np.zeros_like(B)
    _load().oracle_matrix_fwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), k, v, _ptr(A), _ptr(B), _ptr(h0), _ptr(h))
    return h


def matrix_affine_scan_bwd(A, h, dy, h0=None, cu_seqlens=None, reverse=False):
    """Adjoint of matrix_affine_scan_fwd: returns (dA, dB, dh0[nseg, rows, k, v])."""
    A, h, dy = _f64(A), _f64(h), _f64(dy)
    rows, T, k, v = _mat_shapes(A, h)
    assert dy.shape == h.shape
    cu, nseg = _segments(cu_seqlens, T)
    h0 = _h0(h0, nseg, rows, (k, v))
    dA, dB = np.zeros_like(A), np.zeros_like(h)
    dh0 = np.zeros((nseg, rows, k, v))
    _load().oracle_matrix_bwd(rows, T, T, _ptr(cu), nseg, int(bool(reverse)), k, v, _ptr(A), _ptr(h), _ptr(dy),
                              _ptr(h0), _ptr(dA), _ptr(dB), _ptr(dh0))
    return dA, dB, dh0
