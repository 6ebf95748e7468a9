"""Python binding of libmscan, the MI355X (gfx950) affine associative scan.

Thin argument marshalling over the C ABI in ``include/mscan.h``: every step of
every scan runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream. There is no CPU or eager fallback: a missing
library or a missing GPU raises.

Entry points (same names as the C ABI):
    scan_fwd(g, x, h0=None, cu_seqlens=None, reverse=False) -> h
    scan_bwd(g, h, dy, h0=None, cu_seqlens=None, reverse=False) -> (dx, dg, dh0)
    scan_log_fwd(log_a, log_b, log_h0=None, cu_seqlens=None, reverse=False) -> h
    scan_log_bwd(log_a, log_b, h, dy, log_h0=None, cu_seqlens=None, reverse=False) -> (dlog_a, dlog_b, dlog_h0)
    scan_fwd_gated / scan_bwd_gated (gate logits z, g = sigmoid(z)) -> h / (dx, dz, dh0)
    scan_log_fwd_gated / scan_log_bwd_gated (log a = -softplus(z)) -> h / (dz, dlog_b, dlog_h0)
    matrix_affine_scan_fwd(A, B, h0=None, cu_seqlens=None, reverse=False) -> h
    matrix_affine_scan_bwd(A, h, dy, h0=None, cu_seqlens=None, reverse=False) -> (dA, dB, dh0)

Scalar tensors are [..., T] (every leading axis is an independent row, time
contiguous); matrix tensors are [..., T, k, k] and [..., T, k, v]. ``h0`` is
[nseg, rows] ([nseg, rows, k, v] for matrices) or, with one sequence, the shape
of the leading axes. ``cu_seqlens`` is an int32 device tensor in the flash-attn
convention. Inputs are fp32, or bf16 / fp16 for the scalar scan's g and x;
outputs are fp32.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "lib", "library_path", "stress_library_path", "load_library", "Problem", "MscanError",
    "scan_fwd", "scan_bwd", "scan_log_fwd", "scan_log_bwd", "matrix_affine_scan_fwd", "matrix_affine_scan_bwd",
    "scan_fwd_gated", "scan_bwd_gated", "scan_log_fwd_gated", "scan_log_bwd_gated",
    "scan_causal", "scan_bidirectional_branched", "scan_log", "matrix_scan", "GATE_SIGMOID", "GATE_NEG_SOFTPLUS",
    "workspace_bytes", "OP_SCAN_FWD", "OP_SCAN_BWD", "OP_SCAN_LOG_FWD", "OP_MATRIX_FWD", "OP_MATRIX_BWD",
    "OP_SCAN_LOG_BWD", "set_debug", "debug_enabled", "workspace_error", "stream_ceiling", "release_capture_workspaces",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmscan.so")

OP_SCAN_FWD, OP_SCAN_BWD, OP_SCAN_LOG_FWD, OP_MATRIX_FWD, OP_MATRIX_BWD, OP_SCAN_LOG_BWD = range(6)
_F32, _BF16, _F16 = 0, 1, 2
GATE_NONE, GATE_SIGMOID, GATE_NEG_SOFTPLUS = 0, 1, 2
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace too small", 4: "HIP error",
           5: "a look-back wait gave up"}


class MscanError(RuntimeError):
    def __init__(self, fn, status, detail=""):
        self.status = status
        msg = f"{fn}: {_STATUS.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


class Problem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("T", ctypes.c_int64), ("row_stride", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p), ("nseg", ctypes.c_int32), ("reverse", ctypes.c_int32),
    ]


stress_library_path = os.path.join(_HERE, "libmscan_stress.so")


def load_library(path: str):
    """A libmscan build at `path` (e.g. the race-stress build
    libmscan_stress.so) as a ctypes library with every entry point's argument
    types set, for callers that drive the C ABI directly."""
    if not os.path.exists(path):
        raise ImportError(f"{path} not found; build it with `python associative_scan_amd/build.py`")
    L = ctypes.CDLL(path)
    P, p, sz, i32 = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "mscan_workspace_bytes": (sz, [P, i32, i32, i32]),
        "mscan_workspace_init": (i32, [p, sz, p]),
        "scan_fwd": (i32, [P, i32, p, p, p, p, p, sz, p]),
        "scan_bwd": (i32, [P, i32, p, p, p, p, p, p, p, p, sz, p]),
        "scan_log_fwd": (i32, [P, p, p, p, p, p, sz, p]),
        "scan_log_bwd": (i32, [P, p, p, p, p, p, p, p, p, p, sz, p]),
        "scan_fwd_gated": (i32, [P, i32, i32, p, p, p, p, p, sz, p]),
        "scan_bwd_gated": (i32, [P, i32, i32, p, p, p, p, p, p, p, p, sz, p]),
        "scan_log_fwd_gated": (i32, [P, i32, p, p, p, p, p, sz, p]),
        "scan_log_bwd_gated": (i32, [P, i32, p, p, p, p, p, p, p, p, p, sz, p]),
        "matrix_affine_scan_fwd": (i32, [P, i32, i32, p, p, p, p, p, sz, p]),
        "matrix_affine_scan_bwd": (i32, [P, i32, i32, p, p, p, p, p, p, p, p, sz, p]),
        "scan_fwd_noalloc": (i32, [P, i32, p, p, p, p, p]),
        "mscan_workspace_error": (i32, [p, sz, p, p]),
        "mscan_stream_ceiling": (i32, [ctypes.POINTER(p), i32, ctypes.POINTER(p), i32, sz, p]),
        "mscan_debug_partial_fwd": (i32, [P, i32, i32, p, p, p, p, sz, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32,
                                          p]),
        "mscan_status_string": (ctypes.c_char_p, [i32]),
        "mscan_last_hip_error": (ctypes.c_char_p, []),
        "mscan_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    if L.mscan_abi_version() != 1:
        raise ImportError("libmscan ABI version mismatch")
    return L


def _load():
    return load_library(library_path)


lib = _load()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t):
    # a plain int: ctypes converts it for the c_void_p parameters
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device):
    """The current HIP stream of `device` as an integer handle."""
    if _raw_stream is not None:  # no Stream object per call
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _rows_view(t: torch.Tensor, name: str, tail: int = 0):
    """(rows, T, row_stride) of a tensor viewed as [rows, T, *tail] with the
    trailing (T, *tail) block contiguous and a uniform stride between rows."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() < 1 + tail:
        raise ValueError(f"{name} needs at least {1 + tail} dims")
    n = t.numel()
    if n and t.is_contiguous():  # the common case, without the per-axis walk
        T = int(t.shape[t.dim() - 1 - tail])
        block = 1
        for d in t.shape[t.dim() - tail:]:
            block *= int(d)
        return n // (T * block), T, T
    inner = t.shape[t.dim() - 1 - tail:]
    T = int(inner[0])
    block = 1
    for d in inner[1:]:
        block *= int(d)
    # trailing block contiguous
    expect = 1
    for i in range(t.dim() - 1, t.dim() - 2 - tail, -1):
        if t.shape[i] != 1 and t.stride(i) != expect:
            raise ValueError(f"{name}: time (and matrix) axes must be contiguous")
        expect *= t.shape[i]
    lead = t.shape[: t.dim() - 1 - tail]
    rows = 1
    for d in lead:
        rows *= int(d)
    if rows == 0 or T == 0:
        return rows, T, T
    # leading axes must collapse to one uniform stride (in units of the trailing block)
    stride_el = None
    exp = None
    for i in range(len(lead) - 1, -1, -1):
        if lead[i] == 1:
            continue
        if stride_el is None:
            stride_el = t.stride(i)
            exp = stride_el * lead[i]
        else:
            if t.stride(i) != exp:
                raise ValueError(f"{name}: leading axes do not collapse to a single row stride")
            exp *= lead[i]
    if stride_el is None:
        stride_el = T * block
    if stride_el % block:
        raise ValueError(f"{name}: row stride not a multiple of the per-step block")
    return rows, T, stride_el // block


def _out_rows(shape, rows, T, stride, dev, tail=()):
    """An uninitialised fp32 tensor of `shape` whose rows lie `stride` steps
    apart (a view into a [rows, stride, *tail] buffer), matching the row stride
    the C ABI applies to every array of a call."""
    if stride == T:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    buf = torch.empty((rows, stride) + tuple(tail), dtype=torch.float32, device=dev)
    return buf[:, :T].view(shape)


_ws_lock = threading.Lock()
_ws_cache = {}
_capture_ws = []  # workspaces of calls recorded into HIP graphs: kept for the graphs' replays


def release_capture_workspaces() -> None:
    """Drop the workspaces held for calls recorded into HIP graphs. Call only
    once no graph captured through this binding will be replayed again."""
    with _ws_lock:
        _capture_ws.clear()


def _workspace(device, stream_handle, nbytes):
    """A workspace of at least nbytes for (device, stream). Eager calls share
    one cached buffer per (device, stream), grown as needed. A call recorded
    into a HIP graph gets a buffer of its own that is never released (until
    release_capture_workspaces): a graph's replays write the buffer whose
    address it recorded, so it must outlive the graph and must not be shared
    with eager calls or with other graphs, which may be replayed concurrently
    or need a larger buffer later."""
    if torch.cuda.is_current_stream_capturing():
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)  # the graph's memory pool
        with _ws_lock:
            _capture_ws.append(buf)
        return buf
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_handle)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            size = max(nbytes, 1 << 16)
            buf = torch.empty(size, dtype=torch.uint8, device=device)
            st = lib.mscan_workspace_init(_ptr(buf), size, ctypes.c_void_p(stream_handle))
            if st != 0:
                raise MscanError("mscan_workspace_init", st, lib.mscan_last_hip_error().decode())
            _ws_cache[key] = buf
        return buf


def workspace_bytes(prob: Problem, op: int, k: int = 1, v: int = 1) -> int:
    return int(lib.mscan_workspace_bytes(ctypes.byref(prob), op, k, v))


_WS_HEADER_BYTES = 128  # what a scalar-layout op asks for when its rows need no look-back


def _scalar_ws(dev, sh, prob, op):
    """(pointer, bytes) of the workspace a scalar-layout op needs: none when
    every row fits one tile (the library then never reads it)."""
    need = workspace_bytes(prob, op)
    if need <= _WS_HEADER_BYTES:
        return None, 0
    ws = _workspace(dev, sh, need)
    return ws.data_ptr(), ws.numel()


# ---------------------------------------------------------------------------
# debug mode
# ---------------------------------------------------------------------------
_DEBUG = [os.environ.get("MSCAN_DEBUG", "") not in ("", "0")]


def set_debug(on: bool = True) -> None:
    """Debug mode. The contents of cu_seqlens are validated on the host before
    each call (cu[0] = 0, cu[-1] = T, nondecreasing), and after each call that
    chained tiles through a workspace the workspace's error word is read (which
    synchronises the stream): a look-back wait that gave up raises MscanError
    with status 5 instead of leaving NaN in the outputs unnoticed. Off by
    default, since it synchronises every call; MSCAN_DEBUG=1 in the environment
    turns it on at import. Calls made while a HIP graph is being captured skip
    both checks (a capture allows no host copy or synchronisation)."""
    _DEBUG[0] = bool(on)


def debug_enabled() -> bool:
    return _DEBUG[0]


def _validate_cu_host(cu, T):
    """Host check of cu_seqlens contents (debug mode): the flash-attn
    convention, cu[0] = 0, cu[-1] = T, nondecreasing."""
    import numpy as np
    cu = np.asarray(cu)
    if cu.ndim != 1 or cu.size < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    if int(cu[0]) != 0 or int(cu[-1]) != T:
        raise ValueError(f"cu_seqlens must start at 0 and end at T={T} (got {int(cu[0])} ... {int(cu[-1])})")
    bad = np.nonzero(np.diff(cu.astype(np.int64)) < 0)[0]
    if bad.size:
        raise ValueError(f"cu_seqlens must be nondecreasing (cu[{bad[0]}] = {int(cu[bad[0]])} > "
                         f"cu[{bad[0] + 1}] = {int(cu[bad[0] + 1])})")


def _read_ws_error(wsp, wsn, device, stream_handle) -> int:
    """The workspace's error word as an mscan status (0, or 5 when a look-back
    wait of the last call that chained tiles through it gave up); waits for the
    work queued on the stream before it."""
    flag = torch.zeros(1, dtype=torch.int32, device=device)
    _check("mscan_workspace_error", lib.mscan_workspace_error(wsp, wsn, flag.data_ptr(), stream_handle))
    return int(flag.item())


def _raise_if_tripped(fn, wsp, wsn, device, stream_handle):
    code = _read_ws_error(wsp, wsn, device, stream_handle)
    if code != 0:
        raise MscanError(fn, code, "outputs that needed the missing carry are NaN")


def stream_ceiling(srcs, dsts) -> None:
    """Enqueue the streaming diagnostic kernel (mscan_stream_ceiling): reads
    every tensor of `srcs`, writes every tensor of `dsts` (contiguous fp32 GPU
    tensors of one size, a multiple of 4 elements)."""
    n = srcs[0].numel()
    for t in list(srcs) + list(dsts):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
            raise ValueError("stream_ceiling takes contiguous fp32 GPU tensors of one size")
    P = ctypes.c_void_p
    sa = (P * len(srcs))(*[t.data_ptr() for t in srcs])
    da = (P * len(dsts))(*[t.data_ptr() for t in dsts])
    _check("mscan_stream_ceiling", lib.mscan_stream_ceiling(sa, len(srcs), da, len(dsts), n,
                                                            _stream_handle(srcs[0].device)))


def workspace_error(ws: torch.Tensor) -> int:
    """mscan status of a workspace tensor's error word (see mscan_workspace_error)."""
    return _read_ws_error(ws.data_ptr(), ws.numel() * ws.element_size(), ws.device, _stream_handle(ws.device))


def _segments(cu_seqlens, device, T):
    if cu_seqlens is None:
        return None, 1
    if not isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = torch.tensor(cu_seqlens, dtype=torch.int32, device=device)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    if cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    if _DEBUG[0] and not torch.cuda.is_current_stream_capturing():  # no host copy inside a graph capture
        _validate_cu_host(cu_seqlens.cpu().numpy(), T)
    return cu_seqlens, cu_seqlens.numel() - 1


def _h0(h0, nseg, rows, tail, name="h0"):
    if h0 is None:
        return None
    if h0.dtype != torch.float32 or not h0.is_cuda or not h0.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
    need = nseg * rows
    for d in tail:
        need *= d
    if h0.numel() != need:
        raise ValueError(f"{name} must hold nseg*rows states ({need} values), got {h0.numel()}")
    return h0


def _check(fn, status, ws=None):
    """Raise on a failed call; in debug mode also when a call that chained
    tiles through the workspace ws = (ptr, bytes, device, stream) had a wait
    give up."""
    if status != 0:
        raise MscanError(fn, status, lib.mscan_last_hip_error().decode() if status == 4 else "")
    if ws is not None and ws[0] and _DEBUG[0] and not torch.cuda.is_current_stream_capturing():
        _raise_if_tripped(fn, *ws)


def _in_dtype(t, name):
    if t.dtype == torch.float32:
        return _F32
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float16:
        return _F16
    raise ValueError(f"{name}: only float32, bfloat16 and float16 inputs are supported")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def scan_fwd(g, x, h0=None, cu_seqlens=None, reverse=False, out=None):
    """h_t = g_t h_{t-1} + x_t per row and per packed sequence (fp32 result)."""
    return _scan_fwd(g, x, h0, cu_seqlens, reverse, out, GATE_NONE)


def scan_fwd_gated(z, x, h0=None, cu_seqlens=None, reverse=False, out=None):
    """scan_fwd with gates g = sigmoid(z) computed inside the kernel from logits z."""
    return _scan_fwd(z, x, h0, cu_seqlens, reverse, out, GATE_SIGMOID)


def _scan_fwd(g, x, h0, cu_seqlens, reverse, out, gate):
    if g.shape != x.shape or g.dtype != x.dtype:
        raise ValueError("g and x must have the same shape and dtype")
    rows, T, stride = _rows_view(g, "g")
    if not (x.is_cuda and x.is_contiguous() and stride == T) and _rows_view(x, "x")[2] != stride:
        raise ValueError("g and x must share the row stride")
    dt = _in_dtype(g, "g")
    dev = g.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    h0 = _h0(h0, nseg, rows, ())
    if out is None:
        if stride != T:
            raise ValueError("strided rows need an explicit `out` with the same row stride")
        h = torch.empty(g.shape, dtype=torch.float32, device=dev)  # contiguous: stride T
    else:
        h = out
        if h.shape != g.shape or _rows_view(h, "out")[2] != stride:
            raise ValueError("out must match g's shape and row stride")
        if h.dtype != torch.float32:
            raise ValueError("out must be float32")
    if rows == 0 or T == 0:
        return h
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    wsp, wsn = _scalar_ws(dev, sh, prob, OP_SCAN_FWD)
    if gate == GATE_NONE:
        _check("scan_fwd", lib.scan_fwd(ctypes.byref(prob), dt, _ptr(g), _ptr(x), _ptr(h0), _ptr(h), wsp, wsn, sh),
               (wsp, wsn, dev, sh))
    else:
        _check("scan_fwd_gated", lib.scan_fwd_gated(ctypes.byref(prob), dt, gate, _ptr(g), _ptr(x), _ptr(h0), _ptr(h),
                                                    wsp, wsn, sh), (wsp, wsn, dev, sh))
    return h


def scan_bwd(g, h, dy, h0=None, cu_seqlens=None, reverse=False, need_dh0=True):
    """Adjoint of scan_fwd: (dx, dg, dh0) given the forward's output h and dy."""
    return _scan_bwd(g, h, dy, h0, cu_seqlens, reverse, need_dh0, GATE_NONE)


def scan_bwd_gated(z, h, dy, h0=None, cu_seqlens=None, reverse=False, need_dh0=True):
    """Adjoint of scan_fwd_gated: (dx, dz, dh0), dz = dg * g (1 - g)."""
    return _scan_bwd(z, h, dy, h0, cu_seqlens, reverse, need_dh0, GATE_SIGMOID)


def _scan_bwd(g, h, dy, h0, cu_seqlens, reverse, need_dh0, gate):
    if h.dtype != torch.float32 or dy.dtype != torch.float32:
        raise ValueError("h and dy must be float32")
    if g.shape != h.shape or dy.shape != h.shape:
        raise ValueError("g, h and dy must have the same shape")
    rows, T, stride = _rows_view(g, "g")
    if not (h.is_cuda and dy.is_cuda and h.is_contiguous() and dy.is_contiguous() and stride == T):
        for t, n in ((h, "h"), (dy, "dy")):
            if _rows_view(t, n)[2] != stride:
                raise ValueError("g, h and dy must share the row stride")
    dt = _in_dtype(g, "g")
    dev = g.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    h0 = _h0(h0, nseg, rows, ())
    # strided rows: the gradients share the inputs' row stride
    dx = _out_rows(h.shape, rows, T, stride, dev)
    dg = _out_rows(h.shape, rows, T, stride, dev)
    dh0 = torch.empty((nseg, rows), dtype=torch.float32, device=dev) if need_dh0 else None
    if rows == 0 or T == 0:
        if dh0 is not None:
            dh0.zero_()
        return dx, dg, dh0
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    wsp, wsn = _scalar_ws(dev, sh, prob, OP_SCAN_BWD)
    if gate == GATE_NONE:
        _check("scan_bwd", lib.scan_bwd(ctypes.byref(prob), dt, _ptr(g), _ptr(h), _ptr(dy), _ptr(h0), _ptr(dx),
                                        _ptr(dg), _ptr(dh0), wsp, wsn, sh), (wsp, wsn, dev, sh))
    else:
        _check("scan_bwd_gated", lib.scan_bwd_gated(ctypes.byref(prob), dt, gate, _ptr(g), _ptr(h), _ptr(dy), _ptr(h0),
                                                    _ptr(dx), _ptr(dg), _ptr(dh0), wsp, wsn, sh), (wsp, wsn, dev, sh))
    return dx, dg, dh0


def scan_log_fwd(log_a, log_b, log_h0=None, cu_seqlens=None, reverse=False):
    """h = exp of the log-space scan of h_t = a_t h_{t-1} + b_t (fp32 in, fp32 out)."""
    return _scan_log_fwd(log_a, log_b, log_h0, cu_seqlens, reverse, GATE_NONE)


def scan_log_fwd_gated(z, log_b, log_h0=None, cu_seqlens=None, reverse=False):
    """scan_log_fwd with log a = -softplus(z) computed inside the kernel from logits z."""
    return _scan_log_fwd(z, log_b, log_h0, cu_seqlens, reverse, GATE_NEG_SOFTPLUS)


def _scan_log_fwd(log_a, log_b, log_h0, cu_seqlens, reverse, gate):
    if log_a.shape != log_b.shape or log_a.dtype != torch.float32 or log_b.dtype != torch.float32:
        raise ValueError("log_a and log_b must be float32 tensors of one shape")
    rows, T, stride = _rows_view(log_a, "log_a")
    if _rows_view(log_b, "log_b")[2] != stride:
        raise ValueError("log_a and log_b must share the row stride")
    dev = log_a.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    log_h0 = _h0(log_h0, nseg, rows, (), "log_h0")
    h = _out_rows(log_a.shape, rows, T, stride, dev)
    if rows == 0 or T == 0:
        return h
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    wsp, wsn = _scalar_ws(dev, sh, prob, OP_SCAN_LOG_FWD)
    if gate == GATE_NONE:
        _check("scan_log_fwd", lib.scan_log_fwd(ctypes.byref(prob), _ptr(log_a), _ptr(log_b), _ptr(log_h0), _ptr(h),
                                                wsp, wsn, sh), (wsp, wsn, dev, sh))
    else:
        _check("scan_log_fwd_gated", lib.scan_log_fwd_gated(ctypes.byref(prob), gate, _ptr(log_a), _ptr(log_b),
                                                            _ptr(log_h0), _ptr(h), wsp, wsn, sh), (wsp, wsn, dev, sh))
    return h


def scan_log_bwd(log_a, log_b, h, dy, log_h0=None, cu_seqlens=None, reverse=False, need_dh0=True):
    """Adjoint of scan_log_fwd for dL/dh = dy: (dlog_a, dlog_b, dlog_h0)."""
    return _scan_log_bwd(log_a, log_b, h, dy, log_h0, cu_seqlens, reverse, need_dh0, GATE_NONE)


def scan_log_bwd_gated(z, log_b, h, dy, log_h0=None, cu_seqlens=None, reverse=False, need_dh0=True):
    """Adjoint of scan_log_fwd_gated: (dz, dlog_b, dlog_h0), dz = dlog_a * (-sigmoid(z))."""
    return _scan_log_bwd(z, log_b, h, dy, log_h0, cu_seqlens, reverse, need_dh0, GATE_NEG_SOFTPLUS)


def _scan_log_bwd(log_a, log_b, h, dy, log_h0, cu_seqlens, reverse, need_dh0, gate):
    for t, n in ((log_a, "log_a"), (log_b, "log_b"), (h, "h"), (dy, "dy")):
        if t.dtype != torch.float32 or t.shape != log_a.shape:
            raise ValueError(f"{n} must be a float32 tensor of log_a's shape")
    rows, T, stride = _rows_view(log_a, "log_a")
    for t, n in ((log_b, "log_b"), (h, "h"), (dy, "dy")):
        if _rows_view(t, n)[2] != stride:
            raise ValueError("log_a, log_b, h and dy must share the row stride")
    dev = log_a.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    log_h0 = _h0(log_h0, nseg, rows, (), "log_h0")
    dla = _out_rows(log_a.shape, rows, T, stride, dev)
    dlb = _out_rows(log_a.shape, rows, T, stride, dev)
    dlh0 = torch.empty((nseg, rows), dtype=torch.float32, device=dev) if need_dh0 else None
    if rows == 0 or T == 0:
        if dlh0 is not None:
            dlh0.zero_()
        return dla, dlb, dlh0
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    wsp, wsn = _scalar_ws(dev, sh, prob, OP_SCAN_LOG_BWD)
    if gate == GATE_NONE:
        _check("scan_log_bwd", lib.scan_log_bwd(ctypes.byref(prob), _ptr(log_a), _ptr(log_b), _ptr(h), _ptr(dy),
                                                _ptr(log_h0), _ptr(dla), _ptr(dlb), _ptr(dlh0), wsp, wsn, sh),
               (wsp, wsn, dev, sh))
    else:
        _check("scan_log_bwd_gated", lib.scan_log_bwd_gated(ctypes.byref(prob), gate, _ptr(log_a), _ptr(log_b), _ptr(h),
                                                            _ptr(dy), _ptr(log_h0), _ptr(dla), _ptr(dlb), _ptr(dlh0),
                                                            wsp, wsn, sh), (wsp, wsn, dev, sh))
    return dla, dlb, dlh0


def _mat_dims(A, Bh, nameB):
    if A.dtype != torch.float32 or Bh.dtype != torch.float32:
        raise ValueError("matrix scan inputs must be float32")
    if A.dim() < 3 or Bh.dim() < 3:
        raise ValueError("matrix inputs are [..., T, k, k] and [..., T, k, v]")
    k, v = int(A.shape[-1]), int(Bh.shape[-1])
    if A.shape[-2] != k or Bh.shape[-2] != k or A.shape[:-2] != Bh.shape[:-2]:
        raise ValueError(f"A must be [..., T, k, k] and {nameB} [..., T, k, v] with matching leading axes")
    rows, T, stride = _rows_view(A, "A", tail=2)
    if _rows_view(Bh, nameB, tail=2)[2] != stride:
        raise ValueError(f"A and {nameB} must share the row stride (in time steps)")
    return rows, T, stride, k, v


def matrix_affine_scan_fwd(A, B, h0=None, cu_seqlens=None, reverse=False):
    """h_t = A_t h_{t-1} + B_t with k x k transitions and k x v states."""
    rows, T, stride, k, v = _mat_dims(A, B, "B")
    dev = A.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    h0 = _h0(h0, nseg, rows, (k, v))
    h = _out_rows(B.shape, rows, T, stride, dev, (k, v))
    if rows == 0 or T == 0:
        return h
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    ws = _workspace(dev, sh, workspace_bytes(prob, OP_MATRIX_FWD, k, v))
    _check("matrix_affine_scan_fwd", lib.matrix_affine_scan_fwd(
        ctypes.byref(prob), k, v, _ptr(A), _ptr(B), _ptr(h0), _ptr(h), _ptr(ws), ws.numel(), ctypes.c_void_p(sh)),
        (_ptr(ws), ws.numel(), dev, sh))
    return h


def matrix_affine_scan_bwd(A, h, dy, h0=None, cu_seqlens=None, reverse=False, need_dh0=True):
    """Adjoint of matrix_affine_scan_fwd: (dA, dB, dh0)."""
    rows, T, stride, k, v = _mat_dims(A, h, "h")
    if dy.shape != h.shape or dy.dtype != torch.float32:
        raise ValueError("dy must match h")
    if _rows_view(dy, "dy", tail=2)[2] != stride:
        raise ValueError("A, h and dy must share the row stride (in time steps)")
    dev = A.device
    cu, nseg = _segments(cu_seqlens, dev, T)
    h0 = _h0(h0, nseg, rows, (k, v))
    dA = _out_rows(A.shape, rows, T, stride, dev, (k, k))
    dB = _out_rows(h.shape, rows, T, stride, dev, (k, v))
    dh0 = torch.empty((nseg, rows, k, v), dtype=torch.float32, device=dev) if need_dh0 else None
    if rows == 0 or T == 0:
        if dh0 is not None:
            dh0.zero_()
        return dA, dB, dh0
    prob = Problem(rows, T, stride, cu.data_ptr() if cu is not None else None, nseg, int(bool(reverse)))
    sh = _stream_handle(dev)
    ws = _workspace(dev, sh, workspace_bytes(prob, OP_MATRIX_BWD, k, v))
    _check("matrix_affine_scan_bwd", lib.matrix_affine_scan_bwd(
        ctypes.byref(prob), k, v, _ptr(A), _ptr(h), _ptr(dy), _ptr(h0), _ptr(dA), _ptr(dB), _ptr(dh0),
        _ptr(ws), ws.numel(), ctypes.c_void_p(sh)), (_ptr(ws), ws.numel(), dev, sh))
    return dA, dB, dh0


# ---------------------------------------------------------------------------
# differentiable entry points: torch.library custom ops (see _torch_ops.py),
# in the README's calling convention for the scalar scan
# ---------------------------------------------------------------------------
from . import _torch_ops  # noqa: E402  (registers the mscan:: custom ops)


def scan_causal(gates, tokens, cu_seqlens=None, h0=None):
    """Differentiable causal scan h[t] = gates[t] h[t-1] + tokens[t] (fp32 output)."""
    return torch.ops.mscan.scan(gates, tokens, h0, cu_seqlens, False)


def scan_bidirectional_branched(gates_fwd, tokens_fwd, gates_bwd, tokens_bwd, cu_seqlens=None):
    """Two independent branches: a causal scan and a reverse-in-time scan."""
    return (torch.ops.mscan.scan(gates_fwd, tokens_fwd, None, cu_seqlens, False),
            torch.ops.mscan.scan(gates_bwd, tokens_bwd, None, cu_seqlens, True))


def scan_log(log_a, log_b, log_h0=None, cu_seqlens=None, reverse=False):
    """Differentiable log-space scan: h = exp of h_t = a_t h_{t-1} + b_t carried
    in log space, with the native adjoint kernel for the backward."""
    return torch.ops.mscan.scan_log(log_a, log_b, log_h0, cu_seqlens, reverse)


def matrix_scan(A, B, h0=None, cu_seqlens=None, reverse=False):
    """Differentiable matrix-affine scan h_t = A_t h_{t-1} + B_t."""
    return torch.ops.mscan.matrix_scan(A, B, h0, cu_seqlens, reverse)


def matrix_cumprod(A, cu_seqlens=None, reverse=False):
    """Running products Abar_t = A_t Abar_{t-1} with Abar = I before each
    sequence's first step (reverse: Abar_t = A_t Abar_{t+1}), the cumulative-
    product output of the generic affine scan. It is the matrix-affine scan
    with v = k, B = 0 and h0 = I, and runs as that scan (differentiable in A)."""
    k = int(A.shape[-1])
    if A.dim() < 3 or A.shape[-2] != k:
        raise ValueError("A must be [..., T, k, k]")
    rows = A.numel() // (A.shape[-3] * k * k) if A.shape[-3] > 0 else 0
    nseg = 1 if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    eye = torch.eye(k, dtype=torch.float32, device=A.device)
    h0 = eye.expand(nseg, rows, k, k).contiguous()
    return torch.ops.mscan.matrix_scan(A, torch.zeros_like(A), h0, cu_seqlens, reverse)
