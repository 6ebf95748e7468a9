"""Look-back under race stress: the library built with MSCAN_RACE_STRESS
(libmscan_stress.so) waits a pseudo-random time before every publish of a
look-back descriptor or chained state, so tiles publish in unusual orders and
at unusual distances. The chained problems below (many tiles per row, packed
sequences, both directions, every kind of descriptor: the linear scan's three
words, the log-space scan's five, the VALU matrix scans' k^2 + 2kv, the
matrix-core chains' published states) must still give the oracle's results:
bit for bit on exact-mode integer data, within 1e-4 for the log-space scan.
The multi-tile carry is where a race would show ("how it works" of the
associative-scan-triton README: the running prefix carried across chunks)."""
import ctypes

import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m, m.load_library(m.stress_library_path)


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def _p(t):
    return None if t is None else t.data_ptr()


def _ws(m, lib, prob, op, k=1, v=1):
    n = int(lib.mscan_workspace_bytes(ctypes.byref(prob), op, k, v))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)


def _same(gpu, ref, what):
    g = gpu.detach().cpu().double().numpy()
    bad = g != np.asarray(ref, np.float64)
    assert not bad.any(), f"{what}: {int(bad.sum())} mismatches"


@pytest.mark.parametrize("reverse", [False, True])
def test_stress_scalar_exact(L, oracle_lib, reverse):
    m, lib = L
    r = np.random.default_rng(5000 + reverse)
    rows, T = 3, 24 * 4096 + 77
    g, x, dy = gen.exact_mode(r, (rows, T))
    cu = gen.segments_random(r, T, 11)
    h0 = r.integers(-1, 2, (11, rows)).astype(np.float32)
    cu_t, h0_t = _t(cu, torch.int32), _t(h0)
    sh = torch.cuda.current_stream().cuda_stream
    for dt, gd, xd in ((0, _t(g), _t(x)), (1, _t(g).to(torch.bfloat16), _t(x).to(torch.bfloat16))):
        prob = m.Problem(rows, T, T, cu_t.data_ptr(), 11, int(reverse))
        ws = _ws(m, lib, prob, m.OP_SCAN_BWD)
        h = torch.empty((rows, T), device=DEV)
        assert lib.scan_fwd(ctypes.byref(prob), dt, _p(gd), _p(xd), _p(h0_t), _p(h), _p(ws), ws.numel(), sh) == 0
        href = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
        torch.cuda.synchronize()
        _same(h, href, f"h dtype {dt}")
        dx, dg = torch.empty_like(h), torch.empty_like(h)
        dh0 = torch.empty((11, rows), device=DEV)
        assert lib.scan_bwd(ctypes.byref(prob), dt, _p(gd), _p(h), _p(_t(dy)), _p(h0_t), _p(dx), _p(dg), _p(dh0),
                            _p(ws), ws.numel(), sh) == 0
        rx, rg, rh0 = oracle_lib.scan_bwd(g, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
        torch.cuda.synchronize()
        _same(dx, rx, f"dx dtype {dt}")
        _same(dg, rg, f"dg dtype {dt}")
        _same(dh0, rh0, f"dh0 dtype {dt}")
        assert m.workspace_error(ws) == 0


def test_stress_log_space(L, oracle_lib):
    m, lib = L
    r = np.random.default_rng(5100)
    rows, T = 4, 20 * 4096 + 3
    la = -np.log1p(np.exp(r.standard_normal((rows, T)))).astype(np.float32)
    lb = r.standard_normal((rows, T)).astype(np.float32)
    cu = gen.segments_random(r, T, 5)
    cu_t = _t(cu, torch.int32)
    sh = torch.cuda.current_stream().cuda_stream
    for rev in (False, True):
        prob = m.Problem(rows, T, T, cu_t.data_ptr(), 5, int(rev))
        ws = _ws(m, lib, prob, m.OP_SCAN_LOG_FWD)
        h = torch.empty((rows, T), device=DEV)
        assert lib.scan_log_fwd(ctypes.byref(prob), _p(_t(la)), _p(_t(lb)), None, _p(h), _p(ws), ws.numel(), sh) == 0
        ref = oracle_lib.scan_log_fwd(la, lb, cu_seqlens=cu, reverse=rev)
        torch.cuda.synchronize()
        got = h.cpu().double().numpy()
        assert np.max(np.abs(got - ref) / (1 + np.abs(ref))) <= 1e-4
        assert m.workspace_error(ws) == 0


def _signed_perm(r, k, v, rows, T, max_run):
    A = np.zeros((rows, T, k, k), np.float32)
    perm = np.argsort(r.random((rows, T, k)), axis=-1)
    sign = r.choice(np.array([-1.0, 1.0], np.float32), size=(rows, T, k))
    for i in range(k):
        np.put_along_axis(A[:, :, i, :], perm[:, :, i:i + 1], sign[:, :, i:i + 1], axis=-1)
    zero = r.random((rows, T)) < 0.01
    zero[:, max_run - 1::max_run] = True
    A[zero] = 0.0
    B = r.integers(-1, 2, size=(rows, T, k, v)).astype(np.float32)
    dy = r.integers(-1, 2, size=(rows, T, k, v)).astype(np.float32)
    return A, B, dy


@pytest.mark.parametrize("kv,T", [((2, 1), 12 * 2048 + 5), ((4, 1), 30 * 256 + 1), ((4, 4), 40 * 256 + 3),
                                  ((16, 16), 60 * 32 + 7), ((8, 2), 60 * 32 + 1)])
def test_stress_matrix_exact(L, oracle_lib, kv, T):
    m, lib = L
    k, v = kv
    r = np.random.default_rng(5200 + 10 * k + v)
    rows = 2
    A, B, dy = _signed_perm(r, k, v, rows, T, 512 if max(k, v) > 4 else 2048)
    cu = gen.segments_random(r, T, 4)
    cu_t = _t(cu, torch.int32)
    sh = torch.cuda.current_stream().cuda_stream
    Ad, Bd, dyd = _t(A), _t(B), _t(dy)
    for rev in (False, True):
        prob = m.Problem(rows, T, T, cu_t.data_ptr(), 4, int(rev))
        ws = torch.zeros(max(int(lib.mscan_workspace_bytes(ctypes.byref(prob), m.OP_MATRIX_FWD, k, v)),
                             int(lib.mscan_workspace_bytes(ctypes.byref(prob), m.OP_MATRIX_BWD, k, v)), 256),
                         dtype=torch.uint8, device=DEV)
        h = torch.empty((rows, T, k, v), device=DEV)
        assert lib.matrix_affine_scan_fwd(ctypes.byref(prob), k, v, _p(Ad), _p(Bd), None, _p(h), _p(ws), ws.numel(),
                                          sh) == 0
        href = oracle_lib.matrix_affine_scan_fwd(A, B, cu_seqlens=cu, reverse=rev)
        torch.cuda.synchronize()
        _same(h, href, "h")
        dA, dB = torch.empty_like(Ad), torch.empty_like(h)
        assert lib.matrix_affine_scan_bwd(ctypes.byref(prob), k, v, _p(Ad), _p(h), _p(dyd), None, _p(dA), _p(dB),
                                          None, _p(ws), ws.numel(), sh) == 0
        rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A, href, dy, cu_seqlens=cu, reverse=rev)
        torch.cuda.synchronize()
        _same(dB, rB, "dB")
        _same(dA, rA, "dA")
        assert m.workspace_error(ws) == 0
