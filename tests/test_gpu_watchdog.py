"""A look-back wait that gives up is reported, never silent.

The host makes a kernel's own bounded wait run out: a partial launch runs only
the last block of a chained call (its predecessors never publish) with a small
spin limit. Every launched block still ends; its outputs that needed the
missing carry are NaN; the workspace's error word reads MSCAN_ERR_TIMEOUT; the
binding's debug mode raises on it; and the next full call on the same
workspace clears it and is correct ("Triton scan kernels", "The dispatch
seam": failures are reported, not turned into silent wrong results).
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SPIN = 2000  # polls before a wait gives up (about a hundred microseconds)


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _case(r, k, v, rows, T):
    """Transitions of norm just below 1 (gates in [0.998, 1), 0.999 times an
    orthogonal matrix), so that no product over a tile underflows and every
    output of a tile depends on the state entering it."""
    if k == 1 and v == 1:
        a = r.uniform(0.998, 1.0, (rows, T)).astype(np.float32)
        b = r.standard_normal((rows, T)).astype(np.float32)
        return a, b
    q, _ = np.linalg.qr(r.standard_normal((rows, T, k, k)))
    a = (0.999 * q).astype(np.float32)
    b = r.standard_normal((rows, T, k, v)).astype(np.float32)
    return a, b


# (k, v, T, first step of the last row's last tile): the scalar scan (3 tiles
# of 4096), the 2x1 VALU kernel (3 tiles of 2048 steps), the 4x4 matrix-core
# row-segment forward (3 chunks of 1024 steps), the 16x16 and 8x2 matrix-core
# forward chunks (4 chunks of 64 steps)
CASES = [(1, 1, 3 * 4096, 8192), (2, 1, 5000, 4096), (4, 4, 2500, 2048), (16, 16, 200, 192), (8, 2, 200, 192)]


@pytest.mark.parametrize("k,v,T,last", CASES)
def test_tripped_wait_is_reported(m, oracle_lib, k, v, T, last):
    r = np.random.default_rng(2000 + 10 * k + v)
    rows = 2
    a, b = _case(r, k, v, rows, T)
    ad, bd = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    out = torch.full(b.shape, 7.0, device=DEV)
    prob = m.Problem(rows, T, T, None, 1, 0)
    op_bytes = m.workspace_bytes(prob, m.OP_MATRIX_FWD if (k, v) != (1, 1) else m.OP_SCAN_FWD, k, v)
    ws = torch.empty(max(op_bytes, 4096), dtype=torch.uint8, device=DEV)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    # blocks of the call's grid: tiles (or chunks) per row times rows
    per_row = {(1, 1): 3, (2, 1): 3, (4, 4): 3, (16, 16): 4, (8, 2): 4}[(k, v)]
    total = rows * per_row
    # a block range just past the grid is refused on the host
    assert m.lib.mscan_debug_partial_fwd(ctypes.byref(prob), k, v, p(ad), p(bd), p(out), p(ws), ws.numel(),
                                         total, 1, SPIN, sh) == 1
    # only the last block (last tile of the last row): its predecessor never publishes
    assert m.lib.mscan_debug_partial_fwd(ctypes.byref(prob), k, v, p(ad), p(bd), p(out), p(ws), ws.numel(),
                                         total - 1, 1, SPIN, sh) == 0
    torch.cuda.synchronize()
    assert m.workspace_error(ws) == 5
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[rows - 1, last:])), "the block that lost its carry wrote NaN, no plausible value"
    assert np.all(o[:rows - 1] == 7.0) and np.all(o[rows - 1, :last] == 7.0), "blocks not launched wrote nothing"
    # debug mode turns the word into an exception
    old = m.debug_enabled()
    try:
        m.set_debug(True)
        with pytest.raises(m.MscanError) as e:
            m._raise_if_tripped("partial launch", ws.data_ptr(), ws.numel(), ws.device,
                                torch.cuda.current_stream().cuda_stream)
        assert e.value.status == 5
    finally:
        m.set_debug(old)
    # a full call on the same workspace clears the word and is correct (on
    # well-conditioned data: transitions of norm 0.999 over thousands of steps
    # amplify fp32 rounding past the 2e-5 gate)
    if (k, v) == (1, 1):
        a = r.uniform(0.0, 1.0, (rows, T)).astype(np.float32)
    else:
        a = (r.standard_normal((rows, T, k, k)) * (0.9 / np.sqrt(k))).astype(np.float32)
    ad = torch.from_numpy(a).to(DEV)
    if (k, v) == (1, 1):
        assert m.lib.scan_fwd(ctypes.byref(prob), 0, p(ad), p(bd), None, p(out), p(ws), ws.numel(), sh) == 0
        ref = oracle_lib.scan_fwd(a, b)
    else:
        assert m.lib.matrix_affine_scan_fwd(ctypes.byref(prob), k, v, p(ad), p(bd), None, p(out), p(ws), ws.numel(),
                                            sh) == 0
        ref = oracle_lib.matrix_affine_scan_fwd(a, b)
    torch.cuda.synchronize()
    assert m.workspace_error(ws) == 0
    got = out.cpu().double().numpy()
    assert np.max(np.abs(got - ref) / (1 + np.abs(ref))) <= 2e-5


def test_debug_mode_full_calls_do_not_raise(m):
    """Debug mode on ordinary chained calls: the error word stays clear, and a
    malformed cu_seqlens is refused on the host before anything is enqueued."""
    r = np.random.default_rng(2100)
    old = m.debug_enabled()
    try:
        m.set_debug(True)
        g = torch.from_numpy(r.uniform(0, 1, (4, 9000)).astype(np.float32)).to(DEV)
        x = torch.from_numpy(r.standard_normal((4, 9000)).astype(np.float32)).to(DEV)
        cu = torch.tensor([0, 100, 5000, 9000], dtype=torch.int32, device=DEV)
        h = m.scan_fwd(g, x, cu_seqlens=cu)
        m.scan_bwd(g, h, torch.ones_like(h), cu_seqlens=cu)
        m.scan_log_fwd(torch.log(g), x, cu_seqlens=cu)
        A = torch.from_numpy((r.standard_normal((2, 700, 4, 4)) * 0.4).astype(np.float32)).to(DEV)
        B = torch.from_numpy(r.standard_normal((2, 700, 4, 4)).astype(np.float32)).to(DEV)
        hm = m.matrix_affine_scan_fwd(A, B)
        m.matrix_affine_scan_bwd(A, hm, torch.ones_like(hm))
        out = torch.full_like(h, 7.0)
        for bad in ([0, 5000, 100, 9000], [0, 100, 9001], [1, 100, 9000]):
            with pytest.raises(ValueError):
                m.scan_fwd(g, x, cu_seqlens=torch.tensor(bad, dtype=torch.int32, device=DEV), out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)
    finally:
        m.set_debug(old)
