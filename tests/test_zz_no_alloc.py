"""scan_fwd_noalloc (the entry point for callers that cannot allocate) against
scan_fwd, through the C ABI: the same results on two calls in a row, the
second with a smaller problem, and a host-side error for a problem whose
look-back descriptors do not fit the library's fixed scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TAU = 2e-5


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _p(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def _both(m, g, x, h0, cu, reverse, dt):
    """h from scan_fwd (with a workspace) and from scan_fwd_noalloc."""
    rows, T = g.shape
    nseg = 1 if cu is None else cu.numel() - 1
    prob = m.Problem(rows, T, T, None if cu is None else cu.data_ptr(), nseg, int(reverse))
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = m.workspace_bytes(prob, m.OP_SCAN_FWD)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    h_ref = torch.full((rows, T), 7.0, device=DEV)
    h_new = torch.full((rows, T), 7.0, device=DEV)
    assert m.lib.scan_fwd(ctypes.byref(prob), dt, _p(g), _p(x), _p(h0), _p(h_ref), _p(ws), ws.numel(), sh) == 0
    assert m.lib.scan_fwd_noalloc(ctypes.byref(prob), dt, _p(g), _p(x), _p(h0), _p(h_new), sh) == 0
    torch.cuda.synchronize()
    return h_ref, h_new, need


def _close(a, b):
    a, b = a.double().cpu().numpy(), b.double().cpu().numpy()
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    err = np.abs(a - b) / (1 + np.abs(b))
    assert err.max() <= TAU, err.max()


def test_noalloc_matches_scan_fwd_twice_then_smaller(m):
    r = np.random.default_rng(77)
    # call 1: 64 rows of 5 tiles (look-back through the scratch array), packed, h0
    rows, T = 64, 5 * 4096 - 100
    g = torch.from_numpy(r.uniform(0, 1, (rows, T)).astype(np.float32)).to(DEV)
    x = torch.from_numpy(r.standard_normal((rows, T)).astype(np.float32)).to(DEV)
    cu = torch.tensor(gen.segments_random(r, T, 5), dtype=torch.int32, device=DEV)
    h0 = torch.from_numpy(r.standard_normal((5, rows)).astype(np.float32)).to(DEV)
    for rev in (False, True):
        h_ref, h_new, need = _both(m, g, x, h0, cu, rev, 0)
        assert need > 128, "the problem must chain tiles through the scratch array"
        _close(h_new, h_ref)
    # call 2 on the same array right after: fewer rows and tiles, bf16 inputs
    rows2, T2 = 16, 2 * 4096 + 33
    gb = gen.bf16_round(r.uniform(0, 1, (rows2, T2)).astype(np.float32)).reshape(rows2, T2)
    xb = gen.bf16_round(r.standard_normal((rows2, T2)).astype(np.float32)).reshape(rows2, T2)
    g2 = torch.from_numpy(gb.view(np.int16)).to(DEV).view(torch.bfloat16)
    x2 = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    h_ref, h_new, need = _both(m, g2, x2, None, None, False, 1)
    assert need > 128
    _close(h_new, h_ref)


def test_noalloc_exact_mode_bitwise(m):
    """Integer data: both entry points give the oracle's exact integers, so they
    must agree bit for bit (two calls, the second smaller)."""
    r = np.random.default_rng(78)
    for rows, T in ((40, 4 * 4096 + 5), (7, 2 * 4096 + 1)):
        gn, xn, _ = gen.exact_mode(r, (rows, T))
        g, x = torch.from_numpy(gn).to(DEV), torch.from_numpy(xn).to(DEV)
        for rev in (False, True):
            h_ref, h_new, _ = _both(m, g, x, None, None, rev, 0)
            assert torch.equal(h_ref, h_new)


def test_noalloc_rejects_problems_beyond_the_scratch(m):
    """More chained tiles than the fixed array holds: an error on the host,
    nothing enqueued (the output keeps its contents)."""
    g = torch.zeros(16, device=DEV)
    h = torch.full((16,), 7.0, device=DEV)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    prob = m.Problem(12288, 1 << 20, 1 << 20, None, 1, 0)  # 12288 rows x 256 tiles: 75 MB of descriptors
    assert m.workspace_bytes(prob, m.OP_SCAN_FWD) > 8 << 20
    assert m.lib.scan_fwd_noalloc(ctypes.byref(prob), 0, _p(g), _p(g), None, _p(h), sh) == 3
    torch.cuda.synchronize()
    assert torch.all(h == 7.0)
