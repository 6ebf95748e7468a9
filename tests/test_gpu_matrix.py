"""GPU parity of the matrix-affine scan (matrix_affine_scan_fwd / _bwd) against
the fp64 oracle. Tolerances per element: 2e-5 * (1 + |ref|) for h, 1e-4 * (1 + |ref|)
for dA, dB and dh0."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

TAU_FWD, TAU_BWD = 2e-5, 1e-4
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def close(gpu, ref, tau, what):
    g = gpu.detach().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    i = int(np.argmax(err))
    assert err.flat[i] <= tau, f"{what}: max rel err {err.flat[i]:.3e} at {np.unravel_index(i, err.shape)}"


def _random_case(r, k, v, rows, T, reset=0.02):
    A = (r.standard_normal((rows, T, k, k)) * (0.9 / np.sqrt(k))).astype(np.float32)
    A[r.random((rows, T)) < reset] = 0.0
    B = r.standard_normal((rows, T, k, v)).astype(np.float32)
    dy = r.standard_normal((rows, T, k, v)).astype(np.float32)
    return A, B, dy


def run(m, o, A, B, dy, h0=None, cu=None, reverse=False):
    cu_t = None if cu is None else _t(cu, torch.int32)
    h0_t = None if h0 is None else _t(h0)
    Ad = _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = o.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
    close(h, href, TAU_FWD, "h")
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rA, rB, rh0 = o.matrix_affine_scan_bwd(A, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    close(dB, rB, TAU_BWD, "dB")
    close(dA, rA, TAU_BWD, "dA")
    close(dh0, rh0, TAU_BWD, "dh0")


KV = [(2, 1), (2, 2), (4, 1), (4, 4)]


@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("T", [1, 3, 511, 513, 1025, 2049, 5000])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_lengths_lookback(m, oracle_lib, kv, T, reverse):
    """Few rows: tiles of a row chain by look-back."""
    k, v = kv
    r = np.random.default_rng(T * 10 + k * 3 + v + reverse)
    A, B, dy = _random_case(r, k, v, 3, T)
    h0 = r.standard_normal((1, 3, k, v)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, reverse=reverse)


@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_varlen(m, oracle_lib, kv, reverse):
    k, v = kv
    r = np.random.default_rng(50 + k * 3 + v + reverse)
    T = 6000
    A, B, dy = _random_case(r, k, v, 2, T)
    cu = np.array([0, 0, 1, 1000, 1001, 4500, 6000, 6000], dtype=np.int32)
    h0 = r.standard_normal((len(cu) - 1, 2, k, v)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, cu=cu, reverse=reverse)


@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_row_loop(m, oracle_lib, kv, reverse):
    """Many rows: one workgroup walks each row."""
    k, v = kv
    r = np.random.default_rng(90 + k * 3 + v + reverse)
    A, B, dy = _random_case(r, k, v, 1024, 2100)
    cu = np.array([0, 700, 700, 2100], dtype=np.int32)
    h0 = r.standard_normal((3, 1024, k, v)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, cu=cu, reverse=reverse)


def test_matrix_k1_is_scalar_scan(m):
    r = np.random.default_rng(7)
    g = r.uniform(0, 1, (4, 3000)).astype(np.float32)
    x = r.standard_normal((4, 3000)).astype(np.float32)
    hm = m.matrix_affine_scan_fwd(_t(g)[..., None, None], _t(x)[..., None, None])
    hs = m.scan_fwd(_t(g), _t(x))
    assert torch.equal(hm[..., 0, 0], hs)


def test_matrix_reset_gives_B(m):
    d = gen.matrix_orth4(B=1, N=4, T=3000, p_reset=0.05)
    h = m.matrix_affine_scan_fwd(_t(d["A"]), _t(d["B"]), h0=_t(np.ones((1, 4, 4, 4), np.float32)))
    mask = torch.as_tensor(d["reset"], device=DEV)
    assert torch.equal(h[mask], _t(d["B"])[mask])


def test_matrix_unsupported_shapes_raise(m):
    A = torch.zeros(2, 10, 3, 3, device=DEV)
    B = torch.zeros(2, 10, 3, 1, device=DEV)
    with pytest.raises(m.MscanError):
        m.matrix_affine_scan_fwd(A, B)


# ---------------------------------------------------------------------------
# full-size workloads: B=8, 512 state blocks, T=8192
# ---------------------------------------------------------------------------
@pytest.mark.timeout(400)
def test_rotation_2x1_full(m, oracle_lib):
    """A = r Rot(theta), r ~ U(0.5,1), resets with probability 1/2048; every element checked."""
    d = gen.matrix_rot2()
    A, B, dy = d["A"], d["B"], d["dy"]
    Ad = _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B))
    dA, dB, _ = m.matrix_affine_scan_bwd(Ad, h, _t(dy), need_dh0=False)
    href = oracle_lib.matrix_affine_scan_fwd(A, B)
    close(h, href, TAU_FWD, "h")
    rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A, href, dy)
    close(dB, rB, TAU_BWD, "dB")
    close(dA, rA, TAU_BWD, "dA")


@pytest.mark.timeout(400)
def test_orthogonal_4x4_full_sampled(m, oracle_lib):
    """A = 0.9 Q (Q orthogonal), B ~ N(0,1) 4x4, resets 1/2048: full tensors on the GPU,
    the oracle checks a fixed sample of whole rows."""
    d = gen.matrix_orth4()
    A, B, dy = d["A"], d["B"], d["dy"]
    Ad = _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B))
    dA, dB, _ = m.matrix_affine_scan_bwd(Ad, h, _t(dy), need_dh0=False)
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4095])
    idx = torch.as_tensor(rows, device=DEV)
    href = oracle_lib.matrix_affine_scan_fwd(A[rows], B[rows])
    close(h[idx], href, TAU_FWD, "h")
    rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A[rows], href, dy[rows])
    close(dB[idx], rB, TAU_BWD, "dB")
    close(dA[idx], rA, TAU_BWD, "dA")
    assert torch.isfinite(h).all() and torch.isfinite(dA).all()
