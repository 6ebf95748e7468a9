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


@pytest.mark.parametrize("kv", KV + [(16, 16)])
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


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 511, 1025, 5000])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix16_lengths(m, oracle_lib, T, reverse):
    """k = v = 16 (matrix cores): chunk boundaries of 64 steps, ragged tails, h0."""
    r = np.random.default_rng(700 + T + reverse)
    A, B, dy = _random_case(r, 16, 16, 3, T)
    h0 = r.standard_normal((1, 3, 16, 16)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, reverse=reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix16_many_rows(m, oracle_lib, reverse):
    """k = v = 16 with more rows than chunks per row, segments and empty segments."""
    r = np.random.default_rng(800 + reverse)
    A, B, dy = _random_case(r, 16, 16, 96, 700)
    cu = np.array([0, 100, 100, 640, 641, 700], dtype=np.int32)
    h0 = r.standard_normal((5, 96, 16, 16)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, cu=cu, reverse=reverse)


@pytest.mark.parametrize("kv", [(2, 4), (4, 2), (1, 4)])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_core_4x4_tiles_row_groups(m, oracle_lib, kv, reverse):
    """4x4 matrix-core tiles hold 16 rows per wave: 37 rows (three groups, the
    last with 5 rows), chunks across segments, h0 and dh0 per row."""
    k, v = kv
    r = np.random.default_rng(1200 + 10 * k + v + reverse)
    A, B, dy = _random_case(r, k, v, 37, 777)
    cu = np.array([0, 5, 300, 300, 777], dtype=np.int32)
    h0 = r.standard_normal((4, 37, k, v)).astype(np.float32)
    run(m, oracle_lib, A, B, dy, h0=h0, cu=cu, reverse=reverse)


def test_matrix16_no_h0_no_dh0(m, oracle_lib):
    r = np.random.default_rng(900)
    A, B, dy = _random_case(r, 16, 16, 2, 300)
    Ad = _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B))
    href = oracle_lib.matrix_affine_scan_fwd(A, B)
    close(h, href, TAU_FWD, "h")
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, _t(dy), need_dh0=False)
    assert dh0 is None
    rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A, href, dy)
    close(dB, rB, TAU_BWD, "dB")
    close(dA, rA, TAU_BWD, "dA")


ENVELOPE = [(k, v) for k in (1, 2, 4, 8, 16) for v in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("kv", ENVELOPE)
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_envelope(m, oracle_lib, kv, reverse):
    """Every (k, v) of the envelope {1, 2, 4, 8, 16}^2: several 64-step chunks,
    a ragged tail, segments (one empty) with h0."""
    k, v = kv
    r = np.random.default_rng(1000 + 40 * k + v + reverse)
    A, B, dy = _random_case(r, k, v, 2, 333)
    cu = np.array([0, 64, 64, 200, 333], dtype=np.int32)
    h0 = r.standard_normal((4, 2, k, v)).astype(np.float32)
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


@pytest.mark.timeout(400)
def test_orthogonal_16x16_full_sampled(m, oracle_lib):
    """k = v = 16 at the benchmarked size (B=8 x 64 blocks, T=4096): A = 0.9 Q,
    resets 1/2048; the oracle checks whole rows drawn from every 64-row block
    boundary region."""
    d = gen.matrix_orth16()
    A, B, dy = d["A"], d["B"], d["dy"]
    Ad = _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B))
    dA, dB, _ = m.matrix_affine_scan_bwd(Ad, h, _t(dy), need_dh0=False)
    rows = np.array([0, 1, 63, 64, 300, 511])
    idx = torch.as_tensor(rows, device=DEV)
    href = oracle_lib.matrix_affine_scan_fwd(A[rows], B[rows])
    close(h[idx], href, TAU_FWD, "h")
    rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A[rows], href, dy[rows])
    close(dB[idx], rB, TAU_BWD, "dB")
    close(dA[idx], rA, TAU_BWD, "dA")
    assert torch.isfinite(h).all() and torch.isfinite(dA).all()


# ---------------------------------------------------------------------------
# exact mode, strided rows, non-finite containment
# ---------------------------------------------------------------------------
def _signed_perm_case(r, k, v, rows, T, max_run=2048, p_zero=0.02):
    """Integer data whose matrix scan is exact in fp32 in every association order:
    A_t a signed permutation matrix or 0 (a zero at least every max_run steps),
    B, dy in {-1, 0, 1}. Every product has one nonzero term per entry, so
    |h|, |lam| <= max_run and |dA| <= max_run^2 < 2^24."""
    A = np.zeros((rows, T, k, k), np.float32)
    perm = np.argsort(r.random((rows, T, k)), axis=-1)
    sign = r.choice(np.array([-1.0, 1.0], np.float32), size=(rows, T, k))
    for i in range(k):
        np.put_along_axis(A[:, :, i, :], perm[:, :, i:i + 1], sign[:, :, i:i + 1], axis=-1)
    zero = r.random((rows, T)) < p_zero
    zero[:, max_run - 1::max_run] = True
    A[zero] = 0.0
    B = r.integers(-1, 2, size=(rows, T, k, v)).astype(np.float32)
    dy = r.integers(-1, 2, size=(rows, T, k, v)).astype(np.float32)
    return A, B, dy


@pytest.mark.parametrize("kv", KV + [(16, 16), (8, 8), (16, 1), (1, 16), (2, 16), (8, 2)])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_exact_mode_bitwise(m, oracle_lib, kv, reverse):
    """Integer data: the GPU must equal the oracle bit for bit (segments, resets,
    h0 injection, tile and look-back boundaries, reverse, adjoint). An entry of
    dA sums v products, so with v > 4 runs stop at 512 steps: every partial sum
    stays below 16 * 512^2 = 2^22."""
    k, v = kv
    r = np.random.default_rng(300 + 10 * k + v + reverse)
    rows, T = 3, 9001
    A, B, dy = _signed_perm_case(r, k, v, rows, T, max_run=512 if max(k, v) > 4 else 2048)
    cu = gen.segments_random(r, T, 9)
    h0 = r.integers(-1, 2, size=(len(cu) - 1, rows, k, v)).astype(np.float32)
    cu_t, h0_t, Ad = _t(cu, torch.int32), _t(h0), _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(h.cpu().double().numpy(), href)
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(dB.cpu().double().numpy(), rB)
    assert np.array_equal(dA.cpu().double().numpy(), rA)
    assert np.array_equal(dh0.cpu().double().numpy(), rh0)


# Forward chunks are shared by several waves (16x16 tile: waves of 16 steps,
# 64 per chunk; 4x4 tile: waves of 256 steps, 1024 per chunk); backward chunks
# are 2 x 16 and 1 x 256 steps.
@pytest.mark.parametrize("kv,span,chunk", [((16, 16), 16, 64), ((8, 2), 16, 64), ((4, 4), 256, 1024),
                                           ((1, 4), 256, 1024)])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_exact_wave_and_chunk_boundaries(m, oracle_lib, kv, span, chunk, reverse):
    """Integer data, bit for bit against the oracle: sequence starts (in
    processing order) and resets placed on, one before and one after the
    boundaries between the waves of a chunk and between chunks, a sequence
    that is exactly one wave span, a chunk whose second wave starts with a
    reset, and chunks crossed by one long sequence (the carry passed from wave
    to wave and chunk to chunk)."""
    k, v = kv
    r = np.random.default_rng(900 + 10 * k + v + reverse)
    rows, T = 3, 4 * chunk + span // 2 + 3
    A, B, dy = _signed_perm_case(r, k, v, rows, T, max_run=512 if max(k, v) > 4 else 2048, p_zero=0.0)
    # processing-order positions: chunk 0 is cut at its wave edges, chunk 1 by
    # a one-span sequence, chunk 2 has no boundary, chunk 3 is cut just after
    # a chunk edge and just before a wave edge
    starts = {span, 2 * span - 1, chunk - 1, chunk + span, chunk + 2 * span, 3 * chunk + 1, 3 * chunk + 2 * span - 1}
    resets = {chunk + 3 * span, span + 1, 2 * chunk + span - 1, 2 * chunk + 2 * span, 4 * chunk}
    starts = sorted(j for j in starts if 0 < j < T)
    phys = (lambda j: T - 1 - j) if reverse else (lambda j: j)
    # a processing-order start at j is physical step j (forward) or the end of
    # the physical segment ending at T - 1 - j (reverse)
    cuts = sorted({T - j for j in starts} if reverse else set(starts))
    cu = np.array([0] + cuts + [T], np.int64)
    for j in resets:
        if j < T:
            A[:, phys(j)] = 0.0
    h0 = r.integers(-1, 2, size=(len(cu) - 1, rows, k, v)).astype(np.float32)
    cu_t, h0_t, Ad = _t(cu, torch.int32), _t(h0), _t(A)
    h = m.matrix_affine_scan_fwd(Ad, _t(B), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(h.cpu().double().numpy(), href)
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    assert np.array_equal(dB.cpu().double().numpy(), rB)
    assert np.array_equal(dA.cpu().double().numpy(), rA)
    assert np.array_equal(dh0.cpu().double().numpy(), rh0)


@pytest.mark.parametrize("kv", [(2, 1), (4, 4), (16, 16), (8, 2), (1, 4)])
@pytest.mark.parametrize("T", [700, 5001])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_odd_row_stride(m, oracle_lib, kv, T, reverse):
    """row_stride = T + 1 through the C ABI: with k x v = 2, every other row starts
    8 bytes off a 16-byte boundary (the unaligned staging path)."""
    import ctypes
    k, v = kv
    r = np.random.default_rng(400 + T + k + reverse)
    rows, stride = 5, T + 1
    A, B, dy = _random_case(r, k, v, rows, stride)
    h0 = r.standard_normal((1, rows, k, v)).astype(np.float32)
    Ad, Bd, dyd, h0d = _t(A), _t(B), _t(dy), _t(h0)
    h = torch.full((rows, stride, k, v), 7.0, device=DEV)
    prob = m.Problem(rows, T, stride, None, 1, int(reverse))
    ws = torch.zeros(m.workspace_bytes(prob, m.OP_MATRIX_BWD, k, v) + m.workspace_bytes(prob, m.OP_MATRIX_FWD, k, v),
                     dtype=torch.uint8, device=DEV)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(prob), k, v, p(Ad), p(Bd), p(h0d), p(h), p(ws), ws.numel(), sh) == 0
    href = oracle_lib.matrix_affine_scan_fwd(A[:, :T], B[:, :T], h0=h0, reverse=reverse)
    close(h[:, :T], href, TAU_FWD, "h")
    assert torch.all(h[:, T:] == 7.0), "wrote past the row"
    dA = torch.full((rows, stride, k, k), 7.0, device=DEV)
    dB = torch.full((rows, stride, k, v), 7.0, device=DEV)
    dh0 = torch.empty((1, rows, k, v), device=DEV)
    hin = h.clone()
    assert m.lib.matrix_affine_scan_bwd(ctypes.byref(prob), k, v, p(Ad), p(hin), p(dyd), p(h0d), p(dA), p(dB),
                                        p(dh0), p(ws), ws.numel(), sh) == 0
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A[:, :T], href, dy[:, :T], h0=h0, reverse=reverse)
    close(dB[:, :T], rB, TAU_BWD, "dB")
    close(dA[:, :T], rA, TAU_BWD, "dA")
    close(dh0, rh0, TAU_BWD, "dh0")
    assert torch.all(dA[:, T:] == 7.0) and torch.all(dB[:, T:] == 7.0), "wrote past the row"


@pytest.mark.parametrize("kv", [(2, 1), (4, 4), (16, 16), (8, 4)])
def test_matrix_nan_poison_stays_in_its_sequence(m, oracle_lib, kv):
    """A sequence full of NaN/Inf changes nothing in any other sequence (bitwise)."""
    k, v = kv
    r = np.random.default_rng(500 + k)
    T = 7000
    A, B, dy = _random_case(r, k, v, 2, T)
    cu = np.array([0, 1500, 4000, 4001, 7000], dtype=np.int32)
    Ap, Bp = A.copy(), B.copy()
    Ap[:, 1500:4000] = np.nan
    Bp[:, 1500:3000] = np.inf
    cu_t = _t(cu, torch.int32)
    keep = np.r_[0:1500, 4000:7000]
    for rev in (False, True):
        h = m.matrix_affine_scan_fwd(_t(A), _t(B), cu_seqlens=cu_t, reverse=rev)
        hp = m.matrix_affine_scan_fwd(_t(Ap), _t(Bp), cu_seqlens=cu_t, reverse=rev)
        assert torch.equal(h[:, keep], hp[:, keep])
        d1 = m.matrix_affine_scan_bwd(_t(A), h, _t(dy), cu_seqlens=cu_t, reverse=rev)
        d2 = m.matrix_affine_scan_bwd(_t(Ap), hp, _t(dy), cu_seqlens=cu_t, reverse=rev)
        for a, b in zip(d1[:2], d2[:2]):
            assert torch.equal(a[:, keep], b[:, keep])
        assert torch.equal(d1[2][[0, 2, 3]], d2[2][[0, 2, 3]])
        close(h[:, keep], oracle_lib.matrix_affine_scan_fwd(A, B, cu_seqlens=cu, reverse=rev)[:, keep], TAU_FWD, "h")


@pytest.mark.parametrize("k", [2, 4, 16])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_cumprod(m, k, reverse):
    """Running products against explicit fp64 matrix products per sequence,
    and the gradient through the autograd op against finite differences of a
    scalar loss."""
    r = np.random.default_rng(1100 + k + reverse)
    T = 150
    A = (r.standard_normal((2, T, k, k)) * (1.0 / np.sqrt(k))).astype(np.float32)
    cu = np.array([0, 70, 70, 150], dtype=np.int32)
    Ab = m.matrix_cumprod(_t(A), cu_seqlens=_t(cu, torch.int32), reverse=reverse).cpu().double().numpy()
    ref = np.empty(A.shape)
    for row in range(2):
        for s0, s1 in zip(cu[:-1], cu[1:]):
            acc = np.eye(k)
            steps = range(s1 - 1, s0 - 1, -1) if reverse else range(s0, s1)
            for t in steps:
                acc = A[row, t].astype(np.float64) @ acc
                ref[row, t] = acc
    err = np.abs(Ab - ref) / (1.0 + np.abs(ref))
    assert err.max() <= TAU_FWD, err.max()
    # gradient of sum(W * Abar) w.r.t. A, checked on a few entries by central differences in fp64
    W = r.standard_normal(A.shape)
    Ad = _t(A).requires_grad_(True)
    (m.matrix_cumprod(Ad, cu_seqlens=_t(cu, torch.int32), reverse=reverse) * _t(W)).sum().backward()
    g = Ad.grad.cpu().double().numpy()

    def loss(Ax):
        tot = 0.0
        for row in range(2):
            for s0, s1 in zip(cu[:-1], cu[1:]):
                acc = np.eye(k)
                steps = range(s1 - 1, s0 - 1, -1) if reverse else range(s0, s1)
                for t in steps:
                    acc = Ax[row, t] @ acc
                    tot += float((W[row, t] * acc).sum())
        return tot
    A64 = A.astype(np.float64)
    for (row, t, i, j) in [(0, 0, 0, 0), (0, 69, k - 1, 0), (1, 100, 0, k - 1), (1, 149, k - 1, k - 1), (1, 70, 1, 0)]:
        e = np.zeros_like(A64)
        e[row, t, i, j] = 1e-6
        fd = (loss(A64 + e) - loss(A64 - e)) / 2e-6
        assert abs(g[row, t, i, j] - fd) <= 1e-3 * (1 + abs(fd)), (row, t, i, j, g[row, t, i, j], fd)



@pytest.mark.timeout(400)
def test_matrix16_row_beyond_2_31_elements(m, oracle_lib):
    """One 16x16 row of T = 2^23 + 5 steps: 2^31 + 1280 floats per array
    (64-bit element offsets on the matrix cores, 262145 chained chunks).
    A = I with A = 0 every 1000 steps, B = dy = all-ones blocks: h_t =
    (t mod 1000 + 1) J, lam_t = L_t J with L_t the steps to the next reset or
    the row end, dA_t = 16 L_t h_{t-1} J (J the all-ones block), every value an
    integer below 2^24, so exact. Checked over the whole row in slices and
    against the oracle on a window that starts at a reset."""
    T, k = 2**23 + 5, 16
    free, _ = torch.cuda.mem_get_info()
    if free < 96 * 2**30:
        pytest.skip("needs 96 GiB of free device memory")
    A = torch.eye(k, device=DEV).expand(T, k, k).contiguous()
    A[::1000] = 0.0
    B = torch.ones((T, k, k), device=DEV)
    h = m.matrix_affine_scan_fwd(A, B)
    dA, dB, dh0 = m.matrix_affine_scan_bwd(A, h, B)
    step = 2**20
    for lo in range(0, T, step):
        hi = min(lo + step, T)
        t = torch.arange(lo, hi, device=DEV, dtype=torch.int64)
        hv = (t % 1000 + 1).float()
        assert torch.equal(h[lo:hi], hv[:, None, None].expand(-1, k, k)), f"h slice at {lo}"
        L = torch.minimum(1000 - t % 1000, T - t).float()
        assert torch.equal(dB[lo:hi], L[:, None, None].expand(-1, k, k)), f"dB slice at {lo}"
        hprev = torch.where(t % 1000 == 0, 1000.0, (t % 1000).float())
        if lo == 0:
            hprev[0] = 0.0  # no h0
        assert torch.equal(dA[lo:hi], (16.0 * L * hprev)[:, None, None].expand(-1, k, k)), f"dA slice at {lo}"
        del t, hv, L, hprev
    assert torch.count_nonzero(dh0).item() == 0  # A_0 = 0
    w0 = ((T - 1) // 1000) * 1000
    Aw, Bw = A[w0:].cpu().numpy()[None], B[w0:].cpu().numpy()[None]
    href = oracle_lib.matrix_affine_scan_fwd(Aw, Bw)
    assert np.array_equal(h[w0:].cpu().double().numpy()[None], href), "h window"


@pytest.mark.parametrize("k", [2, 4, 16])
def test_matrix_graph_capture_replays(m, oracle_lib, k):
    """Matrix forward + backward (VALU and matrix-core kernels, chained chunks)
    captured in a HIP graph and replayed with new inputs, eager calls between
    replays; every replay matches the oracle."""
    r = np.random.default_rng(4343 + k)
    rows, T = 3, 3000
    A0 = (r.standard_normal((rows, T, k, k)) * (0.9 / np.sqrt(k))).astype(np.float32)
    B0 = r.standard_normal((rows, T, k, k)).astype(np.float32)
    dy = r.standard_normal((rows, T, k, k)).astype(np.float32)
    At, Bt, dyt = _t(A0), _t(B0), _t(dy)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            hw = m.matrix_affine_scan_fwd(At, Bt)
            m.matrix_affine_scan_bwd(At, hw, dyt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h = m.matrix_affine_scan_fwd(At, Bt)
        dA, dB, _ = m.matrix_affine_scan_bwd(At, h, dyt)
    for rep in range(3):
        A = (r.standard_normal((rows, T, k, k)) * (0.9 / np.sqrt(k))).astype(np.float32)
        B = r.standard_normal((rows, T, k, k)).astype(np.float32)
        At.copy_(_t(A))
        Bt.copy_(_t(B))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        href = oracle_lib.matrix_affine_scan_fwd(A, B)
        close(h, href, TAU_FWD, f"h replay {rep}")
        rA, rB, _ = oracle_lib.matrix_affine_scan_bwd(A, href, dy)
        close(dA, rA, TAU_BWD, f"dA replay {rep}")
        close(dB, rB, TAU_BWD, f"dB replay {rep}")
        he = m.matrix_affine_scan_fwd(At, Bt)
        torch.cuda.synchronize()
        close(he, href, TAU_FWD, f"eager h after replay {rep}")


@pytest.mark.parametrize("kv", [(2, 1), (2, 2), (4, 1), (4, 4), (16, 16), (8, 2), (1, 4), (4, 2)])
@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_reset_after_nan_matches_oracle(m, oracle_lib, kv, reverse):
    """NaN inside sequences (injections, output gradients and h0) followed by
    all-zero transitions (resets, "Our RG-LRU GPU audit", "Exact real chunk
    algebra"): on exact-mode data every output equals the oracle bit for bit,
    NaN positions included; a reset on a sequence's first step drops a NaN h0
    and passes no gradient to it."""
    k, v = kv
    r = np.random.default_rng(600 + 10 * k + v + reverse)
    rows, T = 3, 3001
    A, B, dy = _signed_perm_case(r, k, v, rows, T, max_run=512 if max(k, v) > 4 else 2048)
    B[r.random((rows, T, k, v)) < 0.001] = np.nan
    dy[r.random((rows, T, k, v)) < 0.001] = np.nan
    cu = gen.segments_random(r, T, 6)
    h0 = r.integers(-1, 2, size=(6, rows, k, v)).astype(np.float32)
    for s_, row_ in ((1, 0), (3, 2)):
        h0[s_, row_] = np.nan
        if cu[s_] < cu[s_ + 1]:
            A[row_, cu[s_]] = 0.0
            A[row_, cu[s_ + 1] - 1] = 0.0
    cu_t, h0_t, Ad = _t(cu, torch.int32), _t(h0), _t(A)

    def same(gpu, ref, what):
        g = gpu.cpu().double().numpy()
        ok = (g == ref) | (np.isnan(g) & np.isnan(ref))
        assert ok.all(), f"{what}: {int((~ok).sum())} mismatches"

    h = m.matrix_affine_scan_fwd(Ad, _t(B), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu, reverse=reverse)
    same(h, href, "h")
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    same(dB, rB, "dB")
    same(dA, rA, "dA")
    same(dh0, rh0, "dh0")


@pytest.mark.parametrize("kv", [(2, 1), (4, 4), (16, 16)])
def test_matrix_strided_rows_binding(m, oracle_lib, kv):
    """The binding passes a row stride through for every matrix call: rows of a
    larger buffer (views), forward and backward."""
    k, v = kv
    r = np.random.default_rng(700 + k)
    rows, T, stride = 3, 1500, 1503
    A, B, dy = _random_case(r, k, v, rows, stride)
    Ad, Bd, dyd = _t(A)[:, :T], _t(B)[:, :T], _t(dy)[:, :T]
    h = m.matrix_affine_scan_fwd(Ad, Bd)
    href = oracle_lib.matrix_affine_scan_fwd(A[:, :T], B[:, :T])
    close(h, href, TAU_FWD, "h")
    dA, dB, dh0 = m.matrix_affine_scan_bwd(Ad, h, dyd)
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A[:, :T], href, dy[:, :T])
    close(dA, rA, TAU_BWD, "dA")
    close(dB, rB, TAU_BWD, "dB")
    close(dh0, rh0, TAU_BWD, "dh0")
