"""GPU parity of the scalar scan (scan_fwd / scan_bwd) against the fp64 oracle.

Tolerances (per element, every output): |gpu - ref| <= tau * (1 + |ref|) with
tau = 2e-5 for forward states and 1e-4 for gradients; bf16 inputs reach the
oracle already rounded (exact widening). Exact-mode inputs (integer data whose
scan is exact in any association order) must match bit for bit, which pins the
indexing: sequence boundaries, resets, direction, shifts and tile seams.
"""
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


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def close(gpu, ref, tau, what):
    g = gpu.detach().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.flat[i] <= tau, f"{what}: max rel err {err.flat[i]:.3e} at {np.unravel_index(i, err.shape)} (gpu {g.flat[i]!r}, ref {ref.flat[i]!r})"


def exact(gpu, ref, what):
    g = gpu.detach().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    bad = np.nonzero(g != ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} mismatches, first at {tuple(b[0] for b in bad)}: gpu {g[tuple(b[0] for b in bad)]} ref {ref[tuple(b[0] for b in bad)]}"


def run_case(m, o, g, x, dy, h0=None, cu=None, reverse=False, bits=None, check=close):
    """Forward and backward on the GPU vs the oracle; g, x, dy numpy fp32 [rows, T]."""
    cu_t = None if cu is None else _t(cu, torch.int32)
    h0_t = None if h0 is None else _t(h0)
    if bits is None:
        gg, xx = _t(g), _t(x)
    else:
        gg, xx = _bf16(bits[0]), _bf16(bits[1])
    h = m.scan_fwd(gg, xx, h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = o.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=reverse)
    if check is close:
        close(h, href, TAU_FWD, "h")
    else:
        exact(h, href, "h")
    dx, dg, dh0 = m.scan_bwd(gg, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rx, rg, rh0 = o.scan_bwd(g, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    if check is close:
        close(dx, rx, TAU_BWD, "dx")
        close(dg, rg, TAU_BWD, "dg")
        close(dh0, rh0, TAU_BWD, "dh0")
    else:
        exact(dx, rx, "dx")
        exact(dg, rg, "dg")
        exact(dh0, rh0, "dh0")
    return h


# ---------------------------------------------------------------------------
# the README quick-start workload (C=4, T=128, one sequence)
# ---------------------------------------------------------------------------
def test_quickstart(m, oracle_lib):
    d = gen.quickstart()
    run_case(m, oracle_lib, d["g"], d["x"], d["dy"])
    # the same problem stated with cu_seqlens = [0, T] runs the packed kernels
    run_case(m, oracle_lib, d["g"], d["x"], d["dy"], cu=d["cu_seqlens"])


# ---------------------------------------------------------------------------
# dense rows: lengths around the vector width and the 4096-element tile
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 63, 127, 1000, 4095, 4096, 4097, 8192, 9001, 20000])
@pytest.mark.parametrize("reverse", [False, True])
def test_dense_lengths(m, oracle_lib, T, reverse):
    r = np.random.default_rng(T * 2 + reverse)
    rows = 5
    g = r.uniform(0, 1, (rows, T)).astype(np.float32)
    x = r.standard_normal((rows, T)).astype(np.float32)
    dy = r.standard_normal((rows, T)).astype(np.float32)
    h0 = r.standard_normal(rows).astype(np.float32)
    run_case(m, oracle_lib, g, x, dy, h0=h0, reverse=reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_exact_mode_dense(m, oracle_lib, reverse):
    r = np.random.default_rng(11 + reverse)
    g, x, dy = gen.exact_mode(r, (6, 30000))
    h0 = r.integers(-1, 2, 6).astype(np.float32)
    run_case(m, oracle_lib, g, x, dy, h0=h0, reverse=reverse, check=exact)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("nseg", [1, 2, 7, 40, 300])
def test_exact_mode_varlen(m, oracle_lib, reverse, nseg):
    r = np.random.default_rng(100 + nseg + reverse)
    T = 25000
    g, x, dy = gen.exact_mode(r, (3, T))
    cu = gen.segments_random(r, T, nseg, allow_empty=True)
    h0 = r.integers(-1, 2, (nseg, 3)).astype(np.float32)
    run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=reverse, check=exact)


def test_length_one_sequences(m, oracle_lib):
    """Every element its own sequence (more sequences than the tile caches in LDS)."""
    r = np.random.default_rng(5)
    T = 6000
    g = r.uniform(0, 1, (2, T)).astype(np.float32)
    x = r.standard_normal((2, T)).astype(np.float32)
    dy = r.standard_normal((2, T)).astype(np.float32)
    cu = np.arange(T + 1, dtype=np.int32)
    h0 = r.standard_normal((T, 2)).astype(np.float32)
    for rev in (False, True):
        run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=rev)


def test_empty_sequences_everywhere(m, oracle_lib):
    r = np.random.default_rng(6)
    T = 9000
    g = r.uniform(0, 1, (2, T)).astype(np.float32)
    x = r.standard_normal((2, T)).astype(np.float32)
    dy = r.standard_normal((2, T)).astype(np.float32)
    cu = np.array([0, 0, 0, 4096, 4096, 4097, 8999, 9000, 9000, 9000], dtype=np.int32)
    h0 = r.standard_normal((len(cu) - 1, 2)).astype(np.float32)
    for rev in (False, True):
        run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=rev)


def test_nan_poison_stays_in_its_sequence(m, oracle_lib):
    """A sequence full of NaN/Inf changes nothing in any other sequence (bitwise)."""
    r = np.random.default_rng(7)
    T = 12000
    g = r.uniform(0, 1, (3, T)).astype(np.float32)
    x = r.standard_normal((3, T)).astype(np.float32)
    dy = r.standard_normal((3, T)).astype(np.float32)
    cu = np.array([0, 3000, 7000, 7001, 12000], dtype=np.int32)
    gp, xp = g.copy(), x.copy()
    gp[:, 3000:7000] = np.nan
    xp[:, 3000:5000] = np.inf
    cu_t = _t(cu, torch.int32)
    for rev in (False, True):
        h = m.scan_fwd(_t(g), _t(x), cu_seqlens=cu_t, reverse=rev)
        hp = m.scan_fwd(_t(gp), _t(xp), cu_seqlens=cu_t, reverse=rev)
        keep = np.r_[0:3000, 7000:12000]
        assert torch.equal(h[:, keep], hp[:, keep])
        d1 = m.scan_bwd(_t(g), h, _t(dy), cu_seqlens=cu_t, reverse=rev)
        d2 = m.scan_bwd(_t(gp), hp, _t(dy), cu_seqlens=cu_t, reverse=rev)
        for a, b in zip(d1[:2], d2[:2]):
            assert torch.equal(a[:, keep], b[:, keep])
        assert torch.equal(d1[2][[0, 2, 3]], d2[2][[0, 2, 3]])
        close(h[:, keep], oracle_lib.scan_fwd(g, x, cu_seqlens=cu, reverse=rev)[:, keep], TAU_FWD, "h")


@pytest.mark.parametrize("T,stride", [(1001, 1003), (4097, 4099), (8190, 8193), (5, 7)])
def test_unaligned_rows(m, oracle_lib, T, stride):
    """Rows that start at every alignment within a 16-byte vector (row_stride not a multiple of 4)."""
    r = np.random.default_rng(T)
    rows = 9
    full_g = r.uniform(0, 1, (rows, stride)).astype(np.float32)
    full_x = r.standard_normal((rows, stride)).astype(np.float32)
    g, x = full_g[:, :T], full_x[:, :T]
    h0 = r.standard_normal(rows).astype(np.float32)
    gt, xt = _t(full_g)[:, :T], _t(full_x)[:, :T]
    out = torch.full((rows, stride), 7.0, device=DEV)
    for rev in (False, True):
        h = m.scan_fwd(gt, xt, h0=_t(h0), reverse=rev, out=out[:, :T])
        close(h, oracle_lib.scan_fwd(g, x, h0=h0, reverse=rev), TAU_FWD, "h")
        assert torch.all(out[:, T:] == 7.0), "wrote outside the rows"


def test_bf16_inputs(m, oracle_lib):
    r = np.random.default_rng(8)
    T = 15000
    gb = gen.bf16_round(r.uniform(0, 1, (4, T)).astype(np.float32))
    xb = gen.bf16_round(r.standard_normal((4, T)).astype(np.float32))
    g, x = gen.bf16_bits_to_f32(gb).reshape(4, T), gen.bf16_bits_to_f32(xb).reshape(4, T)
    dy = r.standard_normal((4, T)).astype(np.float32)
    cu = gen.segments_random(r, T, 5)
    h0 = r.standard_normal((5, 4)).astype(np.float32)
    for rev in (False, True):
        run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=rev, bits=(gb, xb))


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("T,stride", [(40000, 40000), (40001, 40003), (8192, 8192), (8193, 8195)])
def test_16bit_forward_tiles(m, oracle_lib, dt, T, stride):
    """16-bit forward: rows of several 4096-element tiles (look-back), exactly
    two tiles, two tiles plus one element, rows starting at odd 2-byte offsets;
    packed sequences with h0, both directions."""
    r = np.random.default_rng(50 + T + stride + (dt == "fp16"))
    rows = 3
    g32 = r.uniform(0, 1, (rows, stride)).astype(np.float32)
    x32 = r.standard_normal((rows, stride)).astype(np.float32)
    if dt == "bf16":
        gb = gen.bf16_round(g32).reshape(rows, stride)
        xb = gen.bf16_round(x32).reshape(rows, stride)
        g = gen.bf16_bits_to_f32(gb).reshape(rows, stride)[:, :T]
        x = gen.bf16_bits_to_f32(xb).reshape(rows, stride)[:, :T]
        gt, xt = _bf16(gb)[:, :T], _bf16(xb)[:, :T]
    else:
        g16, x16 = g32.astype(np.float16), x32.astype(np.float16)
        g, x = g16[:, :T].astype(np.float32), x16[:, :T].astype(np.float32)
        gt, xt = torch.from_numpy(g16).to(DEV)[:, :T], torch.from_numpy(x16).to(DEV)[:, :T]
    cu = gen.segments_random(r, T, 6)
    h0 = r.standard_normal((6, rows)).astype(np.float32)
    for rev in (False, True):
        out = torch.full((rows, stride), 7.0, device=DEV)
        h = m.scan_fwd(gt, xt, h0=_t(h0), cu_seqlens=_t(cu, torch.int32), reverse=rev, out=out[:, :T])
        close(h, oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=rev), TAU_FWD, "h")
        assert torch.all(out[:, T:] == 7.0), "wrote outside the rows"
        h = m.scan_fwd(gt, xt, reverse=rev, out=out[:, :T])
        close(h, oracle_lib.scan_fwd(g, x, reverse=rev), TAU_FWD, "h dense")


@pytest.mark.parametrize("T,stride", [(15000, 15000), (4097, 4099)])
def test_fp16_inputs(m, oracle_lib, T, stride):
    """fp16 g and x (widened exactly), packed sequences with h0, both directions;
    odd row strides start rows at every 2-byte offset of an 8-byte vector."""
    r = np.random.default_rng(9 + T)
    rows = 5
    g16 = r.uniform(0, 1, (rows, stride)).astype(np.float16)
    x16 = r.standard_normal((rows, stride)).astype(np.float16)
    g, x = g16[:, :T].astype(np.float32), x16[:, :T].astype(np.float32)
    dy = r.standard_normal((rows, T)).astype(np.float32)
    cu = gen.segments_random(r, T, 4)
    h0 = r.standard_normal((4, rows)).astype(np.float32)
    gt = torch.from_numpy(g16).to(DEV)[:, :T]
    xt = torch.from_numpy(x16).to(DEV)[:, :T]
    cu_t = _t(cu, torch.int32)
    for rev in (False, True):
        out = torch.full((rows, stride), 7.0, device=DEV)
        h = m.scan_fwd(gt, xt, h0=_t(h0), cu_seqlens=cu_t, reverse=rev, out=out[:, :T])
        href = oracle_lib.scan_fwd(g, x, h0=h0, cu_seqlens=cu, reverse=rev)
        close(h, href, TAU_FWD, "h")
        assert torch.all(out[:, T:] == 7.0), "wrote outside the rows"
        if stride == T:
            dx, dg, dh0 = m.scan_bwd(gt, h, _t(dy), h0=_t(h0), cu_seqlens=cu_t, reverse=rev)
            rx, rg, rh0 = oracle_lib.scan_bwd(g, href, dy, h0=h0, cu_seqlens=cu, reverse=rev)
            close(dx, rx, TAU_BWD, "dx")
            close(dg, rg, TAU_BWD, "dg")
            close(dh0, rh0, TAU_BWD, "dh0")


SHORT_T = [1, 200, 256, 257, 253, 700, 1021, 1024, 1025, 1500, 2045, 2048, 2049]


def _inputs(r, rows, stride, dt, gated):
    """(fp32 values the kernel sees for g, x; the device tensors) with g in
    (0, 1) or, gated, logits z ~ N(2, 1) with resets z = -inf."""
    if gated:
        g32 = (r.standard_normal((rows, stride)) + 2.0).astype(np.float32)
        g32[r.random((rows, stride)) < 0.01] = -np.inf
    else:
        g32 = r.uniform(0, 1, (rows, stride)).astype(np.float32)
    x32 = r.standard_normal((rows, stride)).astype(np.float32)
    if dt == "bf16":
        gb, xb = gen.bf16_round(g32).reshape(rows, stride), gen.bf16_round(x32).reshape(rows, stride)
        return (gen.bf16_bits_to_f32(gb).reshape(rows, stride), gen.bf16_bits_to_f32(xb).reshape(rows, stride),
                _bf16(gb), _bf16(xb))
    if dt == "fp16":
        g16, x16 = g32.astype(np.float16), x32.astype(np.float16)
        return (g16.astype(np.float32), x16.astype(np.float32),
                torch.from_numpy(g16).to(DEV), torch.from_numpy(x16).to(DEV))
    return g32, x32, _t(g32), _t(x32)


@pytest.mark.parametrize("dt", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("T", SHORT_T)
def test_short_row_tiles(m, oracle_lib, dt, T):
    """Rows that fit one tile of 256, 1024 or 2048 elements (their own smaller
    workgroups), lengths on both sides of each tile size, rows starting at every
    vector offset, packed sequences with h0, gate values and gate logits, both
    directions, forward and backward."""
    r = np.random.default_rng(700 + T + 10_000 * ("fp32", "bf16", "fp16").index(dt))
    rows = 7
    for gated in (False, True):
        fwd, bwd = (m.scan_fwd_gated, m.scan_bwd_gated) if gated else (m.scan_fwd, m.scan_bwd)
        ofwd, obwd = ((oracle_lib.scan_fwd_gated, oracle_lib.scan_bwd_gated) if gated
                      else (oracle_lib.scan_fwd, oracle_lib.scan_bwd))
        for stride in (T, T + 3):
            g, x, gt, xt = _inputs(r, rows, stride, dt, gated)
            g, x, gt, xt = g[:, :T], x[:, :T], gt[:, :T], xt[:, :T]
            nseg = int(r.integers(1, 5))
            cu = gen.segments_random(r, T, nseg) if nseg > 1 else None
            cu_t = None if cu is None else _t(cu, torch.int32)
            h0 = r.standard_normal((nseg, rows)).astype(np.float32)
            for rev in (False, True):
                out = torch.full((rows, stride), 7.0, device=DEV)
                h = fwd(gt, xt, h0=_t(h0), cu_seqlens=cu_t, reverse=rev, out=out[:, :T])
                href = ofwd(g, x, h0=h0, cu_seqlens=cu, reverse=rev)
                close(h, href, TAU_FWD, f"h stride {stride} rev {rev} gated {gated}")
                assert torch.all(out[:, T:] == 7.0), "wrote outside the rows"
                if stride != T:
                    continue
                dy = r.standard_normal((rows, T)).astype(np.float32)
                d = bwd(gt, h.contiguous(), _t(dy), h0=_t(h0), cu_seqlens=cu_t, reverse=rev)
                rd = obwd(g, href, dy, h0=h0, cu_seqlens=cu, reverse=rev)
                for got, ref, nm in zip(d, rd, ("dx", "dg", "dh0")):
                    close(got, ref, TAU_BWD, f"{nm} rev {rev} gated {gated}")


@pytest.mark.parametrize("T", [256, 1024, 2048])
def test_short_row_tiles_exact(m, oracle_lib, T):
    """Bit-exact results on the short-row tiles (exact-mode inputs)."""
    r = np.random.default_rng(900 + T)
    g, x, dy = gen.exact_mode(r, (5, T))
    cu = gen.segments_random(r, T, 3, allow_empty=True)
    h0 = r.integers(-1, 2, (3, 5)).astype(np.float32)
    for rev in (False, True):
        run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=rev, check=exact)
        run_case(m, oracle_lib, g, x, dy, h0=h0[0], reverse=rev, check=exact)


def test_workspace_reuse_across_calls(m, oracle_lib):
    """Consecutive multi-tile calls of different sizes share one workspace."""
    r = np.random.default_rng(9)
    for T, rows in [(20000, 3), (9000, 11), (70000, 2), (4097, 40), (20000, 3)]:
        g = r.uniform(0, 1, (rows, T)).astype(np.float32)
        x = r.standard_normal((rows, T)).astype(np.float32)
        for rev in (False, True):
            h = m.scan_fwd(_t(g), _t(x), reverse=rev)
            close(h, oracle_lib.scan_fwd(g, x, reverse=rev), TAU_FWD, f"h T={T}")


def test_zero_gates_and_unit_gates(m):
    r = np.random.default_rng(10)
    x = r.standard_normal((3, 9000)).astype(np.float32)
    h = m.scan_fwd(torch.zeros(3, 9000, device=DEV), _t(x))
    assert torch.equal(h, _t(x))
    dy = _t(r.standard_normal((3, 9000)).astype(np.float32))
    dx, dg, _ = m.scan_bwd(torch.zeros(3, 9000, device=DEV), h, dy)
    assert torch.equal(dx, dy)


def test_autograd_wrappers(m, oracle_lib):
    d = gen.quickstart()
    g = _t(d["g"]).requires_grad_(True)
    x = _t(d["x"]).requires_grad_(True)
    h = m.scan_causal(g, x)
    h.backward(_t(d["dy"]))
    href = oracle_lib.scan_fwd(d["g"], d["x"])
    rx, rg, _ = oracle_lib.scan_bwd(d["g"], href, d["dy"])
    close(h, href, TAU_FWD, "h")
    close(x.grad, rx, TAU_BWD, "dx")
    close(g.grad, rg, TAU_BWD, "dg")
    yf, yb = m.scan_bidirectional_branched(_t(d["g"]), _t(d["x"]), _t(d["g"]), _t(d["x"]))
    close(yb, oracle_lib.scan_fwd(d["g"], d["x"], reverse=True), TAU_FWD, "h reverse")


# ---------------------------------------------------------------------------
# many rows: one workgroup walks each row (the mode the large workloads use)
# ---------------------------------------------------------------------------
ROWS_LOOP = 1024


@pytest.mark.parametrize("T", [1, 5, 4095, 4097, 9001])
@pytest.mark.parametrize("reverse", [False, True])
def test_row_loop_lengths(m, oracle_lib, T, reverse):
    r = np.random.default_rng(1000 + T + reverse)
    g = r.uniform(0, 1, (ROWS_LOOP, T)).astype(np.float32)
    x = r.standard_normal((ROWS_LOOP, T)).astype(np.float32)
    dy = r.standard_normal((ROWS_LOOP, T)).astype(np.float32)
    h0 = r.standard_normal(ROWS_LOOP).astype(np.float32)
    run_case(m, oracle_lib, g, x, dy, h0=h0, reverse=reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_row_loop_exact_varlen(m, oracle_lib, reverse):
    r = np.random.default_rng(2000 + reverse)
    T = 13000
    g, x, dy = gen.exact_mode(r, (ROWS_LOOP, T))
    cu = gen.segments_random(r, T, 9, allow_empty=True)
    h0 = r.integers(-1, 2, (9, ROWS_LOOP)).astype(np.float32)
    run_case(m, oracle_lib, g, x, dy, h0=h0, cu=cu, reverse=reverse, check=exact)


def test_row_loop_many_sequences(m, oracle_lib):
    """More sequences than the workgroup caches in LDS: the table is read from global memory."""
    r = np.random.default_rng(2100)
    T = 5000
    g = r.uniform(0, 1, (ROWS_LOOP, T)).astype(np.float32)
    x = r.standard_normal((ROWS_LOOP, T)).astype(np.float32)
    dy = r.standard_normal((ROWS_LOOP, T)).astype(np.float32)
    cu = gen.segments_random(r, T, 3000, allow_empty=True)
    for rev in (False, True):
        run_case(m, oracle_lib, g, x, dy, cu=cu, reverse=rev)


def test_row_loop_unaligned_bf16(m, oracle_lib):
    r = np.random.default_rng(2200)
    T, stride = 9001, 9003
    gb = gen.bf16_round(r.uniform(0, 1, (ROWS_LOOP, stride)).astype(np.float32)).reshape(ROWS_LOOP, stride)
    xb = gen.bf16_round(r.standard_normal((ROWS_LOOP, stride)).astype(np.float32)).reshape(ROWS_LOOP, stride)
    g = gen.bf16_bits_to_f32(gb).reshape(ROWS_LOOP, stride)[:, :T]
    x = gen.bf16_bits_to_f32(xb).reshape(ROWS_LOOP, stride)[:, :T]
    out = torch.full((ROWS_LOOP, stride), 7.0, device=DEV)
    for rev in (False, True):
        h = m.scan_fwd(_bf16(gb)[:, :T], _bf16(xb)[:, :T], reverse=rev, out=out[:, :T])
        close(h, oracle_lib.scan_fwd(g, x, reverse=rev), TAU_FWD, "h")
        assert torch.all(out[:, T:] == 7.0)


# ---------------------------------------------------------------------------
# full-size workloads (the benchmark's launch configuration)
# ---------------------------------------------------------------------------
SAMPLE_ROWS = np.array([0, 1, 63, 64, 777, 1535, 1536, 4095, 6000, 9999, 12286, 12287])


@pytest.mark.timeout(400)
@pytest.mark.parametrize("T", [4096, 65536])
def test_dense_full_size_sampled(m, oracle_lib, T):
    """B=8, C=1536 dense workload, forward then backward on the full tensor;
    the oracle checks a fixed sample of rows (whole rows at full T)."""
    B, C = 8, 1536
    full = gen.dense(B, C, T)
    g, x, h0, dy = (_t(full[k]) for k in ("g", "x", "h0", "dy"))
    del full
    h = m.scan_fwd(g, x, h0=h0)
    dx, dg, dh0 = m.scan_bwd(g, h, dy, h0=h0)
    sub = gen.dense(B, C, T, rows=SAMPLE_ROWS)
    href = oracle_lib.scan_fwd(sub["g"], sub["x"], h0=sub["h0"])
    rx, rg, rh0 = oracle_lib.scan_bwd(sub["g"], href, sub["dy"], h0=sub["h0"])
    idx = torch.as_tensor(SAMPLE_ROWS, device=DEV)
    close(h.view(-1, T)[idx], href, TAU_FWD, "h")
    close(dx.view(-1, T)[idx], rx, TAU_BWD, "dx")
    close(dg.view(-1, T)[idx], rg, TAU_BWD, "dg")
    close(dh0.view(-1)[idx], rh0.reshape(-1), TAU_BWD, "dh0")
    assert torch.isfinite(h).all() and torch.isfinite(dg).all()


@pytest.fixture(scope="module")
def varlen_full():
    return gen.varlen_bidir()


@pytest.mark.timeout(400)
def test_varlen_bidir_full(m, oracle_lib, varlen_full):
    """C=1536, 65536 packed tokens in 16 sequences, bf16 inputs, both branches,
    forward and backward, all elements checked."""
    d = varlen_full
    cu = d["cu_seqlens"]
    cu_t = _t(cu, torch.int32)
    for name in ("fwd", "bwd"):
        b = d[name]
        gg, xx = _bf16(b["g_bf16"]), _bf16(b["x_bf16"])
        h = m.scan_fwd(gg, xx, cu_seqlens=cu_t, reverse=b["reverse"])
        href = oracle_lib.scan_fwd(b["g"], b["x"], cu_seqlens=cu, reverse=b["reverse"])
        close(h, href, TAU_FWD, f"{name} h")
        dx, dg, dh0 = m.scan_bwd(gg, h, _t(b["dy"]), cu_seqlens=cu_t, reverse=b["reverse"])
        rx, rg, rh0 = oracle_lib.scan_bwd(b["g"], href, b["dy"], cu_seqlens=cu, reverse=b["reverse"])
        close(dx, rx, TAU_BWD, f"{name} dx")
        close(dg, rg, TAU_BWD, f"{name} dg")
        close(dh0, rh0, TAU_BWD, f"{name} dh0")


def test_runs_on_the_current_stream(m, oracle_lib):
    """Calls made under a side stream launch on that stream: the handle the
    binding passes is the side stream's, and results produced and consumed on
    it match the oracle."""
    r = np.random.default_rng(77)
    g = r.uniform(0, 1, (6, 9000)).astype(np.float32)
    x = r.standard_normal((6, 9000)).astype(np.float32)
    dy = r.standard_normal((6, 9000)).astype(np.float32)
    s = torch.cuda.Stream()
    dev = torch.device(DEV)
    assert m._stream_handle(dev) == torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.stream(s):
        assert m._stream_handle(dev) == s.cuda_stream
        gt, xt, dyt = _t(g) * 1.0, _t(x) * 1.0, _t(dy) * 1.0  # produced on s
        h = m.scan_fwd(gt, xt)
        dx, dg, _ = m.scan_bwd(gt, h, dyt)
    s.synchronize()
    href = oracle_lib.scan_fwd(g, x)
    close(h, href, TAU_FWD, "h")
    rx, rg, _ = oracle_lib.scan_bwd(g, href, dy)
    close(dx, rx, TAU_BWD, "dx")
    close(dg, rg, TAU_BWD, "dg")


@pytest.mark.timeout(400)
def test_row_of_maximum_length(m, oracle_lib):
    """One row of T = 2^31 - 1 elements, the largest T the library accepts
    (8 GiB per array: 64-bit byte offsets, half a million look-back tiles).
    Resets every 1000 steps and x = dy = 1 make every state and adjoint a small
    integer, exact in any association order: h_t = t mod 1000 + 1, lam_t =
    steps to the next reset or the row end, dg_t = h_{t-1} lam_t (h_{-1} = 0).
    Checked over the whole row on the device in slices, and against the oracle
    on a window that starts at a reset."""
    T = 2**31 - 1
    free, _ = torch.cuda.mem_get_info()
    if free < 64 * 2**30:
        pytest.skip("needs 64 GiB of free device memory")
    g = torch.ones(T, device=DEV)
    g[::1000] = 0.0
    x = torch.ones(T, device=DEV)
    h = m.scan_fwd(g, x)
    dx, dg, dh0 = m.scan_bwd(g, h, x)
    del x
    step = 2**28
    for lo in range(0, T, step):
        hi = min(lo + step, T)
        t = torch.arange(lo, hi, device=DEV, dtype=torch.int64)
        assert torch.equal(h[lo:hi], (t % 1000 + 1).float()), f"h slice at {lo}"
        lam = torch.minimum(1000 - t % 1000, T - t).float()
        assert torch.equal(dx[lo:hi], lam), f"dx slice at {lo}"
        hprev = torch.where(t % 1000 == 0, 1000.0, (t % 1000).float())  # h_{t-1}
        if lo == 0:
            hprev[0] = 0.0  # no h0
        assert torch.equal(dg[lo:hi], hprev * lam), f"dg slice at {lo}"
        del t, lam, hprev
    assert float(dh0.item()) == 0.0  # g_0 = 0
    # the oracle on a window from the last reset to the row end
    w0 = ((T - 1) // 1000) * 1000
    gw = g[w0:].cpu().numpy()[None, :]
    href = oracle_lib.scan_fwd(gw, np.ones_like(gw))
    exact(h[w0:][None, :], href, "h window")


def test_graph_capture_replays(m, oracle_lib):
    """A forward + backward captured in a HIP graph (look-back tiles, packed
    sequences, h0: the workspace clearing is a kernel, not a memset node) and
    replayed several times, with new inputs copied in and eager calls and
    synchronisations between replays; every replay matches the oracle and the
    eager result."""
    r = np.random.default_rng(4242)
    rows, T, nseg = 5, 9000, 3
    cu = gen.segments_random(r, T, nseg)
    g0 = r.uniform(0, 1, (rows, T)).astype(np.float32)
    x0 = r.standard_normal((rows, T)).astype(np.float32)
    dy0 = r.standard_normal((rows, T)).astype(np.float32)
    h00 = r.standard_normal((nseg, rows)).astype(np.float32)
    gt, xt, dyt, h0t, cut = _t(g0), _t(x0), _t(dy0), _t(h00), _t(cu, torch.int32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            hw = m.scan_fwd(gt, xt, h0=h0t, cu_seqlens=cut)
            m.scan_bwd(gt, hw, dyt, h0=h0t, cu_seqlens=cut)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h = m.scan_fwd(gt, xt, h0=h0t, cu_seqlens=cut)
        dx, dg, dh0 = m.scan_bwd(gt, h, dyt, h0=h0t, cu_seqlens=cut)
    for rep in range(4):
        g = r.uniform(0, 1, (rows, T)).astype(np.float32)
        x = r.standard_normal((rows, T)).astype(np.float32)
        gt.copy_(_t(g))
        xt.copy_(_t(x))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        href = oracle_lib.scan_fwd(g, x, h0=h00, cu_seqlens=cu)
        close(h, href, TAU_FWD, f"h replay {rep}")
        rx, rg, rh0 = oracle_lib.scan_bwd(g, href, dy0, h0=h00, cu_seqlens=cu)
        close(dx, rx, TAU_BWD, f"dx replay {rep}")
        close(dg, rg, TAU_BWD, f"dg replay {rep}")
        close(dh0, rh0, TAU_BWD, f"dh0 replay {rep}")
        he = m.scan_fwd(gt, xt, h0=h0t, cu_seqlens=cut)  # eager work between replays
        torch.cuda.synchronize()
        close(he, href, TAU_FWD, f"eager h after replay {rep}")


def test_two_graphs_keep_their_own_workspaces(m, oracle_lib):
    """Two captured graphs whose calls need different workspace sizes (the
    second larger), then an eager call that needs more still: each graph keeps
    the workspace it recorded, so replaying both graphs, in either order and
    with eager calls between, keeps every result correct."""
    r = np.random.default_rng(4343)

    def inputs(rows, T):
        g = r.uniform(0, 1, (rows, T)).astype(np.float32)
        x = r.standard_normal((rows, T)).astype(np.float32)
        return g, x, _t(g), _t(x)

    g1, x1, g1t, x1t = inputs(4, 3 * 4096)     # 12 tiles of descriptors
    g2, x2, g2t, x2t = inputs(16, 6 * 4096)    # 96 tiles
    g3, x3, g3t, x3t = inputs(40, 5 * 4096)    # 200 tiles (eager only)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.scan_fwd(g1t, x1t)
        m.scan_fwd(g2t, x2t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph1, graph2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph1):
        h1 = m.scan_fwd(g1t, x1t)
    with torch.cuda.graph(graph2):
        h2 = m.scan_fwd(g2t, x2t)
    ref1 = oracle_lib.scan_fwd(g1, x1)
    ref2 = oracle_lib.scan_fwd(g2, x2)
    ref3 = oracle_lib.scan_fwd(g3, x3)
    for order in ((graph1, graph2), (graph2, graph1), (graph1, graph2)):
        h1.zero_()
        h2.zero_()
        for gr in order:
            gr.replay()
        h3 = m.scan_fwd(g3t, x3t)  # eager, on a cached workspace larger than either graph's
        torch.cuda.synchronize()
        close(h1, ref1, TAU_FWD, "graph 1")
        close(h2, ref2, TAU_FWD, "graph 2")
        close(h3, ref3, TAU_FWD, "eager")
    # replays on two streams at once: each graph writes only its own workspace
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    h1.zero_()
    h2.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        graph1.replay()
    with torch.cuda.stream(s2):
        graph2.replay()
    torch.cuda.synchronize()
    close(h1, ref1, TAU_FWD, "graph 1 on its own stream")
    close(h2, ref2, TAU_FWD, "graph 2 on its own stream")


def test_binding_rejects_bad_out_and_host_tensors(m):
    """The binding refuses an `out` that is not fp32 or has another shape, and
    host tensors anywhere, before anything reaches the library."""
    g = torch.rand((3, 100), device=DEV)
    x = torch.randn((3, 100), device=DEV)
    with pytest.raises(ValueError):
        m.scan_fwd(g, x, out=torch.empty((3, 100), device=DEV, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        m.scan_fwd(g, x, out=torch.empty((3, 99), device=DEV))
    with pytest.raises(ValueError):
        m.scan_fwd(g, x.cpu())
    h = m.scan_fwd(g, x)
    with pytest.raises(ValueError):
        m.scan_bwd(g, h.cpu(), x)
    with pytest.raises(ValueError):
        m.scan_bwd(g, h, x.cpu())
