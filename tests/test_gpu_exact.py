"""Bit-exact GPU parity on every scalar kernel instantiation, and resets after
Inf / NaN.

Exact mode: integer data (g in {0, 1} with a zero at least every 2048 steps;
x, dy, h0 in {-1, 0, 1}) whose scan is exact in fp32 in every association
order, so the GPU must equal the fp64 oracle bit for bit. The values are exact
in bf16 and fp16 too, so the 16-bit kernels (their 8-byte loads, their
alignment arithmetic, the packed forward's tile-major order) are held to the
same bar, and so are the gate-logit kernels with z in {-inf, +inf}
(sigmoid gives exactly 0 and 1). This pins the indexing: sequence boundaries
from cu_seqlens, resets, direction, the backward's shifts and every tile seam.

Resets after Inf / NaN: a zero gate wipes out the state before it, whatever it
holds ("Our RG-LRU GPU audit", "Exact real chunk algebra": a reset is a_t = 0),
and nothing flows back through it in the adjoint. With Inf and NaN injected
into exact-mode data the GPU must still equal the oracle bit for bit, NaN
positions included.
"""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = ["fp32", "bf16", "fp16"]


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def _dev(a32, dt):
    """Device tensor of dtype dt holding the float32 values a32 (exact in dt)."""
    if dt == "bf16":
        bits = gen.bf16_round(a32).reshape(a32.shape)
        assert np.array_equal(gen.bf16_bits_to_f32(bits).reshape(a32.shape), a32, equal_nan=True)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    if dt == "fp16":
        a16 = a32.astype(np.float16)
        assert np.array_equal(a16.astype(np.float32), a32, equal_nan=True)
        return torch.from_numpy(a16).to(DEV)
    return _t(a32)


def same(gpu, ref, what):
    """Bit-for-bit equality of values, NaN positions included (the sign of a
    zero is not compared: -0 == +0)."""
    g = gpu.detach().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    bad = ~((g == ref) | (np.isnan(g) & np.isnan(ref)))
    if bad.any():
        i = tuple(b[0] for b in np.nonzero(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {i}: gpu {g[i]!r} ref {ref[i]!r}")


def _strided(a, stride, fill):
    """[rows, T] -> a [rows, stride] array holding a in its first T columns."""
    rows, T = a.shape
    out = np.full((rows, stride), fill, a.dtype)
    out[:, :T] = a
    return out


def run_exact(m, o, g, x, dy, h0, cu, rev, dt, gated=False, stride=None):
    """Forward and backward on the GPU against the oracle, bit for bit. g holds
    gate values, or logits z in {-inf, +inf} when gated. With stride > T the
    rows sit stride elements apart (odd strides start rows at every 2-byte
    offset of a vector)."""
    rows, T = g.shape
    stride = stride or T
    gs, xs = _strided(g, stride, 0.0), _strided(x, stride, 0.0)
    gd, xd = _dev(gs, dt)[:, :T], _dev(xs, dt)[:, :T]
    cu_t = None if cu is None else _t(cu, torch.int32)
    h0_t = None if h0 is None else _t(h0)
    out = torch.full((rows, stride), 7.0, device=DEV)
    fwd, bwd = (m.scan_fwd_gated, m.scan_bwd_gated) if gated else (m.scan_fwd, m.scan_bwd)
    ofwd, obwd = ((o.scan_fwd_gated, o.scan_bwd_gated) if gated else (o.scan_fwd, o.scan_bwd))
    h = fwd(gd, xd, h0=h0_t, cu_seqlens=cu_t, reverse=rev, out=out[:, :T])
    href = ofwd(g, x, h0=h0, cu_seqlens=cu, reverse=rev)
    same(h, href, f"h {dt} rev={rev} gated={gated}")
    assert torch.all(out[:, T:] == 7.0), "wrote outside the rows"
    dyd = _t(_strided(dy, stride, 0.0))[:, :T]
    dx, dgz, dh0 = bwd(gd, h, dyd, h0=h0_t, cu_seqlens=cu_t, reverse=rev)
    rx, rgz, rh0 = obwd(g, href, dy, h0=h0, cu_seqlens=cu, reverse=rev)
    same(dx, rx, f"dx {dt} rev={rev} gated={gated}")
    same(dgz, rgz, f"{'dz' if gated else 'dg'} {dt} rev={rev}")
    same(dh0, rh0, f"dh0 {dt} rev={rev} gated={gated}")


def _segments_with_edges(r, T, nseg):
    """Random cu_seqlens with empty sequences (repeated offsets) and length-one
    sequences at a tile seam and at the row's end."""
    cuts = sorted(int(c) for c in r.integers(1, T, size=nseg - 1))
    cuts += [4096, 4097, 4097, T - 1, cuts[2], cuts[2]]
    return np.array([0] + sorted(cuts) + [T], np.int32)


def _exact_inputs(r, rows, T, gated):
    g, x, dy = gen.exact_mode(r, (rows, T))
    if gated:
        g = np.where(g > 0, np.float32(np.inf), np.float32(-np.inf))  # sigmoid: exactly 1 and 0
    return g, x, dy


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("reverse", [False, True])
def test_exact_varlen_every_kernel(m, oracle_lib, dt, gated, reverse):
    """Packed rows over several 4096-element tiles (look-back; the 16-bit
    forward's tile-major order, the packed backward's row-major order), empty
    and length-one sequences, h0 per sequence, both directions."""
    r = np.random.default_rng(1000 + DTYPES.index(dt) * 4 + gated * 2 + reverse)
    rows, T = 3, 3 * 4096 + 1234
    g, x, dy = _exact_inputs(r, rows, T, gated)
    cu = _segments_with_edges(r, T, 12)
    h0 = r.integers(-1, 2, (len(cu) - 1, rows)).astype(np.float32)
    run_exact(m, oracle_lib, g, x, dy, h0, cu, reverse, dt, gated)


def _boundaries_at_every_offset(T):
    """cu_seqlens for 5 tiles and a tail: the first tile holds sequence starts
    at every offset inside a lane's 4-element span, at a wave edge (1024,
    twice: an empty sequence) and on its last element (6 entries inside: the
    wave-uniform pass); the second holds 12 (the per-lane search); the third
    3 at sub-chunk and wave edges; none in the fourth (one sequence spans
    it); a length-one sequence at the row's end."""
    assert T > 5 * 4096
    cuts = [1, 258, 515, 1024, 1024, 4095]
    cuts += [4096 + 3 + 37 * i for i in range(12)]
    cuts += [8192 + 256, 8192 + 1023, 8192 + 2048]
    cuts += [4 * 4096 + 616, T - 1]
    assert all(0 < c < T for c in cuts)
    return np.array([0] + sorted(cuts) + [T], np.int32)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("stride_pad", [0, 1])
@pytest.mark.parametrize("with_h0", [False, True])
def test_exact_varlen_boundary_offsets(m, oracle_lib, dt, gated, reverse, stride_pad, with_h0):
    """Packed rows: the forward finds the boundaries of a tile covered by few
    cu_seqlens entries with one wave-uniform pass (and each start's initial
    state by the entry's index) and falls back to its per-lane search above
    that; both must mark exactly the oracle's sequence starts (ends in
    reverse) and inject the right h0, bit for bit, at every offset and
    alignment."""
    r = np.random.default_rng(3000 + DTYPES.index(dt) * 16 + gated * 8 + reverse * 4 + stride_pad * 2 + with_h0)
    rows, T = 2, 5 * 4096 + 77
    g, x, dy = _exact_inputs(r, rows, T, gated)
    cu = _boundaries_at_every_offset(T)
    h0 = r.integers(-1, 2, (len(cu) - 1, rows)).astype(np.float32) if with_h0 else None
    run_exact(m, oracle_lib, g, x, dy, h0, cu, reverse, dt, gated, stride=T + stride_pad)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("stride_pad", [1, 2, 3])
def test_exact_odd_row_offsets(m, oracle_lib, dt, stride_pad):
    """Rows starting at every element offset of a vector (row_stride = T + 1,
    2, 3), dense and packed, gated and not, both directions."""
    r = np.random.default_rng(1100 + DTYPES.index(dt) * 3 + stride_pad)
    rows, T = 5, 2 * 4096 + 77
    for gated in (False, True):
        g, x, dy = _exact_inputs(r, rows, T, gated)
        cu = gen.segments_random(r, T, 4)
        h0 = r.integers(-1, 2, (4, rows)).astype(np.float32)
        for rev in (False, True):
            run_exact(m, oracle_lib, g, x, dy, h0, cu, rev, dt, gated, stride=T + stride_pad)
            run_exact(m, oracle_lib, g, x, dy, h0[:1], None, rev, dt, gated, stride=T + stride_pad)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("T", [4097, 6001, 8185, 8188, 8191, 8192])
def test_exact_one_wide_tile_rows(m, oracle_lib, dt, T):
    """Rows of 4097 to 8191 elements (8192 for 16-bit inputs) run as one
    8192-element tile; rows that start off a vector boundary near the end need
    a second one (look-back). Dense and packed, gated and not, both
    directions, aligned and odd strides."""
    r = np.random.default_rng(1250 + T + 10000 * DTYPES.index(dt))
    rows = 5
    for gated in (False, True):
        g, x, dy = _exact_inputs(r, rows, T, gated)
        cu = gen.segments_random(r, T, 4, allow_empty=True)
        h0 = r.integers(-1, 2, (4, rows)).astype(np.float32)
        for rev in (False, True):
            for pad in (0, 1, 3):
                run_exact(m, oracle_lib, g, x, dy, h0, cu, rev, dt, gated, stride=T + pad)
                run_exact(m, oracle_lib, g, x, dy, h0[:1], None, rev, dt, gated, stride=T + pad)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("T", [4, 8, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("with_h0", [False, True])
def test_exact_short_power_of_two_rows(m, oracle_lib, dt, T, with_h0):
    """Short dense rows of 4 to 1024 elements stored back to back (37 rows),
    both directions, gate values and logits, with and without h0, bit for
    bit: every row is one tile of the short-row kernel."""
    r = np.random.default_rng(4000 + DTYPES.index(dt) * 64 + T % 61 + with_h0)
    rows = 37
    for gated in (False, True):
        g, x, dy = _exact_inputs(r, rows, T, gated)
        h0 = r.integers(-1, 2, (1, rows)).astype(np.float32) if with_h0 else None
        for rev in (False, True):
            run_exact(m, oracle_lib, g, x, dy, h0, None, rev, dt, gated)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("T", [200, 256, 1000, 1024, 2047, 2048])
def test_exact_short_rows(m, oracle_lib, dt, T):
    """Rows that fit the 256-, 1024- and 2048-element one-per-row tiles."""
    r = np.random.default_rng(1200 + T + DTYPES.index(dt))
    rows = 6
    for gated in (False, True):
        g, x, dy = _exact_inputs(r, rows, T, gated)
        cu = gen.segments_random(r, T, 3, allow_empty=True)
        h0 = r.integers(-1, 2, (3, rows)).astype(np.float32)
        for rev in (False, True):
            run_exact(m, oracle_lib, g, x, dy, h0, cu, rev, dt, gated)
            run_exact(m, oracle_lib, g, x, dy, None, None, rev, dt, gated, stride=T + 1)


def _poison(r, x, frac, values):
    """x with a fraction `frac` of its entries replaced by the given values."""
    x = x.copy()
    idx = r.random(x.shape) < frac
    x[idx] = r.choice(np.array(values, np.float32), size=int(idx.sum()))
    return x


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("gated", [False, True])
def test_reset_after_nonfinite_matches_oracle(m, oracle_lib, dt, gated):
    """Inf and NaN inside sequences (tokens, output gradients and h0), with
    resets after them: every output equals the oracle bit for bit, NaN
    positions included, on look-back rows and on short rows, both directions."""
    r = np.random.default_rng(1300 + DTYPES.index(dt) * 2 + gated)
    for rows, T, nseg in ((3, 3 * 4096 + 500, 7), (4, 1500, 3)):
        g, x, dy = _exact_inputs(r, rows, T, gated)
        x = _poison(r, x, 0.002, [np.nan, np.inf, -np.inf])
        dy = _poison(r, dy, 0.002, [np.nan, np.inf, -np.inf])
        cu = gen.segments_random(r, T, nseg)
        h0 = r.integers(-1, 2, (nseg, rows)).astype(np.float32)
        h0[1, 0], h0[2, 1] = np.nan, np.inf
        gz = g.copy()
        # a reset on the first step of the sequences whose h0 is not finite
        for s_, row_ in ((1, 0), (2, 1)):
            if cu[s_] < cu[s_ + 1]:
                gz[row_, cu[s_]] = -np.inf if gated else 0.0
                gz[row_, cu[s_ + 1] - 1] = -np.inf if gated else 0.0
        for rev in (False, True):
            run_exact(m, oracle_lib, gz, x, dy, h0, cu, rev, dt, gated)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("gated", [False, True])
def test_16bit_nan_poison_stays_in_its_sequence(m, dt, gated):
    """A sequence full of NaN / Inf changes nothing in any other sequence, bit
    for bit, for the 16-bit and gate-logit kernels."""
    r = np.random.default_rng(1400 + gated + 2 * (dt == "fp16"))
    rows, T = 3, 12000
    if gated:
        g = (r.standard_normal((rows, T)) + 2.0).astype(np.float32)
    else:
        g = r.uniform(0, 1, (rows, T)).astype(np.float32)
    x = r.standard_normal((rows, T)).astype(np.float32)
    dy = _t(r.standard_normal((rows, T)).astype(np.float32))
    g, x = _round16(g, dt), _round16(x, dt)
    cu = _t(np.array([0, 3000, 7000, 7001, 12000], np.int32), torch.int32)
    gp, xp = g.copy(), x.copy()
    gp[:, 3000:7000] = np.nan
    xp[:, 3000:5000] = np.inf
    keep = np.r_[0:3000, 7000:12000]
    fwd, bwd = (m.scan_fwd_gated, m.scan_bwd_gated) if gated else (m.scan_fwd, m.scan_bwd)
    for rev in (False, True):
        h = fwd(_dev(g, dt), _dev(x, dt), cu_seqlens=cu, reverse=rev)
        hp = fwd(_dev(gp, dt), _dev(xp, dt), cu_seqlens=cu, reverse=rev)
        assert torch.equal(h[:, keep], hp[:, keep])
        assert torch.isfinite(h).all()
        d1 = bwd(_dev(g, dt), h, dy, cu_seqlens=cu, reverse=rev)
        d2 = bwd(_dev(gp, dt), hp, dy, cu_seqlens=cu, reverse=rev)
        for a, b in zip(d1[:2], d2[:2]):
            assert torch.equal(a[:, keep], b[:, keep])
        assert torch.equal(d1[2][[0, 2, 3]], d2[2][[0, 2, 3]])


def _round16(a, dt):
    if dt == "bf16":
        return gen.bf16_bits_to_f32(gen.bf16_round(a)).reshape(a.shape)
    return a.astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("T", [1800, 3 * 4096 + 5])
def test_log_nan_poison_stays_in_its_sequence(m, gated, T):
    """Log space (and its -softplus gate-logit form): a sequence full of NaN /
    Inf changes nothing in any other sequence, forward and backward, on short
    rows and on look-back rows."""
    r = np.random.default_rng(1500 + gated + T)
    rows = 3
    la = (r.standard_normal((rows, T)) if gated else -np.log1p(np.exp(r.standard_normal((rows, T))))).astype(np.float32)
    lb = r.standard_normal((rows, T)).astype(np.float32)
    dy = _t(r.standard_normal((rows, T)).astype(np.float32))
    a, b = T // 4, T // 2
    cu_np = np.array([0, a, b, b + 1, T], np.int32)
    cu = _t(cu_np, torch.int32)
    lap, lbp = la.copy(), lb.copy()
    lap[:, a:b] = np.nan
    lbp[:, a:(a + b) // 2] = np.inf
    keep = np.r_[0:a, b:T]
    fwd, bwd = (m.scan_log_fwd_gated, m.scan_log_bwd_gated) if gated else (m.scan_log_fwd, m.scan_log_bwd)
    for rev in (False, True):
        h = fwd(_t(la), _t(lb), cu_seqlens=cu, reverse=rev)
        hp = fwd(_t(lap), _t(lbp), cu_seqlens=cu, reverse=rev)
        assert torch.equal(h[:, keep], hp[:, keep])
        assert torch.isfinite(h).all()
        d1 = bwd(_t(la), _t(lb), h, dy, cu_seqlens=cu, reverse=rev)
        d2 = bwd(_t(lap), _t(lbp), hp, dy, cu_seqlens=cu, reverse=rev)
        for u, w in zip(d1[:2], d2[:2]):
            assert torch.equal(u[:, keep], w[:, keep])
        assert torch.equal(d1[2][[0, 2, 3]], d2[2][[0, 2, 3]])


def test_log_reset_drops_h0(m, oracle_lib):
    """log a = -inf on a sequence's first step (in either direction) drops
    log_h0, even a NaN or Inf one, and no gradient reaches log_h0 through it."""
    r = np.random.default_rng(1600)
    rows, T = 4, 3 * 4096 + 9
    la = -np.log1p(np.exp(r.standard_normal((rows, T)))).astype(np.float32)
    lb = r.standard_normal((rows, T)).astype(np.float32)
    cu = np.array([0, 5000, 9000, T], np.int32)
    la[:, [0, 4999, 5000, 8999]] = -np.inf  # both ends of sequences 0 and 1
    lh0 = r.standard_normal((3, rows)).astype(np.float32)
    lh0[0, 0], lh0[1, 1] = np.nan, np.inf
    dy = r.standard_normal((rows, T)).astype(np.float32)
    cu_t = _t(cu, torch.int32)
    for rev in (False, True):
        h = m.scan_log_fwd(_t(la), _t(lb), log_h0=_t(lh0), cu_seqlens=cu_t, reverse=rev)
        href = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=rev)
        hh = h.cpu().double().numpy()
        assert np.all(np.isfinite(hh))
        assert np.max(np.abs(hh - href) / (1 + np.abs(href))) <= 1e-4
        d = m.scan_log_bwd(_t(la), _t(lb), h, _t(dy), log_h0=_t(lh0), cu_seqlens=cu_t, reverse=rev)
        rd = oracle_lib.scan_log_bwd(la, lb, href, dy, log_h0=lh0, cu_seqlens=cu, reverse=rev)
        dlh0 = d[2].cpu().double().numpy()
        assert dlh0[0, 0] == 0.0 and dlh0[1, 1] == 0.0
        assert rd[2][0, 0] == 0.0 and rd[2][1, 1] == 0.0
