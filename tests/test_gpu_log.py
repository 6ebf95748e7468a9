"""GPU parity of the log-space scan (scan_log_fwd) against the fp64 oracle.

Tolerance: |gpu - ref| <= 1e-4 * (1 + |ref|) per element; where values are far
from 1 the test checks the relative error |gpu - ref| / |ref| <= 1e-4 instead.
"""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

TAU_LOG = 1e-4
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def close(gpu, ref, tau, what, relative=False):
    g = gpu.detach().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    den = np.abs(ref) if relative else 1.0 + np.abs(ref)
    err = np.abs(g - ref) / den
    i = int(np.argmax(err))
    assert err.flat[i] <= tau, f"{what}: max err {err.flat[i]:.3e} at {np.unravel_index(i, err.shape)} (gpu {g.flat[i]!r}, ref {ref.flat[i]!r})"


def _inputs(r, rows, T):
    la = -np.log1p(np.exp(r.standard_normal((rows, T)))).astype(np.float32)
    lb = r.standard_normal((rows, T)).astype(np.float32)
    return la, lb


@pytest.mark.timeout(300)
def test_logspace_workload_full(m, oracle_lib):
    """B=8, D=1024, T=8192, log_a = -softplus(N(0,1)), log_b ~ N(0,1): every element."""
    d = gen.logspace()
    h = m.scan_log_fwd(_t(d["log_a"]), _t(d["log_b"]))
    ref = oracle_lib.scan_log_fwd(d["log_a"], d["log_b"])
    close(h, ref, TAU_LOG, "h")


@pytest.mark.parametrize("T", [1, 2, 7, 4095, 4096, 4097, 6000, 8192, 8193, 20000])
@pytest.mark.parametrize("reverse", [False, True])
def test_log_lengths_with_h0(m, oracle_lib, T, reverse):
    r = np.random.default_rng(T + 7 * reverse)
    la, lb = _inputs(r, 5, T)
    lh0 = r.standard_normal(5).astype(np.float32)
    h = m.scan_log_fwd(_t(la), _t(lb), log_h0=_t(lh0), reverse=reverse)
    close(h, oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, reverse=reverse), TAU_LOG, "h")


@pytest.mark.parametrize("rows", [3, 1024])
@pytest.mark.parametrize("reverse", [False, True])
def test_log_varlen(m, oracle_lib, rows, reverse):
    r = np.random.default_rng(rows + reverse)
    T = 15000
    la, lb = _inputs(r, rows, T)
    cu = gen.segments_random(r, T, 11)
    lh0 = r.standard_normal((11, rows)).astype(np.float32)
    h = m.scan_log_fwd(_t(la), _t(lb), log_h0=_t(lh0), cu_seqlens=_t(cu, torch.int32), reverse=reverse)
    close(h, oracle_lib.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse), TAU_LOG, "h")


def test_log_zero_gates_reset(m, oracle_lib):
    """log a = -inf (a = 0) erases the prefix: h_t = b_t there."""
    r = np.random.default_rng(3)
    la, lb = _inputs(r, 4, 9000)
    la[:, ::97] = -np.inf
    h = m.scan_log_fwd(_t(la), _t(lb), log_h0=_t(np.zeros(4, np.float32)))
    ref = oracle_lib.scan_log_fwd(la, lb, log_h0=np.zeros(4))
    close(h, ref, TAU_LOG, "h")
    close(h[:, ::97], np.exp(lb[:, ::97].astype(np.float64)), TAU_LOG, "reset", relative=True)


@pytest.mark.parametrize("shift", [-80.0, 60.0])
def test_log_far_from_one(m, oracle_lib, shift):
    """Values near the ends of fp32's range keep their relative accuracy."""
    r = np.random.default_rng(4)
    la, lb = _inputs(r, 6, 12000)
    lb = (lb + np.float32(shift)).astype(np.float32)
    h = m.scan_log_fwd(_t(la), _t(lb))
    ref = oracle_lib.scan_log_fwd(la, lb)
    assert np.all(ref > 0) and np.all(np.isfinite(ref))
    close(h, ref, TAU_LOG, "h", relative=True)


def test_log_matches_linear_scan_on_exp_inputs(m):
    """The log-space scan and the linear scan on a = e^{log a}, b = e^{log b}
    compute the same states (GPU against GPU, fp32 tolerance)."""
    r = np.random.default_rng(5)
    la, lb = _inputs(r, 1100, 5000)
    h_log = m.scan_log_fwd(_t(la), _t(lb))
    h_lin = m.scan_fwd(_t(np.exp(la)), _t(np.exp(lb)))
    err = ((h_log - h_lin).abs() / (1 + h_lin.abs())).max().item()
    assert err <= 1e-4, err


# ---------------------------------------------------------------------------
# log-space backward (scan_log_bwd): tolerance 1e-4 * (1 + |ref|) per element
# ---------------------------------------------------------------------------
TAU_GRAD = 1e-4


def _log_bwd_case(m, o, la, lb, dy, lh0=None, cu=None, reverse=False):
    cu_t = None if cu is None else _t(cu, torch.int32)
    lh0_t = None if lh0 is None else _t(lh0)
    la_t, lb_t = _t(la), _t(lb)
    h = m.scan_log_fwd(la_t, lb_t, log_h0=lh0_t, cu_seqlens=cu_t, reverse=reverse)
    dla, dlb, dlh0 = m.scan_log_bwd(la_t, lb_t, h, _t(dy), log_h0=lh0_t, cu_seqlens=cu_t, reverse=reverse)
    href = o.scan_log_fwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    ra, rb, rh0 = o.scan_log_bwd(la, lb, href, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    close(dlb, rb, TAU_GRAD, "dlog_b")
    close(dla, ra, TAU_GRAD, "dlog_a")
    if lh0 is not None:
        close(dlh0.reshape(rh0.shape), rh0, TAU_GRAD, "dlog_h0")
    return dla, dlb, dlh0


@pytest.mark.timeout(400)
def test_log_bwd_workload_full(m, oracle_lib):
    """B=8, D=1024, T=8192, log_a = -softplus(N(0,1)), log_b ~ N(0,1), dy ~ N(0,1):
    every element of both gradients."""
    d = gen.logspace()
    dy = np.random.default_rng(41).standard_normal(d["log_a"].shape).astype(np.float32)
    _log_bwd_case(m, oracle_lib, d["log_a"], d["log_b"], dy)


@pytest.mark.parametrize("T", [1, 2, 7, 4095, 4096, 4097, 6000, 8192, 8193, 20000])
@pytest.mark.parametrize("reverse", [False, True])
def test_log_bwd_lengths_with_h0(m, oracle_lib, T, reverse):
    r = np.random.default_rng(100 + T + reverse)
    la, lb = _inputs(r, 5, T)
    dy = r.standard_normal((5, T)).astype(np.float32)
    lh0 = r.standard_normal(5).astype(np.float32)
    _log_bwd_case(m, oracle_lib, la, lb, dy, lh0=lh0, reverse=reverse)


@pytest.mark.parametrize("rows", [3, 1024])
@pytest.mark.parametrize("reverse", [False, True])
def test_log_bwd_varlen(m, oracle_lib, rows, reverse):
    r = np.random.default_rng(200 + rows + reverse)
    T = 15000
    la, lb = _inputs(r, rows, T)
    dy = r.standard_normal((rows, T)).astype(np.float32)
    cu = np.concatenate([[0, 0], gen.segments_random(r, T, 9)[1:], [T]]).astype(np.int32)
    lh0 = r.standard_normal((len(cu) - 1, rows)).astype(np.float32)
    _, _, dlh0 = _log_bwd_case(m, oracle_lib, la, lb, dy, lh0=lh0, cu=cu, reverse=reverse)
    assert torch.all(dlh0[0] == 0) and torch.all(dlh0[-1] == 0), "empty sequences get a zero gradient"


def test_log_bwd_zero_gates(m, oracle_lib):
    """log a = -inf: no gradient reaches log a there, and nothing crosses it."""
    r = np.random.default_rng(6)
    la, lb = _inputs(r, 4, 9000)
    la[:, ::97] = -np.inf
    dy = r.standard_normal((4, 9000)).astype(np.float32)
    dla, _, _ = _log_bwd_case(m, oracle_lib, la, lb, dy, lh0=np.zeros(4, np.float32))
    assert torch.all(dla[:, ::97] == 0)


def test_log_autograd_wrapper(m, oracle_lib):
    """scan_log's autograd backward is the native adjoint kernel."""
    r = np.random.default_rng(7)
    la, lb = _inputs(r, 6, 5000)
    lh0 = r.standard_normal(6).astype(np.float32)
    dy = r.standard_normal((6, 5000)).astype(np.float32)
    la_t, lb_t, lh0_t = (_t(x).requires_grad_() for x in (la, lb, lh0))
    h = m.scan_log(la_t, lb_t, log_h0=lh0_t)
    (h * _t(dy)).sum().backward()
    href = oracle_lib.scan_log_fwd(la, lb, log_h0=lh0)
    ra, rb, rh0 = oracle_lib.scan_log_bwd(la, lb, href, dy, log_h0=lh0)
    close(la_t.grad, ra, TAU_GRAD, "dlog_a")
    close(lb_t.grad, rb, TAU_GRAD, "dlog_b")
    close(lh0_t.grad, rh0.reshape(-1), TAU_GRAD, "dlog_h0")


@pytest.mark.parametrize("T", [1, 100, 256, 257, 1000, 1024, 1025, 2047, 2048, 2049])
def test_log_short_row_tiles(m, oracle_lib, T):
    """Rows that fit one tile of 256, 1024 or 2048 elements (their own smaller
    workgroups): forward and backward, plain and from -softplus logits, with
    packed sequences, h0 and resets (log a = -inf, logits +inf), both
    directions."""
    r = np.random.default_rng(3000 + T)
    rows = 6
    for gated in (False, True):
        fwd, bwd = (m.scan_log_fwd_gated, m.scan_log_bwd_gated) if gated else (m.scan_log_fwd, m.scan_log_bwd)
        ofwd, obwd = ((oracle_lib.scan_log_fwd_gated, oracle_lib.scan_log_bwd_gated) if gated
                      else (oracle_lib.scan_log_fwd, oracle_lib.scan_log_bwd))
        if gated:
            la = r.standard_normal((rows, T)).astype(np.float32)
            la[r.random((rows, T)) < 0.01] = np.inf  # log a = -softplus(+inf) = -inf
        else:
            la, _ = _inputs(r, rows, T)
            la[r.random((rows, T)) < 0.01] = -np.inf
        lb = r.standard_normal((rows, T)).astype(np.float32)
        nseg = int(r.integers(1, 5))
        cu = gen.segments_random(r, T, nseg) if nseg > 1 else None
        cu_t = None if cu is None else _t(cu, torch.int32)
        lh0 = r.standard_normal((nseg, rows)).astype(np.float32)
        for rev in (False, True):
            h = fwd(_t(la), _t(lb), _t(lh0), cu_seqlens=cu_t, reverse=rev)
            href = ofwd(la, lb, log_h0=lh0, cu_seqlens=cu, reverse=rev)
            close(h, href, TAU_LOG, f"h rev {rev} gated {gated}")
            dy = r.standard_normal((rows, T)).astype(np.float32)
            d = bwd(_t(la), _t(lb), h, _t(dy), _t(lh0), cu_seqlens=cu_t, reverse=rev)
            rd = obwd(la, lb, href, dy, log_h0=lh0, cu_seqlens=cu, reverse=rev)
            for got, ref, nm in zip(d, rd, ("dlog_a", "dlog_b", "dlog_h0")):
                close(got, ref, TAU_LOG, f"{nm} rev {rev} gated {gated}")


# ---------------------------------------------------------------------------
# extreme ranges inside one row
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_log_lanes_outside_the_linear_range(m, oracle_lib, reverse):
    """Rows mixing ordinary values with log a far below and above zero (-95,
    +70), log b beyond +-80, partial values near e^80 and runs of tiny terms,
    both directions, against the oracle (relative error)."""
    r = np.random.default_rng(3100 + reverse)
    rows, T = 6, 5 * 4096 + 17
    la, lb = _inputs(r, rows, T)
    la[0, 1000:1003] = -95.0          # log a below the range
    la[1, 5000] = 70.0                # above it
    lb[2, 9000:9004] = 86.0           # log b above the range
    lb[3, 12000:12004] = -90.0        # and below it, alone in its lane
    lb[3, 12004:12016] = -90.0
    la[3, 12000:12016] = 0.0
    lb[4, 15000:15016] = 79.0         # partial values beyond 16 e^80 need the check on M + R
    la[4, 15000:15016] = 0.0
    lb[5, 7000:7016] = -75.0          # every term tiny: log Q must stay accurate
    la[5, 7000:7016] = -0.5
    h = m.scan_log_fwd(_t(la), _t(lb), reverse=reverse)
    ref = oracle_lib.scan_log_fwd(la, lb, reverse=reverse)
    close(h, ref, TAU_LOG, "h", relative=True)


@pytest.mark.parametrize("reverse", [False, True])
def test_log_large_carry_takes_the_exact_apply(m, oracle_lib, reverse):
    """States near e^75 carried across tiles, and a state that decays from
    there back to ordinary values, both directions, against the oracle."""
    r = np.random.default_rng(3200 + reverse)
    rows, T = 4, 3 * 4096 + 5
    la = np.full((rows, T), -0.01, np.float32)
    lb = (70.0 + 0.1 * r.standard_normal((rows, T))).astype(np.float32)
    # row 1 decays from there: log a = -2 after the middle
    la[1, T // 2:] = -2.0
    lb[1, T // 2:] = r.standard_normal(T - T // 2).astype(np.float32)
    h = m.scan_log_fwd(_t(la), _t(lb), reverse=reverse)
    ref = oracle_lib.scan_log_fwd(la, lb, reverse=reverse)
    close(h, ref, TAU_LOG, "h", relative=True)


def test_log_gated_lanes_with_logits(m, oracle_lib):
    """The -softplus gate-logit forward with logits far out (z = 80: log a =
    -80) and a reset (z = +inf), both directions."""
    r = np.random.default_rng(3300)
    rows, T = 4, 3 * 4096 + 100
    z = r.standard_normal((rows, T)).astype(np.float32)
    z[1, 2000:2010] = 80.0
    z[2, 5000] = np.inf  # a reset: log a = -inf
    lb = r.standard_normal((rows, T)).astype(np.float32)
    for rev in (False, True):
        h = m.scan_log_fwd_gated(_t(z), _t(lb), reverse=rev)
        ref = oracle_lib.scan_log_fwd_gated(z, lb, reverse=rev)
        close(h, ref, TAU_LOG, "h", relative=True)
