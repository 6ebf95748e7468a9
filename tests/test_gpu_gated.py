"""GPU parity of the gate-logit scans (scan_fwd_gated / scan_bwd_gated with
g = sigmoid(z), scan_log_fwd_gated / scan_log_bwd_gated with log a = -softplus(z))
against the fp64 oracle, which applies the activation and then runs the plain
scan. Tolerances per element: 2e-5 * (1 + |ref|) for the linear forward, 1e-4 *
(1 + |ref|) for gradients and the log-space scan. bf16 logits reach the oracle
already rounded."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

TAU_FWD, TAU_BWD, TAU_LOG = 2e-5, 1e-4, 1e-4
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def close(gpu, ref, tau, what):
    g = gpu.detach().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    i = int(np.argmax(err))
    assert err.flat[i] <= tau, f"{what}: max rel err {err.flat[i]:.3e} at {np.unravel_index(i, err.shape)}"


def _linear_case(m, o, z, x, dy, h0=None, cu=None, reverse=False, dtype=torch.float32):
    """z, x as float32 arrays holding exactly representable values of `dtype`."""
    cu_t = None if cu is None else _t(cu, torch.int32)
    h0_t = None if h0 is None else _t(h0)
    zt, xt = _t(z, dtype), _t(x, dtype)
    h = m.scan_fwd_gated(zt, xt, h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    href = o.scan_fwd_gated(z, x, h0=h0, cu_seqlens=cu, reverse=reverse)
    close(h, href, TAU_FWD, "h")
    dx, dz, dh0 = m.scan_bwd_gated(zt, h, _t(dy), h0=h0_t, cu_seqlens=cu_t, reverse=reverse)
    rx, rz, rh0 = o.scan_bwd_gated(z, href, dy, h0=h0, cu_seqlens=cu, reverse=reverse)
    close(dx, rx, TAU_BWD, "dx")
    close(dz, rz, TAU_BWD, "dz")
    if h0 is not None:
        close(dh0.reshape(rh0.shape), rh0, TAU_BWD, "dh0")
    return h, dz


@pytest.mark.parametrize("T", [1, 5, 4095, 4097, 20000])
@pytest.mark.parametrize("reverse", [False, True])
def test_sigmoid_gate_lengths(m, oracle_lib, T, reverse):
    r = np.random.default_rng(600 + T + reverse)
    z = (r.standard_normal((6, T)) * 3).astype(np.float32)
    x = r.standard_normal((6, T)).astype(np.float32)
    dy = r.standard_normal((6, T)).astype(np.float32)
    h0 = r.standard_normal(6).astype(np.float32)
    _linear_case(m, oracle_lib, z, x, dy, h0=h0, reverse=reverse)


@pytest.mark.parametrize("reverse", [False, True])
def test_sigmoid_gate_bf16_packed(m, oracle_lib, reverse):
    """bf16 logits z ~ N(2, 1) and inputs, packed sequences (with empty ones), resets
    as z = -inf (sigmoid(-inf) = 0): the packed workload's gates as logits."""
    r = np.random.default_rng(700 + reverse)
    C, T = 96, 30000
    z = gen.bf16_bits_to_f32(gen.bf16_round(r.standard_normal((C, T)) + 2.0))
    z[:, r.random(T) < 1.0 / 1024] = -np.inf
    x = gen.bf16_bits_to_f32(gen.bf16_round(r.standard_normal((C, T))))
    dy = r.standard_normal((C, T)).astype(np.float32)
    cu = np.concatenate([[0], gen.segments_random(r, T, 12)[1:-1], [T, T]]).astype(np.int32)
    _linear_case(m, oracle_lib, z, x, dy, cu=cu, reverse=reverse, dtype=torch.bfloat16)


def test_sigmoid_gate_matches_explicit_gates(m):
    """scan_fwd_gated(z) equals scan_fwd(sigmoid(z)) up to fp32 rounding of the gate."""
    r = np.random.default_rng(8)
    z = torch.randn((512, 5000), device=DEV) * 2
    x = torch.randn((512, 5000), device=DEV)
    h1 = m.scan_fwd_gated(z, x)
    h2 = m.scan_fwd(torch.sigmoid(z), x)
    err = ((h1 - h2).abs() / (1 + h2.abs())).max().item()
    assert err <= 2e-5, err


@pytest.mark.timeout(400)
def test_neg_softplus_gate_log_workload_full(m, oracle_lib):
    """B=8, D=1024, T=8192 with logits z ~ N(0, 1) (log a = -softplus(z)), log b ~ N(0, 1),
    dy ~ N(0, 1): every element of h, dz and dlog_b."""
    B, D, T = 8, 1024, 8192
    r = np.random.default_rng(900)
    z = r.standard_normal((B, D, T)).astype(np.float32)
    lb = r.standard_normal((B, D, T)).astype(np.float32)
    dy = r.standard_normal((B, D, T)).astype(np.float32)
    zt, lbt = _t(z), _t(lb)
    h = m.scan_log_fwd_gated(zt, lbt)
    href = oracle_lib.scan_log_fwd_gated(z, lb)
    close(h, href, TAU_LOG, "h")
    dz, dlb, _ = m.scan_log_bwd_gated(zt, lbt, h, _t(dy), need_dh0=False)
    rz, rb, _ = oracle_lib.scan_log_bwd_gated(z, lb, href, dy)
    close(dz, rz, TAU_BWD, "dz")
    close(dlb, rb, TAU_BWD, "dlog_b")


@pytest.mark.parametrize("reverse", [False, True])
def test_neg_softplus_gate_varlen_h0(m, oracle_lib, reverse):
    r = np.random.default_rng(950 + reverse)
    rows, T = 7, 13000
    z = (r.standard_normal((rows, T)) * 4).astype(np.float32)
    lb = r.standard_normal((rows, T)).astype(np.float32)
    dy = r.standard_normal((rows, T)).astype(np.float32)
    cu = gen.segments_random(r, T, 10)
    lh0 = r.standard_normal((10, rows)).astype(np.float32)
    cu_t, lh0_t, zt, lbt = _t(cu, torch.int32), _t(lh0), _t(z), _t(lb)
    h = m.scan_log_fwd_gated(zt, lbt, log_h0=lh0_t, cu_seqlens=cu_t, reverse=reverse)
    href = oracle_lib.scan_log_fwd_gated(z, lb, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    close(h, href, TAU_LOG, "h")
    dz, dlb, dlh0 = m.scan_log_bwd_gated(zt, lbt, h, _t(dy), log_h0=lh0_t, cu_seqlens=cu_t, reverse=reverse)
    rz, rb, rh0 = oracle_lib.scan_log_bwd_gated(z, lb, href, dy, log_h0=lh0, cu_seqlens=cu, reverse=reverse)
    close(dz, rz, TAU_BWD, "dz")
    close(dlb, rb, TAU_BWD, "dlog_b")
    close(dlh0, rh0, TAU_BWD, "dlog_h0")
