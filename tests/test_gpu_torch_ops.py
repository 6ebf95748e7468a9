"""The torch.library custom ops (mscan::scan, mscan::scan_log, mscan::matrix_scan
and their backward ops): torch.library.opcheck on real GPU tensors, and
torch.compile(fullgraph=True) through forward and backward with no graph break,
giving the eager results. Gradients are also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def m():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import associative_scan_amd as m
    return m


def _r(*shape, lo=None, hi=None, seed=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if lo is None:
        return torch.randn(shape, device=DEV, generator=g)
    return lo + (hi - lo) * torch.rand(shape, device=DEV, generator=g)


def test_opcheck_scan(m):
    g = _r(3, 700, lo=0.0, hi=1.0, seed=1).requires_grad_()
    x = _r(3, 700, seed=2).requires_grad_()
    h0 = _r(2, 3, seed=3).requires_grad_()
    cu = torch.tensor([0, 300, 700], dtype=torch.int32, device=DEV)
    torch.library.opcheck(torch.ops.mscan.scan.default, (g, x, h0, cu, False))
    torch.library.opcheck(torch.ops.mscan.scan.default, (g, x, None, None, True))


def test_opcheck_scan_log(m):
    la = (-torch.nn.functional.softplus(_r(4, 900, seed=4))).requires_grad_()
    lb = _r(4, 900, seed=5).requires_grad_()
    lh0 = _r(1, 4, seed=6).requires_grad_()
    torch.library.opcheck(torch.ops.mscan.scan_log.default, (la, lb, lh0, None, False))


def test_opcheck_matrix_scan(m):
    A = (_r(2, 600, 2, 2, seed=7) * 0.6).requires_grad_()
    B = _r(2, 600, 2, 1, seed=8).requires_grad_()
    torch.library.opcheck(torch.ops.mscan.matrix_scan.default, (A, B, None, None, False))


def test_opcheck_matrix_scan_matrix_cores(m):
    """The custom op over the matrix-core kernels: (8, 4) with h0 and segments."""
    A = (_r(3, 300, 8, 8, seed=21) * 0.3).requires_grad_()
    B = _r(3, 300, 8, 4, seed=22).requires_grad_()
    cu = torch.tensor([0, 100, 100, 300], dtype=torch.int32, device=DEV)
    h0 = _r(3, 3, 8, 4, seed=23).requires_grad_()
    torch.library.opcheck(torch.ops.mscan.matrix_scan.default, (A, B, h0, cu, True))


def test_matrix_scan_16x16_gradients_match_oracle(m, oracle_lib):
    """Autograd through mscan::matrix_scan at (16, 16) against the oracle's adjoint."""
    r = np.random.default_rng(24)
    A = (r.standard_normal((2, 400, 16, 16)) * 0.2).astype(np.float32)
    B = r.standard_normal((2, 400, 16, 16)).astype(np.float32)
    h0 = r.standard_normal((1, 2, 16, 16)).astype(np.float32)
    dy = r.standard_normal((2, 400, 16, 16)).astype(np.float32)
    At, Bt, h0t = (torch.from_numpy(a).to(DEV).requires_grad_() for a in (A, B, h0))
    h = m.matrix_scan(At, Bt, h0=h0t, reverse=True)
    (h * torch.from_numpy(dy).to(DEV)).sum().backward()
    href = oracle_lib.matrix_affine_scan_fwd(A, B, h0=h0, reverse=True)
    rA, rB, rh0 = oracle_lib.matrix_affine_scan_bwd(A, href, dy, h0=h0, reverse=True)
    for got, ref in ((At.grad, rA), (Bt.grad, rB), (h0t.grad, rh0)):
        err = np.max(np.abs(got.cpu().double().numpy() - ref) / (1 + np.abs(ref)))
        assert err <= 1e-4, err


def test_compile_fullgraph_training_step(m):
    """A small 'mixer' step using all three ops compiles into one graph (no break)
    and gives the eager values and gradients."""
    def step(z, x, la, lb, A, B):
        g = torch.sigmoid(z)
        fwd, bwd = m.scan_bidirectional_branched(g, x, g, x * 0.5)
        hl = m.scan_log(la, lb)
        hm = m.matrix_scan(A, B)
        return (fwd * bwd).sum() + hl.square().mean() + hm.sum()

    def inputs():
        return [_r(4, 2048, seed=10).requires_grad_(), _r(4, 2048, seed=11).requires_grad_(),
                (-torch.nn.functional.softplus(_r(4, 2048, seed=12))).detach().requires_grad_(),
                _r(4, 2048, seed=13).requires_grad_(),
                (_r(4, 2048, 2, 2, seed=14) * 0.6).requires_grad_(), _r(4, 2048, 2, 1, seed=15).requires_grad_()]

    a = inputs()
    loss_e = step(*a)
    loss_e.backward()
    b = inputs()
    compiled = torch.compile(step, backend="aot_eager", fullgraph=True)
    loss_c = compiled(*b)
    loss_c.backward()
    assert torch.allclose(loss_c, loss_e, rtol=1e-6, atol=0)
    for ta, tb in zip(a, b):
        assert torch.allclose(tb.grad, ta.grad, rtol=1e-5, atol=1e-6)


def test_custom_op_gradients_match_oracle(m, oracle_lib):
    r = np.random.default_rng(20)
    g = r.uniform(0, 1, (3, 5000)).astype(np.float32)
    x = r.standard_normal((3, 5000)).astype(np.float32)
    h0 = r.standard_normal(3).astype(np.float32)
    dy = r.standard_normal((3, 5000)).astype(np.float32)
    gt, xt, h0t = (torch.from_numpy(a).to(DEV).requires_grad_() for a in (g, x, h0))
    h = m.scan_causal(gt, xt, h0=h0t)
    (h * torch.from_numpy(dy).to(DEV)).sum().backward()
    href = oracle_lib.scan_fwd(g, x, h0=h0)
    rx, rg, rh0 = oracle_lib.scan_bwd(g, href, dy, h0=h0)
    for got, ref in ((xt.grad, rx), (gt.grad, rg), (h0t.grad, rh0.reshape(-1))):
        err = np.max(np.abs(got.cpu().double().numpy() - ref) / (1 + np.abs(ref)))
        assert err <= 1e-4, err
