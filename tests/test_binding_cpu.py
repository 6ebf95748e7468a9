"""Host-side row-view logic of the Python binding (no GPU needed).

`_rows_view` maps a tensor to (rows, T, row_stride) for the C ABI. Its
contiguous fast path must agree with the general per-axis walk, and strided
views must be accepted or refused exactly when their leading axes collapse to
one row stride."""
import pytest
import torch


class _OnDevice:
    """A CPU tensor presented as a device tensor to the view logic."""

    def __init__(self, t):
        self._t = t
        self.is_cuda = True
        self.shape = t.shape

    def dim(self):
        return self._t.dim()

    def stride(self, i):
        return self._t.stride(i)

    def numel(self):
        return self._t.numel()

    def is_contiguous(self):
        return self._t.is_contiguous()


class _Strided(_OnDevice):
    """Same, with the contiguous fast path disabled (forces the general walk)."""

    def is_contiguous(self):
        return False


@pytest.fixture(scope="module")
def m():
    import associative_scan_amd as m
    return m


@pytest.mark.parametrize("shape,tail", [
    ((5, 7), 0), ((2, 3, 9), 0), ((9,), 0), ((1, 1, 8), 0), ((2, 0, 5), 0), ((3, 1), 0),
    ((4, 6, 2, 3), 2), ((3, 5, 16, 16), 2), ((3, 4, 1, 4), 2), ((2, 5, 4, 1), 2), ((7, 2, 1), 2),
])
def test_fast_path_matches_general_walk(m, shape, tail):
    t = torch.zeros(shape)
    assert m._rows_view(_OnDevice(t), "t", tail) == m._rows_view(_Strided(t), "t", tail)


def test_strided_views(m):
    base = torch.zeros((6, 20))
    # rows of a wider buffer: stride 20, T 13
    assert m._rows_view(_OnDevice(base[:, :13]), "t") == (6, 13, 20)
    # every other row: one uniform stride of 40
    assert m._rows_view(_OnDevice(base[::2, :13]), "t") == (3, 13, 40)
    # [2, 3, T] from a [6, 20] buffer: leading axes collapse (3 * 20 = 60)
    assert m._rows_view(_OnDevice(base.view(2, 3, 20)[:, :, :13]), "t") == (6, 13, 20)
    # time axis not contiguous
    with pytest.raises(ValueError):
        m._rows_view(_OnDevice(base[:, ::2]), "t")
    # leading axes that do not collapse to one stride
    with pytest.raises(ValueError):
        m._rows_view(_OnDevice(base.view(2, 3, 20)[:, :2, :13]), "t")
    # host tensors are refused
    with pytest.raises(ValueError):
        m._rows_view(base, "t")


def test_debug_cu_seqlens_host_validation():
    """Debug mode checks cu_seqlens contents on the host (flash-attn convention)."""
    import numpy as np
    import associative_scan_amd as m
    m._validate_cu_host(np.array([0, 0, 5, 9, 9], np.int32), 9)
    for bad, T in (([1, 9], 9), ([0, 8], 9), ([0, 5, 4, 9], 9), ([0], 9)):
        with pytest.raises(ValueError):
            m._validate_cu_host(np.array(bad, np.int32), T)


def test_debug_reporting_path(monkeypatch):
    """A set error word raises MscanError (status 5) in debug mode, a clear one
    does not, and nothing is read with debug mode off (the word itself is read
    on the GPU by mscan_workspace_error; here its value is stubbed)."""
    import associative_scan_amd as m
    seen = []

    def fake_read(wsp, wsn, dev, sh):
        seen.append(wsp)
        return fake_read.code

    monkeypatch.setattr(m, "_read_ws_error", fake_read)
    monkeypatch.setattr(m.torch.cuda, "is_current_stream_capturing", lambda: False)  # no device here
    old = m.debug_enabled()
    try:
        m.set_debug(True)
        fake_read.code = 5
        with pytest.raises(m.MscanError) as e:
            m._check("scan_fwd", 0, (1234, 4096, None, 0))
        assert e.value.status == 5 and "wait gave up" in str(e.value)
        fake_read.code = 0
        m._check("scan_fwd", 0, (1234, 4096, None, 0))
        m._check("scan_fwd", 0, (None, 0, None, 0))  # no workspace used: nothing to read
        assert seen == [1234, 1234]
        m.set_debug(False)
        fake_read.code = 5
        m._check("scan_fwd", 0, (1234, 4096, None, 0))
        assert seen == [1234, 1234]
    finally:
        m.set_debug(old)
