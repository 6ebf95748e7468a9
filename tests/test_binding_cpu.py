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
