"""Host-side checks of libmscan that need no GPU: the library loads, exports
every entry point the header declares, sizes workspaces, and rejects bad
arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mscan.h")


@pytest.fixture(scope="module")
def m():
    import associative_scan_amd as m
    return m


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"MSCAN_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ("scan_fwd", "scan_bwd", "scan_log_fwd", "matrix_affine_scan_fwd", "matrix_affine_scan_bwd",
              "mscan_workspace_bytes", "mscan_workspace_init", "mscan_status_string", "mscan_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(m):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(m.library_path)
    for n in _declared_functions():
        assert getattr(lib, n) is not None


def test_abi_and_status_strings(m):
    assert m.lib.mscan_abi_version() == 1
    for s in range(5):
        assert m.lib.mscan_status_string(s)


def _prob(m, rows=8, T=100, stride=None, cu=None, nseg=1, reverse=0):
    return m.Problem(rows, T, T if stride is None else stride, cu, nseg, reverse)


def test_workspace_sizes(m):
    # a row that fits one 4096-element tile never chains tiles: header only
    assert m.workspace_bytes(_prob(m, rows=12288, T=4096), m.OP_SCAN_FWD) == 128
    assert m.workspace_bytes(_prob(m, rows=3, T=4096), m.OP_SCAN_FWD) == 128
    # longer rows chain tiles by look-back: header (128) + 3 words of 8 bytes
    # per tile of 4096 elements
    assert m.workspace_bytes(_prob(m, rows=12288, T=65536), m.OP_SCAN_FWD) == 128 + 12288 * 16 * 24
    # the log-space scan publishes 5 words per tile
    assert m.workspace_bytes(_prob(m, rows=3, T=65536), m.OP_SCAN_LOG_FWD) == 128 + 3 * 16 * 40
    assert m.workspace_bytes(_prob(m, rows=3, T=65536), m.OP_SCAN_FWD) == 128 + 3 * 16 * 24
    # rows of 4097 to 8191 elements (8192 for 16-bit inputs; 8192 for the
    # log-space scan) take one 8192-element tile: no chain when the rows start
    # 16-byte aligned, two tiles when a row start off that grid pushes the
    # row's last elements past the tile
    assert m.workspace_bytes(_prob(m, rows=3, T=8190, stride=8192), m.OP_SCAN_FWD) == 128
    assert m.workspace_bytes(_prob(m, rows=3, T=8190, stride=8193), m.OP_SCAN_FWD) == 128 + 3 * 2 * 24
    assert m.workspace_bytes(_prob(m, rows=3, T=8192), m.OP_SCAN_LOG_FWD) == 128
    assert m.workspace_bytes(_prob(m, rows=3, T=8193), m.OP_SCAN_LOG_FWD) == 128 + 3 * 3 * 40
    # fp32 rows of 8192 keep two 4096-element tiles
    assert m.workspace_bytes(_prob(m, rows=3, T=8192), m.OP_SCAN_FWD) == 128 + 3 * 2 * 24
    # beyond 8192, 4096-element tiles; rows that do not all start 16-byte
    # aligned may need one more
    assert m.workspace_bytes(_prob(m, rows=3, T=12288), m.OP_SCAN_FWD) == 128 + 3 * 3 * 24
    assert m.workspace_bytes(_prob(m, rows=3, T=12286, stride=12289), m.OP_SCAN_FWD) == 128 + 3 * 4 * 24
    assert m.workspace_bytes(_prob(m, rows=0), m.OP_SCAN_FWD) == 0
    assert m.workspace_bytes(_prob(m, T=10, stride=5), m.OP_SCAN_FWD) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced: validation fails first


@pytest.mark.parametrize("case", [
    dict(rows=0), dict(T=0), dict(stride=50, T=100), dict(nseg=2), dict(reverse=2), dict(nseg=0),
    dict(T=2**31, stride=2**31),  # beyond int32 cu_seqlens offsets
])
def test_scan_fwd_rejects_bad_problem(m, case):
    p = _prob(m, **case)
    st = m.lib.scan_fwd(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, None, 0, None)
    assert st == 1


def test_scan_fwd_rejects_bad_pointers_and_dtypes(m):
    p = _prob(m)
    assert m.lib.scan_fwd(ctypes.byref(p), 0, None, FAKE, None, FAKE, None, 0, None) == 1
    assert m.lib.scan_fwd(ctypes.byref(p), 0, FAKE + 4, FAKE, None, FAKE, None, 0, None) == 1   # misaligned
    assert m.lib.scan_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE + 2, FAKE, None, 0, None) == 1   # h0 misaligned
    assert m.lib.scan_fwd(ctypes.byref(p), 7, FAKE, FAKE, None, FAKE, None, 0, None) == 2       # dtype


def test_scan_fwd_requires_workspace_for_long_rows(m):
    p = _prob(m, rows=4, T=20000)
    need = m.workspace_bytes(p, m.OP_SCAN_FWD)
    assert need > 128
    assert m.lib.scan_fwd(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, None, 0, None) == 3
    assert m.lib.scan_fwd(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, FAKE, need - 8, None) == 3


def test_scan_bwd_validation(m):
    p = _prob(m)
    assert m.lib.scan_bwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, None, FAKE, None, None, 0, None) == 1
    assert m.lib.scan_bwd(ctypes.byref(p), 3, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == 2
    assert m.lib.scan_bwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE + 1, None, 0, None) == 1


def test_null_problem(m):
    st = m.lib.scan_fwd(None, 0, FAKE, FAKE, None, FAKE, None, 0, None)
    assert st == 1


def test_scan_log_bwd_validation(m):
    p = _prob(m)
    # args: prob, log_a, log_b, h, dy, log_h0, dlog_a, dlog_b, dlog_h0, ws, ws_bytes, stream
    assert m.lib.scan_log_bwd(ctypes.byref(p), FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == 1
    assert m.lib.scan_log_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE + 8, None, FAKE, FAKE, None, None, 0, None) == 1
    assert m.lib.scan_log_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE + 1, FAKE, FAKE, None, None, 0, None) == 1
    long = _prob(m, rows=4, T=20000)
    need = m.workspace_bytes(long, m.OP_SCAN_LOG_BWD)
    assert need == 128 + 4 * 5 * 24  # 3 words per 4096-element tile, 5 tiles per row
    assert m.lib.scan_log_bwd(ctypes.byref(long), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, need - 8,
                              None) == 3


def test_gated_entry_points_reject_other_gates(m):
    p = _prob(m)
    # args (scan_fwd_gated): prob, in_dtype, gate, z, x, h0, h, ws, ws_bytes, stream
    assert m.lib.scan_fwd_gated(ctypes.byref(p), 0, 0, FAKE, FAKE, None, FAKE, None, 0, None) == 2
    assert m.lib.scan_fwd_gated(ctypes.byref(p), 0, 2, FAKE, FAKE, None, FAKE, None, 0, None) == 2
    assert m.lib.scan_bwd_gated(ctypes.byref(p), 0, 2, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == 2
    assert m.lib.scan_log_fwd_gated(ctypes.byref(p), 1, FAKE, FAKE, None, FAKE, None, 0, None) == 2
    assert m.lib.scan_log_bwd_gated(ctypes.byref(p), 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, 0,
                                    None) == 2
    # the supported gate still validates its arguments on the host
    assert m.lib.scan_fwd_gated(ctypes.byref(p), 0, 1, None, FAKE, None, FAKE, None, 0, None) == 1
    assert m.lib.scan_log_fwd_gated(ctypes.byref(p), 2, FAKE, FAKE, None, FAKE + 4, None, 0, None) == 1


def test_torch_custom_ops_registered_with_fake_kernels(m):
    """The mscan:: custom ops exist with their schemas, and their fake kernels give
    output shapes on meta tensors (what torch.compile traces with), no GPU needed."""
    import torch
    assert str(torch.ops.mscan.scan.default._schema) == \
        "mscan::scan(Tensor g, Tensor x, Tensor? h0, Tensor? cu_seqlens, bool reverse) -> Tensor"
    for name in ("scan", "scan_backward", "scan_log", "scan_log_backward", "matrix_scan", "matrix_scan_backward"):
        assert hasattr(torch.ops.mscan, name)
    g = torch.empty(3, 5, 100, device="meta", dtype=torch.bfloat16)
    h = torch.ops.mscan.scan(g, g, None, None, False)
    assert h.shape == (3, 5, 100) and h.dtype == torch.float32 and h.device.type == "meta"
    hf = torch.empty(3, 5, 100, device="meta")
    cu = torch.empty(4, device="meta", dtype=torch.int32)
    dx, dg, dh0 = torch.ops.mscan.scan_backward(g, hf, hf, None, cu, True, True)
    assert dx.shape == dg.shape == (3, 5, 100) and dh0.shape == (3, 15)
    A = torch.empty(2, 7, 4, 4, device="meta")
    B = torch.empty(2, 7, 4, 1, device="meta")
    assert torch.ops.mscan.matrix_scan(A, B, None, None, False).shape == (2, 7, 4, 1)
    dA, dB, dh0 = torch.ops.mscan.matrix_scan_backward(A, B, B, None, None, False, True)
    assert dA.shape == A.shape and dB.shape == B.shape and dh0.shape == (1, 2, 4, 1)


def test_matrix_core_workspace_always_required(m):
    # The matrix-core shapes chain their chunks through the workspace on every
    # call: header (128), then per chunk and row the published state after it
    # as tagged 8-byte words, sized for the larger chunk count. k or v above 4:
    # chunks of 64 (forward) / 32 (backward) steps, a padded 16 x 16 state (256
    # words); k, v <= 4: spans of 16 x 16 steps, a padded 4 x 4 state (16 words).
    p = _prob(m, rows=5, T=100)
    need16 = 128 + 5 * 4 * 256 * 8
    for k, v in ((16, 16), (8, 8), (1, 16), (16, 1), (4, 8)):
        assert m.workspace_bytes(p, m.OP_MATRIX_FWD, k, v) == need16
        assert m.workspace_bytes(p, m.OP_MATRIX_BWD, k, v) == need16
    for k, v in ((4, 4), (2, 4), (4, 2), (1, 2), (1, 4)):
        assert m.workspace_bytes(p, m.OP_MATRIX_FWD, k, v) == 128 + 5 * 1 * 16 * 8
    assert m.workspace_bytes(_prob(m, rows=33, T=300), m.OP_MATRIX_BWD, 4, 4) == 128 + 33 * 2 * 16 * 8
    # args (fwd): prob, k, v, A, B, h0, h, ws, ws_bytes, stream
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(p), 16, 16, FAKE, FAKE, None, FAKE, None, 0, None) == 3
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(p), 8, 2, FAKE, FAKE, None, FAKE, FAKE, need16 - 4, None) == 3
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(p), 4, 4, FAKE, FAKE, None, FAKE, None, 0, None) == 3


@pytest.mark.parametrize("kv", [(3, 3), (16, 32), (32, 32), (8, 6), (1, 32), (0, 1), (4, 0), (-2, 2)])
def test_matrix_outside_envelope_unsupported(m, kv):
    """k, v outside {1, 2, 4, 8, 16} is refused on the host, never masked."""
    k, v = kv
    p = _prob(m, rows=5, T=100)
    assert m.workspace_bytes(p, m.OP_MATRIX_FWD, k, v) == 0
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(p), k, v, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, None) == 2
    assert m.lib.matrix_affine_scan_bwd(ctypes.byref(p), k, v, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                                        1 << 20, None) == 2


def test_grid_beyond_one_launch_is_unsupported(m):
    """rows x tiles beyond what one launch can address is refused on the host
    (never launched): 2^20 rows of 2^16 elements are 2^24 tiles of 4096."""
    p = _prob(m, rows=1 << 20, T=1 << 16)
    assert m.lib.scan_fwd(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None) == 2
    assert m.lib.matrix_affine_scan_fwd(ctypes.byref(_prob(m, rows=1 << 22, T=1 << 16)), 16, 16, FAKE, FAKE, None,
                                        FAKE, FAKE, 1 << 40, None) == 2
    # one tile fewer per row is accepted as far as the grid goes (then needs its workspace)
    q = _prob(m, rows=(1 << 20) - 1, T=1 << 16)
    assert m.lib.scan_fwd(ctypes.byref(q), 0, FAKE, FAKE, None, FAKE, None, 0, None) == 3



def test_workspace_error_rejects_bad_arguments_on_host(m):
    """mscan_workspace_error validates before any HIP call (no GPU needed)."""
    flag = FAKE
    assert m.lib.mscan_workspace_error(None, 4096, flag, None) == 1
    assert m.lib.mscan_workspace_error(FAKE, 64, flag, None) == 1       # below the 128-byte header
    assert m.lib.mscan_workspace_error(FAKE + 8, 4096, flag, None) == 1  # misaligned workspace
    assert m.lib.mscan_workspace_error(FAKE, 4096, None, None) == 1
    assert m.lib.mscan_workspace_error(FAKE, 4096, FAKE + 2, None) == 1  # misaligned flag
    assert m.lib.mscan_status_string(5)


@pytest.mark.parametrize("case,k,v,first,n,status", [
    (dict(T=100), 1, 1, 0, 1, 2),            # one tile per row: no wait to run out
    (dict(T=3 * 4096), 1, 1, 0, 0, 1),       # empty block range
    (dict(T=3 * 4096), 1, 1, 23, 2, 1),      # past the grid (8 rows x 3 tiles = 24 blocks)
    (dict(T=3 * 4096), 1, 1, -1, 1, 1),
    (dict(T=3 * 4096), 3, 1, 0, 1, 2),       # outside the envelope
    (dict(T=500), 2, 1, 0, 1, 2),            # a 2x1 row of one tile
])
def test_debug_partial_fwd_host_checks(m, case, k, v, first, n, status):
    p = _prob(m, **case)
    big = 1 << 30
    assert m.lib.mscan_debug_partial_fwd(ctypes.byref(p), k, v, FAKE, FAKE, FAKE, FAKE, big, first, n, 100, None) == status


def test_scan_fwd_noalloc_host_checks(m):
    """scan_fwd_noalloc refuses bad problems and problems whose descriptors do
    not fit its fixed scratch array on the host, before any HIP call."""
    p = _prob(m, rows=0)
    assert m.lib.scan_fwd_noalloc(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, None) == 1
    p = _prob(m, rows=12288, T=1 << 20)  # 12288 rows x 256 tiles of descriptors: 75 MB > 8 MiB
    assert m.workspace_bytes(p, m.OP_SCAN_FWD) > 8 << 20
    assert m.lib.scan_fwd_noalloc(ctypes.byref(p), 0, FAKE, FAKE, None, FAKE, None) == 3
    assert m.lib.scan_fwd_noalloc(ctypes.byref(_prob(m)), 7, FAKE, FAKE, None, FAKE, None) == 2
    assert m.lib.scan_fwd_noalloc(ctypes.byref(_prob(m)), 0, FAKE + 4, FAKE, None, FAKE, None) == 1
