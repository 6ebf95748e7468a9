"""Seeded synthetic inputs for the affine associative scan workloads.

This module only draws random inputs and shapes them; it contains none of the
scan arithmetic. Both the fp64 oracle (``oracle/``) and the HIP path
(``associative_scan_amd``) consume what it returns, so neither side can leak
into the other through their inputs.

Seeding recipe: a workload derives ``numpy.random.SeedSequence([cfg_id, T,
*shape])`` and spawns one child per tensor, in the order each function's
docstring lists. Every tensor is drawn in blocks of 64 rows (the leading,
independent axis); block b uses a PCG64 stream seeded by child b of the
tensor's sequence. Blocks are filled by a thread pool, and since each block has
its own stream the values do not depend on the thread count, and any subset of
rows can be regenerated alone (``dense(rows=...)``). Uniform and normal draws
are float32; derived quantities (sigmoid, softplus, rotations, QR) are formed
in float64 per block and rounded once to float32. bf16 tensors are the float32
values rounded to nearest-even, returned both as raw bf16 bit patterns
(uint16, what the GPU reads) and as their exact float32 widening (what the
oracle reads).

The workloads mirror the shapes and distributions the pages benchmark on:
- the quick-start case of the associative-scan-triton README (C=4, T=128,
  gates U(0,1), tokens N(0,1), one sequence);
- the README's kernel benchmark shape (B=8, C=1536, seqlen swept 128..65536);
- packed variable-length sequences in the flash-attn ``cu_seqlens`` convention
  with two branches in opposite time directions (README, "bidirectional" and
  "how it works");
- the log-space scan of the minGRU Triton page (``parallel_scan_log``);
- the small matrix-affine scan of the minGRU Triton page (k=2, v=1 rotation
  family and generic k=v=4).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits_to_f32",
    "quickstart", "dense", "varlen_lengths", "varlen_bidir", "logspace",
    "matrix_rot2", "matrix_orth4", "exact_mode", "segments_random",
]

_ROWBLOCK = 64
_THREADS = max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def bf16_round(a) -> np.ndarray:
    """Round finite float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _u01(rng, shape):
    return rng.random(shape, dtype=np.float32)


def _n01(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _tensors(cfg_id, T, n, *extra):
    """n child SeedSequences (one per tensor) of SeedSequence([cfg_id, T, *extra])."""
    return np.random.SeedSequence([int(cfg_id), int(T), *[int(e) for e in extra]]).spawn(n)


def _draw(seq, shape, fn, dtype=np.float32, rows=None):
    """Tensor of ``shape`` whose axis-0 blocks of 64 rows are fn(rng_b, block_shape).

    rng_b = PCG64(child b of ``seq``). With ``rows`` (indices into axis 0) only
    those rows are returned, drawing just the blocks that hold them."""
    R = shape[0]
    nblk = (R + _ROWBLOCK - 1) // _ROWBLOCK
    seeds = seq.spawn(nblk)

    def block(b):
        r0, r1 = b * _ROWBLOCK, min(R, (b + 1) * _ROWBLOCK)
        return fn(np.random.Generator(np.random.PCG64(seeds[b])), (r1 - r0,) + tuple(shape[1:]))

    if rows is None:
        out = np.empty(shape, dtype=dtype)

        def fill(b):
            out[b * _ROWBLOCK: min(R, (b + 1) * _ROWBLOCK)] = block(b)

        if nblk == 1:
            fill(0)
        else:
            with ThreadPoolExecutor(_THREADS) as ex:
                list(ex.map(fill, range(nblk)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows),) + tuple(shape[1:]), dtype=dtype)
    for b in np.unique(rows // _ROWBLOCK):
        blk = block(int(b))
        sel = np.nonzero(rows // _ROWBLOCK == b)[0]
        out[sel] = blk[rows[sel] - b * _ROWBLOCK]
    return out


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def quickstart(C: int = 4, T: int = 128, cfg_id: int = 1):
    """README quick start: one sequence, [C, T] contiguous in T.

    Tensors (spawn order): g ~ U(0,1), x ~ N(0,1), dy ~ N(0,1). h0 = 0 (None).
    """
    sg, sx, sdy = _tensors(cfg_id, T, 3, C)
    return {
        "g": _draw(sg, (C, T), _u01), "x": _draw(sx, (C, T), _n01), "dy": _draw(sdy, (C, T), _n01),
        "h0": None, "cu_seqlens": np.array([0, T], dtype=np.int32),
    }


def dense(B: int = 8, C: int = 1536, T: int = 4096, cfg_id: int = 2, rows=None, want=("g", "x", "h0", "dy")):
    """README kernel benchmark layout (B, C, seqlen), fp32.

    Tensors (spawn order): g ~ U(0,1) [B,C,T], x ~ N(0,1) [B,C,T],
    h0 ~ N(0,1) [B,C], dy ~ N(0,1) [B,C,T].

    ``rows`` (indices into the flattened B*C rows) returns the same values for
    just those rows, as [len(rows), T] (h0 as [len(rows)]); ``want`` limits
    which tensors are drawn.
    """
    R = B * C
    sg, sx, sh, sdy = _tensors(cfg_id, T, 4, B, C)
    out = {}
    for name, seq, fn, shp in (("g", sg, _u01, (R, T)), ("x", sx, _n01, (R, T)),
                               ("h0", sh, _n01, (R,)), ("dy", sdy, _n01, (R, T))):
        if name in want:
            out[name] = _draw(seq, shp, fn, rows=rows)
    if rows is None:
        for k in ("g", "x", "dy"):
            if k in out:
                out[k] = out[k].reshape(B, C, T)
        if "h0" in out:
            out["h0"] = out["h0"].reshape(B, C)
    return out


def varlen_lengths(rng, nseq: int = 16, total: int = 65536, lmax: int = 8192):
    """Sequence lengths for the packed workload: nseq-1 lengths i.i.d. U{1..lmax};
    if their sum leaves no room for a last sequence of length >= 1, all nseq-1
    are redrawn from the same stream; the last sequence absorbs the remainder
    (it may exceed lmax)."""
    while True:
        L = rng.integers(1, lmax + 1, size=nseq - 1)
        if L.sum() <= total - 1:
            break
    return np.concatenate([L, [total - L.sum()]]).astype(np.int64)


def varlen_bidir(C: int = 1536, total: int = 65536, nseq: int = 16, lmax: int = 8192,
                 p_reset: float = 1.0 / 1024, cfg_id: int = 3):
    """Packed variable-length, two branches in opposite time directions, bf16 inputs.

    Tensors (spawn order): lengths; then per branch (fwd, bwd): z ~ N(0,1) [C, total]
    -> g = sigmoid(z + 2) -> bf16; a reset mask over token positions (shared by
    all channels, probability p_reset) -> g = 0; x ~ N(0,1) [C, total] -> bf16;
    dy ~ N(0,1) [C, total] fp32.
    """
    seqs = _tensors(cfg_id, total, 9, C, nseq)
    L = varlen_lengths(np.random.Generator(np.random.PCG64(seqs[0])), nseq, total, lmax)
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(L)
    out = {"cu_seqlens": cu, "lengths": L}

    def gate_bits(rng, shp):
        z = _n01(rng, shp).astype(np.float64) + 2.0
        return bf16_round((1.0 / (1.0 + np.exp(-z))).astype(np.float32))

    for bi, name in enumerate(("fwd", "bwd")):
        sz, sm, sx, sdy = seqs[1 + 4 * bi: 5 + 4 * bi]
        gb = _draw(sz, (C, total), gate_bits, dtype=np.uint16)
        reset = np.random.Generator(np.random.PCG64(sm)).random(total) < p_reset
        gb[:, reset] = 0  # +0.0 in bf16
        xb = _draw(sx, (C, total), lambda r, s: bf16_round(_n01(r, s)), dtype=np.uint16)
        out[name] = {
            "g_bf16": gb, "x_bf16": xb,
            "g": bf16_bits_to_f32(gb).reshape(C, total),
            "x": bf16_bits_to_f32(xb).reshape(C, total),
            "reset": reset, "dy": _draw(sdy, (C, total), _n01),
            "reverse": bi == 1,
        }
    return out


def logspace(B: int = 8, D: int = 1024, T: int = 8192, cfg_id: int = 4):
    """Log-space scan inputs, fp32, [B, D, T].

    Tensors (spawn order): z ~ N(0,1) -> log_a = -softplus(z); log_b ~ N(0,1).
    """
    sz, sb = _tensors(cfg_id, T, 2, B, D)

    def neg_softplus(rng, shp):
        z = _n01(rng, shp).astype(np.float64)
        return (-(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))).astype(np.float32)

    R = B * D
    return {"log_a": _draw(sz, (R, T), neg_softplus).reshape(B, D, T),
            "log_b": _draw(sb, (R, T), _n01).reshape(B, D, T)}


def matrix_rot2(B: int = 8, N: int = 512, T: int = 8192, p_reset: float = 1.0 / 2048, cfg_id: int = 51,
                rows=None):
    """k=2, v=1 rotation family, fp32, layout [B*N, T, 2, 2] / [B*N, T, 2, 1].

    Tensors (spawn order): A (r ~ U(0.5,1) and theta ~ U(-pi,pi) from one
    stream per block: A_t = r_t * [[cos, -sin], [sin, cos]]), B ~ N(0,1),
    reset mask i.i.d. per (lane, t) with probability p_reset -> A = 0,
    dy ~ N(0,1). With ``rows`` only those rows of the B*N are drawn.
    """
    R = B * N
    sa, sb, sm, sdy = _tensors(cfg_id, T, 4, B, N)

    def rot(rng, shp):
        n, t = shp[0], shp[1]
        r = 0.5 + 0.5 * rng.random((n, t))
        th = rng.uniform(-np.pi, np.pi, (n, t))
        c, s = r * np.cos(th), r * np.sin(th)
        A = np.empty((n, t, 2, 2), dtype=np.float32)
        A[..., 0, 0], A[..., 0, 1], A[..., 1, 0], A[..., 1, 1] = c, -s, s, c
        return A

    A = _draw(sa, (R, T, 2, 2), rot, rows=rows)
    reset = _draw(sm, (R, T), lambda r, s: r.random(s) < p_reset, dtype=bool, rows=rows)
    A[reset] = 0.0
    return {"A": A, "B": _draw(sb, (R, T, 2, 1), _n01, rows=rows), "dy": _draw(sdy, (R, T, 2, 1), _n01, rows=rows),
            "reset": reset, "k": 2, "v": 1}


def _orthonormal_qr_q(G: np.ndarray) -> np.ndarray:
    """Q factor of the QR decomposition with positive diag(R), for a stack of
    square float64 matrices, by modified Gram-Schmidt on the columns (the
    positive-diagonal QR factor is unique, so this equals Householder QR with
    Q*diag(sign(diag R)))."""
    Q = G.copy()
    k = G.shape[-1]
    for j in range(k):
        for i in range(j):
            proj = np.einsum("...r,...r->...", Q[..., :, i], Q[..., :, j])
            Q[..., :, j] -= proj[..., None] * Q[..., :, i]
        nrm = np.sqrt(np.einsum("...r,...r->...", Q[..., :, j], Q[..., :, j]))
        Q[..., :, j] /= nrm[..., None]
    return Q


def matrix_orth4(B: int = 8, N: int = 512, T: int = 8192, p_reset: float = 1.0 / 2048, cfg_id: int = 52,
                 rows=None):
    """k=4, v=4, fp32: A_t = 0.9 * Q_t with Q_t the Q factor (positive diag R)
    of an N(0,1) 4x4 matrix; B ~ N(0,1) [4,4]; resets A = 0 with probability
    p_reset i.i.d. per (lane, t); dy ~ N(0,1) [4,4]. With ``rows`` only those
    rows of the B*N are drawn.

    Tensors (spawn order): A (from G), B, reset mask, dy.
    """
    R = B * N
    sa, sb, sm, sdy = _tensors(cfg_id, T, 4, B, N)

    def orth(rng, shp):
        G = _n01(rng, shp).astype(np.float64)
        return (0.9 * _orthonormal_qr_q(G)).astype(np.float32)

    A = _draw(sa, (R, T, 4, 4), orth, rows=rows)
    reset = _draw(sm, (R, T), lambda r, s: r.random(s) < p_reset, dtype=bool, rows=rows)
    A[reset] = 0.0
    return {"A": A, "B": _draw(sb, (R, T, 4, 4), _n01, rows=rows), "dy": _draw(sdy, (R, T, 4, 4), _n01, rows=rows),
            "reset": reset, "k": 4, "v": 4}


def matrix_orth16(B: int = 8, N: int = 64, T: int = 4096, p_reset: float = 1.0 / 2048, cfg_id: int = 53,
                  rows=None):
    """k=16, v=16, fp32: A_t = 0.9 * Q_t with Q_t the Q factor (positive diag R)
    of an N(0,1) 16x16 matrix; B ~ N(0,1) [16,16]; resets A = 0 with
    probability p_reset i.i.d. per (lane, t); dy ~ N(0,1) [16,16]. With ``rows``
    only those rows of the B*N are drawn.

    Tensors (spawn order): A (from G), B, reset mask, dy.
    """
    R = B * N
    sa, sb, sm, sdy = _tensors(cfg_id, T, 4, B, N)

    def orth(rng, shp):
        G = _n01(rng, shp).astype(np.float64)
        Q, Rf = np.linalg.qr(G)  # Householder; flip columns so that diag(R) > 0
        Q *= np.sign(np.diagonal(Rf, axis1=-2, axis2=-1))[..., None, :]
        return (0.9 * Q).astype(np.float32)

    A = _draw(sa, (R, T, 16, 16), orth, rows=rows)
    reset = _draw(sm, (R, T), lambda r, s: r.random(s) < p_reset, dtype=bool, rows=rows)
    A[reset] = 0.0
    return {"A": A, "B": _draw(sb, (R, T, 16, 16), _n01, rows=rows),
            "dy": _draw(sdy, (R, T, 16, 16), _n01, rows=rows), "reset": reset, "k": 16, "v": 16}


# ----------------------------------------------------------------------------
# small structured inputs for edge cases
# ----------------------------------------------------------------------------
def segments_random(rng, T: int, nseg: int, allow_empty: bool = True) -> np.ndarray:
    """Random cu_seqlens (int32, nseg+1 entries, cu[0]=0, cu[-1]=T, nondecreasing)."""
    if nseg == 1:
        return np.array([0, T], dtype=np.int32)
    if allow_empty:
        cuts = np.sort(rng.integers(0, T + 1, size=nseg - 1))
    else:
        assert T >= nseg
        cuts = np.sort(rng.choice(np.arange(1, T), size=nseg - 1, replace=False))
    return np.concatenate([[0], cuts, [T]]).astype(np.int32)


def exact_mode(rng, shape, max_run: int = 2048, p_zero: float = 0.02):
    """Integer-valued inputs whose scan is exact in fp32 in every association order.

    g in {0,1} with runs of ones shorter than max_run (a zero every max_run
    steps), x and dy in {-1,0,1}; with |h0| <= 1 every state, adjoint and gate
    gradient is an integer below 2^24. Returned as float32.
    """
    g = (rng.random(shape) >= p_zero).astype(np.float32)
    T = shape[-1]
    flat = g.reshape(-1, T)
    flat[:, max_run - 1::max_run] = 0.0
    x = rng.integers(-1, 2, size=shape).astype(np.float32)
    dy = rng.integers(-1, 2, size=shape).astype(np.float32)
    return g, x, dy
