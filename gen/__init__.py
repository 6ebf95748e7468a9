"""Seeded synthetic inputs for the affine associative scan workloads.

This module only draws random inputs and shapes them; it contains none of the
scan arithmetic. Both the fp64 oracle (``oracle/``) and the HIP path
(``associative_scan_amd``) consume what it returns, so neither side can leak
into the other through their inputs.

Seeding: every workload derives one ``numpy.random.SeedSequence([cfg_id, T,
*extra])`` and spawns one child per tensor, in the order the tensors are listed
in each function's docstring. Uniform and normal draws are made directly in
float32 (PCG64); derived quantities (sigmoid, softplus, rotations, QR) are
formed in float64 and rounded once to float32. bf16 tensors are the float32
draw rounded to nearest-even, returned both as raw bf16 bit patterns (uint16,
what the GPU reads) and as their exact float32 widening (what the oracle
reads).

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

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits_to_f32", "children",
    "quickstart", "dense", "varlen_lengths", "varlen_bidir", "logspace",
    "matrix_rot2", "matrix_orth4", "exact_mode", "segments_random",
]


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def children(cfg_id: int, T: int, n: int, *extra: int):
    """``n`` independent generators spawned from SeedSequence([cfg_id, T, *extra])."""
    ss = np.random.SeedSequence([int(cfg_id), int(T), *[int(e) for e in extra]])
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def bf16_round(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _u01(rng, shape):
    return rng.random(shape, dtype=np.float32)


def _n01(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def quickstart(C: int = 4, T: int = 128, cfg_id: int = 1):
    """README quick start: one sequence, [C, T] contiguous in T.

    Tensors (spawn order): g ~ U(0,1), x ~ N(0,1), dy ~ N(0,1). h0 = 0 (None).
    """
    rg, rx, rdy = children(cfg_id, T, 3, C)
    return {
        "g": _u01(rg, (C, T)), "x": _n01(rx, (C, T)), "dy": _n01(rdy, (C, T)),
        "h0": None, "cu_seqlens": np.array([0, T], dtype=np.int32),
    }


def dense(B: int = 8, C: int = 1536, T: int = 4096, cfg_id: int = 2, rows=None):
    """README kernel benchmark layout (B, C, seqlen), fp32.

    Tensors (spawn order): g ~ U(0,1) [B,C,T], x ~ N(0,1) [B,C,T],
    h0 ~ N(0,1) [B,C], dy ~ N(0,1) [B,C,T].

    ``rows`` (optional, indices into the flattened B*C rows) draws the same
    values for just those rows: each [B*C, T] tensor is drawn in blocks of
    rows, each block from its own child stream, so a subset costs only its
    blocks. The full tensor and any subset agree exactly.
    """
    R = B * C
    ss = np.random.SeedSequence([int(cfg_id), int(T), int(B), int(C)])
    sg, sx, sh, sdy = ss.spawn(4)
    out = {
        "g": _draw_rows(sg, R, T, "u", rows),
        "x": _draw_rows(sx, R, T, "n", rows),
        "dy": _draw_rows(sdy, R, T, "n", rows),
    }
    h0 = _n01(np.random.Generator(np.random.PCG64(sh)), (R,))
    if rows is None:
        for k in ("g", "x", "dy"):
            out[k] = out[k].reshape(B, C, T)
        out["h0"] = h0.reshape(B, C)
    else:
        out["h0"] = h0[np.asarray(rows)]
    return out


_ROWBLOCK = 64


def _draw_rows(seq, R, T, kind, rows):
    """Draw a [R, T] tensor in blocks of _ROWBLOCK rows, block b from child b of
    SeedSequence ``seq``; returns the full tensor or only the given rows."""
    nblk = (R + _ROWBLOCK - 1) // _ROWBLOCK
    seeds = seq.spawn(nblk)
    draw = _u01 if kind == "u" else _n01
    if rows is None:
        out = np.empty((R, T), dtype=np.float32)
        for b in range(nblk):
            r0, r1 = b * _ROWBLOCK, min(R, (b + 1) * _ROWBLOCK)
            out[r0:r1] = draw(np.random.Generator(np.random.PCG64(seeds[b])), (r1 - r0, T))
        return out
    rows = np.asarray(rows)
    out = np.empty((len(rows), T), dtype=np.float32)
    for b in np.unique(rows // _ROWBLOCK):
        r0, r1 = b * _ROWBLOCK, min(R, (b + 1) * _ROWBLOCK)
        blk = draw(np.random.Generator(np.random.PCG64(seeds[b])), (r1 - r0, T))
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        out[sel] = blk[rows[sel] - r0]
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

    Tensors (spawn order): lengths; then per branch (fwd, bwd): z ~ N(0,1)+2
    [C, total] -> g = sigmoid(z) -> bf16; reset mask over token positions
    (shared by all channels) with probability p_reset -> g = 0; x ~ N(0,1)
    [C, total] -> bf16; dy ~ N(0,1) [C, total] fp32.
    """
    gens = children(cfg_id, total, 9, C, nseq)
    L = varlen_lengths(gens[0], nseq, total, lmax)
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(L)
    out = {"cu_seqlens": cu, "lengths": L}
    for bi, name in enumerate(("fwd", "bwd")):
        rz, rm, rx, rdy = gens[1 + 4 * bi: 5 + 4 * bi]
        z = _n01(rz, (C, total)).astype(np.float64) + 2.0
        g32 = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
        del z
        reset = rm.random(total) < p_reset
        g32[:, reset] = 0.0
        gb = bf16_round(g32)
        del g32
        xb = bf16_round(_n01(rx, (C, total)))
        out[name] = {
            "g_bf16": gb, "x_bf16": xb,
            "g": bf16_bits_to_f32(gb).reshape(C, total),
            "x": bf16_bits_to_f32(xb).reshape(C, total),
            "reset": reset, "dy": _n01(rdy, (C, total)),
            "reverse": bi == 1,
        }
    return out


def logspace(B: int = 8, D: int = 1024, T: int = 8192, cfg_id: int = 4):
    """Log-space scan inputs, fp32.

    Tensors (spawn order): z ~ N(0,1) [B,D,T] -> log_a = -softplus(z);
    log_b ~ N(0,1) [B,D,T].
    """
    rz, rb = children(cfg_id, T, 2, B, D)
    z = _n01(rz, (B, D, T)).astype(np.float64)
    # softplus(z) = log(1 + e^z), evaluated stably
    sp = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    log_a = (-sp).astype(np.float32)
    del z, sp
    return {"log_a": log_a, "log_b": _n01(rb, (B, D, T))}


def matrix_rot2(B: int = 8, N: int = 512, T: int = 8192, p_reset: float = 1.0 / 2048, cfg_id: int = 51):
    """k=2, v=1 rotation family, fp32, layout [B*N, T, k, k] / [B*N, T, k, v].

    Tensors (spawn order): r ~ U(0.5,1), theta ~ U(-pi,pi), B ~ N(0,1) [..,2,1],
    reset mask i.i.d. per (lane, t) with probability p_reset -> A = 0,
    dy ~ N(0,1) [..,2,1].
    A_t = r_t * [[cos t, -sin t], [sin t, cos t]].
    """
    R = B * N
    rr, rt, rb, rm, rdy = children(cfg_id, T, 5, B, N)
    r = 0.5 + 0.5 * rr.random((R, T))
    th = rt.uniform(-np.pi, np.pi, (R, T))
    c, s = r * np.cos(th), r * np.sin(th)
    A = np.empty((R, T, 2, 2), dtype=np.float32)
    A[..., 0, 0] = c
    A[..., 0, 1] = -s
    A[..., 1, 0] = s
    A[..., 1, 1] = c
    del r, th, c, s
    Bm = _n01(rb, (R, T, 2, 1))
    reset = rm.random((R, T)) < p_reset
    A[reset] = 0.0
    return {"A": A, "B": Bm, "dy": _n01(rdy, (R, T, 2, 1)), "reset": reset, "k": 2, "v": 1}


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


def matrix_orth4(B: int = 8, N: int = 512, T: int = 8192, p_reset: float = 1.0 / 2048,
                 cfg_id: int = 52, chunk_rows: int = 256):
    """k=4, v=4, fp32: A_t = 0.9 * Q_t with Q_t the Q factor (positive diag R)
    of an N(0,1) 4x4 matrix; B ~ N(0,1) [4,4]; resets A = 0 with probability
    p_reset i.i.d. per (lane, t); dy ~ N(0,1) [4,4].

    Tensors (spawn order): G, B, reset mask, dy.
    """
    R = B * N
    rg, rb, rm, rdy = children(cfg_id, T, 4, B, N)
    A = np.empty((R, T, 4, 4), dtype=np.float32)
    G = _n01(rg, (R, T, 4, 4))
    for r0 in range(0, R, chunk_rows):
        r1 = min(R, r0 + chunk_rows)
        A[r0:r1] = (0.9 * _orthonormal_qr_q(G[r0:r1].astype(np.float64))).astype(np.float32)
    del G
    Bm = _n01(rb, (R, T, 4, 4))
    reset = rm.random((R, T)) < p_reset
    A[reset] = 0.0
    return {"A": A, "B": Bm, "dy": _n01(rdy, (R, T, 4, 4)), "reset": reset, "k": 4, "v": 4}


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

    g in {0,1} with runs of ones no longer than max_run (so |h| <= max_run+1
    given |x|,|h0| <= 1), x, dy in {-1,0,1}. Returned as float32.
    """
    g = (rng.random(shape) >= p_zero).astype(np.float32)
    T = shape[-1]
    flat = g.reshape(-1, T)
    for s in range(max_run, T, max_run):
        flat[:, s] = 0.0
    x = rng.integers(-1, 2, size=shape).astype(np.float32)
    dy = rng.integers(-1, 2, size=shape).astype(np.float32)
    return g, x, dy
