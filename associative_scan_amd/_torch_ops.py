"""torch.library registration of the scans as custom ops with autograd and fake
(meta) implementations, so torch.compile traces through them without graph
breaks ("Triton scan kernels", "Autograd integration and the reversed-scan
backward": the kernels are registered as opaque custom ops whose gradients are
wired with register_autograd).

Ops (namespace ``mscan``):
    scan(g, x, h0?, cu_seqlens?, reverse) -> h
    scan_backward(g, h, dy, h0?, cu_seqlens?, reverse, need_dh0) -> (dx, dg, dh0)
    scan_log(log_a, log_b, log_h0?, cu_seqlens?, reverse) -> h
    scan_log_backward(log_a, log_b, h, dy, log_h0?, cu_seqlens?, reverse, need_dh0) -> (dlog_a, dlog_b, dlog_h0)
    matrix_scan(A, B, h0?, cu_seqlens?, reverse) -> h
    matrix_scan_backward(A, h, dy, h0?, cu_seqlens?, reverse, need_dh0) -> (dA, dB, dh0)
A custom op cannot return None, so a skipped dh0 comes back as an empty tensor.
Every op runs the library's HIP kernels; there is no other implementation.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch
from torch import Tensor

from . import (matrix_affine_scan_bwd, matrix_affine_scan_fwd, scan_bwd, scan_fwd, scan_log_bwd,
               scan_log_fwd)


def _nseg(cu: Optional[Tensor]) -> int:
    return 1 if cu is None else cu.shape[0] - 1


def _rows(t: Tensor, tail: int) -> int:
    n = 1
    for d in t.shape[: t.dim() - 1 - tail]:
        n *= d
    return n


def _dh0_or_empty(dh0: Optional[Tensor], like: Tensor) -> Tensor:
    return dh0 if dh0 is not None else like.new_empty((0,), dtype=torch.float32)


# ---------------------------------------------------------------------------
# scalar scan
# ---------------------------------------------------------------------------
@torch.library.custom_op("mscan::scan", mutates_args=())
def scan_op(g: Tensor, x: Tensor, h0: Optional[Tensor], cu_seqlens: Optional[Tensor], reverse: bool) -> Tensor:
    return scan_fwd(g, x, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse)


@scan_op.register_fake
def _(g, x, h0, cu_seqlens, reverse):
    return torch.empty(g.shape, dtype=torch.float32, device=g.device)


@torch.library.custom_op("mscan::scan_backward", mutates_args=())
def scan_backward_op(g: Tensor, h: Tensor, dy: Tensor, h0: Optional[Tensor], cu_seqlens: Optional[Tensor],
                     reverse: bool, need_dh0: bool) -> Tuple[Tensor, Tensor, Tensor]:
    dx, dg, dh0 = scan_bwd(g, h, dy, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse, need_dh0=need_dh0)
    return dx, dg, _dh0_or_empty(dh0, h)


@scan_backward_op.register_fake
def _(g, h, dy, h0, cu_seqlens, reverse, need_dh0):
    dh0 = (torch.empty((_nseg(cu_seqlens), _rows(h, 0)), dtype=torch.float32, device=h.device) if need_dh0
           else h.new_empty((0,), dtype=torch.float32))
    return torch.empty_like(h), torch.empty_like(h), dh0


def _scan_setup(ctx, inputs, output):
    g, x, h0, cu, reverse = inputs
    ctx.save_for_backward(g, output, h0, cu)
    ctx.reverse = reverse
    ctx.x_dtype = x.dtype


def _scan_backward(ctx, dy):
    g, h, h0, cu = ctx.saved_tensors
    need = h0 is not None and ctx.needs_input_grad[2]
    dx, dg, dh0 = scan_backward_op(g, h, dy.contiguous().float(), h0, cu, ctx.reverse, need)
    return dg.to(g.dtype), dx.to(ctx.x_dtype), (dh0.view(h0.shape) if need else None), None, None


scan_op.register_autograd(_scan_backward, setup_context=_scan_setup)


# ---------------------------------------------------------------------------
# log-space scan
# ---------------------------------------------------------------------------
@torch.library.custom_op("mscan::scan_log", mutates_args=())
def scan_log_op(log_a: Tensor, log_b: Tensor, log_h0: Optional[Tensor], cu_seqlens: Optional[Tensor],
                reverse: bool) -> Tensor:
    return scan_log_fwd(log_a, log_b, log_h0=log_h0, cu_seqlens=cu_seqlens, reverse=reverse)


@scan_log_op.register_fake
def _(log_a, log_b, log_h0, cu_seqlens, reverse):
    return torch.empty_like(log_a)


@torch.library.custom_op("mscan::scan_log_backward", mutates_args=())
def scan_log_backward_op(log_a: Tensor, log_b: Tensor, h: Tensor, dy: Tensor, log_h0: Optional[Tensor],
                         cu_seqlens: Optional[Tensor], reverse: bool,
                         need_dh0: bool) -> Tuple[Tensor, Tensor, Tensor]:
    dla, dlb, dlh0 = scan_log_bwd(log_a, log_b, h, dy, log_h0=log_h0, cu_seqlens=cu_seqlens, reverse=reverse,
                                  need_dh0=need_dh0)
    return dla, dlb, _dh0_or_empty(dlh0, h)


@scan_log_backward_op.register_fake
def _(log_a, log_b, h, dy, log_h0, cu_seqlens, reverse, need_dh0):
    dh0 = (torch.empty((_nseg(cu_seqlens), _rows(h, 0)), dtype=torch.float32, device=h.device) if need_dh0
           else h.new_empty((0,), dtype=torch.float32))
    return torch.empty_like(h), torch.empty_like(h), dh0


def _log_setup(ctx, inputs, output):
    log_a, log_b, log_h0, cu, reverse = inputs
    ctx.save_for_backward(log_a, log_b, output, log_h0, cu)
    ctx.reverse = reverse


def _log_backward(ctx, dy):
    log_a, log_b, h, log_h0, cu = ctx.saved_tensors
    need = log_h0 is not None and ctx.needs_input_grad[2]
    dla, dlb, dlh0 = scan_log_backward_op(log_a, log_b, h, dy.contiguous().float(), log_h0, cu, ctx.reverse, need)
    return dla, dlb, (dlh0.view(log_h0.shape) if need else None), None, None


scan_log_op.register_autograd(_log_backward, setup_context=_log_setup)


# ---------------------------------------------------------------------------
# matrix-affine scan
# ---------------------------------------------------------------------------
@torch.library.custom_op("mscan::matrix_scan", mutates_args=())
def matrix_scan_op(A: Tensor, B: Tensor, h0: Optional[Tensor], cu_seqlens: Optional[Tensor],
                   reverse: bool) -> Tensor:
    return matrix_affine_scan_fwd(A, B, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse)


@matrix_scan_op.register_fake
def _(A, B, h0, cu_seqlens, reverse):
    return torch.empty_like(B)


@torch.library.custom_op("mscan::matrix_scan_backward", mutates_args=())
def matrix_scan_backward_op(A: Tensor, h: Tensor, dy: Tensor, h0: Optional[Tensor], cu_seqlens: Optional[Tensor],
                            reverse: bool, need_dh0: bool) -> Tuple[Tensor, Tensor, Tensor]:
    dA, dB, dh0 = matrix_affine_scan_bwd(A, h, dy, h0=h0, cu_seqlens=cu_seqlens, reverse=reverse,
                                         need_dh0=need_dh0)
    return dA, dB, _dh0_or_empty(dh0, h)


@matrix_scan_backward_op.register_fake
def _(A, h, dy, h0, cu_seqlens, reverse, need_dh0):
    k, v = h.shape[-2], h.shape[-1]
    dh0 = (torch.empty((_nseg(cu_seqlens), _rows(h, 2), k, v), dtype=torch.float32, device=h.device) if need_dh0
           else h.new_empty((0,), dtype=torch.float32))
    return torch.empty_like(A), torch.empty_like(h), dh0


def _matrix_setup(ctx, inputs, output):
    A, B, h0, cu, reverse = inputs
    ctx.save_for_backward(A, output, h0, cu)
    ctx.reverse = reverse


def _matrix_backward(ctx, dy):
    A, h, h0, cu = ctx.saved_tensors
    need = h0 is not None and ctx.needs_input_grad[2]
    dA, dB, dh0 = matrix_scan_backward_op(A, h, dy.contiguous().float(), h0, cu, ctx.reverse, need)
    return dA, dB, (dh0.view(h0.shape) if need else None), None, None


matrix_scan_op.register_autograd(_matrix_backward, setup_context=_matrix_setup)
