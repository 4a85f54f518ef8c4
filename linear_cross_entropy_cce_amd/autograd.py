"""PyTorch autograd wrapper over the C ABI: a drop-in for
cross_entropy(H @ E.T, labels) that never forms the logits.

The per-token loss comes from cce_forward; the reduction is the caller's
and reaches the backward as dloss (mean over non-ignored rows, or sum).
"""
from __future__ import annotations

import torch

from . import binding


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, E, labels, ignore_index, filter_eps, sort_vocab):
        # With the sort, the forward already visits the vocabulary in the
        # backward's order, so that its block-max table (one float per
        # 128 x 128 logit block) describes the backward's blocks: tiles the
        # gradient filter would drop entirely are then not recomputed.
        perm = binding.cce_vocab_order(H, E, labels, ignore_index) if sort_vocab else None
        tb = None
        if filter_eps > 0:
            tb = torch.empty(binding.block_max_elems(H.shape[0], E.shape[0]), dtype=torch.float32, device=H.device)
        loss, lse = binding.cce_forward(H, E, labels, ignore_index, block_max=tb, perm=perm)
        ctx.save_for_backward(H, E, labels, lse, tb, perm)
        ctx.ignore_index = ignore_index
        ctx.filter_eps = filter_eps
        ctx.mark_non_differentiable(lse)
        return loss, lse

    @staticmethod
    def backward(ctx, dloss, _dlse):
        H, E, labels, lse, tb, perm = ctx.saved_tensors
        dH, dE = binding.cce_backward(H, E, labels, lse, dloss.float().contiguous(), ctx.filter_eps,
                                      ctx.ignore_index, perm, block_max=tb)
        return dH, dE, None, None, None, None


class _CompositeLinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, E0, E1, labels, offset1, ignore_index, filter_eps, sort_vocab):
        perm = binding.cce_vocab_order_composite(H, E0, E1, labels, ignore_index) if sort_vocab else None
        tb = None
        if filter_eps > 0:
            tb = torch.empty(binding.block_max_elems(H.shape[0], E0.shape[0] + E1.shape[0]), dtype=torch.float32,
                             device=H.device)
        loss, lse = binding.cce_forward_composite(H, E0, E1, offset1, labels, ignore_index, block_max=tb, perm=perm)
        ctx.save_for_backward(H, E0, E1, labels, lse, tb, perm)
        ctx.offset1 = offset1
        ctx.ignore_index = ignore_index
        ctx.filter_eps = filter_eps
        ctx.mark_non_differentiable(lse)
        return loss, lse

    @staticmethod
    def backward(ctx, dloss, _dlse):
        H, E0, E1, labels, lse, tb, perm = ctx.saved_tensors
        dH, dE0, dE1 = binding.cce_backward_composite(H, E0, E1, ctx.offset1, labels, lse, dloss.float().contiguous(),
                                                      ctx.filter_eps, ctx.ignore_index, perm, block_max=tb)
        return dH, dE0, dE1, None, None, None, None, None


def _reduce(loss, labels, ignore_index, reduction):
    if reduction == "none":
        return loss
    if reduction == "sum":
        return loss.sum()
    if reduction == "mean":
        n = (labels != ignore_index).sum().clamp_min(1)
        return loss.sum() / n
    raise ValueError(f"unknown reduction {reduction!r}")


def linear_cross_entropy_composite(H, E0, E1, offset1, labels, ignore_index=-100, reduction="mean",
                                   filter_eps=2.0 ** -12, sort_vocab=False):
    """linear_cross_entropy for a composite head: token ids [0, V0) are the
    rows of E0 [V0, D], ids [offset1, offset1 + V1) the rows of E1 [V1, D],
    and the ids in between have no row (they add nothing to the softmax and
    are never a label).  Gradients flow to H, E0 and E1."""
    if reduction not in ("none", "sum", "mean"):
        raise ValueError(f"unknown reduction {reduction!r}")
    loss, _ = _CompositeLinearCrossEntropy.apply(H, E0, E1, labels, int(offset1), int(ignore_index),
                                                 float(filter_eps), bool(sort_vocab))
    return _reduce(loss, labels, ignore_index, reduction)


def linear_cross_entropy(H, E, labels, ignore_index=-100, reduction="mean", filter_eps=2.0 ** -12,
                         sort_vocab=False):
    """Cross-entropy of the logits H @ E.T against labels, without the logits.

    H [N, D] and E [V, D] (bf16 or fp32, on the GPU); labels int64 [N].
    reduction: "none" (per-token fp32 loss), "sum", or "mean" over the rows
    whose label is not ignore_index.  filter_eps: gradient-filter threshold
    (0 disables filtering).  sort_vocab: visit the vocabulary by descending
    mean logit (forward and backward) so that surviving blocks cluster.
    """
    if reduction not in ("none", "sum", "mean"):
        raise ValueError(f"unknown reduction {reduction!r}")
    loss, _ = _LinearCrossEntropy.apply(H, E, labels, int(ignore_index), float(filter_eps), bool(sort_vocab))
    return _reduce(loss, labels, ignore_index, reduction)
