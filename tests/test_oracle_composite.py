"""Pins of the oracle's composite head (two classifier blocks with a dead gap
between their ids, the lit note "The loss and the mask: Cut Cross-Entropy +
FlexAttention", section "What transfers to us").

  - torch's cross_entropy (CPU, fp64) on the assembled composite logit row,
    with -inf in the gap, and its autograd gradients: a textbook routine that
    shares nothing with the oracle's segment-wise logaddexp;
  - with no gap, the single-head oracle (pinned on its own) on the
    concatenated classifier;
  - widening the gap (and moving the second block's labels with it) changes
    nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import inputs


def _case(V0, V1, off1, N=24, D=16, seed=0, ignore=0.2, peaked=False):
    x = inputs.make_inputs(N, D, V0 + V1, dtype="f32", e_std=0.3, h_kind="peaked" if peaked else "normal",
                           label_kind="uniform", ignore_frac=ignore, seed=seed)
    H = x.H.astype(np.float64)
    E = x.E.astype(np.float64)
    y = x.labels.copy()
    second = y >= V0
    y[second] = y[second] - V0 + off1
    rng = np.random.default_rng(seed + 100)
    dl = rng.uniform(0.1, 1.0, N)
    return H, E[:V0], E[V0:], y, dl, x.labels


def _torch_reference(H, E0, E1, off1, y, dl):
    Ht = torch.tensor(H, requires_grad=True)
    E0t = torch.tensor(E0, requires_grad=True)
    E1t = torch.tensor(E1, requires_grad=True)
    gap = off1 - E0.shape[0]
    parts = [Ht @ E0t.T]
    if gap:
        parts.append(torch.full((H.shape[0], gap), -float("inf"), dtype=torch.float64))
    parts.append(Ht @ E1t.T)
    Z = torch.cat(parts, dim=1)
    yt = torch.tensor(y)
    loss = torch.nn.functional.cross_entropy(Z, yt, reduction="none", ignore_index=-100)
    (loss * torch.tensor(dl)).sum().backward()
    lse = torch.logsumexp(Z, dim=1)
    return loss.detach().numpy(), lse.detach().numpy(), Ht.grad.numpy(), E0t.grad.numpy(), E1t.grad.numpy()


@pytest.mark.parametrize("V0,V1,off1", [(7, 5, 7), (7, 5, 12), (1, 1, 3), (30, 11, 100)])
def test_matches_torch_cross_entropy(V0, V1, off1):
    H, E0, E1, y, dl, _ = _case(V0, V1, off1)
    loss, lse, dH, dE0, dE1 = oracle.composite(H, E0, E1, off1, y, dl)
    rl, rlse, rdH, rdE0, rdE1 = _torch_reference(H, E0, E1, off1, y, dl)
    valid = y != -100
    np.testing.assert_allclose(loss, rl, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[valid], rlse[valid], rtol=1e-12, atol=1e-12)
    assert np.all(lse[~valid] == 0) and np.all(loss[~valid] == 0)
    for a, b in ((dH, rdH), (dE0, rdE0), (dE1, rdE1)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_no_gap_is_the_single_head_on_the_concatenation():
    H, E0, E1, y, dl, y_cat = _case(20, 13, 20, peaked=True, seed=3)
    loss, lse, dH, dE0, dE1 = oracle.composite(H, E0, E1, 20, y, dl)
    l2, lse2, dH2, dE2 = oracle.backward(H, np.concatenate([E0, E1]), y_cat, dl)
    np.testing.assert_allclose(loss, l2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dH, dH2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([dE0, dE1]), dE2, rtol=1e-10, atol=1e-12)


def test_gap_width_changes_nothing():
    H, E0, E1, y, dl, _ = _case(9, 6, 9, seed=5)
    a = oracle.composite(H, E0, E1, 9, y, dl)
    y2 = np.where(y >= 9, y + 1000, y)
    b = oracle.composite(H, E0, E1, 1009, y2, dl)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_gap_label_is_rejected():
    H, E0, E1, y, dl, _ = _case(9, 6, 20, seed=6)
    y = y.copy()
    y[0] = 12  # in the gap
    with pytest.raises(ValueError):
        oracle.composite(H, E0, E1, 20, y, dl)
