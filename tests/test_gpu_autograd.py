"""The PyTorch autograd wrapper: the reduction reaches the backward as
dloss, and the gradients torch hands back equal the C ABI's on the same
inputs (bit for bit: same kernels, same dloss), for the one-matrix and the
composite head, with and without the vocabulary sort."""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import autograd as A
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _dloss(x, reduction):
    valid = x.labels != x.ignore_index
    if reduction == "mean":
        return np.where(valid, 1.0 / max(valid.sum(), 1), 0.0).astype(np.float32)
    return np.where(valid, 1.0, 0.0).astype(np.float32)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("sort", [False, True])
def test_wrapper_matches_abi(reduction, sort):
    x = inputs.make_workload(3, N=600, D=512, V=5000)
    G.say(f"autograd reduction={reduction} sort={sort}")
    H, E, y = G.to_device(x)
    Hl = H.clone().requires_grad_(True)
    El = E.clone().requires_grad_(True)
    out = A.linear_cross_entropy(Hl, El, y, x.ignore_index, reduction=reduction, filter_eps=x.eps, sort_vocab=sort)
    if reduction == "none":
        out.backward(torch.from_numpy(_dloss(x, "sum")).to(G.DEV))
    else:
        out.backward()
    torch.cuda.synchronize()
    dl = _dloss(x, "mean" if reduction == "mean" else "sum")
    ref = G.run_gpu(x, dl, eps=x.eps, sort=sort)
    valid = x.labels != x.ignore_index
    loss_sum = ref["loss"][valid].sum()
    got = G.t64(out)
    if reduction == "none":
        assert np.array_equal(got, ref["loss"])
    else:
        want = loss_sum / valid.sum() if reduction == "mean" else loss_sum
        assert abs(float(got) - want) <= 1e-5 * max(abs(want), 1.0)  # got is already detached
    assert np.array_equal(G.t64(Hl.grad), ref["dH"])
    assert np.array_equal(G.t64(El.grad), ref["dE"])
    # and against the fp64 oracle: the filtered gradient at the kernel's
    # geometry (vocabulary in id order), or, sorted, the unfiltered one (this
    # flat recipe keeps almost every block at eps = 2^-12)
    LH, LE = G.label_term(x, dl)
    if sort:
        _, _, dH, dE = G.oracle_full(x, dl, f"autograd-{reduction}")
        G.assert_grad("dH", G.t64(Hl.grad), dH, LH, 1e-2)
        G.assert_grad("dE", G.t64(El.grad), dE, LE, 1e-2)
    else:
        fH, fE, _, aH, aE = G.oracle_filtered(x, dl, x.eps, f"autograd-{reduction}")
        G.assert_grad_filtered("dH", G.t64(Hl.grad), fH, aH, LH)
        G.assert_grad_filtered("dE", G.t64(El.grad), fE, aE, LE)


def test_wrapper_full_size():
    """The Gemma-2-2B head at full size through the wrapper (mean reduction):
    the C ABI's bits, which the full-size parity tests check against the
    oracle."""
    x = inputs.make_workload(2)
    G.say(f"autograd full size N={x.N} D={x.D} V={x.V}")
    H, E, y = G.to_device(x)
    Hl = H.clone().requires_grad_(True)
    El = E.clone().requires_grad_(True)
    out = A.linear_cross_entropy(Hl, El, y, x.ignore_index, reduction="mean", filter_eps=x.eps)
    out.backward()
    torch.cuda.synchronize()
    ref = G.run_gpu(x, _dloss(x, "mean"), eps=x.eps)
    valid = x.labels != x.ignore_index
    want = ref["loss"][valid].sum() / valid.sum()
    assert abs(float(out.detach()) - want) <= 1e-5 * max(abs(want), 1.0)
    assert np.array_equal(G.t64(Hl.grad), ref["dH"])
    assert np.array_equal(G.t64(El.grad), ref["dE"])


def test_composite_wrapper_matches_oracle():
    x = inputs.make_workload(1)  # fp32, 10 % ignored
    V0, gap = 2500, 300
    y = x.labels.copy()
    y[y >= V0] += gap
    G.say("autograd composite")
    H, E, _ = G.to_device(x)
    yt = torch.from_numpy(y).to(G.DEV)
    Hl = H.clone().requires_grad_(True)
    E0 = E[:V0].clone().requires_grad_(True)
    E1 = E[V0:].clone().requires_grad_(True)
    loss = A.linear_cross_entropy_composite(Hl, E0, E1, V0 + gap, yt, x.ignore_index, filter_eps=0.0)
    loss.backward()
    torch.cuda.synchronize()
    dl = _dloss(x, "mean").astype(np.float64)
    Hf = oracle.as_f64(x.H, x.dtype)
    Ef = oracle.as_f64(x.E, x.dtype)
    rl, _, dH, dE0, dE1 = oracle.composite(Hf, Ef[:V0], Ef[V0:], V0 + gap, y, dl, x.ignore_index)
    valid = y != x.ignore_index
    want = rl[valid].mean()
    assert abs(float(loss.detach()) - want) <= 1e-5 * max(abs(want), 1.0)
    for name, g, r in (("dH", Hl.grad, dH), ("dE0", E0.grad, dE0), ("dE1", E1.grad, dE1)):
        g = G.t64(g)
        assert np.linalg.norm(g - r) <= 1e-5 * np.linalg.norm(r), name
