"""The GPU parity criteria can fail.  On the CPU, emulated kernel outputs --
the oracle's float64 gradient entries at the kernel's 128 x 128 filter
blocks, formed as dloss (p [kept] - onehot), rounded to bf16, multiplied in
float64 and rounded to bf16 again -- must pass the checks of tests/_gpu.py,
while outputs with a planted mistake must fail them:
  - p rounded to bf16 before the -1 of the label entry (p_y near 1 cancels);
  - the label term alone (the softmax part dropped);
  - all zeros.
Recipes: the moderately peaked Gemma-head recipe (median 1 - p_y = 0.03),
unfiltered and filtered, and the flat Llama-3-head recipe, filtered."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

BLOCK = 128


def _bf16(a):
    return inputs.bf16_bits_as_f32(inputs.round_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def _emulate(x, dl, eps, plant=None):
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    valid = x.labels != x.ignore_index
    rows = np.nonzero(valid)[0]
    _, lse = oracle.forward(H, E, x.labels, x.ignore_index)
    P = np.exp(H[rows] @ E.T - lse[rows, None])
    onehot = np.zeros_like(P)
    onehot[np.arange(rows.size), x.labels[rows]] = 1.0
    keep = onehot > 0
    other = np.where(keep, -1.0, P)
    for r0 in range(0, rows.size, BLOCK):
        for c0 in range(0, x.V, BLOCK):
            if eps == 0 or other[r0:r0 + BLOCK, c0:c0 + BLOCK].max() >= eps:
                keep[r0:r0 + BLOCK, c0:c0 + BLOCK] = True
    Pk = np.where(keep, P, 0.0)
    if plant == "bf16 p":
        Pk = _bf16(Pk)
    g = dl[rows, None].astype(np.float64) * (Pk - onehot)
    if plant == "label only":
        g = -dl[rows, None].astype(np.float64) * onehot
    g = _bf16(g)
    dH = np.zeros((x.N, x.D))
    dH[rows] = _bf16(g @ E)
    dE = _bf16(g.T @ H[rows])
    if plant == "zero":
        dH[:] = 0.0
        dE[:] = 0.0
    return dH, dE


def _check_unfiltered(x, dl, out):
    _, _, dH, dE = oracle.backward(oracle.as_f64(x.H, x.dtype), oracle.as_f64(x.E, x.dtype), x.labels,
                                   dl.astype(np.float64), x.ignore_index)
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dH", out[0], dH, LH, 1e-2)
    G.assert_grad("dE", out[1], dE, LE, 1e-2)
    valid = np.nonzero(x.labels != x.ignore_index)[0]
    G.assert_rows_rel("dH rows", out[0], dH, valid, 1e-2)


def _check_filtered(x, dl, eps, out):
    fH, fE, _, aH, aE = oracle.backward_filtered(oracle.as_f64(x.H, x.dtype), oracle.as_f64(x.E, x.dtype), x.labels,
                                                 dl.astype(np.float64), eps, BLOCK, BLOCK, x.ignore_index)
    LH, LE = G.label_term(x, dl)
    G.assert_grad_filtered("dH", out[0], fH, aH, LH)
    G.assert_grad_filtered("dE", out[1], fE, aE, LE)


@pytest.fixture(scope="module")
def moderate():
    x = G.moderate_peaked()
    return x, G.mean_dloss(x)


@pytest.fixture(scope="module")
def flat():
    x = inputs.make_workload(3, N=600, D=512, V=5000)
    return x, G.mean_dloss(x)


def test_recipe_is_moderately_peaked(moderate):
    x, _ = moderate
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    loss, _ = oracle.forward(H, E, x.labels, x.ignore_index)
    gap = 1.0 - np.exp(-loss[x.labels != x.ignore_index])  # 1 - p_y
    assert 1e-2 <= np.median(gap) <= 0.3, np.median(gap)


def test_correct_outputs_pass(moderate, flat):
    x, dl = moderate
    _check_unfiltered(x, dl, _emulate(x, dl, 0.0))
    _check_filtered(x, dl, 2.0 ** -12, _emulate(x, dl, 2.0 ** -12))
    x, dl = flat
    _check_filtered(x, dl, 2.0 ** -12, _emulate(x, dl, 2.0 ** -12))


@pytest.mark.parametrize("plant", ["bf16 p", "label only", "zero"])
def test_planted_mistakes_fail_unfiltered(moderate, plant):
    x, dl = moderate
    with pytest.raises(AssertionError):
        _check_unfiltered(x, dl, _emulate(x, dl, 0.0, plant))


@pytest.mark.parametrize("plant", ["bf16 p", "label only", "zero"])
def test_planted_mistakes_fail_filtered(moderate, flat, plant):
    x, dl = moderate
    with pytest.raises(AssertionError):
        _check_filtered(x, dl, 2.0 ** -12, _emulate(x, dl, 2.0 ** -12, plant))
    if plant != "bf16 p":  # p_y ~ 1/V on a flat softmax: rounding p first costs nothing there
        x, dl = flat
        with pytest.raises(AssertionError):
            _check_filtered(x, dl, 2.0 ** -12, _emulate(x, dl, 2.0 ** -12, plant))
