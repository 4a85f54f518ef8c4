"""Pins for the oracle's filtered gradient (oracle.backward_filtered), the
block filter of the CCE paper summary "Cut Your Losses in Large-Vocabulary
Language Models", section "Approach", at a stated block geometry.  Each pin
fixes its answer from something other than the function itself: the
unfiltered C oracle at eps = 0 (a separate implementation), the label-term
closed form at eps > 1, a designed input whose keep decisions are worked out
by hand, the identity sum <dE, E> = sum <dH, H>, monotonicity in eps and the
elementwise error bound against the unfiltered gradient.  Planted mistakes in
a copy of the function's source must each fail one of them."""
import inspect
import math

import numpy as np
import pytest

import oracle

IGN = -100


def _rand(seed, N=37, D=9, V=300, ign=(2, 11, 12)):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((N, D)) * 1.5
    E = rng.standard_normal((V, D)) / math.sqrt(D)
    y = rng.integers(0, V, size=N).astype(np.int64)
    y[list(ign)] = IGN
    dl = rng.uniform(0.5, 2.0, size=N)
    return H, E, y, dl


def pin_eps0_is_unfiltered(fn):
    H, E, y, dl = _rand(1)
    dH, dE, kept, aH, aE = fn(H, E, y, dl, 0.0, block_rows=8, block_vocab=16)
    _, _, rH, rE = oracle.backward(H, E, y, dl, IGN)
    np.testing.assert_allclose(dH, rH, rtol=0, atol=1e-13 * np.abs(rH).max())
    np.testing.assert_allclose(dE, rE, rtol=0, atol=1e-13 * np.abs(rE).max())
    assert kept.all() and aH == 0 and aE == 0


def pin_eps_above_one_is_label_term(fn):
    # every p < 1 < eps: only label entries keep their gradient dloss (p_y - 1)
    H, E, y, dl = _rand(2)
    dH, dE, kept, _, _ = fn(H, E, y, dl, 2.0, block_rows=8, block_vocab=16)
    loss, _ = oracle.forward(H, E, y, IGN)
    valid = y != IGN
    g = np.where(valid, dl * (np.exp(-loss) - 1.0), 0.0)  # p_y = exp(z_y - lse) = exp(-loss)
    want_H = g[:, None] * E[np.where(valid, y, 0)]
    want_H[~valid] = 0.0
    want_E = np.zeros_like(E)
    for i in np.nonzero(valid)[0]:
        want_E[y[i]] += g[i] * H[i]
    np.testing.assert_allclose(dH, want_H, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dE, want_E, rtol=1e-12, atol=1e-15)
    assert not kept.any()


# Designed problem: E = I (D = V = 6), so z_i = h_i, dH_i = g_i and the keep
# decisions can be worked out by hand.  Row 1 is ignored, so the non-ignored
# rows 0, 2, 3, 4 form row blocks {0, 2} and {3, 4} (block_rows = 2); the
# vocabulary blocks are {0, 1, 2} and {3, 4, 5} (block_vocab = 3); eps = 0.05.
#   row 0, label 0, h = (10, 0, 0, 0, 0, 0): non-label p = 4.5e-5 each
#   row 2, label 4, h = (0, 0, 0, 0, 10, 0): non-label p = 4.5e-5 each
#   row 3, label 2, h = (0, 4, 5, 0, 0, 0): p_1 = 0.264 (>= eps), p_3..5 = 0.0048
#   row 4, label 5, h = (0, 0, 0, 0, 0, 2.5): non-label p = 0.058 (>= eps, < 2 eps)
# Block (0, 0): its only large p is row 0's label entry -> dropped.
# Block (0, 1): row 2's label entry only -> dropped.  Block (1, 0): row 3's
# p_1 -> kept, with every entry in it (row 4's ids 0-2 too).  Block (1, 1):
# row 4's p_3 = p_4 = 0.058 -> kept (row 3's ids 3-5 too).
DESIGN_H = np.array([[10, 0, 0, 0, 0, 0], [0, 0, 0, 0, 0, 0], [0, 0, 0, 0, 10, 0],
                     [0, 4, 5, 0, 0, 0], [0, 0, 0, 0, 0, 2.5]], dtype=np.float64)
DESIGN_Y = np.array([0, IGN, 4, 2, 5], dtype=np.int64)
DESIGN_KEPT = np.array([[False, False], [True, True]])
# entries (row, id) whose softmax part survives: label entries, and blocks (1, 0), (1, 1)
DESIGN_KEEP = {(0, 0), (2, 4)} | {(i, v) for i in (3, 4) for v in range(6)}


def pin_designed_blocks(fn):
    dl = np.array([1.0, 7.0, 0.5, 2.0, 0.25])
    dH, dE, kept, _, _ = fn(DESIGN_H, np.eye(6), DESIGN_Y, dl, 0.05, block_rows=2, block_vocab=3)
    assert np.array_equal(kept, DESIGN_KEPT), kept
    want = np.zeros((5, 6))
    for i in (0, 2, 3, 4):
        ex = [math.exp(v) for v in DESIGN_H[i]]
        s = sum(ex)
        for v in range(6):
            p = ex[v] / s if (i, v) in DESIGN_KEEP else 0.0
            want[i, v] = dl[i] * (p - (1.0 if v == DESIGN_Y[i] else 0.0))
    np.testing.assert_allclose(dH, want, rtol=1e-13, atol=1e-16)


def pin_identity_and_bound(fn):
    # sum_vd dE E = sum_id dH H (both are sum_iv g_iv z_iv, whatever is kept);
    # kept blocks never grow with eps; every dropped entry has p < eps, so
    # |dH - dH_unfiltered| <= dloss_i eps sum_v |e_vd| elementwise.
    H, E, y, dl = _rand(3, N=50, D=7, V=400)
    H = H * 2.0
    _, _, rH, rE = oracle.backward(H, E, y, dl, IGN)
    prev = None
    for eps in (0.0, 1e-4, 1e-3, 1e-2, 0.1, 0.5):
        dH, dE, kept, _, _ = fn(H, E, y, dl, eps, block_rows=8, block_vocab=32)
        assert abs(np.sum(dE * E) - np.sum(dH * H)) <= 1e-10 * (np.abs(dE * E).sum() + 1e-30)
        n = int(kept.sum())
        assert prev is None or n <= prev
        prev = n
        bound = dl[:, None] * eps * np.abs(E).sum(axis=0)[None, :]
        assert np.all(np.abs(dH - rH) <= bound + 1e-13)
        valid = y != IGN
        bE = eps * (dl[valid, None] * np.abs(H[valid])).sum(axis=0)[None, :]
        assert np.all(np.abs(dE - rE) <= bE + 1e-13)
    assert prev < int(kept.size)


PINS = [pin_eps0_is_unfiltered, pin_eps_above_one_is_label_term, pin_designed_blocks, pin_identity_and_bound]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.backward_filtered)


def test_allowance_counts_near_threshold_blocks():
    # a block whose largest non-label p equals eps to within the margin gets
    # an allowance; far from eps none
    dl = np.ones(5)
    ex = [math.exp(v) for v in DESIGN_H[3]]
    p1 = ex[1] / sum(ex)
    _, _, _, aH, aE = oracle.backward_filtered(DESIGN_H, np.eye(6), DESIGN_Y, dl, p1 * (1 + 2.0 ** -16),
                                               block_rows=2, block_vocab=3)
    assert aH > 0 and aE > 0
    _, _, _, aH, aE = oracle.backward_filtered(DESIGN_H, np.eye(6), DESIGN_Y, dl, p1 * (1 + 2.0 ** -12),
                                               block_rows=2, block_vocab=3)
    assert aH == 0 and aE == 0


# (name, text in the function's source, replacement)
MUTANTS = [
    ("label entries count in the block maximum",
     "other = np.where(is_label[r0:r1, c0:c1], -np.inf, p[r0:r1, c0:c1])", "other = p[r0:r1, c0:c1]"),
    ("a dropped block also drops its label entry's p",
     "keep_entry = is_label.copy()", "keep_entry = np.zeros((n, V), dtype=bool)"),
    ("the one-hot term is left out", "(np.where(keep_entry, p, 0.0) - is_label)", "(np.where(keep_entry, p, 0.0))"),
    ("eps = 0 keeps nothing", "else top > -np.inf", "else False"),
    ("vocabulary blocks cut with the row block size",
     "c0, c1 = cb * block_vocab, min(V, (cb + 1) * block_vocab)",
     "c0, c1 = cb * block_rows, min(V, (cb + 1) * block_rows)"),
    ("row blocks over all rows, ignored ones included",
     "r0, r1 = rb * block_rows, min(n, (rb + 1) * block_rows)",
     "r0, r1 = rb * block_rows - rb, min(n, (rb + 1) * block_rows - rb)"),
    ("threshold doubled", "top >= eps if eps > 0", "top >= 2 * eps if eps > 0"),
    ("dE from the wrong operand", "dE[:] = g.T @ Hv", "dE[:] = g.T @ (Hv - Hv.mean(axis=0))"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.backward_filtered)
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    return ns["backward_filtered"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    fn = _mutant(old, new)
    caught = 0
    for pin in PINS:
        try:
            pin(fn)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"no pin caught: {name}"


def test_unmodified_source_passes_as_copy():
    fn = _mutant("keep_entry = is_label.copy()", "keep_entry = is_label.copy()")
    for pin in PINS:
        pin(fn)
