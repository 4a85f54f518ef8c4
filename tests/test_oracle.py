"""Pins for the fp64 oracle: each check fixes its answer from something other
than the oracle itself -- a hand-worked example, a closed form, an invariant,
finite differences, or a textbook library routine (torch's CPU
cross_entropy / logsumexp in float64).  A dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
IGN = -100


def _rand(rng, N, D, V, ign_rows=(), scale=1.0):
    H = rng.standard_normal((N, D)) * scale
    E = rng.standard_normal((V, D)) / math.sqrt(D)
    y = rng.integers(0, V, size=N).astype(np.int64)
    for r in ign_rows:
        y[r] = IGN
    dl = rng.uniform(0.5, 2.0, size=N)
    return H, E, y, dl


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    ns = {"e": math.e, "log": math.log, "__builtins__": {}}

    def ev(a):
        return np.array(eval(a, ns)) if isinstance(a, str) else np.array([ev(x) for x in a])

    H = np.array(g["H"], dtype=np.float64)
    E = np.array(g["E"], dtype=np.float64)
    y = np.array(g["labels"], dtype=np.int64)
    dl = np.array(g["dloss"], dtype=np.float64)
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, g["ignore_index"])
    np.testing.assert_allclose(lse, ev(g["lse"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(loss, ev(g["loss"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dH, ev(g["dH"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dE, ev(g["dE"]), rtol=0, atol=1e-14)


def test_zero_classifier_closed_form(rng):
    # E = 0: every logit is 0, softmax is uniform 1/V.
    N, D, V = 9, 6, 11
    H, _, y, dl = _rand(rng, N, D, V, ign_rows=(3,))
    E = np.zeros((V, D))
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, IGN)
    valid = y != IGN
    np.testing.assert_allclose(lse[valid], math.log(V), rtol=1e-15)
    np.testing.assert_allclose(loss[valid], math.log(V), rtol=1e-15)
    assert np.all(lse[~valid] == 0) and np.all(loss[~valid] == 0)
    assert np.all(dH == 0)
    want = np.zeros((V, D))
    for i in np.nonzero(valid)[0]:
        want += dl[i] * (1.0 / V) * H[i]
        want[y[i]] -= dl[i] * H[i]
    np.testing.assert_allclose(dE, want, rtol=0, atol=1e-14)


def test_equal_rows_closed_form(rng):
    # All e_v equal to e: lse_i = <h_i, e> + log V, loss = log V.
    N, D, V = 7, 5, 13
    H, _, y, dl = _rand(rng, N, D, V)
    e = rng.standard_normal(D)
    E = np.tile(e, (V, 1))
    loss, lse = oracle.forward(H, E, y, IGN)
    np.testing.assert_allclose(lse, H @ e + math.log(V), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(loss, math.log(V), rtol=1e-13)


def test_single_class():
    # V = 1: lse = z, loss = 0, both gradients vanish.
    H = np.array([[0.5, -2.0, 3.0]])
    E = np.array([[1.5, 0.25, -1.0]])
    loss, lse, dH, dE = oracle.backward(H, E, np.array([0]), np.array([0.7]), IGN)
    assert lse[0] == pytest.approx(H[0] @ E[0], abs=1e-15)
    assert loss[0] == pytest.approx(0.0, abs=1e-15)
    np.testing.assert_allclose(dH, 0, atol=1e-15)
    np.testing.assert_allclose(dE, 0, atol=1e-15)


def test_shift_invariance(rng):
    # e_v -> e_v + c for every v: lse_i shifts by <h_i, c>; loss and the
    # gradient with respect to H are unchanged.
    N, D, V = 10, 8, 17
    H, E, y, dl = _rand(rng, N, D, V, ign_rows=(0,))
    c = rng.standard_normal(D)
    loss0, lse0, dH0, _ = oracle.backward(H, E, y, dl, IGN)
    loss1, lse1, dH1, _ = oracle.backward(H, E + c, y, dl, IGN)
    valid = y != IGN
    np.testing.assert_allclose(lse1[valid] - lse0[valid], (H @ c)[valid], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(loss1, loss0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dH1, dH0, rtol=1e-10, atol=1e-12)


def test_gradient_rows_sum_to_zero(rng):
    # sum_v g_iv = 0 for every row, so sum_v dE_v = 0 and
    # sum_v <dE_v, e_v> = sum_i <dH_i, h_i> (both are sum_iv g_iv z_iv).
    N, D, V = 12, 7, 19
    H, E, y, dl = _rand(rng, N, D, V, ign_rows=(2, 5))
    _, _, dH, dE = oracle.backward(H, E, y, dl, IGN)
    np.testing.assert_allclose(dE.sum(axis=0), 0, atol=1e-13)
    assert float(np.sum(dE * E)) == pytest.approx(float(np.sum(dH * H)), rel=1e-12, abs=1e-13)


def test_ignored_rows_contribute_nothing(rng):
    N, D, V = 8, 6, 9
    H, E, y, dl = _rand(rng, N, D, V, ign_rows=(1, 4, 7))
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, IGN)
    ign = y == IGN
    assert np.all(loss[ign] == 0) and np.all(lse[ign] == 0) and np.all(dH[ign] == 0)
    # Changing an ignored row's hidden state or dloss leaves dE exactly as is.
    H2, dl2 = H.copy(), dl.copy()
    H2[ign] = rng.standard_normal((int(ign.sum()), D)) * 100
    dl2[ign] = 1e6
    _, _, _, dE2 = oracle.backward(H2, E, y, dl2, IGN)
    assert np.array_equal(dE, dE2)


def test_all_rows_ignored(rng):
    H, E, y, dl = _rand(rng, 4, 3, 5, ign_rows=(0, 1, 2, 3))
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, IGN)
    for a in (loss, lse, dH, dE):
        assert np.all(a == 0)


def test_finite_differences():
    # Central differences of L = sum_i dloss_i loss_i on N=3, D=5, V=7 (fp64).
    rng = np.random.default_rng(7)
    H, E, y, dl = _rand(rng, 3, 5, 7)

    def L(Hx, Ex):
        loss, _ = oracle.forward(Hx, Ex, y, IGN)
        return float(np.sum(dl * loss))

    _, _, dH, dE = oracle.backward(H, E, y, dl, IGN)
    h = 1e-6
    for X, G in ((H, dH), (E, dE)):
        num = np.empty_like(X)
        for idx in np.ndindex(*X.shape):
            xp, xm = X.copy(), X.copy()
            xp[idx] += h
            xm[idx] -= h
            if X is H:
                num[idx] = (L(xp, E) - L(xm, E)) / (2 * h)
            else:
                num[idx] = (L(H, xp) - L(H, xm)) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("shape", [(64, 32, 512), (33, 24, 257), (5, 8, 3)])
def test_against_torch_cross_entropy(shape):
    # Textbook routine: torch.nn.functional.cross_entropy (CPU, float64) and
    # its autograd gradients, with ignore_index rows.
    N, D, V = shape
    rng = np.random.default_rng(N * 1000 + V)
    H, E, y, dl = _rand(rng, N, D, V, ign_rows=tuple(range(0, N, 5)), scale=2.0)
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, IGN)
    Ht = torch.tensor(H, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    logits = Ht @ Et.T
    lt = torch.nn.functional.cross_entropy(logits, torch.tensor(y), ignore_index=IGN, reduction="none")
    (lt * torch.tensor(dl)).sum().backward()
    valid = y != IGN
    lse_t = torch.logsumexp(logits, dim=1).detach().numpy()
    np.testing.assert_allclose(loss, lt.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[valid], lse_t[valid], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_sampled_rows_match_full(rng):
    # The row-sampled entry points agree with the full computation.
    N, D, V = 20, 6, 31
    H, E, y, dl = _rand(rng, N, D, V, ign_rows=(3,))
    loss, lse, dH, dE = oracle.backward(H, E, y, dl, IGN)
    rows = np.array([19, 3, 0, 7])
    l2, s2, h2 = oracle.rows(H, E, y, dl, rows, IGN)
    assert np.array_equal(l2, lse[rows]) and np.array_equal(s2, loss[rows]) and np.array_equal(h2, dH[rows])
    vids = np.array([30, 0, 11])
    assert np.array_equal(oracle.dE_rows(H, E, y, lse, dl, vids, IGN), dE[vids])


def test_mean_logit_identity(rng):
    # key_v = mean_i z_iv equals <mean_i h_i, e_v> (linearity), over valid rows.
    N, D, V = 15, 9, 40
    H, E, y, _ = _rand(rng, N, D, V, ign_rows=(1, 2))
    key = oracle.mean_logit(H, E, y, IGN)
    hbar = H[y != IGN].mean(axis=0)
    np.testing.assert_allclose(key, E @ hbar, rtol=1e-12, atol=1e-13)


def test_vocab_order_descending_stable():
    keys = np.array([0.5, 2.0, -1.0, 2.0, 0.5, 3.0])
    assert list(oracle.vocab_order(keys)) == [5, 1, 3, 0, 4, 2]


def test_bf16_conversion_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049], dtype=np.uint16)
    want = [1.0, -1.0, 2.0 ** -133, 3.3895313892515355e38, 3.140625]
    np.testing.assert_array_equal(oracle.as_f64(bits, "bf16"), want)


def test_lse_matmul_against_torch(rng):
    # The matmul-based lse (used for full-size checks) is the same definition:
    # pin it to torch.logsumexp and to the loop oracle.
    N, D, V = 70, 16, 300
    H, E, y, _ = _rand(rng, N, D, V, ign_rows=(4,), scale=3.0)
    got = oracle.lse_matmul(H, E, y, IGN, row_chunk=32)
    want = torch.logsumexp(torch.tensor(H) @ torch.tensor(E).T, dim=1).numpy()
    valid = y != IGN
    np.testing.assert_allclose(got[valid], want[valid], rtol=1e-13, atol=1e-13)
    assert got[4] == 0
    _, lse_loop = oracle.forward(H, E, y, IGN)
    np.testing.assert_allclose(got, lse_loop, rtol=1e-12, atol=1e-12)

