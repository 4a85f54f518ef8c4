"""Gradient filter contract (a block keeps the softmax part of its entries
only if one of them, other than a label entry, reaches eps; a label entry
always keeps its whole gradient dloss (p - 1)), checked against the fp64
oracle and closed forms."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _pow2_dloss(x, k=10):
    return np.where(x.labels != x.ignore_index, 2.0 ** -k, 0.0).astype(np.float32)


@pytest.mark.parametrize("recipe", ["flat", "peaked"])
def test_eps_above_one_is_the_label_term_closed_form(recipe):
    # eps > 1 > every p: no block keeps the softmax part of its other
    # entries, and each label entry keeps its own, so
    #   dH_i = dloss_i (p_{i,y_i} - 1) e_{y_i},  dE_v = sum_{i: y_i = v} dloss_i (p_{i,y_i} - 1) h_i
    # with p_{i,y_i} = exp(z_{i,y_i} - lse_i) from the oracle.  The gradient
    # entry and the output are each rounded to bf16 once (8 significant bits:
    # up to 2^-8 each, 2^-7 together).
    # Flat: p_y ~ 1/V.  Peaked (median 1 - p_y = 0.03): p_y - 1 must be formed
    # in fp32 before rounding; rounding p_y to bf16 first misses by up to
    # 2^-9 / (1 - p_y), far above 2^-7.
    x = inputs.make_workload(4, N=600, D=256, V=3000) if recipe == "flat" else G.moderate_peaked()
    G.say(f"filter eps=2 closed form {recipe}")
    dl = _pow2_dloss(x)
    out = G.run_gpu(x, dl, eps=2.0)
    assert out["stats"][0] == 0 and out["stats"][1] > 0
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    valid = x.labels != x.ignore_index
    loss, lse = oracle.forward(H, E, x.labels, x.ignore_index)
    g = np.zeros(x.N)
    g[valid] = dl[valid].astype(np.float64) * (np.exp(-loss[valid]) - 1.0)  # p_y = exp(z_y - lse) = exp(-loss)
    want_dH = g[:, None] * np.where(valid[:, None], E[np.where(valid, x.labels, 0)], 0.0)
    err = np.abs(out["dH"] - want_dH)
    assert np.all(err <= 2.0 ** -7 * np.abs(want_dH) + 1e-12), float(err.max())
    want_dE = np.zeros_like(E)
    mag = np.zeros_like(E)
    np.add.at(want_dE, x.labels[valid], g[valid, None] * H[valid])
    np.add.at(mag, x.labels[valid], np.abs(g[valid, None] * H[valid]))
    err = np.abs(out["dE"] - want_dE)
    assert np.all(err <= 2.0 ** -7 * mag + 1e-12), float(err.max())


def test_kept_blocks_do_not_grow_with_eps():
    x = inputs.make_workload(2, N=640, D=128, V=6000)  # peaked at small D: partial filtering
    dl = G.mean_dloss(x)
    kept = []
    for eps in (0.0, 2.0 ** -24, 2.0 ** -16, 2.0 ** -12, 2.0 ** -8, 0.5, 2.0):
        G.say(f"filter monotone eps={eps}")
        out = G.run_gpu(x, dl, eps=eps)
        kept.append(int(out["stats"][0]))
        assert out["stats"][0] + out["stats"][1] <= out["stats"][2]
    assert all(a >= b for a, b in zip(kept, kept[1:])), kept
    assert kept[0] == out["stats"][2] and kept[-1] == 0


@pytest.mark.parametrize("k,N,D,V,eps", [(3, 600, 512, 5000, 2.0 ** -8), (4, 512, 384, 3000, 2.0 ** -8),
                                         (2, 700, 256, 9000, 2.0 ** -12)])
def test_filtered_error_within_bound(k, N, D, V, eps):
    # Every skipped entry has p < eps, so elementwise
    #   |dH_gpu - dH| <= dloss_i (eps sum_v |e_vd| + 2^-8 max_v |e_vd|) + 2^-8 |dH|
    #   |dE_gpu - dE| <= eps sum_i dloss_i |h_id| + 2^-8 max_i |h_id| sum_i |g_iv| + 2^-8 |dE|
    # where the 2^-8 terms cover bf16 rounding of the gradient tile and of
    # the outputs.  The bound does not depend on the block geometry.
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"filter bound w{k} eps={eps}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps)
    _, lse, dH, dE = G.oracle_full(x, dl, "mean")
    G.assert_filter_bound(x, dl, eps, out, lse, dH, dE)
    assert out["stats"][0] < out["stats"][2] or eps < 2.0 ** -10  # something was skipped at 2^-8
