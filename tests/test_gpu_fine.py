"""Filtering per 32 x 32 sub-tile (CCE_BWD_FINE_FILTER; the summary "Cut Your
Losses in Large-Vocabulary Language Models" names block-granular control
flow as a limitation of its kernel, section "Limitations").  A sub-tile
keeps the softmax part of its entries iff one of them other than a label
entry has p >= eps; the dH / dE products skip the sub-tiles left all zero.

  - against the oracle's filtered gradient at 32 x 32 geometry, on the
    partially peaked recipe (two regimes: every 128 x 128 block kept but 58 %
    of the sub-tiles; 37 % against 2.8 %), the moderately peaked and the
    flat recipes (75 % of the sub-tiles kept), fp32, and a problem cut into
    several passes; dE checked as label-free rows (the softmax part alone)
    and label rows;
  - the elementwise filter bound against the unfiltered gradient;
  - eps = 0 keeps every sub-tile: bit-identical to the default filter;
  - the block counts are those of the default filter (a block survives iff
    one of its sub-tiles does), the kept sub-tiles those of the oracle."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

FINE = B.CCE_BWD_FINE_FILTER


def _partial(N, D, V, seed=77):
    # workload 7's recipe at a reduced size
    return inputs.make_inputs(N, D, V, dtype="bf16", e_std=0.02, h_kind="peaked", label_kind="zipf", seed=seed,
                              eps=2.0 ** -10, name="gemma-recipe-partial", peak_scale=0.35, h_noise=2.0)


CASES = [
    ("partial-a", lambda: _partial(768, 512, 12000), 2.0 ** -10),
    ("partial-b", lambda: _partial(640, 1024, 20000), 2.0 ** -8),
    ("moderate", lambda: G.moderate_peaked(), 2.0 ** -12),
    ("flat-w3", lambda: inputs.make_workload(3, N=600, D=512, V=5000), 2.0 ** -10.5),
    ("fp32-w1", lambda: inputs.make_workload(1), 2.0 ** -10),
    ("passes-w3", lambda: inputs.make_workload(3, N=2300, D=512, V=20000), 2.0 ** -13),
]


@pytest.mark.parametrize("name,make,eps", CASES, ids=[c[0] for c in CASES])
def test_fine_filter_matches_oracle(name, make, eps):
    x = make()
    G.say(f"fine filter {name} N={x.N} D={x.D} V={x.V} eps={eps}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, flags=FINE)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    br, bv = B.FINE_SUBTILE
    fH, fE, kept, aH, aE = oracle.backward_filtered(H, E, x.labels, dl.astype(np.float64), eps, br, bv,
                                                    x.ignore_index)
    LH, LE = G.label_term(x, dl)
    tol = 1e-5 if x.dtype == "f32" else 1e-2
    G.assert_grad_filtered("dH", out["dH"], fH, aH, LH, tol)
    G.assert_grad_filtered("dE", out["dE"], fE, aE, LE, tol, split=x.dtype == "bf16")
    if aH == 0 and aE == 0:
        assert out["stats"][6] == int(kept.sum()), (out["stats"], int(kept.sum()))
    # a block survives iff one of its sub-tiles does: the default filter's counts
    ref = G.run_gpu(x, dl, eps=eps)
    assert np.array_equal(out["stats"][:5], ref["stats"][:5])
    assert out["stats"][6] <= ref["stats"][6]
    # and the geometry-free bound against the unfiltered gradient
    _, lse, dH, dE = G.oracle_full(x, dl, "mean")
    G.assert_filter_bound(x, dl, eps, out, lse, dH, dE)


@pytest.mark.parametrize("k,N,D,V", [(3, 600, 512, 5000), (2, 700, 256, 9000), (1, None, None, None)])
def test_fine_filter_at_eps_zero_is_the_default(k, N, D, V):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"fine filter eps=0 w{k}")
    dl = G.random_dloss(x, seed=4)
    a = G.run_gpu(x, dl, eps=0.0, flags=FINE)
    b = G.run_gpu(x, dl, eps=0.0)
    for key in ("dH", "dE"):
        assert np.array_equal(a[key], b[key]), key


def test_fine_filter_sorted_within_bound():
    x = _partial(768, 512, 12000)
    eps = 2.0 ** -10
    G.say("fine filter sorted")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, flags=FINE, sort=True)
    _, lse, dH, dE = G.oracle_full(x, dl, "mean")
    G.assert_filter_bound(x, dl, eps, out, lse, dH, dE)
