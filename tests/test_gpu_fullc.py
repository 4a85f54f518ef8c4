"""The full-classifier-gradient variant (CCE_BWD_FULL_DE): dE from every
block, unfiltered and Kahan-compensated, while dH stays filtered.  Its dE must
equal, bit for bit, the dE of an unfiltered run (every block kept, same
values, same order), and its dH the dH of the ordinary filtered run; both are
also held to the fp64 oracle."""
import numpy as np
import pytest

from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

CASES = [
    (2, 700, 256, 9000, 2.0 ** -12),   # peaked: almost every block dropped by the filter
    (3, 600, 512, 5000, 2.0 ** -12),   # flat, 40 % ignored: some blocks dropped
    (1, None, None, None, 2.0 ** -10), # fp32
]


@pytest.mark.parametrize("k,N,D,V,eps,sort", [c + (False,) for c in CASES] + [(5, 480, 256, 9500, 2.0 ** -12, True)],
                         ids=[f"w{c[0]}" for c in CASES] + ["w5-sort"])
def test_full_de(k, N, D, V, eps, sort):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"full dE w{k} N={x.N} D={x.D} V={x.V} eps={eps} sort={sort}")
    dl = G.random_dloss(x, seed=5)
    full = G.run_gpu(x, dl, eps=eps, flags=B.CCE_BWD_FULL_DE, sort=sort)
    filt = G.run_gpu(x, dl, eps=eps, sort=sort)
    dense = G.run_gpu(x, dl, eps=0.0, sort=sort)
    assert np.array_equal(full["dE"], dense["dE"]), "dE must be the unfiltered dE"
    assert np.array_equal(full["dH"], filt["dH"]), "dH must be the filtered dH"
    assert np.array_equal(full["stats"][:4], filt["stats"][:4])
    # against the oracle: dE unfiltered, dH filtered (the oracle's filtered
    # gradient at the kernel's geometry; with the sort, the label-term floor
    # of this peaked recipe)
    _, _, dH, dE = G.oracle_full(x, dl, "full_de")
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dE", full["dE"], dE, LE, 1e-5 if x.dtype == "f32" else 1e-2)
    if sort:
        G.assert_grad("dH", full["dH"], dH, LH, 2e-2, "label")
    else:
        fH, _, _, aH, _ = G.oracle_filtered(x, dl, eps, "full_de")
        G.assert_grad_filtered("dH", full["dH"], fH, aH, LH)
