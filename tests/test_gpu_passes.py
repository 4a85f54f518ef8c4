"""The backward's pass structure: the listed tiles are cut into passes whose
kept blocks fit the block store.  With the block-max table fewer tiles are
listed, so the same problem is cut into fewer passes; dH carries its fp32
running sum across passes block by block, so the outputs must not depend on
the cut (bit-identical with and without the table), and a problem cut into
several passes must still match the fp64 oracle."""
import numpy as np
import pytest

from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# The block store holds max(row blocks x 128, 1024) blocks (with 2300 rows:
# 18 x 128 = 2304), so these vocabularies take several passes.
CASES = [
    (2, 2300, 256, 40000, 2.0 ** -12),   # peaked: three passes without the table, one with it
    (3, 2300, 512, 20000, 2.0 ** -12),   # flat, 40 % ignored: several passes either way
    (4, 2300, 72, 20000, 2.0 ** -6),     # D * 2 not a multiple of 128: VGPR-staged recompute
]


@pytest.mark.parametrize("k,N,D,V,eps", CASES, ids=[f"w{c[0]}-{c[2]}-{c[3]}" for c in CASES])
def test_pass_cut_does_not_change_results(k, N, D, V, eps):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"pass cut w{k} N={x.N} D={x.D} V={x.V} eps={eps}")
    dl = G.random_dloss(x, seed=3)
    a = G.run_gpu(x, dl, eps=eps, bound=True)
    b = G.run_gpu(x, dl, eps=eps, bound=False)
    for key in ("dH", "dE"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["stats"][:4], b["stats"][:4])


def test_multi_pass_matches_oracle():
    """A flat case with every block kept, cut into several passes."""
    x = inputs.make_workload(3, N=2300, D=512, V=20000)
    G.say(f"multi-pass parity N={x.N} D={x.D} V={x.V}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=0.0)
    _, _, dH, dE = G.oracle_full(x, dl, "mean")
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dH", out["dH"], dH, LH, 1e-2)
    G.assert_dE_split("dE", out["dE"], dE, LE, 1e-2)
    assert out["stats"][0] == out["stats"][2]


def test_multi_pass_matches_oracle_f32():
    """The same in fp32 (fp32 store, fp32 products): a flat recipe with 40 %
    ignored rows, every block kept: 1380 valid rows (11 row blocks) x 313
    vocabulary blocks = 3443 blocks, more than the store's 2304, so at least
    two passes."""
    x = inputs.make_inputs(2300, 256, 40000, dtype="f32", e_std=0.05, h_kind="normal", label_kind="uniform",
                           ignore_frac=0.4, seed=3, name="flat-f32-passes")
    G.say(f"multi-pass parity fp32 N={x.N} D={x.D} V={x.V}")
    dl = G.random_dloss(x, seed=4)
    out = G.run_gpu(x, dl, eps=0.0)
    loss, lse, dH, dE = G.oracle_full(x, dl, "random4")
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dH", out["dH"], dH, LH, 1e-5)
    G.assert_grad("dE", out["dE"], dE, LE, 1e-5)
    assert out["stats"][0] == out["stats"][2]


def test_unfiltered_few_rows_vgpr_recompute():
    """eps = 0 with one row block of valid tokens and a row block of padding,
    on the VGPR-staged recompute (D * 2 not a multiple of 128), which computes
    every block of a tile: the padding block's entries (p = 0) must not count
    as kept, or the pass would hold more blocks than the plan made room for
    and drop some.  782 vocabulary tiles x 2 real blocks: two passes."""
    x = inputs.make_workload(3, N=100, D=72, V=200000)
    G.say(f"unfiltered few rows N={x.N} D={x.D} V={x.V}")
    dl = G.random_dloss(x, seed=9)
    out = G.run_gpu(x, dl, eps=0.0)
    _, _, dH, dE = G.oracle_full(x, dl, "random9")
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dH", out["dH"], dH, LH, 1e-2)
    G.assert_dE_split("dE", out["dE"], dE, LE, 1e-2)
    # every real block kept, every real block recomputed, none other
    assert out["stats"][0] == out["stats"][2] == out["stats"][4], out["stats"]
