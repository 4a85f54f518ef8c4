"""Hot vocabulary blocks: a block of 128 vocabulary entries that more than
512 valid tokens are labelled with (with Zipf labels, the block of the most
frequent ids).  When every kept block of such a column is label-only, its dE
rows are sums of g_i h_i over its label entries; the backward groups the
entries by row once per call and sums each row's entries in pieces of 32
(token order within a piece, pieces in order) over 32-feature tiles.

The static route (with the forward's block-max table the column is known to
keep only label-only blocks before any recompute) and the dynamic route
(without the table the tiles are recomputed and the column's items find only
label-only blocks) must give the same bits; both are checked against the
oracle's filtered gradient, which here keeps the label entries only, with
label gradients dloss (p_y - 1) well away from zero.
"""
import numpy as np
import pytest

from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

HOT = 512  # a column with more label entries than this is hot


def _label_only_hot(N, D, V, dtype, seed, ignore_frac=0.0):
    """The Gemma-head recipe (peaked H, Zipf labels, peak 3.0): no non-label
    p reaches 2^-12, and with N in the thousands the first vocabulary block
    holds more than 512 of the label entries."""
    return inputs.make_inputs(N, D, V, dtype=dtype, e_std=0.02, h_kind="peaked", label_kind="zipf", seed=seed,
                              eps=2.0 ** -12, name="gemma-recipe-label-only-hot", peak_scale=3.0,
                              ignore_frac=ignore_frac)


def _hot_columns(x, perm=None):
    valid = x.labels != x.ignore_index
    pos = x.labels[valid] if perm is None else np.argsort(perm)[x.labels[valid]]
    counts = np.bincount(pos // 128)
    return np.nonzero(counts > HOT)[0], counts


# (N, D, V, dtype, ignored fraction, hot blocks at least): D = 264 leaves a
# partial last 32-feature tile (and a ragged 256-feature tile); the fp32
# case takes 8 segments of 4 features; the third has two hot blocks, ignored
# rows, and eight token slices for the grouping.
CASES = [(4096, 264, 9000, "bf16", 0.0, 1), (2048, 264, 5000, "f32", 0.0, 1), (8192, 264, 5000, "bf16", 0.1, 2)]


@pytest.mark.parametrize("sort", [False, True])
@pytest.mark.parametrize("N,D,V,dtype,ign,n_hot", CASES)
def test_hot_columns_static_and_dynamic(N, D, V, dtype, ign, n_hot, sort):
    x = _label_only_hot(N, D, V, dtype, seed=7, ignore_frac=ign)
    eps = 2.0 ** -12
    G.say(f"hot columns N={N} D={D} V={V} {dtype} sort={sort}")
    dl = G.random_dloss(x, seed=11)
    a = G.run_gpu(x, dl, eps=eps, bound=True, sort=sort)
    b = G.run_gpu(x, dl, eps=eps, bound=False, sort=sort)
    hot, counts = _hot_columns(x, a.get("perm"))
    G.say(f"  hot columns {hot.tolist()} (largest column {counts.max()} entries)")
    if not sort:
        assert len(hot) >= n_hot, counts.max()  # the case exercises the hot path
    for key in ("loss", "lse", "dH", "dE"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["stats"][:4], b["stats"][:4])
    assert a["stats"][0] == 0 and a["stats"][1] > 0, a["stats"]  # only label-only blocks kept
    if not sort:
        fH, fE, kept, aH, aE = G.oracle_filtered(x, dl, eps, "label-only-hot")
        assert not kept.any()
        LH, LE = G.label_term(x, dl)
        G.assert_grad_filtered("dH", a["dH"], fH, aH, LH)
        G.assert_grad_filtered("dE", a["dE"], fE, aE, LE)
        # the hot block's own rows, elementwise against the oracle, relative
        # to the largest entry of the row: a row summed from another row's
        # entries is off by O(1).  (The bound is not the output rounding:
        # g_i = dloss (p_y - 1) is formed from fp32 logits with p_y near 1,
        # so it carries a relative error of about ulp(z) / (1 - p_y), here
        # up to a few 1e-3 in either dtype.)
        for cb in hot.tolist():
            rows = np.arange(cb * 128, min(cb * 128 + 128, V))
            rows = rows[np.any(fE[rows] != 0, axis=1)]
            assert len(rows) > 0
            scale = np.max(np.abs(fE[rows]), axis=1, keepdims=True)
            err = np.max(np.abs(a["dE"][rows] - fE[rows]) / scale)
            assert err <= 2.0 ** -7, (cb, err)
