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

import oracle
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
# rows, and eight token slices for the grouping; the fourth has 2^18 tokens
# (1024 token tiles, 64 token slices) and every vocabulary block hot, the
# first with about 187 000 label entries (one of its rows with tens of
# thousands).
CASES = [(4096, 264, 9000, "bf16", 0.0, 1), (2048, 264, 5000, "f32", 0.0, 1), (8192, 264, 5000, "bf16", 0.1, 2),
         (262144, 264, 1000, "bf16", 0.1, 8)]


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
        # the hot blocks' own rows, elementwise against the oracle.  The
        # label gradient g_i = dloss_i (p_y - 1) is formed from the float32
        # lse and label logit, each within a few float32 ulps of |lse| of
        # the exact values; with p_y near 1 that absolute error is all of
        # g_i's error (a relative 2e-3 at 1 - p_y = 2e-3, 3e-2 at 2e-4, the
        # 2^18-token case), and it comes out alike for the tokens of one label.
        # So entry (v, d) may be off by u sum_{i: y_i = v} dloss_i |h_id|,
        # u = 8 ulps of max |lse|, plus the output's rounding; the bound is
        # asserted to reject an all-zero row.
        H64 = oracle.as_f64(x.H, x.dtype)
        valid = x.labels != x.ignore_index
        u = 8 * 2.0 ** -24 * np.max(np.abs(a["lse"]))
        for cb in hot.tolist():
            for v in range(cb * 128, min(cb * 128 + 128, V)):
                sel = valid & (x.labels == v)
                if not sel.any():
                    continue
                bound = u * (dl[sel, None].astype(np.float64) * np.abs(H64[sel])).sum(axis=0) + \
                    2.0 ** -8 * np.abs(fE[v]) + 1e-30
                j = int(np.argmax(np.abs(fE[v])))
                assert bound[j] < 0.5 * abs(fE[v][j]), (v, bound[j], fE[v][j])  # zero fails
                err = np.abs(a["dE"][v] - fE[v])
                assert np.all(err <= bound), (v, int(np.argmax(err / bound)), float(np.max(err / bound)))
