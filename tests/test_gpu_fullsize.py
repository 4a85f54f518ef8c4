"""The seven workloads at their full sizes, in the launch configuration the
benchmark times.  The oracle computes sampled outputs one by one (lse, loss
and dH rows; dE rows where every row's lse is affordable), every row's lse of
the Gemma-2-2B and Phi-3.5-mini heads (numpy float64 matrix products), and
properties that hold at any size check the rest:
  sum_v dE_v = 0 (every logit-gradient row sums to zero), and
  sum_v <dE_v, e_v> = sum_i <dH_i, h_i> (both are sum_iv g_iv z_iv)."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6])
def test_full_size(k):
    x = inputs.make_workload(k)
    eps = x.eps
    sort = k >= 5
    G.say(f"full size w{k} N={x.N} D={x.D} V={x.V} eps={eps} sort={sort}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, sort=sort)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    valid = x.labels != x.ignore_index
    rng = np.random.default_rng(k)
    vrows = np.nonzero(valid)[0]
    rows = np.unique(np.concatenate([vrows[:2], vrows[-2:], rng.choice(vrows, 8, replace=False)]))
    lse, loss, dH = oracle.rows(H, E, x.labels, dl.astype(np.float64), rows, x.ignore_index)
    tol = G.lse_tol(x)
    m = np.ones(rows.size, dtype=bool)
    G.assert_rows("lse", out["lse"][rows], lse, m, tol)
    G.assert_rows("loss", out["loss"][rows], loss, m, tol, lse)
    assert np.all(out["lse"][~valid] == 0) and np.all(out["loss"][~valid] == 0)
    assert np.all(out["dH"][~valid] == 0)
    # dH rows: relative Frobenius over the sample.  The peaked heads are
    # degenerate (margin ~120 nats: the true gradient is below float32
    # resolution of the label term), so they take the label-term floor.  On
    # the flat heads the softmax part averages out over the large vocabulary:
    # the label-term-only output is 2.1-2.2e-2 off (dH) and 8.7e-3 (w4 dE
    # rows) while bf16 rounding costs ~2e-3, hence the tighter tolerances.
    floor, tol_h, tol_e = {1: ("ref", 1e-5, 1e-5), 3: ("ref", 1e-2, 4e-3), 4: ("ref", 1e-2, 4e-3)}.get(
        k, ("label", 2e-2, 2e-2))
    LH = -dl[rows, None].astype(np.float64) * E[x.labels[rows]]
    G.assert_grad("dH rows", out["dH"][rows], dH, LH, tol_h, floor)
    if k in (2, 4):
        # every row's lse, which covers every segment of the forward's
        # partition (workgroup ranges that cross token tiles included)
        G.say(f"full size w{k}: every row's lse (float64 matrix products)")
        lse_all = oracle.lse_matmul(H, E, x.labels, x.ignore_index)
        G.assert_rows("lse (all rows)", out["lse"], lse_all, valid, tol)
    # properties over the whole of dE
    dEg, dHg = out["dE"], out["dH"]
    label_scale = np.linalg.norm((dl[valid, None].astype(np.float64) * H[valid]).sum(axis=0)) + \
        np.sqrt((dl[valid].astype(np.float64) ** 2 * (H[valid] ** 2).sum(axis=1)).sum())
    assert np.linalg.norm(dEg.sum(axis=0)) <= 2e-2 * label_scale
    s_e = float(np.sum(dEg * E))
    s_h = float(np.sum(dHg * H))
    scale = float(np.sum(dl[valid].astype(np.float64) * np.abs((H[valid] * E[x.labels[valid]]).sum(axis=1))))
    assert abs(s_e - s_h) <= 2e-2 * max(scale, 1e-30), (s_e, s_h, scale)
    if k in (1, 4):
        # every row's lse is affordable here: sample dE rows from the oracle
        if k == 1:
            lse_all = oracle.lse_matmul(H, E, x.labels, x.ignore_index)
        vids = np.unique(np.concatenate([x.labels[vrows[:6]], rng.integers(0, x.V, 6)]))
        dE = oracle.dE_rows(H, E, x.labels, lse_all, dl.astype(np.float64), vids, x.ignore_index)
        LE = np.zeros_like(dE)
        for j, v in enumerate(vids):
            sel = x.labels == v
            LE[j] = -(dl[sel, None].astype(np.float64) * H[sel]).sum(axis=0)
        G.assert_grad("dE rows", dEg[vids], dE, LE, tol_e, floor)


@pytest.mark.parametrize("fine,sort", [(False, False), (True, False), (False, True)])
def test_full_size_partially_peaked(fine, sort):
    """The Gemma-2-2B head with a partially peaked softmax (workload 7) at
    full size, with the default filter and with the fine filter: most blocks
    keep a softmax part, so the backward runs its worst-case number of store
    passes with real work in each.  The filtered gradient of a row depends
    only on the rows of its 128-row block (the decisions of the blocks or
    sub-tiles it lies in) and on its own logits, so the oracle's filtered
    backward on a few whole row blocks (all V columns) gives those rows' dH
    exactly; every row of those blocks is compared with it, and their lse
    with the float64 matrix products.  With the vocabulary sorted, the blocks
    are those of the sorted order: the oracle gets the classifier rows and
    the labels in that order (dH does not depend on the order otherwise)."""
    k = 7
    x = inputs.make_workload(k)
    eps = x.eps
    assert not np.any(x.labels == x.ignore_index)  # row blocks = blocks of 128 consecutive rows
    G.say(f"full size w{k} N={x.N} D={x.D} V={x.V} eps={eps} (partially peaked) fine={fine} sort={sort}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, flags=B.CCE_BWD_FINE_FILTER if fine else 0, sort=sort)
    stats = out["stats"]
    assert stats[0] > 0, stats  # blocks that kept a softmax part
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    n_rb = x.N // 128
    rng = np.random.default_rng(k)
    blocks = np.unique(np.concatenate([[0, n_rb - 1], rng.choice(np.arange(1, n_rb - 1), 1)]))
    R = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
    G.say(f"full size w{k}: filtered oracle on row blocks {blocks.tolist()}")
    dl64 = dl.astype(np.float64)
    br, bv = B.FINE_SUBTILE if fine else B.filter_block()
    if sort:
        perm = out["perm"].astype(np.int64)  # sorted position -> vocabulary id
        inv = np.empty_like(perm)
        inv[perm] = np.arange(x.V)
        assert np.array_equal(np.sort(perm), np.arange(x.V))
        fH, _, kept, aH, _ = oracle.backward_filtered(H[R], E[perm], inv[x.labels[R]], dl64[R], eps, br, bv,
                                                      x.ignore_index)
    else:
        fH, _, kept, aH, _ = oracle.backward_filtered(H[R], E, x.labels[R], dl64[R], eps, br, bv, x.ignore_index)
    assert kept.any() and not kept.all(), kept.mean()  # the partial regime
    lse = oracle.lse_matmul(H[R], E, x.labels[R], x.ignore_index)
    G.assert_rows("lse", out["lse"][R], lse, np.ones(R.size, dtype=bool), G.lse_tol(x))
    LH = -dl64[R, None] * E[x.labels[R]]
    G.assert_grad_filtered("dH rows", out["dH"][R], fH, aH, LH)
    # sum_v <dE_v, e_v> = sum_i <dH_i, h_i> holds for the filtered gradient
    # too (both products use the same kept entries)
    s_e = float(np.sum(out["dE"] * E))
    s_h = float(np.sum(out["dH"] * H))
    scale = float(np.sum(dl64 * np.abs((H * E[x.labels]).sum(axis=1))))
    assert abs(s_e - s_h) <= 2e-2 * max(scale, 1e-30), (s_e, s_h, scale)
