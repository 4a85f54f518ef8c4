"""Composite head on the GPU: two classifier blocks, ids [0, V0) in E0 and
[off1, off1 + V1) in E1 with a dead gap between (the lit note "The loss and
the mask: Cut Cross-Entropy + FlexAttention", section "What transfers to us").

  - parity with the fp64 composite oracle (forward rows, unfiltered and
    filtered gradients of both blocks);
  - the kernels see the concatenated vocabulary, so a composite call gives
    the same bits as the one-matrix call on cat(E0, E1) with the labels moved
    down by the gap (sort and block-max table on and off);
  - a label in the gap is out of range: its row gets NaN, the others are
    unchanged.
Inputs: a workload recipe with V = V0 + V1 split into the two blocks, labels
of the second block moved up by the gap.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _case(k, N, D, V0, V1, gap):
    x = inputs.make_workload(k, N=N, D=D, V=V0 + V1)
    y = x.labels.copy()
    second = y >= V0
    y[second] += gap
    return x, y


def _dev(x, V0):
    H, E, ycat = G.to_device(x)
    E0 = E[:V0].contiguous()
    E1 = E[V0:].contiguous()  # a separate allocation
    return H, E0, E1, ycat


def _run(x, y, V0, off1, dl, eps, sort=False, bound=True, flags=0):
    H, E0, E1, _ = _dev(x, V0)
    yt = torch.from_numpy(y).to(G.DEV)
    V = x.V
    perm = B.cce_vocab_order_composite(H, E0, E1, yt, x.ignore_index) if sort else None
    tb = torch.empty(B.block_max_elems(x.N, V), dtype=torch.float32, device=G.DEV) if bound else None
    loss, lse = B.cce_forward_composite(H, E0, E1, off1, yt, x.ignore_index, block_max=tb, perm=perm)
    stats = torch.zeros(7, dtype=torch.int64, device=G.DEV)
    dH = torch.full_like(H, float("nan"))
    dE0 = torch.full_like(E0, float("nan"))
    dE1 = torch.full_like(E1, float("nan"))
    B.cce_backward_composite(H, E0, E1, off1, yt, lse, torch.from_numpy(dl).to(G.DEV), eps, x.ignore_index, perm,
                             flags, dH=dH, dE0=dE0, dE1=dE1, stats=stats, block_max=tb)
    torch.cuda.synchronize()
    return dict(loss=G.t64(loss), lse=G.t64(lse), dH=G.t64(dH), dE0=G.t64(dE0), dE1=G.t64(dE1),
                stats=stats.cpu().numpy(), perm=None if perm is None else perm.cpu().numpy())


CASES = [
    (1, 256, 128, 2500, 1596, 404),     # fp32, flat, 10 % ignored; blocks meet inside a 128-block
    (2, 700, 256, 6000, 3000, 1000),    # peaked, Zipf labels (most in the first block)
    (3, 600, 512, 3000, 2000, 7),       # flat, 40 % ignored
    (4, 300, 72, 1000, 777, 0),         # D * 2 not a multiple of 128; no gap
]


@pytest.mark.parametrize("k,N,D,V0,V1,gap", CASES, ids=[f"w{c[0]}" for c in CASES])
@pytest.mark.parametrize("filtered", [False, True])
def test_composite_matches_oracle(k, N, D, V0, V1, gap, filtered):
    x, y = _case(k, N, D, V0, V1, gap)
    off1 = V0 + gap
    eps = (x.eps or 2.0 ** -12) if filtered else 0.0
    G.say(f"composite parity w{k} N={N} D={D} V0={V0} V1={V1} gap={gap} eps={eps}")
    dl = G.random_dloss(x, seed=k)
    out = _run(x, y, V0, off1, dl, eps)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    loss, lse, dH, dE0, dE1 = oracle.composite(H, E[:V0], E[V0:], off1, y, dl.astype(np.float64), x.ignore_index)
    valid = y != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)
    # label-term floor of the tolerance, per block
    LH = np.zeros_like(H)
    LE = np.zeros_like(E)
    ycat = x.labels
    LH[valid] = -dl[valid, None] * E[ycat[valid]]
    np.add.at(LE, ycat[valid], -dl[valid, None] * H[valid])
    if filtered:
        # the kernels filter blocks of the concatenated vocabulary (E0's rows,
        # then E1's): the oracle's filtered gradient over that vocabulary
        fH, fE, _, aH, aE = oracle.backward_filtered(H, E, ycat, dl.astype(np.float64), eps, *B.filter_block(),
                                                     x.ignore_index)
        G.assert_grad_filtered("dH", out["dH"], fH, aH, LH)
        G.assert_grad_filtered("dE", np.concatenate([out["dE0"], out["dE1"]]), fE, aE, LE)
    else:
        tol = 1e-5 if x.dtype == "f32" else 1e-2
        G.assert_grad("dH", out["dH"], dH, LH, tol)
        G.assert_grad("dE0", out["dE0"], dE0, LE[:V0], tol)
        G.assert_grad("dE1", out["dE1"], dE1, LE[V0:], tol)
    assert np.all(out["dH"][~valid] == 0)


@pytest.mark.parametrize("sort", [False, True])
# (the last case: the Gemma-2-2B head at full size split into two blocks of
# 128 000 rows, two allocations of 590 MB)
@pytest.mark.parametrize("k,N,D,V0,V1,gap", [CASES[1], CASES[2], (2, None, None, 128000, 128000, 1000)],
                         ids=["w2", "w3", "w2-full"])
def test_composite_equals_concatenated_head(k, N, D, V0, V1, gap, sort):
    x, y = _case(k, N, D, V0, V1, gap)
    eps = x.eps or 2.0 ** -12
    G.say(f"composite == concatenated w{k} N={x.N} D={x.D} V0={V0} V1={V1} sort={sort}")
    dl = G.random_dloss(x, seed=11)
    a = _run(x, y, V0, V0 + gap, dl, eps, sort=sort)
    b = G.run_gpu(x, dl, eps=eps, sort=sort)
    if sort:
        assert np.array_equal(a["perm"], b["perm"])
    for key in ("loss", "lse", "dH"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(np.concatenate([a["dE0"], a["dE1"]]), b["dE"])
    assert np.array_equal(a["stats"], b["stats"])


def test_table_skip_is_bit_identical():
    x, y = _case(2, 700, 256, 6000, 3000, 1000)
    G.say("composite block-max skip")
    dl = G.random_dloss(x, seed=12)
    a = _run(x, y, 6000, 7000, dl, x.eps, bound=True)
    b = _run(x, y, 6000, 7000, dl, x.eps, bound=False)
    for key in ("loss", "lse", "dH", "dE0", "dE1"):
        assert np.array_equal(a[key], b[key]), key
    assert a["stats"][4] < b["stats"][4]


def test_gap_label_gives_nan_row():
    x, y = _case(3, 600, 512, 3000, 2000, 50)
    G.say("composite gap label")
    H, E0, E1, _ = _dev(x, 3000)
    valid_rows = np.nonzero(y != x.ignore_index)[0]
    bad = int(valid_rows[3])
    y2 = y.copy()
    y2[bad] = 3000 + 10  # in the gap
    l1, s1 = B.cce_forward_composite(H, E0, E1, 3050, torch.from_numpy(y).to(G.DEV), x.ignore_index)
    l2, s2 = B.cce_forward_composite(H, E0, E1, 3050, torch.from_numpy(y2).to(G.DEV), x.ignore_index)
    torch.cuda.synchronize()
    l1, s1, l2, s2 = (G.t64(t) for t in (l1, s1, l2, s2))
    assert np.isnan(l2[bad]) and np.isnan(s2[bad])
    keep = np.arange(x.N) != bad
    assert np.array_equal(l1[keep], l2[keep]) and np.array_equal(s1[keep], s2[keep])


def test_one_row_blocks():
    x, y = _case(1, 40, 64, 1, 1, 5)
    G.say("composite V0 = V1 = 1")
    dl = G.random_dloss(x, seed=2)
    out = _run(x, y, 1, 6, dl, 0.0)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    loss, lse, dH, dE0, dE1 = oracle.composite(H, E[:1], E[1:], 6, y, dl.astype(np.float64), x.ignore_index)
    valid = y != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, 1e-5)
    G.assert_rows("loss", out["loss"], loss, valid, 1e-5, lse)
    for name, g, r in (("dH", out["dH"], dH), ("dE0", out["dE0"], dE0), ("dE1", out["dE1"], dE1)):
        assert np.linalg.norm(g - r) <= 1e-5 * max(np.linalg.norm(r), 1e-30) + 1e-7, name
