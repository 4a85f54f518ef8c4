"""The block-max table and the recompute skip it allows.

cce_forward can record the largest logit of every 128-token x 128-vocabulary
block; cce_backward, given that table, leaves out the logit recompute of
256 x 256 tiles whose every softmax entry is provably below filter_eps / 2.
The gradient filter would drop all of such a tile's softmax part, so the
outputs must be bit-identical to a run without the table; only the count of
recomputed blocks (stats[4]) changes.  The table itself is checked against the
definition: the largest fp64 logit of each block of the valid rows (in order),
-inf for blocks past the valid rows.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

BLK = 128
CASES = [
    (1, None, None, None),    # fp32, flat, 10 % ignored
    (2, 700, 256, 9000),      # peaked, two vocabulary chunks, ragged
    (3, 600, 512, 5000),      # flat, 40 % ignored
    (5, 480, 256, 9500),      # peaked, Zipf labels
]


def _ref_block_max(x):
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    valid = np.nonzero(x.labels != x.ignore_index)[0]
    Z = H[valid] @ E.T  # the logits of the valid rows, in order
    nrb, ncb = 2 * -(-x.N // 256), 2 * -(-x.V // 256)
    ref = np.full((nrb, ncb), -np.inf)
    for rb in range(-(-valid.size // BLK)):
        rows = Z[rb * BLK:(rb + 1) * BLK]
        for cb in range(-(-x.V // BLK)):
            ref[rb, cb] = rows[:, cb * BLK:(cb + 1) * BLK].max()
    return ref


@pytest.mark.parametrize("k,N,D,V", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_table_is_block_max(k, N, D, V):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"block-max table w{k} N={x.N} D={x.D} V={x.V}")
    out = G.run_gpu(x, G.mean_dloss(x), eps=x.eps or 2.0 ** -12)
    ref = _ref_block_max(x)
    got = out["block_max"].reshape(ref.shape)
    fin = np.isfinite(ref)
    assert np.all(got[~fin] == -np.inf), "blocks past the valid rows or vocabulary must stay -inf"
    err = np.abs(got[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), 1.0)
    tol = 1e-5 if x.dtype == "f32" else 1e-3
    assert err.max() <= tol, err.max()


@pytest.mark.parametrize("k,N,D,V", CASES, ids=[f"w{c[0]}" for c in CASES])
@pytest.mark.parametrize("eps", [2.0 ** -12, 2.0 ** -6])
def test_skip_is_bit_identical(k, N, D, V, eps):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"bound skip bit identity w{k} N={x.N} D={x.D} V={x.V} eps={eps}")
    dl = G.random_dloss(x, seed=7)
    a = G.run_gpu(x, dl, eps=eps, bound=True)
    b = G.run_gpu(x, dl, eps=eps, bound=False)
    for key in ("loss", "lse", "dH", "dE"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["stats"][:4], b["stats"][:4])
    # without the table every valid block is recomputed
    assert b["stats"][4] == b["stats"][2]
    assert a["stats"][4] <= b["stats"][4]
    # a recomputed block is never needed where the filter kept something
    assert a["stats"][4] >= a["stats"][0]
    if x.name.startswith(("gemma", "large-vocab")):
        # peaked softmax: tiles without a label need no logits
        assert a["stats"][4] < a["stats"][2], a["stats"]


def test_table_unused_with_sort_or_without_filter():
    x = inputs.make_workload(5, N=480, D=256, V=9500)
    G.say("bound ignored with sort / eps=0")
    dl = G.mean_dloss(x)
    s = G.run_gpu(x, dl, eps=2.0 ** -12, sort=True)
    assert s["stats"][4] == s["stats"][2]
    z = G.run_gpu(x, dl, eps=0.0)
    assert z["stats"][4] == z["stats"][2] and z["stats"][0] == z["stats"][2]


def _device_run(x, tb, eps, dl):
    H, E, y = G.to_device(x)
    _, lse = B.cce_forward(H, E, y, x.ignore_index, block_max=tb)
    stats = torch.zeros(5, dtype=torch.int64, device=G.DEV)
    dH, dE = B.cce_backward(H, E, y, lse, dl, eps, x.ignore_index, None, 0, stats=stats, block_max=tb)
    torch.cuda.synchronize()
    return dH, dE, stats.cpu().numpy()


@pytest.mark.parametrize("k", [2, 5])
def test_full_size_skip_is_bit_identical(k):
    """At the full head shapes of the peaked workloads, with the launch
    configuration the benchmark times, compared on the device."""
    x = inputs.make_workload(k)
    G.say(f"bound skip full size w{k} N={x.N} D={x.D} V={x.V}")
    dl = torch.from_numpy(G.mean_dloss(x)).to(G.DEV)
    tb = torch.empty(B.block_max_elems(x.N, x.V), dtype=torch.float32, device=G.DEV)
    dH_a, dE_a, st_a = _device_run(x, tb, x.eps, dl)
    dH_b, dE_b, st_b = _device_run(x, None, x.eps, dl)
    assert torch.equal(dH_a, dH_b) and torch.equal(dE_a, dE_b)
    assert np.array_equal(st_a[:4], st_b[:4])
    G.say(f"  recomputed blocks {st_a[4]} of {st_a[2]} (kept {st_a[0]}, label-only {st_a[1]})")
    assert st_a[4] < st_a[2] // 4
