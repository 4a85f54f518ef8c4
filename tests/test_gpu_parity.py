"""Parity of the HIP path with the fp64 oracle, element by element, on the
six workloads' recipes at sizes the oracle finishes in seconds (several
tiles, ragged tails, more than one vocabulary chunk), plus edge cases."""
import numpy as np
import pytest

from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# (workload, N, D, V): reduced sizes that keep each recipe's regime.
SMALL = [
    (1, None, None, None),   # the tiny workload at full size
    (2, 700, 256, 9000),     # peaked; two vocabulary chunks; ragged N and V
    (3, 600, 512, 5000),     # flat, 40 % ignored rows
    (4, 512, 384, 3000),     # flat, small V / D
    (5, 480, 256, 9500),     # peaked, Zipf labels; run with and without sort
    (6, 480, 256, 9500),     # as 5 with the Zipf ranks scattered over the ids
]


def _case(k, N, D, V):
    return inputs.make_workload(k, N=N, D=D, V=V)


@pytest.mark.parametrize("k,N,D,V", SMALL, ids=[f"w{c[0]}" for c in SMALL])
def test_forward_matches_oracle(k, N, D, V):
    x = _case(k, N, D, V)
    G.say(f"forward w{k} N={x.N} D={x.D} V={x.V} {x.dtype}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=0.0)
    loss, lse, _, _ = G.oracle_full(x, dl, "mean")
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)


@pytest.mark.parametrize("k,N,D,V", SMALL, ids=[f"w{c[0]}" for c in SMALL])
@pytest.mark.parametrize("dkind", ["mean", "random"])
def test_backward_unfiltered(k, N, D, V, dkind):
    x = _case(k, N, D, V)
    G.say(f"backward eps=0 w{k} N={x.N} D={x.D} V={x.V} dloss={dkind}")
    dl = G.mean_dloss(x) if dkind == "mean" else G.random_dloss(x, seed=k)
    out = G.run_gpu(x, dl, eps=0.0)
    _, _, dH, dE = G.oracle_full(x, dl, dkind)
    LH, LE = G.label_term(x, dl)
    tol = 1e-5 if x.dtype == "f32" else 1e-2
    G.assert_grad("dH", out["dH"], dH, LH, tol)
    G.assert_grad("dE", out["dE"], dE, LE, tol)
    valid = x.labels != x.ignore_index
    assert np.all(out["dH"][~valid] == 0)
    # eps = 0 keeps every block
    assert out["stats"][0] == out["stats"][2] and out["stats"][1] == 0
    assert out["stats"][3] == valid.sum()


@pytest.mark.parametrize("k,N,D,V", SMALL[1:], ids=[f"w{c[0]}" for c in SMALL[1:]])
@pytest.mark.parametrize("sort", [False, True])
def test_backward_filtered(k, N, D, V, sort):
    x = _case(k, N, D, V)
    eps = inputs.WORKLOADS[k].eps
    G.say(f"backward eps={eps} sort={sort} w{k} N={x.N} D={x.D} V={x.V}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, sort=sort)
    _, _, dH, dE = G.oracle_full(x, dl, "mean")
    LH, LE = G.label_term(x, dl)
    G.assert_grad("dH", out["dH"], dH, LH, 2e-2)
    G.assert_grad("dE", out["dE"], dE, LE, 2e-2)


EDGE = [
    # (N, D, V, dtype, ignore_frac, h_kind)
    (1, 8, 1, "bf16", 0.0, "normal"),        # V = 1: lse = z, loss = 0, zero gradients
    (1, 64, 130, "f32", 0.0, "normal"),      # single row, ragged vocabulary
    (3, 8, 7, "f32", 0.0, "normal"),         # smallest D
    (129, 136, 257, "bf16", 0.0, "normal"),  # one past tile edges everywhere
    (200, 64, 300, "bf16", 1.0, "normal"),   # every row ignored
    (300, 96, 1000, "f32", 0.5, "peaked"),
]


@pytest.mark.parametrize("N,D,V,dt,ign,hk", EDGE, ids=[f"{e[0]}x{e[1]}x{e[2]}-{e[3]}-ign{e[4]}" for e in EDGE])
def test_edge_shapes(N, D, V, dt, ign, hk):
    x = inputs.make_inputs(N, D, V, dtype=dt, e_std=0.5 if dt == "f32" else 0.05, h_kind=hk,
                           label_kind="uniform", ignore_frac=ign, seed=N + D + V)
    G.say(f"edge N={N} D={D} V={V} {dt} ign={ign}")
    dl = G.random_dloss(x, seed=3)
    dl = np.where(x.labels != x.ignore_index, dl, 0).astype(np.float32)
    out = G.run_gpu(x, dl, eps=0.0)
    loss, lse, dH, dE = G.oracle_full(x, dl, "edge")
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)
    LH, LE = G.label_term(x, dl)
    tol = 1e-5 if dt == "f32" else 1e-2
    if valid.any():
        G.assert_grad("dH", out["dH"], dH, LH, tol)
        G.assert_grad("dE", out["dE"], dE, LE, tol)
    else:
        assert np.all(out["dH"] == 0) and np.all(out["dE"] == 0)
        assert np.all(out["loss"] == 0) and np.all(out["lse"] == 0)
    if V == 1:
        assert np.all(out["dE"] == 0) and np.all(out["dH"] == 0)
