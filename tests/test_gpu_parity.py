"""Parity of the HIP path with the fp64 oracle, element by element, on the
six workloads' recipes at sizes the oracle finishes in seconds (several
tiles, ragged tails, more than one vocabulary chunk), a moderately peaked
recipe whose gradient is dominated by the label entry's dloss (p_y - 1) with
p_y near 1, forward cases whose workgroup ranges cross token tiles, and edge
cases.  Gradient checks assert first that they can fail (see tests/_gpu.py)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

# (workload, N, D, V): reduced sizes that keep each recipe's regime; "2m" is
# the Gemma-head recipe with a moderate peak (median 1 - p_y = 0.03).
SMALL = [
    (1, None, None, None),   # the tiny workload at full size
    (2, 700, 256, 9000),     # peaked (1 - p_y ~ 3e-3); two vocabulary chunks; ragged N and V
    ("2m", 700, 256, 9000),  # moderately peaked
    (3, 600, 512, 5000),     # flat, 40 % ignored rows
    (4, 512, 384, 3000),     # flat, small V / D
    (5, 480, 256, 9500),     # peaked, Zipf labels; run with and without sort
    (6, 480, 256, 9500),     # as 5 with the Zipf ranks scattered over the ids
]
IDS = [f"w{c[0]}" for c in SMALL]
PEAKED = {2, "2m", 5, 6}


def _case(k, N, D, V):
    if k == "2m":
        return G.moderate_peaked(N, D, V)
    return inputs.make_workload(k, N=N, D=D, V=V)


def _eps(k):
    return 2.0 ** -12 if k == "2m" else inputs.WORKLOADS[k].eps


@pytest.mark.parametrize("k,N,D,V", SMALL, ids=IDS)
def test_forward_matches_oracle(k, N, D, V):
    x = _case(k, N, D, V)
    G.say(f"forward w{k} N={x.N} D={x.D} V={x.V} {x.dtype}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=0.0)
    loss, lse, _, _ = G.oracle_full(x, dl, "mean")
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)


def _forward_split(n_valid, V, groups):
    """The forward's work split, as the kernels choose it (token tiles x
    vocabulary ranges, a x bb blocks per XCD group, m range groups): returns
    (ranges per token tile, steps per workgroup, block shape)."""
    R = -(-n_valid // 256)
    C = -(-V // 256)
    G_ = min(groups, 1024, R * C)
    if G_ >= 8:
        G_ &= ~7
    nx = 8 if G_ % 8 == 0 else 1
    P = G_ // nx
    best, cfg = None, (1, 1, 1)
    a = 1
    while a <= P:
        if P % a == 0:
            bb = P // a
            m = 1
            while bb * m <= min(C, 32):
                steps = (-(-R // a) * m + nx - 1) // nx
                cost = (steps * -(-C // (bb * m)), 0 if a == 4 else 1)
                if best is None or cost < best:
                    best, cfg = cost, (a, bb, m)
                m += 1
        a *= 2
    a, bb, m = cfg
    return bb * m, (-(-R // a) * m + nx - 1) // nx, (a, bb)


# several vocabulary ranges per token tile, several blocks per workgroup, and
# a block shape other than 4 x 8: the ordered merge combines many segments
SPLIT = [(3, 2300, 512, 20000), (5, 9500, 64, 20000), (5, 9500, 64, 10000)]


@pytest.mark.parametrize("k,N,D,V", SPLIT, ids=[f"w{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in SPLIT])
def test_forward_split_ranges_and_steps(k, N, D, V):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    # one forward workgroup per CU (its LDS buffers take 128 KB)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ranges, steps, shape = _forward_split(x.n_valid, x.V, cus)
    G.say(f"forward split w{k} N={x.N} D={x.D} V={x.V}: {ranges} ranges per token tile, {steps} steps, blocks {shape}")
    assert ranges >= 2
    out = G.run_gpu(x, G.mean_dloss(x), eps=0.0, backward=False)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    loss, lse = oracle.forward(H, E, x.labels, x.ignore_index)
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)


@pytest.mark.parametrize("k,N,D,V", SMALL, ids=IDS)
@pytest.mark.parametrize("dkind", ["mean", "random"])
def test_backward_unfiltered(k, N, D, V, dkind):
    x = _case(k, N, D, V)
    G.say(f"backward eps=0 w{k} N={x.N} D={x.D} V={x.V} dloss={dkind}")
    dl = G.mean_dloss(x) if dkind == "mean" else G.random_dloss(x, seed=zlib.crc32(str(k).encode()) % 97)
    out = G.run_gpu(x, dl, eps=0.0)
    _, _, dH, dE = G.oracle_full(x, dl, dkind)
    LH, LE = G.label_term(x, dl)
    tol = 1e-5 if x.dtype == "f32" else 1e-2
    G.assert_grad("dH", out["dH"], dH, LH, tol)
    G.assert_grad("dE", out["dE"], dE, LE, tol)
    valid = x.labels != x.ignore_index
    assert np.all(out["dH"][~valid] == 0)
    if k == "2m":
        # row by row: every row's gradient is dominated by its label entry
        G.assert_rows_rel("dH rows", out["dH"], dH, np.nonzero(valid)[0], 1e-2)
    # eps = 0 keeps every block
    assert out["stats"][0] == out["stats"][2] and out["stats"][1] == 0
    assert out["stats"][3] == valid.sum()


@pytest.mark.parametrize("k,N,D,V", SMALL[1:], ids=IDS[1:])
def test_backward_filtered(k, N, D, V):
    """Against the oracle's filtered gradient at the kernel's block geometry."""
    x = _case(k, N, D, V)
    eps = _eps(k)
    G.say(f"backward eps={eps} w{k} N={x.N} D={x.D} V={x.V}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps)
    fH, fE, kept, aH, aE = G.oracle_filtered(x, dl, eps, "mean")
    LH, LE = G.label_term(x, dl)
    G.assert_grad_filtered("dH", out["dH"], fH, aH, LH)
    G.assert_grad_filtered("dE", out["dE"], fE, aE, LE)
    # the kernel keeps the same number of blocks, up to near-threshold ones
    if aH == 0 and aE == 0:
        assert out["stats"][0] == int(kept.sum()), (out["stats"], int(kept.sum()))


@pytest.mark.parametrize("k,N,D,V", SMALL[1:], ids=IDS[1:])
def test_backward_filtered_sorted(k, N, D, V):
    """Sorted vocabulary: the blocks follow the sort, so the check is the
    geometry-free one -- the elementwise filter bound against the unfiltered
    gradient -- and the relative Frobenius error (label-term floor where the
    softmax is peaked)."""
    x = _case(k, N, D, V)
    eps = _eps(k)
    G.say(f"backward eps={eps} sort=True w{k} N={x.N} D={x.D} V={x.V}")
    dl = G.mean_dloss(x)
    out = G.run_gpu(x, dl, eps=eps, sort=True)
    _, lse, dH, dE = G.oracle_full(x, dl, "mean")
    G.assert_filter_bound(x, dl, eps, out, lse, dH, dE)
    LH, LE = G.label_term(x, dl)
    floor, tol = ("label", 2e-2) if k in PEAKED else ("ref", 1e-2)
    G.assert_grad("dH", out["dH"], dH, LH, tol, floor)
    G.assert_grad("dE", out["dE"], dE, LE, tol, floor)


EDGE = [
    # (N, D, V, dtype, ignore_frac, h_kind)
    (1, 8, 1, "bf16", 0.0, "normal"),        # V = 1: lse = z, loss = 0, zero gradients
    (1, 64, 130, "f32", 0.0, "normal"),      # single row, ragged vocabulary
    (3, 8, 7, "f32", 0.0, "normal"),         # smallest D
    (129, 136, 257, "bf16", 0.0, "normal"),  # one past tile edges everywhere
    (200, 64, 300, "bf16", 1.0, "normal"),   # every row ignored
    (300, 64, 700, "bf16", 0.1, "normal"),   # D = 64: one 128-byte K stage per vocabulary tile
    (300, 96, 1000, "f32", 0.5, "peaked"),   # z_y ~ 144: every non-label p below fp32 resolution
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
    if V == 1:
        assert np.all(out["dE"] == 0) and np.all(out["dH"] == 0)
    elif valid.any():
        floor = "label" if hk == "peaked" else "ref"
        G.assert_grad("dH", out["dH"], dH, LH, tol, floor)
        G.assert_grad("dE", out["dE"], dE, LE, tol, floor)
    else:
        assert np.all(out["dH"] == 0) and np.all(out["dE"] == 0)
        assert np.all(out["loss"] == 0) and np.all(out["lse"] == 0)
