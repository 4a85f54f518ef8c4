"""Forward parity on seeded random shapes: every valid row's lse and loss
against the fp64 oracle.  Most shapes take the 4-wave forward (bf16, D a
multiple of 64): token counts that leave a partial token tile or a single
one, vocabularies that leave a partial last tile or fit one tile, one to
eight 128-byte K stages per tile, ignored rows, peaked rows (where most
tiles skip their exponentials) and flat ones; a few take the other forward
kernels (fp32, D not a multiple of 64), with the block-max table on and
off and the vocabulary sort on and off."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("normal", "peaked")[i % 2]
        dt = "f32" if i % 8 == 7 else "bf16"
        D = int(64 * rng.integers(1, 9)) if i % 5 != 4 else int(8 * rng.integers(1, 40))
        N = int(rng.integers(1, 1500))
        V = int(rng.integers(1, 6000))
        ign = float(rng.choice([0.0, 0.0, 0.3]))
        lab = ("uniform", "zipf")[int(rng.integers(0, 2))]
        out.append((i, N, D, V, dt, kind, lab, ign, bool(i % 3 == 0), bool(i % 4 == 1)))
    return out


# plus a single token, and a single 64-byte-per-row K stage pair with a token
# count one past a tile
CASES = _shapes() + [(16, 1, 64, 300, "bf16", "peaked", "uniform", 0.0, False, False),
                     (17, 257, 64, 257, "bf16", "normal", "zipf", 0.0, False, True)]


@pytest.mark.parametrize("i,N,D,V,dt,kind,lab,ign,nobound,sort", CASES,
                         ids=[f"s{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}-{c[5]}" for c in CASES])
def test_forward_random_shape(i, N, D, V, dt, kind, lab, ign, nobound, sort):
    x = inputs.make_inputs(N, D, V, dtype=dt, e_std=0.5 if dt == "f32" else 0.05, h_kind=kind,
                           label_kind=lab, ignore_frac=ign, seed=1000 + i, peak_scale=2.0)
    G.say(f"random shape {i}: N={N} D={D} V={V} {dt} {kind} {lab} ignore={ign} table={not nobound} sort={sort}")
    out = G.run_gpu(x, G.mean_dloss(x), eps=0.0, backward=False, bound=not nobound, sort=sort)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    loss, lse = oracle.forward(H, E, x.labels, x.ignore_index)
    valid = x.labels != x.ignore_index
    G.assert_rows("lse", out["lse"], lse, valid, G.lse_tol(x))
    G.assert_rows("loss", out["loss"], loss, valid, G.lse_tol(x), lse)
    ign_rows = ~valid
    assert np.all(out["lse"][ign_rows] == 0) and np.all(out["loss"][ign_rows] == 0), "ignored rows are zero"
