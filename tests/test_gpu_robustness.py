"""Error reporting on the device: the label check counts labels outside
[0, V) that are not ignore_index, and a pass whose block store fills up
(forced from the host with CCE_BWD_DEBUG_STORE_LIMIT, which halves the slots
the epilogue may take) drops the blocks it cannot store and counts them in
stats[5] instead of writing past the store."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_check_labels_counts_out_of_range():
    G.say("check labels small")
    y = torch.tensor([0, 5, -100, 7, -1, 8, 100000, -100, -7], dtype=torch.int64, device=G.DEV)
    assert B.cce_check_labels(y, 8, -100) == 4      # -1, 8, 100000, -7
    assert B.cce_check_labels(y, 100001, -100) == 2  # -1, -7
    assert B.cce_check_labels(y, 8, -1) == 5         # -100 (twice), 8, 100000, -7; -1 is ignored


def test_check_labels_large():
    G.say("check labels large")
    rng = np.random.default_rng(4)
    N, V = 300_001, 50_000
    y = rng.integers(0, V, size=N)
    y[rng.choice(N, 1000, replace=False)] = -100
    bad = rng.choice(N, 37, replace=False)
    y[bad[:20]] = V + rng.integers(0, 10, 20)
    y[bad[20:]] = -rng.integers(1, 99, 17)
    want = int(np.count_nonzero((y != -100) & ((y < 0) | (y >= V))))
    assert B.cce_check_labels(torch.from_numpy(y).to(G.DEV), V, -100) == want == 37


def test_store_overflow_is_counted():
    # Phi-head recipe, no ignored rows, eps = 0: every one of the 4 x 24
    # blocks is kept in one pass whose store holds exactly 96 blocks; with
    # the debug limit only 48 get a slot.
    x = inputs.make_workload(4, N=512, D=384, V=3000)
    dl = G.mean_dloss(x)
    G.say("store overflow report")
    ok = G.run_gpu(x, dl, eps=0.0)
    assert ok["stats"][5] == 0 and ok["stats"][0] == ok["stats"][2] == 96
    bad = G.run_gpu(x, dl, eps=0.0, flags=B.CCE_BWD_DEBUG_STORE_LIMIT)
    assert bad["stats"][5] == 48 and bad["stats"][0] == 48
    assert bad["stats"][0] + bad["stats"][5] == bad["stats"][2]
    assert np.all(np.isfinite(bad["dH"])) and np.all(np.isfinite(bad["dE"]))
    assert not np.array_equal(bad["dE"], ok["dE"])  # the dropped blocks are missing
