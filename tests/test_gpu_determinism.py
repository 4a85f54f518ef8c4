"""Same inputs, same bits: the forward merges its vocabulary splits in a fixed
order and the backward owns every output element in one workgroup."""
import numpy as np
import pytest

from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k,N,D,V,sort", [(3, 900, 256, 9000, False), (5, 480, 256, 9500, True)])
def test_bit_identical_reruns(k, N, D, V, sort):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"determinism w{k} sort={sort}")
    dl = G.random_dloss(x, seed=5)
    runs = [G.run_gpu(x, dl, eps=inputs.WORKLOADS[k].eps, sort=sort) for _ in range(3)]
    for r in runs[1:]:
        for key in ("loss", "lse", "dH", "dE", "stats"):
            assert np.array_equal(r[key], runs[0][key]), key
