"""Kahan compensation of the classifier gradient across row blocks.  The
input makes one large contribution to dE arrive first and many small ones
after it (fp32 so the output keeps the difference); compensated
accumulation must land closer to the fp64 oracle than plain fp32."""
import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _adversarial():
    N, D, V = 128 * 48, 64, 256
    rng = np.random.default_rng(42)
    H = (rng.standard_normal((N, D)) * 1e-3).astype(np.float32)
    # First row block: a large constant, so its block product is exact in fp32
    # (g = 1/256 or 1/256 - 1, both powers-of-two sums) and the only rounding
    # left is where the later, small block products meet the large sum.
    H[:128] = np.float32(2.0 ** 13)
    E = np.zeros((V, D), dtype=np.float32)  # uniform softmax: g_iv = dloss_i (1/V - [v = y_i])
    labels = rng.integers(0, V, size=N).astype(np.int64)
    return inputs.Inputs("kahan-adversarial", 42, N, D, V, "f32", H, E, labels, 0.0)


def test_kahan_reduces_error():
    x = _adversarial()
    G.say("kahan adversarial")
    dl = np.ones(x.N, dtype=np.float32)
    on = G.run_gpu(x, dl, eps=0.0)
    off = G.run_gpu(x, dl, eps=0.0, flags=B.CCE_BWD_NO_KAHAN)
    _, _, _, dE = G.oracle_full(x, dl, "ones")
    e_on = np.abs(on["dE"] - dE).sum()
    e_off = np.abs(off["dE"] - dE).sum()
    assert e_on < e_off / 2, (e_on, e_off)
    # and both are right to fp32 precision of the partial sums
    assert np.linalg.norm(on["dE"] - dE) / np.linalg.norm(dE) < 1e-5
