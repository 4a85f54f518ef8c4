"""Vocabulary order by mean logit: a stable descending permutation whose keys
match the oracle's definition, and which leaves the gradients unchanged up
to fp32 reassociation."""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _keys_perm(x):
    H, E, y = G.to_device(x)
    perm, keys = B.cce_vocab_order(H, E, y, x.ignore_index, want_keys=True)
    torch.cuda.synchronize()
    return perm.cpu().numpy().astype(np.int64), keys.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("k,N,D,V", [(5, 480, 256, 9500), (3, 600, 512, 5000), (1, None, None, None)])
def test_perm_is_stable_descending_by_mean_logit(k, N, D, V):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"sort w{k}")
    perm, keys = _keys_perm(x)
    assert np.array_equal(np.sort(perm), np.arange(x.V))
    kp = keys[perm]
    assert np.all(kp[:-1] >= kp[1:])
    ties = kp[:-1] == kp[1:]
    assert np.all(perm[:-1][ties] < perm[1:][ties])
    # keys against the definition (fp64 mean of the logits over valid rows)
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    ref = oracle.mean_logit(H, E, x.labels, x.ignore_index)
    hbar = np.abs(H[x.labels != x.ignore_index]).mean(axis=0)
    scale = np.abs(E) @ hbar  # sum_d |hbar_d e_vd| bounds the terms of the dot
    tol = 1e-5 * scale + 1e-30
    assert np.all(np.abs(keys - ref) <= tol), float(np.max(np.abs(keys - ref) / tol))
    # the order is descending in the oracle's keys up to that tolerance
    assert np.all(ref[perm[:-1]] >= ref[perm[1:]] - tol[perm[:-1]] - tol[perm[1:]])


def test_equal_rows_tie_by_ascending_id():
    x = inputs.make_inputs(64, 32, 300, dtype="bf16", seed=11)
    for r in (10, 20, 30, 299):
        x.E[r] = x.E[5]
    perm, keys = _keys_perm(x)
    pos = {int(v): i for i, v in enumerate(perm)}
    group = [5, 10, 20, 30, 299]
    assert [pos[v] for v in group] == sorted(pos[v] for v in group)
    assert all(keys[v] == keys[5] for v in group)


def test_no_valid_row_gives_identity():
    x = inputs.make_inputs(40, 16, 100, dtype="f32", ignore_frac=1.0, seed=3)
    perm, keys = _keys_perm(x)
    assert np.array_equal(perm, np.arange(100)) and np.all(keys == 0)


@pytest.mark.parametrize("k,N,D,V", [(5, 480, 256, 9500), (4, 512, 384, 3000)])
def test_sorted_and_unsorted_backward_agree(k, N, D, V):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"sort on/off agreement w{k}")
    dl = G.mean_dloss(x)
    a = G.run_gpu(x, dl, eps=0.0, sort=False)
    b = G.run_gpu(x, dl, eps=0.0, sort=True)
    for name in ("dH", "dE"):
        n = max(np.linalg.norm(a[name]), 1e-30)
        assert np.linalg.norm(a[name] - b[name]) / n <= 2e-3, name
    # the sorted forward visits the vocabulary in another order: rounding only
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(b["loss"], a["loss"], rtol=1e-5, atol=1e-5)
