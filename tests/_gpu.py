"""Helpers for the GPU parity tests: move generated inputs to the device, run
the HIP path through the C ABI binding, run the fp64 oracle on the same bits,
and apply the tolerances.

Tolerances (floating point):
  lse         per valid row |gpu - ref| <= tol * max(|ref|, 1)
  loss        per valid row |gpu - ref| <= tol * max(|ref|, 1) + 2^-20 |lse_ref|
              tol = 1e-3 for bf16 inputs, 1e-5 for fp32 inputs.  The 1-nat
              floor makes the bound meaningful where the true loss is ~0
              (peaked softmax); loss = lse - z_y is a difference of two
              O(lse) fp32 numbers, so it also admits 16 fp32 ulps of lse.
  dH, dE      ||gpu - ref||_F <= gtol * max(||ref||_F, ||L||_F), where L is
              the label-term-only gradient (dH_i = -dloss_i e_{y_i},
              dE_v = -sum_{i: y_i = v} dloss_i h_i).  gtol = 2e-2 with
              filtering on; tighter without filtering (1e-2 bf16, 1e-5 fp32).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs

DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x: inputs.Inputs):
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H).view(torch.bfloat16).to(DEV)
        E = torch.from_numpy(x.E).view(torch.bfloat16).to(DEV)
    else:
        H = torch.from_numpy(x.H).to(DEV)
        E = torch.from_numpy(x.E).to(DEV)
    y = torch.from_numpy(x.labels).to(DEV)
    return H, E, y


def mean_dloss(x: inputs.Inputs) -> np.ndarray:
    nv = max(x.n_valid, 1)
    return np.where(x.labels != x.ignore_index, 1.0 / nv, 0.0).astype(np.float32)


def random_dloss(x: inputs.Inputs, seed=0) -> np.ndarray:
    r = np.random.default_rng(seed).uniform(0.5, 1.5, size=x.N) / max(x.n_valid, 1)
    return r.astype(np.float32)


def t64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(x: inputs.Inputs, dloss: np.ndarray, eps: float, sort=False, flags=0, prefill_nan=True, bound=True):
    """Forward + backward through the C ABI; returns fp64 numpy arrays.
    bound: the forward writes the block-max table and the backward gets it
    (as the autograd wrapper does); False runs the backward without it.
    sort: both passes visit the vocabulary in cce_vocab_order's order."""
    H, E, y = to_device(x)
    loss = torch.full((x.N,), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((x.N,), float("nan"), dtype=torch.float32, device=DEV)
    tb = torch.full((B.block_max_elems(x.N, x.V),), float("nan"), dtype=torch.float32, device=DEV) \
        if bound else None
    perm = B.cce_vocab_order(H, E, y, x.ignore_index) if sort else None
    B.cce_forward(H, E, y, x.ignore_index, loss=loss, lse=lse, block_max=tb, perm=perm)
    dl = torch.from_numpy(dloss).to(DEV)
    dH = torch.full_like(H, float("nan")) if prefill_nan else None
    dE = torch.full_like(E, float("nan")) if prefill_nan else None
    stats = torch.zeros(5, dtype=torch.int64, device=DEV)
    dH, dE = B.cce_backward(H, E, y, lse, dl, eps, x.ignore_index, perm, flags, dH=dH, dE=dE, stats=stats,
                            block_max=tb)
    torch.cuda.synchronize()
    out = dict(loss=t64(loss), lse=t64(lse), dH=t64(dH), dE=t64(dE), stats=stats.cpu().numpy())
    if perm is not None:
        out["perm"] = perm.cpu().numpy()
    if tb is not None:
        out["block_max"] = tb.cpu().numpy().astype(np.float64)
    return out


_ORACLE = {}


def oracle_full(x: inputs.Inputs, dloss: np.ndarray, tag: str):
    """Full fp64 oracle (loss, lse, dH, dE) for a small case, cached per tag."""
    key = (x.name, x.seed, x.N, x.D, x.V, tag)
    if key not in _ORACLE:
        H = oracle.as_f64(x.H, x.dtype)
        E = oracle.as_f64(x.E, x.dtype)
        _ORACLE[key] = oracle.backward(H, E, x.labels, dloss.astype(np.float64), x.ignore_index)
    return _ORACLE[key]


def label_term(x: inputs.Inputs, dloss: np.ndarray):
    """Gradient of the indexed-logit term alone (the floor of the tolerance)."""
    H = oracle.as_f64(x.H, x.dtype)
    E = oracle.as_f64(x.E, x.dtype)
    valid = x.labels != x.ignore_index
    LH = np.zeros_like(H)
    LH[valid] = -dloss[valid, None] * E[x.labels[valid]]
    LE = np.zeros_like(E)
    np.add.at(LE, x.labels[valid], -dloss[valid, None] * H[valid])
    return LH, LE


def lse_tol(x):
    return 1e-5 if x.dtype == "f32" else 1e-3


def assert_rows(name, got, ref, valid, tol, lse_ref=None):
    g, r = got[valid], ref[valid]
    slack = 0.0 if lse_ref is None else 2.0 ** -20 * np.abs(lse_ref[valid])
    err = np.maximum(np.abs(g - r) - slack, 0.0) / np.maximum(np.abs(r), 1.0)
    worst = int(np.argmax(err)) if err.size else 0
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err.size == 0 or err.max() <= tol, \
        f"{name}: max rel err {err.max():.3e} > {tol:g} at valid row {worst} (gpu {g[worst]!r}, ref {r[worst]!r})"
    assert np.all(got[~valid] == 0), f"{name}: ignored rows must be exactly 0"


def frob_err(got, ref, floor):
    scale = max(np.linalg.norm(ref), np.linalg.norm(floor), 1e-300)
    return np.linalg.norm(got - ref) / scale


def assert_grad(name, got, ref, floor, tol):
    assert np.all(np.isfinite(got)), f"{name}: non-finite (unwritten?) output"
    e = frob_err(got, ref, floor)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:g}"
    return e
