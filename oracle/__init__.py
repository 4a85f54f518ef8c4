"""fp64 CPU oracle for the fused classifier-head + cross-entropy (CCE).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The HIP path never
imports or calls it and shares no code with it; the two meet only in the
seeded input generator.

The arithmetic of the plain definition lives in cce_oracle.c (double
precision, see its header).  This wrapper converts the stored input bits to
float64 exactly, calls the C library, and sorts vocabulary keys with a library
sort.  Three numpy functions use a library matrix product as their logit step:
lse_matmul (every row's lse at full sizes), backward_filtered (the gradient
with the block filter at a stated geometry) and composite (a two-block head).

Sources: the lit note "The loss and the mask: Cut Cross-Entropy +
FlexAttention", section "Contribution"; the paper summary "Cut Your Losses in
Large-Vocabulary Language Models", section "Approach".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcce_oracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile the C oracle with the host compiler (make)."""
    subprocess.run(["make", "-s", "-C", _HERE], check=True)
    return _LIB_PATH


def use_library(path=None):
    """Point the wrapper at another build of cce_oracle.c (the mutation tests
    load deliberately broken copies); None restores the default library."""
    global _lib, _lib_override
    _lib_override = path
    _lib = None


_lib_override = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_override
    if path is None:
        path = _LIB_PATH
        src = os.path.join(_HERE, "cce_oracle.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            build()
    lib = ctypes.CDLL(path)
    lib.cce_oracle_rows.argtypes = [_d, _d, _i64, _d, _i64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, _d, _d, _d]
    lib.cce_oracle_rows.restype = ctypes.c_int
    lib.cce_oracle_dE.argtypes = [_d, _d, _i64, _d, _d, ctypes.c_int64, _i64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, _d]
    lib.cce_oracle_dE.restype = ctypes.c_int
    lib.cce_oracle_mean_logit.argtypes = [_d, _d, _i64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, _d]
    lib.cce_oracle_mean_logit.restype = ctypes.c_int
    lib.cce_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.cce_oracle_max_threads.restype = ctypes.c_int
    ncpu = len(os.sched_getaffinity(0))
    lib.cce_oracle_set_threads(min(ncpu, 16))
    _lib = lib
    return lib


def threads() -> int:
    return _load().cce_oracle_max_threads()


def set_threads(n: int) -> None:
    _load().cce_oracle_set_threads(int(n))


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input -> exact float64 values.  bf16 inputs arrive as uint16
    bit patterns (the upper half of an IEEE float32)."""
    if dtype == "bf16":
        return (np.asarray(x).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(dtype)


def _p(a, t):
    return a.ctypes.data_as(t)


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def rows(H64, E64, labels, dloss, row_ids, ignore_index=-100, want_dH=True):
    """lse, loss (and dH rows) for the listed rows; full logit rows in fp64."""
    lib = _load()
    H64, E64 = _c64(H64), _c64(E64)
    N, D = H64.shape
    V = E64.shape[0]
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    dloss = _c64(np.zeros(N) if dloss is None else dloss)
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    n = row_ids.size
    lse = np.empty(n)
    loss = np.empty(n)
    dH = np.empty((n, D)) if want_dH else None
    rc = lib.cce_oracle_rows(_p(H64, _d), _p(E64, _d), _p(labels, _i64), _p(dloss, _d),
                             _p(row_ids, _i64), n, D, V, int(ignore_index),
                             _p(lse, _d), _p(loss, _d), _p(dH, _d) if want_dH else None)
    if rc != 0:
        raise MemoryError("oracle: cannot allocate a logit row")
    return lse, loss, dH


def forward(H64, E64, labels, ignore_index=-100):
    """Per-token loss and lse for every row (fp64)."""
    N = H64.shape[0]
    lse, loss, _ = rows(H64, E64, labels, None, np.arange(N), ignore_index, want_dH=False)
    return loss, lse


def dE_rows(H64, E64, labels, lse, dloss, vids, ignore_index=-100):
    """Rows vids of dE = sum_i g_iv h_i, given every row's lse."""
    lib = _load()
    H64, E64 = _c64(H64), _c64(E64)
    N, D = H64.shape
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    lse, dloss = _c64(lse), _c64(dloss)
    vids = np.ascontiguousarray(vids, dtype=np.int64)
    out = np.empty((vids.size, D))
    lib.cce_oracle_dE(_p(H64, _d), _p(E64, _d), _p(labels, _i64), _p(lse, _d), _p(dloss, _d), N,
                      _p(vids, _i64), vids.size, D, int(ignore_index), _p(out, _d))
    return out


def backward(H64, E64, labels, dloss, ignore_index=-100):
    """Full forward + unfiltered gradient: loss, lse, dH [N,D], dE [V,D] (fp64)."""
    N = H64.shape[0]
    V = E64.shape[0]
    lse, loss, dH = rows(H64, E64, labels, dloss, np.arange(N), ignore_index, want_dH=True)
    dE = dE_rows(H64, E64, labels, lse, dloss, np.arange(V), ignore_index)
    return loss, lse, dH, dE


def mean_logit(H64, E64, labels, ignore_index=-100):
    """key_v = mean over non-ignored rows of z_iv (fp64, from the definition)."""
    lib = _load()
    H64, E64 = _c64(H64), _c64(E64)
    N, D = H64.shape
    V = E64.shape[0]
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    key = np.empty(V)
    lib.cce_oracle_mean_logit(_p(H64, _d), _p(E64, _d), _p(labels, _i64), N, D, V,
                              int(ignore_index), _p(key, _d))
    return key


def vocab_order(keys):
    """Vocabulary permutation: descending key, ties by ascending id (a stable
    sort).  perm[k] is the original id at sorted position k."""
    keys = np.asarray(keys)
    ids = np.arange(keys.size)
    return np.lexsort((ids, -keys)).astype(np.int64)


def lse_matmul(H64, E64, labels, ignore_index=-100, row_chunk=512):
    """lse_i for every row, with a library matrix product (numpy, float64)
    as the logit step: z = H E^T in row chunks, then the definition
    lse = m + log sum exp(z - m).  Used where the full C loop would take
    minutes (full-size workloads); ignored rows get 0."""
    H64, E64 = _c64(H64), _c64(E64)
    N = H64.shape[0]
    out = np.zeros(N)
    for r0 in range(0, N, row_chunk):
        z = H64[r0:r0 + row_chunk] @ E64.T
        m = z.max(axis=1, keepdims=True)
        out[r0:r0 + row_chunk] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    out[np.asarray(labels) == ignore_index] = 0.0
    return out



def backward_filtered(H64, E64, labels, dloss, eps, block_rows=128, block_vocab=128, ignore_index=-100,
                      margin=2.0 ** -14):
    """Gradient with the block filter of the CCE paper summary "Cut Your
    Losses in Large-Vocabulary Language Models", section "Approach": the
    backward skips the blocks of the logit matrix whose softmax entries all
    fall below a threshold.  The pages fix neither the block shape nor what
    happens at a label entry; the reading taken here:
      - the logit matrix is that of the non-ignored rows, in order (ignored
        rows are dropped first), with the vocabulary in id order; blocks are
        block_rows consecutive such rows x block_vocab consecutive ids;
      - a block keeps the softmax part p of all its entries iff one entry other
        than a label entry (i, y_i) has p >= eps; eps = 0 keeps every block;
      - the gradient of the indexed-logit term (-1 at a label entry) is always
        kept, and so is the label entry's own p (the whole dloss_i (p - 1)).
    Steps, in the pages' order: full logit rows (numpy matmul, float64), lse
    by its definition, p = exp(z - lse), the per-block keep decision, then
    g = dloss (p [kept or label entry] - onehot), dH = g E, dE = g^T H.

    Several results are correct when a block's largest non-label p lies
    within a relative `margin` of eps (a float32 kernel may decide it either
    way: its p carries a relative error of about 1e-5 from float32 logits and
    lse, against the default margin of 2^-14 = 6e-5); for those blocks the sum
    of the Frobenius norms of their softmax part's contributions to dH and to
    dE is returned as an allowance.
    Returns dH [N, D], dE [V, D], kept [row blocks, vocab blocks] (bool),
    allow_dH, allow_dE (floats).  Ignored rows get dH = 0, add nothing."""
    H64, E64 = _c64(H64), _c64(E64)
    labels = np.asarray(labels, dtype=np.int64)
    dloss = np.asarray(dloss, dtype=np.float64)
    N, D = H64.shape
    V = E64.shape[0]
    rows = np.nonzero(labels != ignore_index)[0]
    n = rows.size
    dH = np.zeros((N, D))
    dE = np.zeros((V, D))
    n_rb = -(-n // block_rows)
    n_cb = -(-V // block_vocab)
    kept = np.zeros((n_rb, n_cb), dtype=bool)
    if n == 0:
        return dH, dE, kept, 0.0, 0.0
    Hv = H64[rows]
    y = labels[rows]
    z = Hv @ E64.T
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    p = np.exp(z - lse)
    is_label = np.zeros((n, V), dtype=bool)
    is_label[np.arange(n), y] = True
    allow_dH = allow_dE = 0.0
    keep_entry = is_label.copy()
    for rb in range(n_rb):
        r0, r1 = rb * block_rows, min(n, (rb + 1) * block_rows)
        for cb in range(n_cb):
            c0, c1 = cb * block_vocab, min(V, (cb + 1) * block_vocab)
            other = np.where(is_label[r0:r1, c0:c1], -np.inf, p[r0:r1, c0:c1])
            top = other.max()
            kept[rb, cb] = top >= eps if eps > 0 else top > -np.inf
            if kept[rb, cb]:
                keep_entry[r0:r1, c0:c1] = True
            if eps > 0 and abs(top - eps) <= margin * eps:
                soft = dloss[rows[r0:r1], None] * np.where(is_label[r0:r1, c0:c1], 0.0, p[r0:r1, c0:c1])
                allow_dH += np.linalg.norm(soft @ E64[c0:c1])
                allow_dE += np.linalg.norm(soft.T @ Hv[r0:r1])
    g = dloss[rows, None] * (np.where(keep_entry, p, 0.0) - is_label)
    dH[rows] = g @ E64
    dE[:] = g.T @ Hv
    return dH, dE, kept, allow_dH, allow_dE


def composite(H64, E0, E1, off1, labels, dloss, ignore_index=-100):
    """Composite head (the lit note "The loss and the mask: Cut Cross-Entropy +
    FlexAttention", section "What transfers to us"): ids [0, V0) are rows of
    E0, ids [off1, off1 + V1) rows of E1, the ids between have no row.  The
    log-sum-exp is composed over the two blocks with logaddexp (the gap adds
    exp(-inf) = 0), the label logit comes from the block that holds the label,
    and the gradient of each block uses the composed lse.
    Returns loss, lse [N], dH [N, D], dE0 [V0, D], dE1 [V1, D] (fp64); ignored
    rows get 0 and add nothing.  Matrix products are numpy's (float64)."""
    H64, E0, E1 = _c64(H64), _c64(E0), _c64(E1)
    labels = np.asarray(labels, dtype=np.int64)
    dloss = np.asarray(dloss, dtype=np.float64)
    N = H64.shape[0]
    V0, V1 = E0.shape[0], E1.shape[0]
    if off1 < V0:
        raise ValueError("the second block must start at or after the end of the first")
    valid = labels != ignore_index
    in0 = valid & (labels >= 0) & (labels < V0)
    in1 = valid & (labels >= off1) & (labels < off1 + V1)
    if np.any(valid & ~in0 & ~in1):
        raise ValueError("a label outside both blocks (in the gap or past the end)")
    Z0 = H64 @ E0.T
    Z1 = H64 @ E1.T
    m0 = Z0.max(axis=1)
    m1 = Z1.max(axis=1)
    lse0 = m0 + np.log(np.exp(Z0 - m0[:, None]).sum(axis=1))
    lse1 = m1 + np.log(np.exp(Z1 - m1[:, None]).sum(axis=1))
    lse = np.logaddexp(lse0, lse1)
    zy = np.zeros(N)
    rows = np.arange(N)
    zy[in0] = Z0[rows[in0], labels[in0]]
    zy[in1] = Z1[rows[in1], labels[in1] - off1]
    loss = np.where(valid, lse - zy, 0.0)
    lse = np.where(valid, lse, 0.0)
    w = np.where(valid, dloss, 0.0)
    G0 = w[:, None] * np.exp(Z0 - lse[:, None])
    G1 = w[:, None] * np.exp(Z1 - lse[:, None])
    G0[~valid] = 0.0
    G1[~valid] = 0.0
    G0[rows[in0], labels[in0]] -= w[in0]
    G1[rows[in1], labels[in1] - off1] -= w[in1]
    dH = G0 @ E0 + G1 @ E1
    dE0 = G0.T @ H64
    dE1 = G1.T @ H64
    return loss, lse, dH, dE0, dE1
