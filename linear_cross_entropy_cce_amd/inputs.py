"""Seeded synthetic inputs for the fused classifier-head + cross-entropy workloads.

This module is the one place both sides of every parity check draw their data
from: the HIP path and the fp64 oracle receive the same bits.  It holds none of
the method's arithmetic -- only random draws, the round-to-nearest-even
conversion of those draws to bfloat16 bit patterns, and the label / ignore
layout.

Workload recipes.  The pages measure real heads (Gemma 2 2B, Llama 3 8B,
Phi 3.5 Mini) during fine-tuning and pretraining runs ("Cut Your Losses in
Large-Vocabulary Language Models" summary, sections "Key results",
"Limitations" and "Experimental setup"), and a 1024-anchor x 24-position head
over a 248 320-token vocabulary ("The Defensive Edit: Chunking Cross-Entropy
Loss After an OOM Wake-Up Call", section "The OOM: A 12.2 GB Softmax Wall").
Weights, tokens and hidden states of those runs are not available, so each
workload keeps the head shape and draws the values:

  E  ~ N(0, s_E^2) per element (s_E = 0.02, or 1/sqrt(D) for the tiny case)
  H  ~ N(0, 1) per element ("flat": an early-training softmax), or
  H  = 3 sqrt(D) e_y / ||e_y|| + N(0, I)  ("peaked": a trained-like softmax,
       e_y the bf16-rounded classifier row of the token's label), or
  H  = a sqrt(D) e_y / ||e_y|| + s N(0, I) with a = 0.35, s = 2 ("partially
       peaked", workload 7): the label takes a median 80 % of the softmax
       and about 0.02 % of the other entries reach 2^-12, the sparsity the
       summary reports for trained models ("Surprising findings").  With unit
       noise no scale a gets there: the other logits' spread is too narrow
       for any of them to come within ln(2^12) of the lse.
  labels uniform over [0, V), or Zipf(1.1): P(id = r - 1) ~ r^-1.1, r = 1..V,
       or the same Zipf ranks sent through a seeded permutation of the ids
       (frequent tokens scattered over the vocabulary, as in a tokenizer
       whose ids do not follow frequency)
  exactly round(f N) rows, chosen by a seeded permutation, set to -100.

Streams: numpy PCG64 seeded by SeedSequence([seed, stream]) with stream
0 = E, 1 = labels, 2 = ignore mask, 3 = H noise, 4 = id permutation.  Values are drawn in float32
and, for bf16 workloads, rounded to nearest-even bfloat16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

IGNORE_INDEX = -100

_ROW_CHUNK_ELEMS = 1 << 25  # draw big matrices in bounded slabs


@dataclasses.dataclass(frozen=True)
class Recipe:
    name: str
    N: int
    D: int
    V: int
    dtype: str            # "f32" or "bf16"
    e_std: float | None   # None -> 1/sqrt(D)
    h_kind: str           # "normal" | "peaked"
    label_kind: str       # "uniform" | "zipf"
    ignore_frac: float
    eps: float            # default filter threshold for this workload
    sort_vocab: tuple     # vocabulary-sort settings the workload is run with
    peak_scale: float = 3.0  # a of a peaked H
    h_noise: float = 1.0     # s of a peaked H


# The five workloads, by number.  Sizes are the head shapes named above.
WORKLOADS = {
    1: Recipe("tiny-f32", 256, 128, 4096, "f32", None, "normal", "uniform", 0.10, 0.0, (False,)),
    2: Recipe("gemma2-2b-head", 8192, 2304, 256000, "bf16", 0.02, "peaked", "zipf", 0.0, 2.0 ** -12, (False,)),
    3: Recipe("llama3-8b-head", 16384, 4096, 128256, "bf16", 0.02, "normal", "zipf", 0.40, 2.0 ** -12, (False,)),
    4: Recipe("phi3.5-mini-head", 8192, 3072, 32064, "bf16", 0.02, "normal", "uniform", 0.0, 2.0 ** -12, (False,)),
    5: Recipe("large-vocab-1024x24", 24576, 2048, 248320, "bf16", 0.02, "peaked", "zipf", 0.0, 2.0 ** -12, (False, True)),
    # workload 5 with the Zipf ranks scattered over the ids: what the sort is for
    6: Recipe("large-vocab-1024x24-scattered", 24576, 2048, 248320, "bf16", 0.02, "peaked", "zipf-scattered", 0.0,
              2.0 ** -12, (False, True)),
    # the Gemma-2-2B head with a partially peaked softmax (filtering at a
    # granularity finer than the 128 x 128 block is what pays there)
    7: Recipe("gemma2-2b-head-partial", 8192, 2304, 256000, "bf16", 0.02, "peaked", "zipf", 0.0, 2.0 ** -12, (False,),
              peak_scale=0.35, h_noise=2.0),
}


@dataclasses.dataclass
class Inputs:
    """One drawn problem.  H, E are float32 arrays (f32) or uint16 bf16 bit
    patterns (bf16), row-major [N, D] and [V, D]; labels is int64 [N]."""
    name: str
    seed: int
    N: int
    D: int
    V: int
    dtype: str
    H: np.ndarray
    E: np.ndarray
    labels: np.ndarray
    eps: float
    ignore_index: int = IGNORE_INDEX

    @property
    def n_valid(self) -> int:
        return int(np.count_nonzero(self.labels != self.ignore_index))


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.
    (Inputs are finite draws; no NaN handling is needed.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 numbers they denote (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_matrix(rng, rows, cols, std, dtype):
    """Draw a [rows, cols] N(0, std^2) matrix in float32 slabs; return float32
    or bf16 bits.  The slab size does not change the drawn sequence."""
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    step = max(1, _ROW_CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = rng.standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = x if dtype == "f32" else round_to_bf16_bits(x)
    return out


def zipf_labels(rng, n, V, s=1.1):
    """P(id = r - 1) proportional to r^-s for r = 1..V, by inverse-CDF draws."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)


def make_inputs(N, D, V, dtype="bf16", e_std=0.02, h_kind="normal", label_kind="uniform",
                ignore_frac=0.0, seed=0, eps=0.0, name="custom", peak_scale=3.0, h_noise=1.0) -> Inputs:
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    std = (1.0 / math.sqrt(D)) if e_std is None else float(e_std)
    E = _normal_matrix(_rng(seed, 0), V, D, std, dtype)

    lrng = _rng(seed, 1)
    if label_kind == "uniform":
        labels = lrng.integers(0, V, size=N, dtype=np.int64)
    elif label_kind == "zipf":
        labels = zipf_labels(lrng, N, V)
    elif label_kind == "zipf-scattered":
        labels = _rng(seed, 4).permutation(V).astype(np.int64)[zipf_labels(lrng, N, V)]
    else:
        raise ValueError(f"unknown label kind {label_kind!r}")

    hrng = _rng(seed, 3)
    if h_kind == "normal":
        H = _normal_matrix(hrng, N, D, 1.0, dtype)
    elif h_kind == "peaked":
        # h_i = peak_scale * sqrt(D) * e_{y_i} / ||e_{y_i}|| + xi_i, built from
        # the classifier rows as stored (after bf16 rounding).
        Ef = E if dtype == "f32" else None
        H = np.empty((N, D), dtype=np.float32 if dtype == "f32" else np.uint16)
        step = max(1, _ROW_CHUNK_ELEMS // D)
        for r0 in range(0, N, step):
            r1 = min(N, r0 + step)
            rows = labels[r0:r1]
            ey = (Ef[rows] if Ef is not None else bf16_bits_as_f32(E[rows])).astype(np.float64)
            ey *= (peak_scale * math.sqrt(D)) / np.linalg.norm(ey, axis=1, keepdims=True)
            noise = hrng.standard_normal(size=(r1 - r0, D), dtype=np.float32)
            if h_noise != 1.0:
                noise *= np.float32(h_noise)
            x = (ey + noise).astype(np.float32)
            H[r0:r1] = x if dtype == "f32" else round_to_bf16_bits(x)
    else:
        raise ValueError(f"unknown H kind {h_kind!r}")

    n_ignore = int(round(ignore_frac * N))
    if n_ignore:
        drop = _rng(seed, 2).permutation(N)[:n_ignore]
        labels = labels.copy()
        labels[drop] = IGNORE_INDEX
    return Inputs(name, seed, N, D, V, dtype, H, E, labels, eps)


def make_workload(k: int, seed: int | None = None, N: int | None = None, D: int | None = None,
                  V: int | None = None) -> Inputs:
    """Workload k (1..7) at its full size, or with any of N, D, V overridden
    (the same recipe at a size the oracle finishes quickly)."""
    r = WORKLOADS[k]
    return make_inputs(N or r.N, D or r.D, V or r.V, dtype=r.dtype, e_std=r.e_std, h_kind=r.h_kind,
                       label_kind=r.label_kind, ignore_frac=r.ignore_frac,
                       seed=k if seed is None else seed, eps=r.eps, name=r.name, peak_scale=r.peak_scale,
                       h_noise=r.h_noise)
