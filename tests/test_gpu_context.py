"""PyTorch's own cross-entropy on materialised logits and in row chunks
(bench.py --torch-context), the baseline technique of "The Defensive Edit:
Chunking Cross-Entropy Loss After an OOM Wake-Up Call" (sections "The OOM: A
12.2 GB Softmax Wall" and the chunked-computation option): its mean loss
matches the fp64 oracle, chunking lowers its peak memory, and the
materialised form takes more extra device memory than this path's whole
workspace (forward + backward + block-max table)."""
import os
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_torch_context_small():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    x = inputs.make_workload(3, N=2048, D=512, V=32000)  # flat, 40 % ignored rows
    G.say(f"torch context N={x.N} D={x.D} V={x.V}")
    H, E, y = G.to_device(x)
    ctx = bench.torch_context(H, E, y, x.ignore_index, reps=1, chunk=512)
    loss, _ = oracle.forward(oracle.as_f64(x.H, x.dtype), oracle.as_f64(x.E, x.dtype), x.labels, x.ignore_index)
    want = loss[x.labels != x.ignore_index].mean()
    mat, chk = ctx["materialised"], ctx["chunked_512_rows"]
    for name, c in (("materialised", mat), ("chunked", chk)):
        # bf16 logits (8 significant bits) upcast to fp32: a few 1e-4 of the mean loss
        assert abs(c["mean_loss"] - want) <= 1e-3 * max(abs(want), 1.0), (name, c["mean_loss"], want)
        assert c["ms_per_step"] > 0
    assert chk["extra_memory_GB"] < mat["extra_memory_GB"]
    dt = B.CCE_BF16
    ours = (B.forward_workspace_bytes(x.N, x.D, x.V, dt) + B.backward_workspace_bytes(x.N, x.D, x.V, dt)
            + 4 * B.block_max_elems(x.N, x.V)) / 1e9
    logits = x.N * x.V * 2 / 1e9
    assert mat["extra_memory_GB"] > max(ours, logits), (mat, ours, logits)
