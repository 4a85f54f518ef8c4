"""Calls on caller-given streams.  Every entry point enqueues all of its work on
the stream it is handed, and the library keeps no state between calls (each
call brings its own workspace).  So two problems enqueued at once on two
streams, their kernels free to overlap, give the same bits as the same problems
run one after the other on the default stream; and so does one problem run on
two streams at once with separate outputs and workspaces."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu

KEYS = ("loss", "lse", "dH", "dE", "stats", "block_max")


def _enqueue(x, dl_np, eps, sort, stream):
    """Forward + backward of one problem, every allocation, copy and kernel on
    `stream`; returns the device outputs (read after a device synchronize)."""
    with torch.cuda.stream(stream):
        H, E, y = G.to_device(x)
        loss = torch.full((x.N,), float("nan"), dtype=torch.float32, device=G.DEV)
        lse = torch.full((x.N,), float("nan"), dtype=torch.float32, device=G.DEV)
        tb = torch.full((B.block_max_elems(x.N, x.V),), float("nan"), dtype=torch.float32, device=G.DEV)
        perm = B.cce_vocab_order(H, E, y, x.ignore_index, stream=stream) if sort else None
        B.cce_forward(H, E, y, x.ignore_index, loss=loss, lse=lse, block_max=tb, perm=perm, stream=stream)
        dl = torch.from_numpy(dl_np).to(G.DEV)
        dH = torch.full_like(H, float("nan"))
        dE = torch.full_like(E, float("nan"))
        stats = torch.zeros(7, dtype=torch.int64, device=G.DEV)
        B.cce_backward(H, E, y, lse, dl, eps, x.ignore_index, perm, 0, dH=dH, dE=dE, stats=stats,
                       block_max=tb, stream=stream)
    return dict(loss=loss, lse=lse, dH=dH, dE=dE, stats=stats, block_max=tb)


def _host(out):
    return {k: (v.cpu().numpy() if k == "stats" else G.t64(v)) for k, v in out.items()}


CASES = {
    "peaked": (2, dict(N=1100, D=512, V=20000), False),
    "flat-sorted": (3, dict(N=900, D=256, V=9000), True),
}


def test_two_problems_on_two_streams():
    probs = []
    for name, (k, shape, sort) in CASES.items():
        x = inputs.make_workload(k, **shape)
        probs.append((name, x, G.random_dloss(x, seed=11), inputs.WORKLOADS[k].eps, sort))
    G.say("streams: sequential on the default stream")
    ref = [G.run_gpu(x, dl, eps=eps, sort=sort) for _, x, dl, eps, sort in probs]
    G.say("streams: both problems enqueued at once on two streams")
    streams = [torch.cuda.Stream() for _ in probs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [_enqueue(x, dl, eps, sort, s) for (_, x, dl, eps, sort), s in zip(probs, streams)]
    torch.cuda.synchronize()
    for (name, *_), r, o in zip(probs, ref, outs):
        got = _host(o)
        for key in KEYS:
            assert np.array_equal(got[key], r[key], equal_nan=True), f"{name}: {key}"


def test_one_problem_twice_at_once():
    x = inputs.make_workload(5, N=700, D=256, V=12000)
    dl = G.random_dloss(x, seed=3)
    eps = inputs.WORKLOADS[5].eps
    G.say("streams: one problem on two streams at once")
    ref = G.run_gpu(x, dl, eps=eps, sort=True)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [_enqueue(x, dl, eps, True, s) for s in streams]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        got = _host(o)
        for key in KEYS:
            assert np.array_equal(got[key], ref[key], equal_nan=True), f"stream {i}: {key}"
