"""The library enqueues kernels only (no allocation, no host synchronisation,
no memset), so a forward + backward can be captured in a HIP graph and
replayed.  Each replay, with eager work of the program in between, must give
the eager run's bits."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


# (the last case: the Gemma-2-2B head at full size, whose backward runs
# every worst-case store pass and the hot-column items)
@pytest.mark.parametrize("k,N,D,V,sort", [(2, 700, 256, 9000, False), (3, 600, 512, 20000, True),
                                          (2, None, None, None, False)])
def test_graph_replays_match_eager(k, N, D, V, sort):
    x = inputs.make_workload(k, N=N, D=D, V=V)
    G.say(f"graph capture w{k} N={x.N} D={x.D} V={x.V} sort={sort}")
    H, E, y = G.to_device(x)
    dt = B.CCE_BF16 if x.dtype == "bf16" else B.CCE_F32
    dl = torch.from_numpy(G.random_dloss(x, seed=1)).to(G.DEV)
    loss = torch.empty(x.N, dtype=torch.float32, device=G.DEV)
    lse = torch.empty_like(loss)
    dH = torch.empty_like(H)
    dE = torch.empty_like(E)
    stats = torch.zeros(7, dtype=torch.int64, device=G.DEV)
    tb = torch.empty(B.block_max_elems(x.N, x.V), dtype=torch.float32, device=G.DEV)
    perm = torch.empty(x.V, dtype=torch.int32, device=G.DEV) if sort else None
    ws_f = torch.empty(B.forward_workspace_bytes(x.N, x.D, x.V, dt), dtype=torch.uint8, device=G.DEV)
    ws_b = torch.empty(B.backward_workspace_bytes(x.N, x.D, x.V, dt), dtype=torch.uint8, device=G.DEV)
    ws_s = torch.empty(B.vocab_order_workspace_bytes(x.N, x.D, x.V, dt), dtype=torch.uint8, device=G.DEV)

    def step(stream=None):
        if sort:
            B.cce_vocab_order(H, E, y, x.ignore_index, perm=perm, ws=ws_s, stream=stream)
        B.cce_forward(H, E, y, x.ignore_index, loss=loss, lse=lse, block_max=tb, ws=ws_f, stream=stream, perm=perm)
        B.cce_backward(H, E, y, lse, dl, x.eps, x.ignore_index, perm, 0, dH=dH, dE=dE, stats=stats, ws=ws_b,
                       stream=stream, block_max=tb)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (loss, lse, dH, dE, stats)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(stream=s)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (loss, lse, dH, dE):
            t.fill_(float("nan"))  # eager work between replays: the replay must rewrite everything
        stats.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "lse", "dH", "dE", "stats"), (loss, lse, dH, dE, stats), want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
