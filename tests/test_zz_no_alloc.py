"""The allocation-free forward, cce_forward_noalloc (for callers that cannot
allocate: its workspace is a device array the library holds per GPU), called
through the C ABI: it gives the bits of cce_forward with a caller workspace,
loss, lse and the block-max table, on two calls in a row with the second on a
smaller problem (the array keeps the first call's contents), with and
without a vocabulary permutation."""
import numpy as np
import pytest
import torch

from linear_cross_entropy_cce_amd import binding as B
from linear_cross_entropy_cce_amd import inputs
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _run(x, sort):
    H, E, y = G.to_device(x)
    perm = B.cce_vocab_order(H, E, y, x.ignore_index) if sort else None
    n = B.block_max_elems(x.N, x.V)
    out = {}
    for kind in ("workspace", "noalloc"):
        loss = torch.full((x.N,), float("nan"), dtype=torch.float32, device=G.DEV)
        lse = torch.full((x.N,), float("nan"), dtype=torch.float32, device=G.DEV)
        tb = torch.full((n,), float("nan"), dtype=torch.float32, device=G.DEV)
        torch.cuda.synchronize()
        if kind == "workspace":
            B.cce_forward(H, E, y, x.ignore_index, loss=loss, lse=lse, block_max=tb, perm=perm)
        else:
            B.cce_forward_noalloc(H, E, y, loss, lse, x.ignore_index, block_max=tb, perm=perm)
        torch.cuda.synchronize()
        out[kind] = [t.cpu().numpy() for t in (loss, lse, tb)]
    return out


@pytest.mark.parametrize("sort", [False, True])
def test_noalloc_forward_equals_forward(sort):
    # a larger problem, then a smaller one: the second call sees the first's
    # partials in the shared array and must not be affected by them
    for x in (inputs.make_workload(5, N=3800, D=256, V=40000), inputs.make_workload(3, N=600, D=512, V=5000)):
        G.say(f"noalloc forward N={x.N} D={x.D} V={x.V} sort={sort}")
        out = _run(x, sort)
        valid = x.labels != x.ignore_index
        assert np.all(np.isfinite(out["noalloc"][1][valid]))
        for name, a, b in zip(("loss", "lse", "block_max"), out["workspace"], out["noalloc"]):
            assert np.array_equal(a, b, equal_nan=True), name


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    N, D, V = 1 << 20, 8, 64  # labels, row indices and partials need more than 16 MiB
    assert B.forward_workspace_bytes(N, D, V, B.CCE_BF16) > B.NOALLOC_SCRATCH_BYTES
    G.say("noalloc oversize")
    H = torch.zeros((N, D), dtype=torch.bfloat16, device=G.DEV)
    E = torch.zeros((V, D), dtype=torch.bfloat16, device=G.DEV)
    y = torch.zeros(N, dtype=torch.int64, device=G.DEV)
    loss = torch.full((N,), 7.0, dtype=torch.float32, device=G.DEV)
    lse = torch.full((N,), 7.0, dtype=torch.float32, device=G.DEV)
    with pytest.raises(B.CCEError) as e:
        B.cce_forward_noalloc(H, E, y, loss, lse, -100)
    assert e.value.status == B.CCE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(loss == 7.0) and torch.all(lse == 7.0)  # nothing was enqueued
