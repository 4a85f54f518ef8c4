"""The C ABI on the host: the library loads, exports every entry point the
header declares, sizes its workspace without an N x V term, and rejects bad
arguments before enqueuing anything.  Nothing here runs a kernel: every
argument error is detected on the host, and pointers passed are never
dereferenced (they are fake, suitably aligned addresses)."""
import ctypes
import os
import re

import pytest

from linear_cross_entropy_cce_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # aligned, never dereferenced


def _header_functions():
    text = open(os.path.join(ROOT, "include", "cce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cce_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = B.lib()
    declared = _header_functions()
    assert declared == sorted(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_block():
    assert B.version() >= 10000
    r, v = B.filter_block()
    assert r > 0 and v > 0 and r % 32 == 0 and v % 32 == 0


def test_status_strings():
    for s in range(8):
        assert len(B.status_string(s)) > 0
    assert B.status_string(99) == "unknown status"


@pytest.mark.parametrize("dt", [B.CCE_F32, B.CCE_BF16])
def test_workspace_has_no_per_logit_term(dt):
    # Doubling N and V together at most roughly doubles the workspace: the
    # buffers are O((N + V) D) plus byte-sized maps, one entry per 128 x 128
    # logit block (6 bytes) and per 256 x 256 tile (5 bytes).
    f = B.backward_workspace_bytes
    D = 2048
    a = f(8192, D, 256000, dt)
    b = f(16384, D, 512000, dt)
    assert a > 0 and b < 2.2 * a
    g = B.forward_workspace_bytes
    assert g(16384, D, 512000, dt) < 2.2 * g(8192, D, 256000, dt)
    # per vocabulary entry at fixed N: inverse permutation (4 bytes), the
    # block maps (N / 16384 blocks x 8 bytes: label flag, status, store slot,
    # sub-tile mask), the tile maps (N / 65536 tiles x 5 bytes) and the plan's
    # per-tile scratch; nothing per logit
    N = 8192
    per_v = (f(N, D, 512000, dt) - f(N, D, 256000, dt)) / 256000
    assert per_v <= 4 + 8 * N / 16384 + 5 * N / 65536 + 1
    # per row at fixed V: the fp32 dH accumulator, H^T and the block store
    # (as many blocks as a dense slice of 16384 vocabulary columns, two
    # layouts), the row index, label logit and mapped label (4 + 4 + 8 bytes),
    # the label positions and hot-block entry lists (4 + 4 bytes) and the hot
    # blocks' per-slice row counts (at most N / 513 hot blocks x 64 slices x
    # 512 bytes: 64 bytes per row)
    elem = 4 if dt == B.CCE_F32 else 2
    V = 256000
    per_n = (f(2 * N, D, V, dt) - f(N, D, V, dt)) / N
    assert per_n <= 4 * D + elem * D + 2 * elem * 16384 + 8 * V / 16384 + 5 * V / 65536 + 16 + 16 + 8 + 64


def test_workspace_invalid_sizes_return_zero():
    vmax = (1 << 31) - (1 << 16)
    for args in [(0, 64, 10), (10, 0, 10), (10, 12, 10), (10, 64, 0), (10, 64, 1 << 31), (10, 64, 10),
                 (10, 64, vmax), (10, 64, vmax + 1), (vmax, 64, 10), (vmax + 1, 64, 10)]:
        n, d, v = args
        want_zero = not (1 <= n <= vmax and 1 <= v <= vmax and d >= 8 and d % 8 == 0)
        assert (B.forward_workspace_bytes(n, d, v, 1) == 0) == want_zero
    assert B.forward_workspace_bytes(10, 64, 10, 7) == 0


def _fwd(**kw):
    a = dict(H=FAKE, E=FAKE, labels=FAKE, N=16, D=64, V=100, dt=B.CCE_BF16, ign=-100, perm=None, loss=FAKE,
             lse=FAKE, tb=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.lib().cce_forward(a["H"], a["E"], a["labels"], a["N"], a["D"], a["V"], a["dt"], a["ign"], a["perm"],
                               a["loss"], a["lse"], a["tb"], a["ws"], a["ws_bytes"], a["stream"])


def _bwd(**kw):
    a = dict(H=FAKE, E=FAKE, labels=FAKE, lse=FAKE, dloss=FAKE, tb=None, N=16, D=64, V=100, dt=B.CCE_BF16,
             ign=-100, eps=0.0, perm=None, flags=0, dH=FAKE, dE=FAKE, stats=None, ws=FAKE, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return B.lib().cce_backward(a["H"], a["E"], a["labels"], a["lse"], a["dloss"], a["tb"], a["N"], a["D"], a["V"],
                                a["dt"], a["ign"], a["eps"], a["perm"], a["flags"], a["dH"], a["dE"], a["stats"],
                                a["ws"], a["ws_bytes"], a["stream"])


def _vord(**kw):
    a = dict(H=FAKE, E=FAKE, labels=FAKE, N=16, D=64, V=100, dt=B.CCE_BF16, ign=-100, perm=FAKE, keys=None,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.lib().cce_vocab_order(a["H"], a["E"], a["labels"], a["N"], a["D"], a["V"], a["dt"], a["ign"],
                                   a["perm"], a["keys"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("call", [_fwd, _bwd, _vord])
def test_argument_errors_before_launch(call):
    assert call(H=None) == B.CCE_ERR_NULL
    assert call(E=None) == B.CCE_ERR_NULL
    assert call(labels=None) == B.CCE_ERR_NULL
    assert call(ws=None) == B.CCE_ERR_NULL
    assert call(N=0) == B.CCE_ERR_SHAPE
    assert call(V=0) == B.CCE_ERR_SHAPE
    assert call(D=12) == B.CCE_ERR_SHAPE
    assert call(D=0) == B.CCE_ERR_SHAPE
    assert call(V=1 << 31) == B.CCE_ERR_SHAPE
    assert call(V=(1 << 31) - (1 << 16) + 1) == B.CCE_ERR_SHAPE  # a tile's positions must stay 32-bit
    assert call(N=(1 << 31) - (1 << 16) + 1) == B.CCE_ERR_SHAPE
    assert call(dt=5) == B.CCE_ERR_DTYPE
    assert call(H=FAKE + 8) == B.CCE_ERR_ALIGN
    assert call(E=FAKE + 4) == B.CCE_ERR_ALIGN
    assert call(ws=FAKE + 2) == B.CCE_ERR_ALIGN
    assert call(ws_bytes=16) == B.CCE_ERR_WORKSPACE


def test_forward_specific_errors():
    assert _fwd(loss=None) == B.CCE_ERR_NULL
    assert _fwd(lse=None) == B.CCE_ERR_NULL
    assert _fwd(lse=FAKE + 2) == B.CCE_ERR_ALIGN
    assert _fwd(tb=FAKE + 2) == B.CCE_ERR_ALIGN
    assert _fwd(perm=FAKE + 2) == B.CCE_ERR_ALIGN
    need = B.forward_workspace_bytes(16, 64, 100, B.CCE_BF16)
    assert _fwd(ws_bytes=need - 1) == B.CCE_ERR_WORKSPACE


def test_backward_specific_errors():
    assert _bwd(dH=None) == B.CCE_ERR_NULL
    assert _bwd(dE=None) == B.CCE_ERR_NULL
    assert _bwd(lse=None) == B.CCE_ERR_NULL
    assert _bwd(dloss=None) == B.CCE_ERR_NULL
    assert _bwd(eps=-1.0) == B.CCE_ERR_ARG
    assert _bwd(eps=float("nan")) == B.CCE_ERR_ARG
    assert _bwd(eps=float("inf")) == B.CCE_ERR_ARG
    assert _bwd(flags=16) == B.CCE_ERR_ARG  # no such flag
    assert _bwd(flags=B.CCE_BWD_FINE_FILTER | B.CCE_BWD_FULL_DE) == B.CCE_ERR_ARG  # not combined
    assert _bwd(dE=FAKE + 8) == B.CCE_ERR_ALIGN
    assert _bwd(perm=FAKE + 2) == B.CCE_ERR_ALIGN
    assert _bwd(stats=FAKE + 4) == B.CCE_ERR_ALIGN
    assert _bwd(tb=FAKE + 2) == B.CCE_ERR_ALIGN
    need = B.backward_workspace_bytes(16, 64, 100, B.CCE_BF16)
    assert _bwd(ws_bytes=need - 1) == B.CCE_ERR_WORKSPACE


def test_block_max_elems():
    # one entry per 128 x 128 logit block, over whole 256 x 256 tiles, then one
    # label logit per row; 0 on invalid sizes
    assert B.block_max_elems(1, 1) == 4 + 1
    assert B.block_max_elems(256, 256) == 4 + 256
    assert B.block_max_elems(257, 256) == 8 + 257
    assert B.block_max_elems(8192, 256000) == 64 * 2000 + 8192
    assert B.block_max_elems(24576, 248320) == 192 * 1940 + 24576
    assert B.block_max_elems(0, 10) == 0
    assert B.block_max_elems(10, 0) == 0


def test_check_labels_errors():
    L = B.lib()
    assert L.cce_check_labels(None, 10, 10, -100, FAKE, None) == B.CCE_ERR_NULL
    assert L.cce_check_labels(FAKE, 0, 10, -100, FAKE, None) == B.CCE_ERR_SHAPE
    assert L.cce_check_labels(FAKE + 4, 10, 10, -100, FAKE, None) == B.CCE_ERR_ALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="libcce.so not found"):
        B.lib()


def _fwd_c(**kw):
    a = dict(H=FAKE, E0=FAKE, V0=60, E1=FAKE + 4096, V1=40, off1=70, labels=FAKE, N=16, D=64, dt=B.CCE_BF16,
             ign=-100, perm=None, loss=FAKE, lse=FAKE, tb=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.lib().cce_forward_composite(a["H"], a["E0"], a["V0"], a["E1"], a["V1"], a["off1"], a["labels"], a["N"],
                                         a["D"], a["dt"], a["ign"], a["perm"], a["loss"], a["lse"], a["tb"], a["ws"],
                                         a["ws_bytes"], a["stream"])


def _bwd_c(**kw):
    a = dict(H=FAKE, E0=FAKE, V0=60, E1=FAKE + 4096, V1=40, off1=70, labels=FAKE, lse=FAKE, dloss=FAKE, tb=None,
             N=16, D=64, dt=B.CCE_BF16, ign=-100, eps=0.0, perm=None, flags=0, dH=FAKE, dE0=FAKE, dE1=FAKE + 8192,
             stats=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return B.lib().cce_backward_composite(a["H"], a["E0"], a["V0"], a["E1"], a["V1"], a["off1"], a["labels"],
                                          a["lse"], a["dloss"], a["tb"], a["N"], a["D"], a["dt"], a["ign"], a["eps"],
                                          a["perm"], a["flags"], a["dH"], a["dE0"], a["dE1"], a["stats"], a["ws"],
                                          a["ws_bytes"], a["stream"])


def test_composite_argument_errors():
    for f in (_fwd_c, _bwd_c):
        assert f(E1=None) == B.CCE_ERR_NULL
        assert f(V0=0) == B.CCE_ERR_SHAPE
        assert f(V1=0) == B.CCE_ERR_SHAPE
        assert f(off1=59) == B.CCE_ERR_SHAPE          # the second block may not overlap the first
        assert f(V0=1 << 30, V1=1 << 30, off1=1 << 30) == B.CCE_ERR_SHAPE  # V0 + V1 >= 2^31
        assert f(E1=FAKE + 8) == B.CCE_ERR_ALIGN
        assert f(dt=5) == B.CCE_ERR_DTYPE
        # the workspace query takes V = V0 + V1
        need = B.backward_workspace_bytes(16, 64, 100, B.CCE_BF16) if f is _bwd_c else \
            B.forward_workspace_bytes(16, 64, 100, B.CCE_BF16)
        assert f(ws_bytes=need - 1) == B.CCE_ERR_WORKSPACE
    assert _bwd_c(dE1=None) == B.CCE_ERR_NULL
    assert _bwd_c(dE1=FAKE + 8) == B.CCE_ERR_ALIGN
    assert _bwd_c(eps=-1.0) == B.CCE_ERR_ARG
    L = B.lib()
    assert L.cce_vocab_order_composite(FAKE, FAKE, 60, None, 40, FAKE, 16, 64, B.CCE_BF16, -100, FAKE, None, FAKE,
                                       1 << 40, None) == B.CCE_ERR_NULL
    assert L.cce_vocab_order_composite(FAKE, FAKE, 0, FAKE, 40, FAKE, 16, 64, B.CCE_BF16, -100, FAKE, None, FAKE,
                                       1 << 40, None) == B.CCE_ERR_SHAPE


def test_noalloc_forward_argument_errors():
    # checked on the host before the device is touched
    L = B.lib()
    def call(H=FAKE, E=FAKE, y=FAKE, N=16, D=64, V=100, dt=B.CCE_BF16, loss=FAKE, lse=FAKE):
        return L.cce_forward_noalloc(H, E, y, N, D, V, dt, -100, None, loss, lse, None, None)
    assert call(H=None) == B.CCE_ERR_NULL
    assert call(loss=None) == B.CCE_ERR_NULL
    assert call(dt=9) == B.CCE_ERR_DTYPE
    assert call(D=12) == B.CCE_ERR_SHAPE
    assert call(E=FAKE + 8) == B.CCE_ERR_ALIGN
    # beyond the 16 MiB scratch: a million tokens, or four million vocabulary entries
    assert B.forward_workspace_bytes(1 << 20, 64, 100, B.CCE_BF16) > B.NOALLOC_SCRATCH_BYTES
    assert call(N=1 << 20) == B.CCE_ERR_WORKSPACE
    assert call(V=1 << 22) == B.CCE_ERR_WORKSPACE
    # the workloads' shapes fit
    for N, D, V in ((8192, 2304, 256000), (16384, 4096, 128256), (24576, 2048, 248320)):
        assert B.forward_workspace_bytes(N, D, V, B.CCE_BF16) <= B.NOALLOC_SCRATCH_BYTES
