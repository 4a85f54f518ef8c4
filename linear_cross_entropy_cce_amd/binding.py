"""ctypes binding of libcce.so, with the C ABI's names (include/cce.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the ABI.  PyTorch supplies device memory (outputs and
workspace) and the stream.  Tensors a call allocates (default outputs and the
workspace) are allocated while the call's stream is current, so PyTorch's
caching allocator hands their memory to other work only in that stream's
order.  If the library is missing or cannot be loaded, every call raises:
there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcce.so")

CCE_OK = 0
CCE_ERR_NULL = 1
CCE_ERR_SHAPE = 2
CCE_ERR_DTYPE = 3
CCE_ERR_ALIGN = 4
CCE_ERR_WORKSPACE = 5
CCE_ERR_HIP = 6
CCE_ERR_ARG = 7

CCE_F32 = 0
CCE_BF16 = 1

CCE_BWD_NO_KAHAN = 1
CCE_BWD_FULL_DE = 2
CCE_BWD_DEBUG_STORE_LIMIT = 4
CCE_BWD_FINE_FILTER = 8
FINE_SUBTILE = (32, 32)  # (tokens, vocabulary entries) of a sub-tile of CCE_BWD_FINE_FILTER

STATS_LEN = 7  # entries of the backward's stats buffer (include/cce.h)

# Every entry point include/cce.h declares.
EXPORTS = (
    "cce_status_string", "cce_version", "cce_filter_block",
    "cce_forward_workspace_bytes", "cce_backward_workspace_bytes", "cce_vocab_order_workspace_bytes",
    "cce_block_max_elems", "cce_forward", "cce_vocab_order", "cce_backward", "cce_check_labels",
    "cce_forward_composite", "cce_vocab_order_composite", "cce_backward_composite", "cce_forward_noalloc",
)

NOALLOC_SCRATCH_BYTES = 16 << 20  # CCE_NOALLOC_SCRATCH_BYTES


class CCEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load libcce.so (built in-tree by linear_cross_entropy_cce_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcce.so not found at {LIB_PATH}; build it with "
                           "`python -m linear_cross_entropy_cce_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.cce_status_string.argtypes = [ctypes.c_int]
    L.cce_status_string.restype = ctypes.c_char_p
    L.cce_version.restype = ctypes.c_int
    L.cce_filter_block.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.cce_filter_block.restype = None
    for f in ("cce_forward_workspace_bytes", "cce_backward_workspace_bytes", "cce_vocab_order_workspace_bytes"):
        getattr(L, f).argtypes = [_i64, _i64, _i64, ctypes.c_int]
        getattr(L, f).restype = ctypes.c_size_t
    L.cce_block_max_elems.argtypes = [_i64, _i64]
    L.cce_block_max_elems.restype = ctypes.c_size_t
    L.cce_forward.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _i64, _vp, _vp, _vp, _vp, _vp,
                              ctypes.c_size_t, _vp]
    L.cce_forward.restype = ctypes.c_int
    L.cce_vocab_order.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _i64, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
    L.cce_vocab_order.restype = ctypes.c_int
    L.cce_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _i64, ctypes.c_float,
                               _vp, ctypes.c_uint, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.cce_backward.restype = ctypes.c_int
    L.cce_forward_composite.argtypes = [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, ctypes.c_int, _i64, _vp,
                                        _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.cce_forward_composite.restype = ctypes.c_int
    L.cce_vocab_order_composite.argtypes = [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _i64, ctypes.c_int, _i64, _vp,
                                            _vp, _vp, ctypes.c_size_t, _vp]
    L.cce_vocab_order_composite.restype = ctypes.c_int
    L.cce_backward_composite.argtypes = [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                                         ctypes.c_int, _i64, ctypes.c_float, _vp, ctypes.c_uint, _vp, _vp, _vp, _vp,
                                         _vp, ctypes.c_size_t, _vp]
    L.cce_backward_composite.restype = ctypes.c_int
    L.cce_forward_noalloc.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _i64, _vp, _vp, _vp, _vp, _vp]
    L.cce_forward_noalloc.restype = ctypes.c_int
    L.cce_check_labels.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp]
    L.cce_check_labels.restype = ctypes.c_int
    _lib = L
    return L


def status_string(s: int) -> str:
    return lib().cce_status_string(int(s)).decode()


def _check(fn, s):
    if s != CCE_OK:
        raise CCEError(fn, s, status_string(s))


def version() -> int:
    return lib().cce_version()


def filter_block() -> tuple[int, int]:
    """(rows, vocabulary entries) of one gradient-filter block."""
    r, v = ctypes.c_int(), ctypes.c_int()
    lib().cce_filter_block(ctypes.byref(r), ctypes.byref(v))
    return r.value, v.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CCE_BF16
    if t.dtype == torch.float32:
        return CCE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def forward_workspace_bytes(N, D, V, dtype_code) -> int:
    return lib().cce_forward_workspace_bytes(N, D, V, dtype_code)


def backward_workspace_bytes(N, D, V, dtype_code) -> int:
    return lib().cce_backward_workspace_bytes(N, D, V, dtype_code)


def vocab_order_workspace_bytes(N, D, V, dtype_code) -> int:
    return lib().cce_vocab_order_workspace_bytes(N, D, V, dtype_code)


def block_max_elems(N, V) -> int:
    """fp32 entries of the block-max table (one per 128 x 128 logit block)."""
    return lib().cce_block_max_elems(N, V)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the call's allocations are made: the call's stream."""
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check_rowvec(name, t, N, device):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.float32 or t.dim() != 1 or t.numel() != N or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 [{N}] tensor on {device}")


def _check_stats(stats):
    import torch
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < STATS_LEN or not stats.is_contiguous()):
        raise ValueError(f"stats must be contiguous int64 with at least {STATS_LEN} entries")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _workspace(nbytes, device, ws):
    import torch
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _shapes(H, E, labels):
    if H.dim() != 2 or E.dim() != 2 or H.shape[1] != E.shape[1]:
        raise ValueError(f"H must be [N, D] and E [V, D]; got {tuple(H.shape)} and {tuple(E.shape)}")
    if H.dtype != E.dtype:
        raise TypeError("H and E must share one dtype")
    if labels.dim() != 1 or labels.shape[0] != H.shape[0]:
        raise ValueError("labels must be [N]")
    for name, t in (("H", H), ("E", E), ("labels", labels)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    import torch
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    return H.shape[0], H.shape[1], E.shape[0]


def _check_perm(perm, V):
    import torch
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != V or not perm.is_contiguous()):
        raise ValueError(f"perm must be contiguous int32 with {V} entries")


def cce_forward(H, E, labels, ignore_index=-100, loss=None, lse=None, block_max=None, ws=None, stream=None,
                perm=None):
    """loss, lse (fp32 [N]) of the fused head + cross-entropy.  block_max:
    None, or an fp32 tensor of block_max_elems(N, V) entries to receive the
    largest non-label logit of every 128 x 128 block of the logits and the label
    logit of every row (for cce_backward).
    perm: None, or the int32 [V] vocabulary order to visit (the table is then
    in that order, for a cce_backward given the same perm)."""
    import torch
    N, D, V = _shapes(H, E, labels)
    dt = _dtype_code(H)
    _check_perm(perm, V)
    with _on(stream):
        loss = torch.empty(N, dtype=torch.float32, device=H.device) if loss is None else loss
        lse = torch.empty(N, dtype=torch.float32, device=H.device) if lse is None else lse
        ws = _workspace(forward_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_rowvec("loss", loss, N, H.device)
    _check_rowvec("lse", lse, N, H.device)
    if block_max is not None and (block_max.dtype != torch.float32 or
                                  block_max.numel() < block_max_elems(N, V) or not block_max.is_contiguous()):
        raise ValueError(f"block_max must be contiguous fp32 with at least {block_max_elems(N, V)} entries")
    s = lib().cce_forward(_ptr(H), _ptr(E), _ptr(labels), N, D, V, dt, int(ignore_index), _ptr(perm), _ptr(loss),
                          _ptr(lse), _ptr(block_max), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_forward", s)
    return loss, lse


def cce_forward_noalloc(H, E, labels, loss, lse, ignore_index=-100, block_max=None, stream=None, perm=None):
    """cce_forward with the library's own device scratch instead of a
    workspace: the C entry point allocates nothing, so the caller passes the
    outputs (fp32 [N] loss and lse)."""
    import torch
    N, D, V = _shapes(H, E, labels)
    dt = _dtype_code(H)
    _check_perm(perm, V)
    _check_rowvec("loss", loss, N, H.device)
    _check_rowvec("lse", lse, N, H.device)
    if block_max is not None and (block_max.dtype != torch.float32 or
                                  block_max.numel() < block_max_elems(N, V) or not block_max.is_contiguous()):
        raise ValueError(f"block_max must be contiguous fp32 with at least {block_max_elems(N, V)} entries")
    s = lib().cce_forward_noalloc(_ptr(H), _ptr(E), _ptr(labels), N, D, V, dt, int(ignore_index), _ptr(perm),
                                  _ptr(loss), _ptr(lse), _ptr(block_max), _stream(stream))
    _check("cce_forward_noalloc", s)
    return loss, lse


def cce_vocab_order(H, E, labels, ignore_index=-100, perm=None, keys=None, want_keys=False, ws=None, stream=None):
    """perm (int32 [V]): vocabulary ids by descending mean logit (stable)."""
    import torch
    N, D, V = _shapes(H, E, labels)
    dt = _dtype_code(H)
    with _on(stream):
        perm = torch.empty(V, dtype=torch.int32, device=H.device) if perm is None else perm
        if want_keys and keys is None:
            keys = torch.empty(V, dtype=torch.float32, device=H.device)
        ws = _workspace(vocab_order_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_perm(perm, V)
    if keys is not None:
        _check_rowvec("keys", keys, V, H.device)
    s = lib().cce_vocab_order(_ptr(H), _ptr(E), _ptr(labels), N, D, V, dt, int(ignore_index), _ptr(perm),
                              _ptr(keys), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_vocab_order", s)
    return (perm, keys) if want_keys else perm


def cce_backward(H, E, labels, lse, dloss, filter_eps=2.0 ** -12, ignore_index=-100, perm=None, flags=0,
                 dH=None, dE=None, stats=None, ws=None, stream=None, block_max=None):
    """dH [N, D], dE [V, D] (input dtype) of sum_i dloss_i loss_i.  stats:
    None or int64 [7] (see include/cce.h); block_max: None or the table
    cce_forward wrote for the same H, E, labels and perm."""
    import torch
    N, D, V = _shapes(H, E, labels)
    dt = _dtype_code(H)
    _check_perm(perm, V)
    _check_rowvec("lse", lse, N, H.device)
    _check_rowvec("dloss", dloss, N, H.device)
    _check_stats(stats)
    if block_max is not None and (block_max.dtype != torch.float32 or block_max.numel() < block_max_elems(N, V)
                                  or not block_max.is_contiguous()):
        raise ValueError(f"block_max must be contiguous fp32 with at least {block_max_elems(N, V)} entries")
    with _on(stream):
        dH = torch.empty_like(H) if dH is None else dH
        dE = torch.empty_like(E) if dE is None else dE
        ws = _workspace(backward_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_grad("dH", dH, H)
    _check_grad("dE", dE, E)
    s = lib().cce_backward(_ptr(H), _ptr(E), _ptr(labels), _ptr(lse), _ptr(dloss), _ptr(block_max), N, D, V, dt,
                           int(ignore_index),
                           float(filter_eps), _ptr(perm), int(flags), _ptr(dH), _ptr(dE), _ptr(stats), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_backward", s)
    return dH, dE


def _check_grad(name, g, like):
    if g.shape != like.shape or g.dtype != like.dtype or not g.is_contiguous() or g.device != like.device:
        raise ValueError(f"{name} must be a contiguous {like.dtype} {tuple(like.shape)} tensor on {like.device}")


def _composite_shapes(H, E0, E1, labels):
    N, D, V0 = _shapes(H, E0, labels)
    _, _, V1 = _shapes(H, E1, labels)
    return N, D, V0, V1


def cce_forward_composite(H, E0, E1, off1, labels, ignore_index=-100, loss=None, lse=None, block_max=None, ws=None,
                          stream=None, perm=None):
    """loss, lse (fp32 [N]) of a composite head: ids [0, V0) are rows of E0,
    ids [off1, off1 + V1) rows of E1, the ids between them have no row.
    block_max / perm are over the V0 + V1 rows (E0's, then E1's)."""
    import torch
    N, D, V0, V1 = _composite_shapes(H, E0, E1, labels)
    V = V0 + V1
    dt = _dtype_code(H)
    _check_perm(perm, V)
    with _on(stream):
        loss = torch.empty(N, dtype=torch.float32, device=H.device) if loss is None else loss
        lse = torch.empty(N, dtype=torch.float32, device=H.device) if lse is None else lse
        ws = _workspace(forward_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_rowvec("loss", loss, N, H.device)
    _check_rowvec("lse", lse, N, H.device)
    if block_max is not None and (block_max.dtype != torch.float32 or
                                  block_max.numel() < block_max_elems(N, V) or not block_max.is_contiguous()):
        raise ValueError(f"block_max must be contiguous fp32 with at least {block_max_elems(N, V)} entries")
    s = lib().cce_forward_composite(_ptr(H), _ptr(E0), V0, _ptr(E1), V1, int(off1), _ptr(labels), N, D, dt,
                                    int(ignore_index), _ptr(perm), _ptr(loss), _ptr(lse), _ptr(block_max), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_forward_composite", s)
    return loss, lse


def cce_vocab_order_composite(H, E0, E1, labels, ignore_index=-100, perm=None, keys=None, want_keys=False, ws=None,
                              stream=None):
    """perm (int32 [V0 + V1]) over E0's rows then E1's, by descending mean logit."""
    import torch
    N, D, V0, V1 = _composite_shapes(H, E0, E1, labels)
    V = V0 + V1
    dt = _dtype_code(H)
    with _on(stream):
        perm = torch.empty(V, dtype=torch.int32, device=H.device) if perm is None else perm
        if want_keys and keys is None:
            keys = torch.empty(V, dtype=torch.float32, device=H.device)
        ws = _workspace(vocab_order_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_perm(perm, V)
    if keys is not None:
        _check_rowvec("keys", keys, V, H.device)
    s = lib().cce_vocab_order_composite(_ptr(H), _ptr(E0), V0, _ptr(E1), V1, _ptr(labels), N, D, dt,
                                        int(ignore_index), _ptr(perm), _ptr(keys), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_vocab_order_composite", s)
    return (perm, keys) if want_keys else perm


def cce_backward_composite(H, E0, E1, off1, labels, lse, dloss, filter_eps=2.0 ** -12, ignore_index=-100, perm=None,
                           flags=0, dH=None, dE0=None, dE1=None, stats=None, ws=None, stream=None, block_max=None):
    """dH [N, D], dE0 [V0, D], dE1 [V1, D] of sum_i dloss_i loss_i for a
    composite head (see cce_forward_composite)."""
    import torch
    N, D, V0, V1 = _composite_shapes(H, E0, E1, labels)
    V = V0 + V1
    dt = _dtype_code(H)
    _check_perm(perm, V)
    _check_rowvec("lse", lse, N, H.device)
    _check_rowvec("dloss", dloss, N, H.device)
    _check_stats(stats)
    if block_max is not None and (block_max.dtype != torch.float32 or block_max.numel() < block_max_elems(N, V)
                                  or not block_max.is_contiguous()):
        raise ValueError(f"block_max must be contiguous fp32 with at least {block_max_elems(N, V)} entries")
    with _on(stream):
        dH = torch.empty_like(H) if dH is None else dH
        dE0 = torch.empty_like(E0) if dE0 is None else dE0
        dE1 = torch.empty_like(E1) if dE1 is None else dE1
        ws = _workspace(backward_workspace_bytes(N, D, V, dt), H.device, ws)
    _check_grad("dH", dH, H)
    _check_grad("dE0", dE0, E0)
    _check_grad("dE1", dE1, E1)
    s = lib().cce_backward_composite(_ptr(H), _ptr(E0), V0, _ptr(E1), V1, int(off1), _ptr(labels), _ptr(lse),
                                     _ptr(dloss), _ptr(block_max), N, D, dt, int(ignore_index), float(filter_eps),
                                     _ptr(perm), int(flags), _ptr(dH), _ptr(dE0), _ptr(dE1), _ptr(stats), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check("cce_backward_composite", s)
    return dH, dE0, dE1


def cce_check_labels(labels, V, ignore_index=-100, stream=None) -> int:
    """Number of labels neither ignore_index nor in [0, V)."""
    import torch
    with _on(stream):
        n_bad = torch.empty(1, dtype=torch.int64, device=labels.device)
    s = lib().cce_check_labels(_ptr(labels), labels.shape[0], int(V), int(ignore_index), _ptr(n_bad),
                               _stream(stream))
    _check("cce_check_labels", s)
    return int(n_bad.item())
