"""MI355X-native fused classifier-head + cross-entropy (Cut Cross-Entropy).

The compute path is the HIP library libcce.so (hand-written gfx950 kernels
behind the C ABI declared in include/cce.h); the Python layer only marshals
arguments and allocates device memory through PyTorch.  Nothing here falls
back to another implementation: without the library every call raises.
"""
from .binding import (CCEError, cce_backward, cce_backward_composite, cce_check_labels,  # noqa: F401
                      cce_forward, cce_forward_composite, cce_vocab_order, cce_vocab_order_composite,
                      filter_block)
from .inputs import IGNORE_INDEX  # noqa: F401


def linear_cross_entropy(*args, **kwargs):
    from .autograd import linear_cross_entropy as f
    return f(*args, **kwargs)


def linear_cross_entropy_composite(*args, **kwargs):
    from .autograd import linear_cross_entropy_composite as f
    return f(*args, **kwargs)


__all__ = ["cce_forward", "cce_backward", "cce_vocab_order", "cce_check_labels", "filter_block",
           "cce_forward_composite", "cce_backward_composite", "cce_vocab_order_composite",
           "linear_cross_entropy", "linear_cross_entropy_composite", "CCEError", "IGNORE_INDEX"]
