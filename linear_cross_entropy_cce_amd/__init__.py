"""MI355X-native fused classifier-head + cross-entropy (Cut Cross-Entropy).

The compute path is the HIP library libcce.so (hand-written gfx950 kernels
behind a C ABI declared in include/cce.h); the Python layer only marshals
arguments and allocates device memory through PyTorch.
"""
