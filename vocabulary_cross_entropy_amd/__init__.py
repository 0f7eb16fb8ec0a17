"""Fused cross-entropy over a large vocabulary for AMD MI355X (gfx950).

The computation lives in ``libvce.so`` (HIP kernels behind the C-ABI declared
in ``include/vce.h``); ``binding`` marshals torch tensors into it.
"""
from .binding import (ce_backward, ce_forward, gemm_bf16, lce_backward, lce_forward,  # noqa: F401
                      lce_workspace, lce_workspace_size, lib, strerror,
                      VceError)
