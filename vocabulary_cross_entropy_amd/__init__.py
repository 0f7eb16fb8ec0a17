"""Fused cross-entropy over a large vocabulary for AMD MI355X (gfx950).

The computation lives in ``libvce.so`` (HIP kernels behind the C-ABI declared
in ``include/vce.h``); ``binding`` marshals torch tensors into it.
"""
from .binding import (ce_backward, ce_backward_shard, ce_forward,  # noqa: F401
                      ce_forward_backward, ce_forward_shard, ce_merge_shards, gemm_bf16,
                      lce_backward, lce_backward_f32,
                      lce_backward_shard, lce_forward, lce_forward_f32, lce_forward_noalloc,
                      lce_forward_shard,
                      lce_workspace, lce_workspace_size, lce_workspace_size_f32, lib,
                      shift_targets, strerror, VceError)
