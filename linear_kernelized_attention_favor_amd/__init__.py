"""FAVOR+ attention for AMD Instinct MI355X (gfx950): forward and backward passes.

Positive orthogonal random features and linear-time attention, bidirectional
and causal, with their gradients, computed by hand-written HIP kernels in libfavor.so (C ABI in
include/favor.h).  This package is the thin Python binding over that library.
"""
from ._binding import (BF16, F32, GAUSSIAN, LIB_PATH, RELU, SOFTMAX, FavorError,  # noqa: F401
                       bwd, bwd_workspace_bytes, decode, draw_projection,
                       draw_projection_device, feature_map,
                       fwd_bidir, fwd_causal, fwd_noalloc, NOALLOC_SCRATCH_BYTES,
                       plan_describe, prefill, state_bytes, state_new,
                       state_reset,
                       status_string, timing_start, timing_stop, workspace_bytes)

__all__ = ["fwd_bidir", "fwd_causal", "fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "bwd", "bwd_workspace_bytes", "prefill", "decode",
           "draw_projection_device",
           "state_bytes", "state_new", "state_reset", "feature_map", "draw_projection", "workspace_bytes",
           "status_string", "plan_describe", "timing_start", "timing_stop", "FavorError", "LIB_PATH", "F32",
           "BF16", "SOFTMAX", "GAUSSIAN", "RELU"]
