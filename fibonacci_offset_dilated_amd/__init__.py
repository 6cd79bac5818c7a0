"""Fibonacci-offset dilated sparse attention on AMD MI355X (gfx950).

The attention layer of "Depth-Staggered Fibonacci Spacing for Sparse Attention" (gist.science
summaries of arXiv 2606.28560): causal self-attention over a dense local window of W keys
plus one key per base offset f_k scaled by a per-layer alpha, with RoPE applied before the
gather and linear K/V interpolation at non-integer offsets. The compute runs in the
hand-written HIP kernels of libfibattn.so; this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    BF16, F32, INT, INTERP, SCHED_COPRIME, SCHED_FIXED, SCHED_LINEAR,
    NOALLOC_SCRATCH_BYTES, FibError, bwd, bwd_dev, bwd_layers, bwd_noalloc, bwd_workspace_size, decode, decode_dev, decode_layers, dense_lse,
    dropped_mass, fwd, fwd_dev, fwd_layers, index_set, layers_plan_bytes, lib, offset_table, plan_bytes,
    schedule_alpha, status_string,
)
