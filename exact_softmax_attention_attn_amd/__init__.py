"""Exact causal softmax-attention backward by score recomputation, for MI355X (gfx950).

The compute lives in ``libattn.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/attn.h``); :mod:`.binding` marshals torch tensors into
that ABI.  :mod:`.workloads` holds the seeded synthetic inputs.
"""

__all__ = ["binding", "workloads"]
