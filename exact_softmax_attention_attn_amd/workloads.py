"""Seeded synthetic inputs for the attention backward, shared by tests and bench.

This module holds shapes, seeds and value recipes only: none of the attention
arithmetic lives here, so the oracle and the HIP path can both draw from it
without sharing any of the method.

The first five workloads stand in for the pages' own workloads (no dataset
or trained weights exist for them); five more take c5's shape beyond square
causal attention, to head dim 256, or through the backward of the backward:

* ``c1_tiny``  -- the toy of ddx issue #217's repro script: 3 sequences, 2
  heads, 8 positions, 4 channels per head, scale 1/2, and Q/K/V filled with
  sin(flat_index * 0.37 + phase) for phases 0, 1, 2 over the row-major
  (sequence, position, head, channel) flattening.  dO ~ N(0, 1) from the seed.
* ``c2_nanogpt_cpu`` -- the GPT demo size of issue #217: batch 12, 4 heads,
  64 positions, 128 channels (head dim 32), scale 1/sqrt(32).
* ``c3_single_seq`` -- PR #162's timing workload: one sequence of 256 tokens
  with 64 features, one head, scale 1/8.
* ``c4_batched`` -- 1,024 tokens as in issue #243 item 1, batch 4 x 16 heads,
  head dim 64, bf16 in / fp32 accumulate, scale 1/8 (1/sqrt(d); unstated).
* ``c5_long`` -- 16,384 tokens as in issue #243 item 2, 16 heads, head dim 128,
  bf16 in / fp32 accumulate, scale 1/sqrt(128).
* ``c5_full`` -- c5_long with full (non-causal) attention.
* ``c5_ragged`` -- c5_long at 16,383 tokens, a length no tile size divides.
* ``c5_d256`` -- 16,384 tokens, 8 heads of head dim 256 (c5_long's FLOPs).
* ``c5_bob`` -- c5_long's inputs through the backward of the backward, with
  cotangents gQ, gK, gV from ``make_cotangents``.
* ``c5_window`` -- c5_long under a block-sparse mask: each query block keeps
  the 16 key blocks up to its own (a 2,048-token local window) and the first
  block (attention sink), causal inside the window.
* ``c5_fwd`` -- c5_long's inputs through the forward alone (O and L).

Random draws use numpy's PCG64 ``default_rng(seed)`` in fp64, in the order
Q, K, V, dO, each of shape [B, N, H, d]; Q/K/V are multiplied by ``qkv_std``.
bf16 workloads are rounded fp64 -> fp32 -> bf16, each step round-to-nearest-
even, and returned as fp32 arrays that hold bf16 values exactly.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "make_random", "bf16_round",
           "MASK_BLOCK", "make_block_mask", "window_block_mask", "workload_mask",
           "make_cotangents", "make_peaked", "make_shifted"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    scale: float
    dtype: str            # "f32" or "bf16": the device input/output type
    qkv_std: float = 1.0
    qkv: str = "normal"   # "normal" or "sin" (the issue #217 toy recipe)
    causal: bool = True
    description: str = ""
    mask: str = ""        # "" (no block mask) or "window<W>": window_block_mask(N, W, 1)
    op: str = "bwd"       # "bwd" (the backward), "bob" (the backward of the backward), "fwd"

    @property
    def shape(self):
        return (self.B, self.N, self.H, self.d)


WORKLOADS = (
    Workload("c1_tiny", 3, 2, 8, 4, 0.5, "f32", qkv="sin",
             description="toy of issue #217: 3 seq x 2 heads x 8 pos x d 4, scale 1/2, sin inputs"),
    Workload("c2_nanogpt_cpu", 12, 4, 64, 32, 1.0 / math.sqrt(32), "f32",
             description="nanoGPT CPU size: batch 12, 4 heads, 64 pos, d 32"),
    Workload("c3_single_seq", 1, 1, 256, 64, 1.0 / 8.0, "f32",
             description="one sequence, 256 tokens x 64 features"),
    Workload("c4_batched", 4, 16, 1024, 64, 1.0 / 8.0, "bf16", qkv_std=0.5,
             description="batch 4 x 16 heads x 1024 tokens x d 64, bf16"),
    Workload("c5_long", 1, 16, 16384, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5,
             description="1 x 16 heads x 16384 tokens x d 128, bf16"),
    # c5's shape beyond square causal: full (non-causal) attention, and a
    # length that no tile size divides (every walk ends on a ragged tile)
    Workload("c5_full", 1, 16, 16384, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5,
             causal=False, description="c5_long without the causal mask"),
    Workload("c5_ragged", 1, 16, 16383, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5,
             description="c5_long one token shorter: ragged last tile everywhere"),
    Workload("c5_window", 1, 16, 16384, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5,
             mask="window16",
             description="c5_long under a block mask: 2048-token local window + first block"),
    # the backward of the backward at c5_long's shape (cotangents from make_cotangents)
    Workload("c5_bob", 1, 16, 16384, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5, op="bob",
             description="c5_long through the backward of the backward"),
    # head dim 256 at the same FLOPs as c5_long (half the heads)
    Workload("c5_d256", 1, 8, 16384, 256, 1.0 / 16.0, "bf16", qkv_std=0.5,
             description="16384 tokens x 8 heads x d 256, bf16"),
    # the forward that supplies O and L, at c5_long's shape
    Workload("c5_fwd", 1, 16, 16384, 128, 1.0 / math.sqrt(128), "bf16", qkv_std=0.5, op="fwd",
             description="c5_long through the forward (O and L)"),
)


def get(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def bf16_round(x) -> np.ndarray:
    """Round to bf16 (via fp32), nearest-even at each step; returns fp32 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


def _sin_fill(shape, phase: float) -> np.ndarray:
    n = int(np.prod(shape))
    return np.sin(np.arange(n) * 0.37 + phase).reshape(shape)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Q, K, V, dO for a workload as fp32 arrays [B, N, H, d] (bf16-exact for bf16)."""
    rng = np.random.default_rng(seed)
    shape = w.shape
    if w.qkv == "sin":
        q, k, v = (_sin_fill(shape, ph) for ph in (0.0, 1.0, 2.0))
    else:
        q = rng.standard_normal(shape) * w.qkv_std
        k = rng.standard_normal(shape) * w.qkv_std
        v = rng.standard_normal(shape) * w.qkv_std
    do = rng.standard_normal(shape)
    return {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype),
            "do": _cast(do, w.dtype)}


MASK_BLOCK = 128   # rows and keys per block of a block-sparse mask


def make_block_mask(N: int, density: float = 0.5, seed: int = 0, heads=None,
                    keep_diagonal: bool = True, empty_rows=()) -> np.ndarray:
    """A random block mask: uint8 [nb, nb], or [B, H, nb, nb] for heads = (B, H).

    Each block is kept with probability ``density`` (PCG64 ``default_rng``);
    ``keep_diagonal`` keeps block (r, r) so every row keeps a key; the block
    rows listed in ``empty_rows`` keep nothing.
    """
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    rng = np.random.default_rng(seed)
    shape = (nb, nb) if heads is None else tuple(heads) + (nb, nb)
    m = (rng.random(shape) < density).astype(np.uint8)
    if keep_diagonal:
        idx = np.arange(nb)
        m[..., idx, idx] = 1
    for r in empty_rows:
        m[..., r, :] = 0
    return np.ascontiguousarray(m)


def window_block_mask(N: int, window_blocks: int, sink_blocks: int = 1) -> np.ndarray:
    """Local attention with attention sinks, at block granularity: block (r, c)
    is kept when r - window_blocks < c <= r or c < sink_blocks."""
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    r = np.arange(nb)[:, None]
    c = np.arange(nb)[None, :]
    return (((c <= r) & (c > r - window_blocks)) | (c < sink_blocks)).astype(np.uint8)


def make_cotangents(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0) -> dict:
    """Cotangents gQ, gK, gV of the backward's outputs, ~ N(0, 1) [B, N, H, d]
    (PCG64 ``default_rng(seed + 1000)``, drawn in that order), cast like inputs."""
    rng = np.random.default_rng(seed + 1000)
    shape = (B, N, H, d)
    return {n: _cast(rng.standard_normal(shape), dtype) for n in ("gq", "gk", "gv")}


def workload_mask(w: Workload):
    """The workload's block mask (uint8 [nb, nb], shared by every head) or None."""
    if not w.mask:
        return None
    if w.mask.startswith("window"):
        return window_block_mask(w.N, int(w.mask[len("window"):]), 1)
    raise ValueError(w.mask)


def make_random(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                qkv_std: float = 1.0) -> dict:
    """Normal inputs of any shape (edge cases: ragged N, small d, N = 1, ...)."""
    w = Workload("random", B, H, N, d, 1.0 / math.sqrt(d), dtype, qkv_std=qkv_std)
    return make_inputs(w, seed)


def make_peaked(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                qkv_std: float = 2.0, growth: float = 3.0) -> dict:
    """Sharply peaked softmax rows whose maximum keeps rising along the sequence.

    Q, K, V ~ N(0, qkv_std^2) and dO ~ N(0, 1) as in ``make_inputs``; then key
    row j is multiplied by 1 + growth * j / N, so later keys score higher and
    a row's running maximum climbs as the walk reaches them.  Rounded like
    the other inputs.
    """
    x = make_random(B, H, N, d, "f32", seed=seed, qkv_std=qkv_std)
    ramp = (1.0 + growth * np.arange(N) / N)[None, :, None, None]
    x["k"] = x["k"].astype(np.float64) * ramp
    return {n: _cast(v, dtype) for n, v in x.items()}


def make_shifted(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                 q_shift: float = 1296.0, k_shift: float = 1.0, qkv_std: float = 0.5) -> dict:
    """Inputs whose scores all sit far below zero by the same amount per row.

    Normal inputs as in ``make_random``; then channel 0 of every query is set
    to +q_shift and channel 0 of every key to -k_shift: the keys share a
    component anti-aligned with every query, which lowers every score by
    scale * q_shift * k_shift (a constant per row, to which the softmax is
    blind) and leaves the rest of the scores as they were.  Both shifts must
    be exactly representable in the device type.
    """
    assert _cast(np.array([q_shift, k_shift]), dtype).tolist() == [q_shift, k_shift]
    x = make_random(B, H, N, d, "f32", seed=seed, qkv_std=qkv_std)
    x["q"][..., 0] = q_shift
    x["k"][..., 0] = -k_shift
    return {n: _cast(v, dtype) for n, v in x.items()}

