"""attn_bwd_noalloc against attn_bwd, through the C ABI.

attn_bwd_noalloc runs attn_bwd's kernels on the library's static per-GPU
workspace array instead of a caller's workspace, so on the same inputs its
dQ, dK and dV must be attn_bwd's bit for bit.  Two calls in a row, the
second on a smaller problem (the array keeps the first call's contents),
then the other way round and on float32; no device memory is taken by the
calls once the array exists.
"""

import math
import sys

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu no-alloc case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_softmax_attention_attn_amd import binding
    binding.load()
    return binding


def _case(binding, b, h, n, d, dtype, causal):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = workloads.make_random(b, h, n, d, dtype, seed=n + d, qkv_std=0.5 if dtype == "bf16" else 1.0)
    q, k, v, do = (torch.from_numpy(x[t]).cuda().to(tdt) for t in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = binding.attn_fwd_lse(q, k, v, causal=causal, scale=scale)
    ref = binding.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    outs = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    return (q, k, v, o, do, lse, scale), ref, outs


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_equals_attn_bwd_bitwise(B, order):
    import torch
    shapes = [(4, 16, 1024, 64, "bf16", True), (1, 2, 300, 128, "bf16", False)]
    if order == "small_then_large":
        shapes = shapes[::-1]
    shapes.append((2, 2, 77, 32, "f32", True))
    for shape in shapes:
        _say(f"{order} {shape}")
        (q, k, v, o, do, lse, scale), ref, outs = _case(B, *shape)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        alloc0 = torch.cuda.memory_allocated()
        B.attn_bwd_noalloc(q, k, v, o, do, lse, *outs, causal=shape[5], scale=scale)
        torch.cuda.synchronize()
        # nothing taken from torch's allocator, and (once the array exists,
        # after the process's first call) nothing from the device
        assert torch.cuda.memory_allocated() == alloc0, shape
        if shape != shapes[0]:
            assert abs(torch.cuda.mem_get_info()[0] - free0) < (1 << 20), shape
        for name, a, r in zip(("dQ", "dK", "dV"), outs, ref):
            assert torch.isfinite(a.float()).all(), (shape, name)
            bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.view(bits), r.view(bits)), (shape, name)
        del q, k, v, o, do, lse, ref, outs


def test_noalloc_rejects_a_workspace_beyond_its_array(B):
    import ctypes
    import torch
    lib = B.load()
    rows = B.ATTN_MASK_BLOCK  # any small size for the pointers' shapes
    q = torch.zeros((1, rows, 1, 8), device="cuda")
    lse = torch.zeros((1, 1, rows), device="cuda")
    p = [ctypes.c_void_p(t.data_ptr()) for t in (q, q, q, q, q, lse, q, q, q)]
    # B*H*N = 2,097,153 rows needs 8 bytes more than the 16 MiB array holds
    st = lib.attn_bwd_noalloc(*p, 1, 1, 2097153, 8, 1, 0.5, 0, ctypes.c_void_p(0))
    assert st == B.ATTN_ERR_UNSUPPORTED
    assert b"exceeds" in lib.attn_last_error()


def test_noalloc_replays_under_graph_capture(B):
    """The callers it is for: a HIP graph captures the allocation-free call
    once and replays it; each replay, with eager work and synchronisation in
    between, must give attn_bwd's dQ, dK, dV bit for bit."""
    import torch
    shape = (1, 4, 700, 128, "bf16", True)
    _say(f"graph capture {shape}")
    (q, k, v, o, do, lse, scale), ref, outs = _case(B, *shape)
    # the first call on a device finds the array's address; it runs outside the capture
    B.attn_bwd_noalloc(q, k, v, o, do, lse, *outs, causal=True, scale=scale)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.attn_bwd_noalloc(q, k, v, o, do, lse, *outs, causal=True, scale=scale)
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))                  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, r in zip(("dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a.view(torch.int16), r.view(torch.int16)), (i, name)
    del g
