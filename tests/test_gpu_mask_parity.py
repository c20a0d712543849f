"""Block-sparse masks: HIP path vs the fp64 oracle through the C ABI.

Same bar as the unmasked parity tests (relative Frobenius error per tensor,
per (b, h) and per row, ``tests/gpu_check.py``: 1e-5 float32, 2e-2 bf16),
plus exact checks that the masks make exact: an
all-ones mask reproduces the unmasked call bit for bit, an all-zeros mask
gives zeros (and L = -inf), and rows that keep no key give O = 0, L = -inf
and dQ = 0.
"""

import math
import sys

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc
from tests import gpu_check

pytestmark = pytest.mark.gpu

TOL = gpu_check.TOL


def _say(msg):
    print(f"[gpu mask case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_softmax_attention_attn_amd import binding
    binding.load()
    return binding


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t if dtype == "f32" else t.to(torch.bfloat16)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


# B, H, N, d, dtype, causal, mask recipe
CASES = [
    (1, 2, 1000, 128, "bf16", True, "random"),          # pipelined kernels, d = 128
    (1, 2, 1000, 128, "bf16", False, "random_heads"),
    (2, 2, 700, 64, "bf16", False, "random_empty"),     # d = 64, rows keeping no key
    (2, 2, 700, 64, "bf16", True, "random_empty"),      # d = 64 causal (one-half dQ form)
    (1, 2, 513, 128, "bf16", True, "random_empty"),     # ragged last tile
    (1, 1, 1100, 128, "bf16", True, "window"),           # local window + sink blocks
    (1, 2, 300, 64, "f32", True, "random_heads"),        # generic kernels, float32
    (2, 1, 260, 32, "f32", False, "random_empty"),
    (1, 2, 257, 40, "bf16", False, "random"),            # generic bf16 (odd head dim)
    (1, 2, 400, 256, "bf16", True, "random_empty"),      # head dim 256
]


def _mask(recipe, Bn, H, N, seed):
    nb = (N + 127) // 128
    if recipe == "random":
        return workloads.make_block_mask(N, 0.5, seed)
    if recipe == "random_heads":
        return workloads.make_block_mask(N, 0.5, seed, heads=(Bn, H))
    if recipe == "random_empty":
        return workloads.make_block_mask(N, 0.6, seed, heads=(Bn, H), empty_rows=(1,))
    if recipe == "window":
        return workloads.window_block_mask(N, window_blocks=3, sink_blocks=1)
    raise ValueError(recipe)


def _run_masked(binding, x, m, scale, causal, dtype, feed=None):
    import torch
    q, k, v, do = (_dev(x[n], dtype) for n in ("q", "k", "v", "do"))
    mask = torch.from_numpy(m).cuda()
    o, lse = binding.attn_fwd_lse_masked(q, k, v, mask, causal=causal, scale=scale)
    if feed is not None:
        o_in = _dev(feed[0], dtype)
        l_in = torch.from_numpy(np.ascontiguousarray(feed[1], dtype=np.float32)).cuda()
    else:
        o_in, l_in = o, lse
    dq, dk, dv = binding.attn_bwd_masked(q, k, v, o_in, do, l_in, mask, causal=causal,
                                         scale=scale)
    torch.cuda.synchronize()
    return {"O": _host(o), "L": _host(lse), "dQ": _host(dq), "dK": _host(dk), "dV": _host(dv)}


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_masked_parity(B, case):
    Bn, H, N, d, dtype, causal, recipe = case
    x = workloads.make_random(Bn, H, N, d, dtype, seed=N + d,
                              qkv_std=0.5 if dtype == "bf16" else 1.0)
    m = _mask(recipe, Bn, H, N, seed=N)
    scale = 1.0 / math.sqrt(d)
    xs = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "do")}
    O, L = orc.attn_fwd(xs["q"], xs["k"], xs["v"], scale, causal, m)
    g = orc.attn_bwd(xs["q"], xs["k"], xs["v"], xs["do"], scale, causal, m)
    for feed in ("own", "oracle"):
        _say(f"{case} feed={feed}")
        got = _run_masked(B, x, m, scale, causal, dtype, None if feed == "own" else (O, L))
        assert all(np.isfinite(got[t]).all() for t in ("O", "dQ", "dK", "dV")), (case, feed)
        # rows that keep no key: L = -inf on both sides; compared as 0 below
        assert np.array_equal(np.isneginf(got["L"]), np.isneginf(L)), (case, feed)
        ref = dict(g, O=O, L=np.where(np.isneginf(L), 0.0, L))
        got["L"] = np.where(np.isneginf(got["L"]), 0.0, got["L"])
        gpu_check.check(f"masked {case} feed={feed}", got, ref, dtype)
        # rows that keep no key: exactly zero output and dQ
        empty = np.isneginf(L)                                    # [B, H, N]
        if empty.any():
            o_rows = np.transpose(got["O"], (0, 2, 1, 3))[empty]
            dq_rows = np.transpose(got["dQ"], (0, 2, 1, 3))[empty]
            assert np.all(o_rows == 0.0) and np.all(dq_rows == 0.0), (case, feed)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(1000, 128), (700, 64), (300, 32)])
def test_all_ones_mask_equals_the_unmasked_call_bitwise(B, causal, n, d):
    import torch
    _say(f"all-ones mask n={n} d={d} causal={causal}")
    x = workloads.make_random(1, 2, n, d, "bf16", seed=7, qkv_std=0.5)
    q, k, v, do = (_dev(x[t], "bf16") for t in ("q", "k", "v", "do"))
    ones = torch.ones(((n + 127) // 128,) * 2, dtype=torch.uint8, device="cuda")
    o0, l0 = B.attn_fwd_lse(q, k, v, causal=causal)
    o1, l1 = B.attn_fwd_lse_masked(q, k, v, ones, causal=causal)
    g0 = B.attn_bwd(q, k, v, o0, do, l0, causal=causal)
    g1 = B.attn_bwd_masked(q, k, v, o0, do, l0, ones, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_all_zeros_mask_gives_zeros(B, dtype, d):
    import torch
    _say(f"all-zeros mask {dtype} d={d}")
    n = 384
    x = workloads.make_random(1, 2, n, d, dtype, seed=3, qkv_std=0.5)
    q, k, v, do = (_dev(x[t], dtype) for t in ("q", "k", "v", "do"))
    zeros = torch.zeros((3, 3), dtype=torch.uint8, device="cuda")
    o, lse = B.attn_fwd_lse_masked(q, k, v, zeros)
    dq, dk, dv = B.attn_bwd_masked(q, k, v, o, do, lse, zeros)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    for t in (dq, dk, dv):
        assert torch.all(t == 0)
