"""The entry points against their own stages, bit for bit.

attn_bwd (and attn_bwd_masked) may run dQ first with the preprocess done
inside it for the block's own rows, then dK/dV: two launches.  The stage entry
points run the preprocess kernel, dK/dV and dQ on their own.  Both must leave
the same bits in dQ, dK, dV and in the workspace (-D, -L log2 e): the fused
preprocess uses the preprocess kernel's lanes and summation order.  Cases span
both head dims of the pipelined kernels, causal and full, ragged and short
sequences, block masks (with rows that keep no key), and shapes that take the
three-launch path (float32, head dim 256) as controls.
"""

import sys

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu stages case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_softmax_attention_attn_amd import binding
    binding.load()
    return binding


CASES = [
    # B, H, N, d, dtype, causal, mask recipe (None: no mask)
    (1, 2, 1000, 128, "bf16", True, None),
    (2, 2, 700, 128, "bf16", False, None),
    (1, 3, 513, 64, "bf16", True, None),
    (2, 1, 7, 64, "bf16", True, None),
    (1, 2, 63, 128, "bf16", False, None),
    (1, 2, 1100, 128, "bf16", True, "window"),
    (1, 2, 900, 64, "bf16", False, "random_empty"),
    (1, 2, 300, 64, "f32", True, None),
    (1, 2, 300, 256, "bf16", True, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_entry_point_equals_stages_bitwise(B, case):
    import torch
    from tests.test_gpu_mask_parity import _mask
    Bn, H, N, d, dtype, causal, recipe = case
    _say(f"{case}")
    x = workloads.make_random(Bn, H, N, d, dtype, seed=N + d + 5,
                              qkv_std=0.5 if dtype == "bf16" else 1.0)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v, do = (torch.from_numpy(np.ascontiguousarray(x[n], dtype=np.float32)).cuda().to(tdt)
                   for n in ("q", "k", "v", "do"))
    mask = None
    if recipe is not None:
        mask = torch.from_numpy(_mask(recipe, Bn, H, N, seed=N + 9)).cuda()
        o, lse = B.attn_fwd_lse_masked(q, k, v, mask, causal=causal)
    else:
        o, lse = B.attn_fwd_lse(q, k, v, causal=causal)
    ws_e = torch.full((2, Bn, H, N), float("nan"), dtype=torch.float32, device="cuda")
    ws_s = torch.full_like(ws_e, float("nan"))
    if mask is None:
        ge = B.attn_bwd(q, k, v, o, do, lse, causal=causal, workspace=ws_e)
    else:
        ge = B.attn_bwd_masked(q, k, v, o, do, lse, mask, causal=causal, workspace=ws_e)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    B.attn_bwd_preprocess(o, do, lse, ws_s)
    if mask is None:
        B.attn_bwd_dkdv(q, k, v, do, ws_s, dk, dv, causal=causal)
        B.attn_bwd_dq(q, k, v, do, ws_s, dq, causal=causal)
    else:
        B.attn_bwd_dkdv_masked(q, k, v, do, ws_s, dk, dv, mask, causal=causal)
        B.attn_bwd_dq_masked(q, k, v, do, ws_s, dq, mask, causal=causal)
    torch.cuda.synchronize()
    iview = torch.int32 if dtype == "f32" else torch.int16
    for name, a, b in (("dQ", ge[0], dq), ("dK", ge[1], dk), ("dV", ge[2], dv)):
        assert torch.equal(a.view(iview), b.view(iview)), (case, name)
    assert torch.equal(ws_e.view(torch.int32), ws_s.view(torch.int32)), (case, "workspace")
    for a in ge:
        assert torch.isfinite(a.float()).all(), case
