"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerance (relative Frobenius error per tensor, max over dQ, dK, dV):
1e-5 for the float32 path and 2e-2 for the bf16 path.  Two feeds for the
backward: (i) O and L from the library's own forward (the user flow) and
(ii) the oracle's O and L cast to the device type (isolates the backward).
"""

import math
import sys

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _say(msg):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_softmax_attention_attn_amd import binding
    binding.load()
    return binding


def _tdtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _dev(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(_tdtype(dtype))


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def _run(binding, x, scale, causal, dtype, feed_oracle=None):
    import torch
    q, k, v, do = (_dev(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = binding.attn_fwd_lse(q, k, v, causal=causal, scale=scale)
    if feed_oracle is not None:
        o_in = _dev(feed_oracle[0], dtype)
        l_in = torch.from_numpy(np.ascontiguousarray(feed_oracle[1], dtype=np.float32)).cuda()
    else:
        o_in, l_in = o, lse
    dq, dk, dv = binding.attn_bwd(q, k, v, o_in, do, l_in, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return {"O": _host(o), "L": _host(lse), "dQ": _host(dq), "dK": _host(dk), "dV": _host(dv)}


def _check_full(binding, x, scale, causal, dtype, tag):
    xs = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "do")}
    O, L = orc.attn_fwd(xs["q"], xs["k"], xs["v"], scale, causal)
    g = orc.attn_bwd(xs["q"], xs["k"], xs["v"], xs["do"], scale, causal)
    tol = TOL[dtype]
    for feed in ("own", "oracle"):
        _say(f"{tag} feed={feed}")
        got = _run(binding, x, scale, causal, dtype, None if feed == "own" else (O, L))
        errs = {t: rel_fro(got[t], g[t]) for t in ("dQ", "dK", "dV")}
        errs["O"] = rel_fro(got["O"], O)
        errs["L"] = rel_fro(got["L"], L)
        assert all(np.isfinite(v) for v in errs.values()), (tag, feed, errs)
        assert max(errs[t] for t in ("dQ", "dK", "dV")) <= tol, (tag, feed, errs)
        assert errs["O"] <= tol and errs["L"] <= tol, (tag, feed, errs)
    return errs


@pytest.mark.parametrize("name", ["c1_tiny", "c2_nanogpt_cpu", "c3_single_seq", "c4_batched"])
def test_parity_workload(B, name):
    w = workloads.get(name)
    x = workloads.make_inputs(w, seed=0)
    _check_full(B, x, w.scale, w.causal, w.dtype, name)


def test_parity_c1_with_the_pages_loss(B):
    # loss = sum(O^2)/2, so the output cotangent is O itself
    w = workloads.get("c1_tiny")
    x = workloads.make_inputs(w, seed=0)
    O, _ = orc.attn_fwd(x["q"], x["k"], x["v"], w.scale, True)
    x = dict(x, do=O.astype(np.float32))
    _check_full(B, x, w.scale, True, "f32", "c1_pages_loss")


EDGE = [
    # B, H, N, d, dtype, causal
    (1, 1, 1, 8, "f32", True),
    (1, 1, 1, 8, "bf16", True),
    (2, 3, 7, 4, "f32", True),
    (1, 2, 65, 32, "f32", True),
    (1, 2, 65, 64, "bf16", True),
    (1, 1, 1000, 64, "f32", True),
    (1, 1, 1000, 128, "bf16", True),
    (2, 1, 200, 128, "f32", True),      # float32 128 bucket: two column parts per block
    (1, 2, 150, 128, "f32", False),
    (1, 2, 129, 8, "bf16", True),
    (1, 2, 300, 40, "bf16", True),
    (1, 1, 300, 128, "bf16", True),   # odd tile counts per key block
    (1, 2, 300, 100, "f32", True),
    (2, 2, 77, 32, "f32", False),
    (1, 2, 190, 128, "bf16", False),
    (1, 2, 1000, 128, "bf16", False),  # long non-causal walks through the pipelined main loops
    (1, 2, 700, 64, "bf16", False),
    (1, 1, 257, 64, "f32", False),
    (1, 1, 1, 16, "bf16", False),
    (1, 2, 300, 256, "bf16", True),    # head dim 256 (bf16 only)
    (2, 1, 200, 256, "bf16", False),
    (1, 2, 129, 192, "bf16", True),    # 192 runs in the 256 bucket, zero padded
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_parity_edge_shapes(B, case):
    b, h, n, d, dtype, causal = case
    x = workloads.make_random(b, h, n, d, dtype, seed=n + d, qkv_std=0.5 if dtype == "bf16" else 1.0)
    _check_full(B, x, 1.0 / math.sqrt(d), causal, dtype, f"edge {case}")


def test_bitwise_repeatable(B):
    import torch
    w = workloads.get("c4_batched")
    x = workloads.make_inputs(w, seed=0)
    q, k, v, do = (_dev(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    o, lse = B.attn_fwd_lse(q, k, v, causal=True, scale=w.scale)
    first = B.attn_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale)
    for _ in range(2):
        again = B.attn_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    torch.cuda.synchronize()


def test_no_device_allocation_during_backward(B):
    import torch
    w = workloads.get("c4_batched")
    x = workloads.make_inputs(w, seed=1)
    q, k, v, do = (_dev(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    o, lse = B.attn_fwd_lse(q, k, v, causal=True, scale=w.scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = B.new_workspace(w.B, w.H, w.N, "cuda")
    B.attn_bwd(q, k, v, o, do, lse, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        B.attn_bwd(q, k, v, o, do, lse, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert abs(free1 - free0) < (2 << 20)


@pytest.mark.parametrize("name", ["c5_long", "c5_full", "c5_ragged", "c5_window", "c5_d256"])
def test_c5_full_size_sampled_against_oracle(B, name):
    """N = 16,384 (or 16,383), d = 128, bf16: sampled rows and columns of two heads."""
    import torch
    w = workloads.get(name)
    _say(f"{name} inputs")
    x = workloads.make_inputs(w, seed=0)
    q, k, v, do = (_dev(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    _say(f"{name} forward + backward on the GPU")
    bm = workloads.workload_mask(w)
    if bm is None:
        o, lse = B.attn_fwd_lse(q, k, v, causal=w.causal, scale=w.scale)
        dq, dk, dv = B.attn_bwd(q, k, v, o, do, lse, causal=w.causal, scale=w.scale)
    else:
        mask = torch.from_numpy(bm).cuda()
        o, lse = B.attn_fwd_lse_masked(q, k, v, mask, causal=w.causal, scale=w.scale)
        dq, dk, dv = B.attn_bwd_masked(q, k, v, o, do, lse, mask, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    N = w.N
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 8191, 8192, N - 1], rng.integers(0, N, 40)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 8191, 8192, N - 1], rng.integers(0, N, 40)]))
    errs = []
    for h in (0, w.H - 5):
        _say(f"{name} oracle sample head {h}")
        s = orc.attn_bwd_sampled(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal, 0, h, rows, cols,
                                 row_block=1024, block_mask=bm)
        got_dq = dq[0, rows, h].float().cpu().numpy()
        got_o = o[0, rows, h].float().cpu().numpy()
        got_dk = dk[0, cols, h].float().cpu().numpy()
        got_dv = dv[0, cols, h].float().cpu().numpy()
        got_l = lse[0, h].cpu().numpy()
        e = {"dQ": rel_fro(got_dq, s["dQ"]), "dK": rel_fro(got_dk, s["dK"]),
             "dV": rel_fro(got_dv, s["dV"]), "O": rel_fro(got_o, s["O"]),
             "L": rel_fro(got_l, s["L"])}
        errs.append(e)
        assert max(e.values()) <= TOL["bf16"], (h, e)
    # properties over the whole tensor: sum_j dV_j = sum_i dO_i; sum_j dK_j = 0
    sdv = dv.double().sum(dim=1).cpu().numpy()
    sdo = do.double().sum(dim=1).cpu().numpy()
    assert rel_fro(sdv, sdo) <= TOL["bf16"]
    sdk = dk.double().sum(dim=1).cpu().numpy()
    adk = dk.double().abs().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(sdk) <= TOL["bf16"] * adk + 1e-6)
    print(f"{name} sampled errors", errs, flush=True)
