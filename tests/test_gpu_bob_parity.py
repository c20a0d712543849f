"""Backward of the backward: HIP path vs the fp64 oracle through the C ABI.

Relative Frobenius error per output tensor (hQ, hK, hV, hdO) and for the two
row scalars r and E the kernels leave in the workspace, gated per tensor, per
(b, h) and per row as in the first backward's tests (``tests/gpu_check.py``).
Two feeds of O and L: the library's own forward, and the oracle's O and L
cast to the device type.
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
    print(f"[gpu bob case] {msg}", flush=True)
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


CASES = [
    # B, H, N, d, dtype, causal
    (3, 2, 8, 4, "f32", True),
    (2, 2, 77, 32, "f32", False),
    (1, 2, 300, 64, "f32", True),
    (1, 2, 257, 64, "bf16", True),
    (1, 2, 300, 128, "bf16", False),
    (1, 1, 700, 128, "bf16", True),
    (2, 1, 129, 40, "bf16", True),
]


# every score of a row lowered by scale * q_shift > 100 (L < -88; keys share
# channel 0 = -1, queries have channel 0 = q_shift), ragged N: the padded keys
# of the last tile must not reach the products
SHIFTED = [
    (1, 2, 1000, 64, "f32", False, 900.0),
    (1, 2, 1000, 128, "bf16", False, 1296.0),
    (1, 1, 1000, 128, "bf16", True, 1296.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_bwd_parity(B, case):
    Bn, H, N, d, dtype, causal = case
    x = workloads.make_random(Bn, H, N, d, dtype, seed=N + d,
                              qkv_std=0.5 if dtype == "bf16" else 1.0)
    _bob_case(B, x, case)


@pytest.mark.parametrize("case", SHIFTED, ids=lambda c: "x".join(map(str, c)))
def test_bwd_bwd_parity_shifted_scores(B, case):
    from tests.test_gpu_parity import shifted_tol
    Bn, H, N, d, dtype, causal, q_shift = case
    x = workloads.make_shifted(Bn, H, N, d, dtype, seed=5 + d, q_shift=q_shift, k_shift=1.0)
    _bob_case(B, x, case[:6], tol=shifted_tol(dtype, 1.0 / math.sqrt(d), q_shift, 1.0))


def _bob_case(B, x, case, tol=None):
    import torch
    Bn, H, N, d, dtype, causal = case
    scale = 1.0 / math.sqrt(d)
    x.update(workloads.make_cotangents(Bn, H, N, d, dtype, seed=N))
    xs = {n: x[n].astype(np.float64) for n in x}
    O, L = orc.attn_fwd(xs["q"], xs["k"], xs["v"], scale, causal)
    ref = orc.attn_bwd_bwd(xs["q"], xs["k"], xs["v"], xs["do"], xs["gq"], xs["gk"], xs["gv"],
                           scale, causal)
    t = {n: _dev(x[n], dtype) for n in x}
    for feed in ("own", "oracle"):
        _say(f"{case} feed={feed}")
        if feed == "own":
            o, lse = B.attn_fwd_lse(t["q"], t["k"], t["v"], causal=causal, scale=scale)
        else:
            o = _dev(O, dtype)
            lse = torch.from_numpy(np.ascontiguousarray(L, dtype=np.float32)).cuda()
        ws = torch.empty((4, Bn, H, N), dtype=torch.float32, device="cuda")
        hq, hk, hv, hdo = B.attn_bwd_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, t["gq"],
                                         t["gk"], t["gv"], causal=causal, scale=scale,
                                         workspace=ws)
        torch.cuda.synchronize()
        got = {"hQ": _host(hq), "hK": _host(hk), "hV": _host(hv), "hdO": _host(hdo),
               "r": _host(ws[2]), "E": _host(ws[3])}
        gpu_check.check(f"bob {case} feed={feed}", got, ref, dtype,
                        names=("hQ", "hK", "hV", "hdO", "r", "E"), tol=tol)


def test_c5_bob_full_size_sampled_against_oracle(B):
    """N = 16,384, d = 128, bf16: sampled rows and columns of two heads."""
    import torch
    w = workloads.get("c5_bob")
    _say("c5_bob inputs")
    x = workloads.make_inputs(w, seed=0)
    x.update(workloads.make_cotangents(w.B, w.H, w.N, w.d, w.dtype, seed=0))
    t = {n: _dev(x[n], w.dtype) for n in x}
    _say("c5_bob forward + backward of the backward on the GPU")
    o, lse = B.attn_fwd_lse(t["q"], t["k"], t["v"], causal=True, scale=w.scale)
    ws = torch.empty((4, w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    hq, hk, hv, hdo = B.attn_bwd_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, t["gq"], t["gk"],
                                     t["gv"], causal=True, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    N = w.N
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 8191, 8192, N - 1], rng.integers(0, N, 24)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 8191, 8192, N - 1], rng.integers(0, N, 24)]))
    for h in (0, 9):
        _say(f"c5_bob oracle sample head {h}")
        s = orc.attn_bwd_bwd_sampled(x["q"], x["k"], x["v"], x["do"], x["gq"], x["gk"], x["gv"],
                                     w.scale, True, 0, h, rows, cols, row_block=1024)
        got = {"hQ": _host(hq[0, rows, h]), "hdO": _host(hdo[0, rows, h]),
               "hK": _host(hk[0, cols, h]), "hV": _host(hv[0, cols, h])}
        # sampled rows as one (b, h) slice [1, rows, 1, d]; r and E [1, 1, N]
        g = {n: v[None, :, None, :] for n, v in got.items()}
        r = {n: s[n][None, :, None, :] for n in got}
        for n, i in (("r", 2), ("E", 3)):
            g[n], r[n] = _host(ws[i, 0, h])[None, None, :], s[n][None, None, :]
        gpu_check.check(f"c5_bob sampled head {h}", g, r, "bf16",
                        names=("hQ", "hK", "hV", "hdO", "r", "E"))
