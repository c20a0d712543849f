"""Backward of the backward: HIP path vs the fp64 oracle through the C ABI.

Relative Frobenius error per output tensor (hQ, hK, hV, hdO) and for the two
row scalars r and E the kernels leave in the workspace, gated per tensor, per
(b, h) and per row as in the first backward's tests (``tests/gpu_check.py``).
Two feeds of O and L: the library's own forward, and the oracle's O and L
cast to the device type.  The block-masked form is checked the same way
against the oracle with the mask, plus two exact checks: an all-ones mask
reproduces the unmasked call bit for bit, and an all-zeros mask gives zeros.
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


# block masks: B, H, N, d, dtype, causal, mask recipe (tests/test_gpu_mask_parity.py)
MASKED = [
    (1, 2, 300, 64, "f32", True, "random_heads"),
    (2, 1, 260, 32, "f32", False, "random_empty"),      # rows keeping no key
    (1, 2, 1000, 128, "bf16", True, "random"),
    (1, 2, 700, 128, "bf16", False, "random_empty"),
    (1, 1, 1100, 128, "bf16", True, "window"),           # local window + sink blocks
    (1, 2, 513, 64, "bf16", True, "random_empty"),       # ragged last tile
]


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "x".join(map(str, c)))
def test_masked_bwd_bwd_parity(B, case):
    import torch
    from tests.test_gpu_mask_parity import _mask
    Bn, H, N, d, dtype, causal, recipe = case
    scale = 1.0 / math.sqrt(d)
    x = workloads.make_random(Bn, H, N, d, dtype, seed=N + d + 1,
                              qkv_std=0.5 if dtype == "bf16" else 1.0)
    x.update(workloads.make_cotangents(Bn, H, N, d, dtype, seed=N + 1))
    m = _mask(recipe, Bn, H, N, seed=N + 2)
    xs = {n: x[n].astype(np.float64) for n in x}
    O, L = orc.attn_fwd(xs["q"], xs["k"], xs["v"], scale, causal, m)
    ref = orc.attn_bwd_bwd(xs["q"], xs["k"], xs["v"], xs["do"], xs["gq"], xs["gk"], xs["gv"],
                           scale, causal, m)
    t = {n: _dev(x[n], dtype) for n in x}
    mask = torch.from_numpy(m).cuda()
    empty = np.isneginf(L)                                         # rows keeping no key
    for feed in ("own", "oracle"):
        _say(f"masked {case} feed={feed}")
        if feed == "own":
            o, lse = B.attn_fwd_lse_masked(t["q"], t["k"], t["v"], mask, causal=causal,
                                           scale=scale)
        else:
            o = _dev(O, dtype)
            lse = torch.from_numpy(np.ascontiguousarray(L, dtype=np.float32)).cuda()
        ws = torch.empty((4, Bn, H, N), dtype=torch.float32, device="cuda")
        hq, hk, hv, hdo = B.attn_bwd_bwd_masked(t["q"], t["k"], t["v"], o, t["do"], lse, t["gq"],
                                                t["gk"], t["gv"], mask, causal=causal,
                                                scale=scale, workspace=ws)
        torch.cuda.synchronize()
        got = {"hQ": _host(hq), "hK": _host(hk), "hV": _host(hv), "hdO": _host(hdo),
               "r": _host(ws[2]), "E": _host(ws[3])}
        for n, a in got.items():
            assert np.isfinite(a).all(), (case, feed, n)
        gpu_check.check(f"masked bob {case} feed={feed}", got, ref, dtype,
                        names=("hQ", "hK", "hV", "hdO", "r", "E"))
        if empty.any():
            for n in ("hQ", "hdO"):
                assert np.all(np.transpose(got[n], (0, 2, 1, 3))[empty] == 0.0), (case, feed, n)
            assert np.all(got["r"][empty] == 0.0) and np.all(got["E"][empty] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_masked_bwd_bwd_all_ones_equals_unmasked_bitwise(B, causal):
    import torch
    n, d = 700, 128
    _say(f"bob all-ones mask causal={causal}")
    x = workloads.make_random(1, 2, n, d, "bf16", seed=11, qkv_std=0.5)
    x.update(workloads.make_cotangents(1, 2, n, d, "bf16", seed=12))
    t = {k: _dev(v, "bf16") for k, v in x.items()}
    ones = torch.ones(((n + 127) // 128,) * 2, dtype=torch.uint8, device="cuda")
    o, lse = B.attn_fwd_lse(t["q"], t["k"], t["v"], causal=causal)
    args = (t["q"], t["k"], t["v"], o, t["do"], lse, t["gq"], t["gk"], t["gv"])
    ws0 = torch.empty((4, 1, 2, n), dtype=torch.float32, device="cuda")
    ws1 = torch.empty_like(ws0)
    g0 = B.attn_bwd_bwd(*args, causal=causal, workspace=ws0)
    g1 = B.attn_bwd_bwd_masked(*args, ones, causal=causal, workspace=ws1)
    torch.cuda.synchronize()
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ws0, ws1)


def test_masked_bwd_bwd_all_zeros_gives_zeros(B):
    import torch
    n, d = 384, 64
    _say("bob all-zeros mask")
    x = workloads.make_random(1, 2, n, d, "bf16", seed=13, qkv_std=0.5)
    x.update(workloads.make_cotangents(1, 2, n, d, "bf16", seed=14))
    t = {k: _dev(v, "bf16") for k, v in x.items()}
    zeros = torch.zeros((3, 3), dtype=torch.uint8, device="cuda")
    o, lse = B.attn_fwd_lse_masked(t["q"], t["k"], t["v"], zeros)
    out = B.attn_bwd_bwd_masked(t["q"], t["k"], t["v"], o, t["do"], lse, t["gq"], t["gk"],
                                t["gv"], zeros)
    torch.cuda.synchronize()
    for a in out:
        assert torch.all(a == 0)
