"""Pins for the oracle's backward of the backward (CPU only).

l2 = <gQ, dQ> + <gK, dK> + <gV, dV> is a scalar function of (Q, K, V, dO)
through the first backward.  The oracle's closed form of its gradient is
checked against: torch's CPU fp64 double backward (autograd through an
attention written with plain tensor ops, create_graph=True); central
finite differences of l2 evaluated with the first-backward oracle (which
shares no step with the closed form); masks (causal, full, block-sparse,
rows that keep no key); and invariants of the two row scalars.
"""

import math

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc


def _rand(B, H, N, d, seed, std=1.0):
    x = workloads.make_random(B, H, N, d, "f32", seed=seed, qkv_std=std)
    rng = np.random.default_rng(seed + 100)
    g = {n: rng.standard_normal((B, N, H, d)) for n in ("gq", "gk", "gv")}
    return dict({k: v.astype(np.float64) for k, v in x.items()}, **g)


def _l2(x, scale, causal, bm=None, mb=orc.MASK_BLOCK):
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal, bm, mb)
    return float((x["gq"] * g["dQ"]).sum() + (x["gk"] * g["dK"]).sum()
                 + (x["gv"] * g["dV"]).sum())


def _bob(x, scale, causal, bm=None, mb=orc.MASK_BLOCK):
    return orc.attn_bwd_bwd(x["q"], x["k"], x["v"], x["do"], x["gq"], x["gk"], x["gv"],
                            scale, causal, bm, mb)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_fp64_double_backward(causal):
    torch = pytest.importorskip("torch")
    for (B, H, N, d, seed) in ((1, 2, 9, 4, 0), (2, 1, 23, 8, 1)):
        x = _rand(B, H, N, d, seed)
        scale = 1 / math.sqrt(d)
        t = {n: torch.tensor(x[n], dtype=torch.float64).permute(0, 2, 1, 3).contiguous()
             for n in x}
        for n in ("q", "k", "v", "do"):
            t[n].requires_grad_(True)
        s = scale * t["q"] @ t["k"].transpose(-1, -2)
        if causal:
            s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
        o = torch.softmax(s, dim=-1) @ t["v"]
        dq, dk, dv = torch.autograd.grad(o, (t["q"], t["k"], t["v"]), t["do"], create_graph=True)
        l2 = (t["gq"] * dq).sum() + (t["gk"] * dk).sum() + (t["gv"] * dv).sum()
        hq, hk, hv, hdo = torch.autograd.grad(l2, (t["q"], t["k"], t["v"], t["do"]))
        got = _bob(x, scale, causal)

        def back(a):
            return a.detach().permute(0, 2, 1, 3).numpy()
        for name, ref in (("hQ", hq), ("hK", hk), ("hV", hv), ("hdO", hdo)):
            np.testing.assert_allclose(got[name], back(ref), rtol=1e-10, atol=1e-12,
                                       err_msg=name)


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_of_the_first_backward(causal):
    x = _rand(1, 2, 7, 3, seed=5)
    scale = 0.6
    got = _bob(x, scale, causal)
    grads = {"q": got["hQ"], "k": got["hK"], "v": got["hV"], "do": got["hdO"]}
    worst = 0.0
    for key in ("q", "k", "v", "do"):
        for idx in np.ndindex(*x[key].shape):
            y = {k: v.copy() for k, v in x.items()}
            y[key][idx] += 1e-6
            lp = _l2(y, scale, causal)
            y[key][idx] -= 2e-6
            lm = _l2(y, scale, causal)
            worst = max(worst, abs((lp - lm) / 2e-6 - grads[key][idx]))
    assert worst <= 1e-7, worst


def test_finite_differences_with_a_block_mask_and_empty_rows():
    n, mb = 7, 2
    x = _rand(1, 1, n, 3, seed=6)
    bm = np.array([[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 1]], dtype=np.uint8)
    for causal in (True, False):
        got = _bob(x, 0.7, causal, bm, mb)
        grads = {"q": got["hQ"], "k": got["hK"], "v": got["hV"], "do": got["hdO"]}
        worst = 0.0
        for key in ("q", "k", "v", "do"):
            for idx in np.ndindex(*x[key].shape):
                y = {k: v.copy() for k, v in x.items()}
                y[key][idx] += 1e-6
                lp = _l2(y, 0.7, causal, bm, mb)
                y[key][idx] -= 2e-6
                lm = _l2(y, 0.7, causal, bm, mb)
                worst = max(worst, abs((lp - lm) / 2e-6 - grads[key][idx]))
        assert worst <= 1e-7, (causal, worst)
        # rows 2, 3 keep no key: nothing flows through them
        assert np.all(got["hQ"][:, 2:4] == 0.0) and np.all(got["hdO"][:, 2:4] == 0.0)
        assert np.all(got["r"][:, :, 2:4] == 0.0) and np.all(got["E"][:, :, 2:4] == 0.0)


def test_row_scalars_are_weighted_sums():
    # r_i = sum_j P_ij G_ij with G = scale (gQ K^T + Q gK^T) equals
    # scale (gQ_i . (P K)_i + Q_i . (P gK)_i): two attention outputs
    x = _rand(1, 1, 11, 5, seed=8)
    scale = 0.4
    got = _bob(x, scale, True)
    q, k, gq, gk = (x[n][0, :, 0] for n in ("q", "k", "gq", "gk"))
    _, _, p = orc.head_forward(q, k, x["v"][0, :, 0], scale, True)
    r = scale * ((gq * (p @ k)).sum(axis=1) + (q * (p @ gk)).sum(axis=1))
    np.testing.assert_allclose(got["r"][0, 0], r, rtol=1e-12, atol=1e-14)


def test_zero_cotangents_give_zero_and_gv_alone_is_linear():
    x = _rand(1, 2, 6, 4, seed=9)
    z = dict(x, gq=0 * x["gq"], gk=0 * x["gk"], gv=0 * x["gv"])
    got = _bob(z, 0.5, True)
    for n in ("hQ", "hK", "hV", "hdO"):
        assert np.all(got[n] == 0.0)
    # l2 is linear in the cotangents: doubling them doubles every output
    two = dict(x, gq=2 * x["gq"], gk=2 * x["gk"], gv=2 * x["gv"])
    a, b = _bob(x, 0.5, False), _bob(two, 0.5, False)
    for n in ("hQ", "hK", "hV", "hdO"):
        np.testing.assert_allclose(b[n], 2 * a[n], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_evaluator_equals_full_oracle(causal):
    x = _rand(2, 2, 70, 16, seed=11)
    full = _bob(x, 0.25, causal)
    rows, cols = [0, 1, 33, 69], [0, 5, 64, 69]
    s = orc.attn_bwd_bwd_sampled(x["q"], x["k"], x["v"], x["do"], x["gq"], x["gk"], x["gv"],
                                 0.25, causal, 1, 0, rows, cols, row_block=16)
    for name, idx in (("hQ", rows), ("hdO", rows), ("hK", cols), ("hV", cols)):
        np.testing.assert_allclose(s[name], full[name][1, idx, 0], rtol=1e-11, atol=1e-13,
                                   err_msg=name)
    np.testing.assert_allclose(s["r"], full["r"][1, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["E"], full["E"][1, 0], rtol=1e-11, atol=1e-13)
