"""Pins for the oracle's block-sparse masks (CPU only).

A block mask keeps or drops whole mask_block x mask_block groups of (query,
key) pairs, on top of the causal rule.  Each test ties the masked oracle to
something other than itself: the unmasked oracle (all-ones mask), separate
sequences (block-diagonal mask), torch's CPU fp64 attention with an explicit
boolean mask and autograd, central finite differences of the loss, a
brute-force loop over pairs, and the closed form of a row with no kept key.
"""

import math

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc


def _rand(B, H, N, d, seed, std=1.0):
    x = workloads.make_random(B, H, N, d, "f32", seed=seed, qkv_std=std)
    return {k: v.astype(np.float64) for k, v in x.items()}


def _nb(n, mb):
    return (n + mb - 1) // mb


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,mb", [(10, 4), (200, 128)])
def test_all_ones_mask_is_the_unmasked_oracle(causal, n, mb):
    x = _rand(2, 2, n, 8, seed=n)
    ones = np.ones((_nb(n, mb), _nb(n, mb)), dtype=np.uint8)
    O0, L0 = orc.attn_fwd(x["q"], x["k"], x["v"], 0.3, causal)
    O1, L1 = orc.attn_fwd(x["q"], x["k"], x["v"], 0.3, causal, ones, mb)
    g0 = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.3, causal)
    g1 = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.3, causal, ones, mb)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(L0, L1)
    for key in ("dQ", "dK", "dV"):
        np.testing.assert_array_equal(g0[key], g1[key])


@pytest.mark.parametrize("causal", [True, False])
def test_block_diagonal_mask_is_independent_sequences(causal):
    # blocks [0, 4), [4, 8), [8, 10): attention never crosses a block, so each
    # block is a sequence of its own
    n, mb = 10, 4
    x = _rand(1, 2, n, 6, seed=3)
    bm = np.eye(_nb(n, mb), dtype=np.uint8)
    O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.4, causal, bm, mb)
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.4, causal, bm, mb)
    for r0 in range(0, n, mb):
        r1 = min(n, r0 + mb)
        part = {k: v[:, r0:r1] for k, v in x.items()}
        Op, Lp = orc.attn_fwd(part["q"], part["k"], part["v"], 0.4, causal)
        gp = orc.attn_bwd(part["q"], part["k"], part["v"], part["do"], 0.4, causal)
        np.testing.assert_allclose(O[:, r0:r1], Op, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(L[:, :, r0:r1], Lp, rtol=1e-13, atol=1e-15)
        for key in ("dQ", "dK", "dV"):
            np.testing.assert_allclose(g[key][:, r0:r1], gp[key], rtol=1e-12, atol=1e-14)


def _mask_with_live_rows(rng, nb, causal):
    bm = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    np.fill_diagonal(bm, 1)          # every row keeps its own block, so no row is empty
    return bm


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_cpu_fp64_sdpa_with_boolean_mask(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    for (B, H, N, d, mb) in ((2, 2, 13, 8, 3), (1, 3, 40, 16, 8)):
        x = _rand(B, H, N, d, seed=N)
        scale = 1 / math.sqrt(d)
        bm = np.stack([np.stack([_mask_with_live_rows(rng, _nb(N, mb), causal) for _ in range(H)])
                       for _ in range(B)])
        keep = np.stack([np.stack([orc.keep_mask(N, N, causal, bm[b, h], mb) for h in range(H)])
                         for b in range(B)])
        t = {n: torch.tensor(x[n], dtype=torch.float64).permute(0, 2, 1, 3).contiguous()
             for n in ("q", "k", "v", "do")}
        for n in ("q", "k", "v"):
            t[n].requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            t["q"], t["k"], t["v"], attn_mask=torch.tensor(keep), scale=scale)
        o.backward(t["do"])
        O, _ = orc.attn_fwd(x["q"], x["k"], x["v"], scale, causal, bm, mb)
        g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal, bm, mb)

        def back(a):
            return a.detach().permute(0, 2, 1, 3).numpy()
        assert np.allclose(O, back(o), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dQ"], back(t["q"].grad), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dK"], back(t["k"].grad), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dV"], back(t["v"].grad), rtol=1e-12, atol=1e-14)


def _brute_forward_head(q, k, v, scale, keep):
    """O and L by explicit loops over pairs, with no array softmax."""
    n, dv = q.shape[0], v.shape[1]
    o = np.zeros((n, dv))
    lse = np.full(n, -np.inf)
    for i in range(n):
        kept = [j for j in range(n) if keep[i][j]]
        if not kept:
            continue
        sc = {j: scale * sum(q[i, c] * k[j, c] for c in range(q.shape[1])) for j in kept}
        top = max(sc.values())
        z = sum(math.exp(sc[j] - top) for j in kept)
        for j in kept:
            o[i] += math.exp(sc[j] - top) / z * v[j]
        lse[i] = top + math.log(z)
    return o, lse


def test_brute_force_loops_with_an_empty_block_row():
    n, mb = 7, 2
    x = _rand(1, 1, n, 3, seed=9)
    bm = np.array([[1, 0, 0, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 1]], dtype=np.uint8)
    for causal in (True, False):
        keep = orc.keep_mask(n, n, causal, bm, mb)
        O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.7, causal, bm, mb)
        ob, lb = _brute_forward_head(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], 0.7, keep)
        np.testing.assert_allclose(O[0, :, 0], ob, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(np.isinf(L[0, 0]), np.isinf(lb))
        live = np.isfinite(lb)
        np.testing.assert_allclose(L[0, 0][live], lb[live], rtol=1e-13)


def _loss(x, scale, causal, bm, mb, key=None, idx=None, delta=0.0):
    y = {k: v.copy() for k, v in x.items()}
    if key is not None:
        y[key][idx] += delta
    O, _ = orc.attn_fwd(y["q"], y["k"], y["v"], scale, causal, bm, mb)
    return float((y["do"] * O).sum())


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_with_empty_rows(causal):
    # block row 1 keeps nothing: rows 2, 3 have no kept key
    n, mb = 7, 2
    x = _rand(1, 2, n, 3, seed=4)
    bm = np.array([[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 1]], dtype=np.uint8)
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.6, causal, bm, mb)
    grads = {"q": g["dQ"], "k": g["dK"], "v": g["dV"]}
    worst = 0.0
    for key in "qkv":
        for idx in np.ndindex(*x[key].shape):
            fd = (_loss(x, 0.6, causal, bm, mb, key, idx, 1e-6)
                  - _loss(x, 0.6, causal, bm, mb, key, idx, -1e-6)) / 2e-6
            worst = max(worst, abs(fd - grads[key][idx]))
    assert worst <= 1e-7, worst


def test_empty_rows_closed_form():
    n, mb = 9, 3
    x = _rand(2, 1, n, 4, seed=2)
    bm = np.ones((3, 3), dtype=np.uint8)
    bm[1] = 0                                         # rows 3, 4, 5 keep no key
    for causal in (True, False):
        O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.5, causal, bm, mb)
        g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.5, causal, bm, mb)
        assert np.all(O[:, 3:6] == 0.0)
        assert np.all(np.isneginf(L[:, :, 3:6]))
        assert np.all(np.isfinite(L[:, :, :3])) and np.all(np.isfinite(L[:, :, 6:]))
        assert np.all(g["dQ"][:, 3:6] == 0.0)
        assert np.all(g["D"][:, :, 3:6] == 0.0)
        # sum rules over the rows that keep keys: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
        live = np.r_[0:3, 6:9]
        np.testing.assert_allclose(g["dV"].sum(axis=1), x["do"][:, live].sum(axis=1), atol=1e-12)
        np.testing.assert_allclose(g["dK"].sum(axis=1), 0.0, atol=1e-12)


def test_mask_per_head_selects_each_heads_mask():
    n, mb = 8, 4
    x = _rand(2, 3, n, 4, seed=8)
    rng = np.random.default_rng(1)
    bm = (rng.random((2, 3, 2, 2)) < 0.6).astype(np.uint8)
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.5, False, bm, mb)
    for b in range(2):
        for h in range(3):
            one = {k: v[b:b + 1, :, h:h + 1] for k, v in x.items()}
            gh = orc.attn_bwd(one["q"], one["k"], one["v"], one["do"], 0.5, False, bm[b, h], mb)
            for key in ("dQ", "dK", "dV"):
                np.testing.assert_array_equal(g[key][b, :, h], gh[key][0, :, 0])


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_evaluator_with_mask_equals_full_oracle(causal):
    n, mb = 70, 16
    x = _rand(1, 2, n, 8, seed=12)
    rng = np.random.default_rng(3)
    bm = (rng.random((2, _nb(n, mb), _nb(n, mb))) < 0.5).astype(np.uint8)[None]
    bm[0, 1, 2, :] = 0                                # query rows 32..47 of head 1 keep nothing
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.25, causal, bm, mb)
    O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.25, causal, bm, mb)
    rows = [0, 1, 33, 40, 69]
    cols = [0, 5, 33, 64, 69]
    s = orc.attn_bwd_sampled(x["q"], x["k"], x["v"], x["do"], 0.25, causal, 0, 1, rows, cols,
                             row_block=16, block_mask=bm, mask_block=mb)
    np.testing.assert_allclose(s["dQ"], g["dQ"][0, rows, 1], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["O"], O[0, rows, 1], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["dK"], g["dK"][0, cols, 1], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["dV"], g["dV"][0, cols, 1], rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(s["L"], L[0, 1])
