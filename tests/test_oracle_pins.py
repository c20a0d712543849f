"""Pins that tie the fp64 oracle to something other than itself (CPU only).

Each test checks the oracle against a fact fixed by the pages or by the
mathematics: printed table sizes, central finite differences of the loss,
the shift-cancellation identity, sum rules, metamorphic shifts, closed forms,
scipy's logsumexp and torch's CPU fp64 attention with autograd.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c1(seed=0):
    w = workloads.get("c1_tiny")
    x = workloads.make_inputs(w, seed)
    return w, {k: v.astype(np.float64) for k, v in x.items()}


def _rand(B, H, N, d, seed, std=1.0):
    x = workloads.make_random(B, H, N, d, "f32", seed=seed, qkv_std=std)
    return {k: v.astype(np.float64) for k, v in x.items()}


# ---------------------------------------------------------------- P1 counts

def test_pair_counts_match_printed_table_sizes():
    with open(os.path.join(GOLDEN, "plan_row_counts.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if "pairs" in c:
            assert orc.pair_count(c["B"], c["H"], c["N"], c["causal"]) == c["pairs"], c["cite"]
        elif "pairs_approx" in c:
            got = orc.pair_count(c["B"], c["H"], c["N"], c["causal"])
            assert abs(got - c["pairs_approx"]) <= c["rel_tol"] * c["pairs_approx"], c["cite"]
        elif "rows" in c:
            q = np.zeros((c["B"], c["N"], c["H"], 4))
            _, L = orc.attn_fwd(q, q, q, 0.5, True)
            assert L.size == c["rows"], c["cite"]
        elif "elements" in c:
            q = np.zeros((c["B"], c["N"], c["H"], c["d"]))
            O, _ = orc.attn_fwd(q, q, q, 0.5, True)
            assert O.size == c["elements"], c["cite"]


def test_c1_inputs_follow_the_repro_recipe():
    # sin(flat * 0.37 + phase), row-major over (seq, pos, head, channel)
    w, x = _c1()
    assert x["q"].shape == (3, 8, 2, 4)
    flat = np.arange(192)
    for name, ph in (("q", 0.0), ("k", 1.0), ("v", 2.0)):
        want = np.sin(flat * 0.37 + ph).astype(np.float32).astype(np.float64)
        np.testing.assert_array_equal(x[name].ravel(), want)
    # index (s, t, h, c) -> flat = ((s*8 + t)*2 + h)*4 + c
    assert x["k"][2, 5, 1, 3] == np.float32(np.sin((((2 * 8 + 5) * 2 + 1) * 4 + 3) * 0.37 + 1.0))


# ---------------------------------------------------------------- P2 finite differences

def _head_loss(x, b, h, scale, causal, key=None, idx=None, delta=0.0):
    q = x["q"][b, :, h].copy()
    k = x["k"][b, :, h].copy()
    v = x["v"][b, :, h].copy()
    if key is not None:
        {"q": q, "k": k, "v": v}[key][idx] += delta
    o, _, _ = orc.head_forward(q, k, v, scale, causal)
    return float((x["do"][b, :, h] * o).sum())


def _fd_check(x, scale, causal, entries, step=1e-6, atol=1e-7):
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
    grads = {"q": g["dQ"], "k": g["dK"], "v": g["dV"]}
    worst = 0.0
    for key, (b, n, h, c) in entries:
        lp = _head_loss(x, b, h, scale, causal, key, (n, c), +step)
        lm = _head_loss(x, b, h, scale, causal, key, (n, c), -step)
        fd = (lp - lm) / (2 * step)
        worst = max(worst, abs(fd - grads[key][b, n, h, c]))
    assert worst <= atol, worst
    return worst


def test_finite_differences_c1_every_input():
    w, x = _c1()
    entries = [(key, idx) for key in "qkv" for idx in np.ndindex(*w.shape)]
    assert len(entries) == 576
    _fd_check(x, w.scale, True, entries)


def test_finite_differences_c1_pages_loss():
    # The pages' own loss is sum(O^2)/2, whose output cotangent is dO = O.
    w, x = _c1()
    O, _ = orc.attn_fwd(x["q"], x["k"], x["v"], w.scale, True)
    x = dict(x, do=O)

    def half_sq(b, h, key, idx, delta):
        q = x["q"][b, :, h].copy(); k = x["k"][b, :, h].copy(); v = x["v"][b, :, h].copy()
        {"q": q, "k": k, "v": v}[key][idx] += delta
        o, _, _ = orc.head_forward(q, k, v, w.scale, True)
        return 0.5 * float((o * o).sum())

    g = orc.attn_bwd(x["q"], x["k"], x["v"], O, w.scale, True)
    grads = {"q": g["dQ"], "k": g["dK"], "v": g["dV"]}
    worst = 0.0
    for key in "qkv":
        for (b, n, h, c) in np.ndindex(*w.shape):
            fd = (half_sq(b, h, key, (n, c), 1e-6) - half_sq(b, h, key, (n, c), -1e-6)) / 2e-6
            worst = max(worst, abs(fd - grads[key][b, n, h, c]))
    assert worst <= 1e-7, worst


def test_finite_differences_c2_sampled_entries():
    w = workloads.get("c2_nanogpt_cpu")
    x = {k: v.astype(np.float64) for k, v in workloads.make_inputs(w, 0).items()}
    rng = np.random.default_rng(123)
    entries = []
    for _ in range(200):
        key = "qkv"[rng.integers(3)]
        entries.append((key, tuple(int(rng.integers(s)) for s in w.shape)))
    _fd_check(x, w.scale, True, entries)


def test_finite_differences_noncausal():
    x = _rand(1, 2, 9, 8, seed=5)
    entries = [(key, idx) for key in "qkv" for idx in np.ndindex(1, 9, 2, 8)][::3]
    _fd_check(x, 1.0 / math.sqrt(8), False, entries)


# ---------------------------------------------------------------- P3 shift cancels

@pytest.mark.parametrize("causal", [True, False])
def test_ds_rows_sum_to_zero_and_max_shift_gradient_cancels(causal):
    x = _rand(2, 3, 33, 16, seed=1)
    scale = 0.25
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
    for b in range(2):
        for h in range(3):
            q, k, v, do = (x[n][b, :, h] for n in ("q", "k", "v", "do"))
            _, _, _, _, _, p, _, _ = orc.head_backward(q, k, v, do, scale, causal)
            dp = do @ v.T
            ds, _ = orc.softmax_backward(p, dp)
            bound = 1e-12 * np.abs(ds).sum(axis=1) + 1e-300
            assert np.all(np.abs(g["dS_rowsum"][b, h]) <= bound)
            sbar, mbar = orc.literal_backward_head(q, k, v, do, scale, causal)
            np.testing.assert_allclose(sbar, ds, rtol=1e-11, atol=1e-14)
            assert np.all(np.abs(mbar) <= 1e-12 * np.abs(sbar).sum(axis=1) + 1e-300)


# ---------------------------------------------------------------- P4 / P5 sum rules

def test_sum_rules():
    x = _rand(2, 2, 40, 8, seed=2)
    scale = 1 / math.sqrt(8)
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, True)
    # softmax rows sum to 1  =>  sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(g["dV"].sum(axis=1), x["do"].sum(axis=1), rtol=1e-12, atol=1e-12)
    # rows of dS sum to 0  =>  sum_j dK_j = 0
    assert np.all(np.abs(g["dK"].sum(axis=1)) <= 1e-12 * np.abs(g["dK"]).sum(axis=1) + 1e-300)
    # <Q, dQ> = <K, dK> per (b, h): both equal scale * sum_ij dS_ij q_i.k_j
    lhs = np.einsum("bnhc,bnhc->bh", x["q"], g["dQ"])
    rhs = np.einsum("bnhc,bnhc->bh", x["k"], g["dK"])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- P6 metamorphic

def test_constant_shift_of_values_or_keys_leaves_gradients_unchanged():
    x = _rand(1, 2, 24, 8, seed=3)
    scale = 0.3
    base = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, True)
    c = np.random.default_rng(9).standard_normal(8)
    for key in ("v", "k"):
        y = dict(x)
        y[key] = x[key] + c
        got = orc.attn_bwd(y["q"], y["k"], y["v"], y["do"], scale, True)
        for t in ("dQ", "dK", "dV"):
            np.testing.assert_allclose(got[t], base[t], rtol=1e-10, atol=1e-12)
    # and O shifts by exactly c when V does
    O0, _ = orc.attn_fwd(x["q"], x["k"], x["v"], scale, True)
    O1, _ = orc.attn_fwd(x["q"], x["k"], x["v"] + c, scale, True)
    np.testing.assert_allclose(O1 - O0, np.broadcast_to(c, O0.shape), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P7 D and L

def test_D_equals_rowsum_dO_O_and_L_is_logsumexp():
    x = _rand(2, 2, 50, 16, seed=4)
    scale = 0.25
    for causal in (True, False):
        O, L = orc.attn_fwd(x["q"], x["k"], x["v"], scale, causal)
        g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
        D2 = np.einsum("bnhc,bnhc->bhn", x["do"], O)
        np.testing.assert_allclose(g["D"], D2, rtol=1e-12, atol=1e-12)
        for b in range(2):
            for h in range(2):
                s = scale * np.einsum("ic,jc->ij", x["q"][b, :, h], x["k"][b, :, h])
                if causal:
                    s = np.where(np.tril(np.ones((50, 50), dtype=bool)), s, -np.inf)
                np.testing.assert_allclose(L[b, h], scipy.special.logsumexp(s, axis=1),
                                           rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- P8 closed forms

def test_closed_form_zero_queries():
    # Q = 0: every kept score is 0, so P_ij = 1/(i+1) for j <= i.
    rng = np.random.default_rng(7)
    N, d, scale = 12, 4, 0.7
    q = np.zeros((1, N, 1, d))
    k = rng.standard_normal((1, N, 1, d))
    v = rng.standard_normal((1, N, 1, d))
    do = rng.standard_normal((1, N, 1, d))
    O, L = orc.attn_fwd(q, k, v, scale, True)
    g = orc.attn_bwd(q, k, v, do, scale, True)
    K, V, G = k[0, :, 0], v[0, :, 0], do[0, :, 0]
    for i in range(N):
        assert abs(L[0, 0, i] - math.log(i + 1)) <= 1e-14
        mean_v = sum(V[j] for j in range(i + 1)) / (i + 1)
        np.testing.assert_allclose(O[0, i, 0], mean_v, rtol=1e-13, atol=1e-14)
        want_dq = np.zeros(d)
        for j in range(i + 1):
            want_dq += (G[i] @ (V[j] - mean_v)) * K[j]
        want_dq *= scale / (i + 1)
        np.testing.assert_allclose(g["dQ"][0, i, 0], want_dq, rtol=1e-12, atol=1e-14)
    for j in range(N):
        want_dv = sum(G[i] / (i + 1) for i in range(j, N))
        np.testing.assert_allclose(g["dV"][0, j, 0], want_dv, rtol=1e-12, atol=1e-14)
    assert np.all(g["dK"] == 0.0)


def test_closed_form_single_position_and_first_row():
    x = _rand(2, 3, 1, 8, seed=8)
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.5, True)
    O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.5, True)
    np.testing.assert_array_equal(O, x["v"])
    np.testing.assert_array_equal(g["dV"], x["do"])
    assert np.all(g["dQ"] == 0.0) and np.all(g["dK"] == 0.0)
    # causal row 0 attends only to itself: its dS row is exactly zero
    y = _rand(1, 2, 16, 8, seed=9)
    g = orc.attn_bwd(y["q"], y["k"], y["v"], y["do"], 0.5, True)
    assert np.all(g["dQ"][:, 0] == 0.0)


# ---------------------------------------------------------------- P9 library routine

@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_cpu_fp64_sdpa_autograd(causal):
    torch = pytest.importorskip("torch")
    for (B, H, N, d, seed) in ((3, 2, 8, 4, 0), (2, 3, 37, 16, 1)):
        if (B, N) == (3, 8):
            w, x = _c1()
            scale = w.scale
        else:
            x = _rand(B, H, N, d, seed)
            scale = 1 / math.sqrt(d)
        t = {n: torch.tensor(x[n], dtype=torch.float64).permute(0, 2, 1, 3).contiguous()
             for n in ("q", "k", "v", "do")}
        for n in ("q", "k", "v"):
            t[n].requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            t["q"], t["k"], t["v"], is_causal=causal, scale=scale)
        o.backward(t["do"])
        O, _ = orc.attn_fwd(x["q"], x["k"], x["v"], scale, causal)
        g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)

        def back(a):
            return a.detach().permute(0, 2, 1, 3).numpy()
        # the pages' own tolerance for gradient agreement in fp64
        assert np.allclose(O, back(o), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dQ"], back(t["q"].grad), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dK"], back(t["k"].grad), rtol=1e-12, atol=1e-14)
        assert np.allclose(g["dV"], back(t["v"].grad), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- sampled evaluator

@pytest.mark.parametrize("causal", [True, False])
def test_sampled_evaluator_equals_full_oracle(causal):
    x = _rand(2, 2, 70, 16, seed=11)
    scale = 0.25
    g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
    O, L = orc.attn_fwd(x["q"], x["k"], x["v"], scale, causal)
    rows = [0, 1, 33, 69]
    cols = [0, 5, 64, 69]
    s = orc.attn_bwd_sampled(x["q"], x["k"], x["v"], x["do"], scale, causal, 1, 0,
                             rows, cols, row_block=16)
    np.testing.assert_allclose(s["dQ"], g["dQ"][1, rows, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["O"], O[1, rows, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["dK"], g["dK"][1, cols, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["dV"], g["dV"][1, cols, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s["L"], L[1, 0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["D"], g["D"][1, 0], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- forward outputs of attn_bwd

def test_attn_bwd_reports_the_forward_outputs_of_attn_fwd():
    # attn_bwd hands back O and L as computed on its way to the gradient; they
    # must be attn_fwd's values bit for bit (attn_fwd is pinned above by
    # scipy's logsumexp, closed forms and torch), causal and full, with a
    # block mask too.
    x = _rand(2, 3, 150, 16, seed=11)
    bm = workloads.make_block_mask(150, 0.6, seed=3, keep_diagonal=False, empty_rows=(1,))
    for causal, mask in ((True, None), (False, None), (True, bm)):
        O, L = orc.attn_fwd(x["q"], x["k"], x["v"], 0.25, causal, mask)
        g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.25, causal, mask)
        np.testing.assert_array_equal(g["O"], O)
        np.testing.assert_array_equal(g["L"], L)
