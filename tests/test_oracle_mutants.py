"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch them.

Each mutant replaces one step function of the oracle module for the duration
of a test.  A quick battery of the pins (pair count, finite differences,
shift cancellation, sum rules, torch's fp64 attention) must report at least
one failure for every mutant, and none for the unmodified oracle.
"""

import math

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc


def _battery():
    """Return the names of the pins that fail for the oracle as it stands."""
    torch = pytest.importorskip("torch")
    fails = []
    w = workloads.get("c1_tiny")
    x = {k: v.astype(np.float64) for k, v in workloads.make_inputs(w, 0).items()}
    with np.errstate(all="ignore"):
        # P1: the causal mask keeps 216 pairs at the toy size
        try:
            if orc.pair_count(3, 2, 8, True) != 216:
                fails.append("P1")
        except Exception:
            fails.append("P1")
        try:
            g = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], w.scale, True)
        except Exception:
            return fails + ["crash"]
        # P2: central differences on a sample of inputs
        rng = np.random.default_rng(0)
        worst = 0.0
        for _ in range(40):
            key = "qkv"[rng.integers(3)]
            b, n, h, c = (int(rng.integers(s)) for s in w.shape)
            vals = []
            for sgn in (1, -1):
                y = {kk: vv.copy() for kk, vv in x.items()}
                y[key][b, n, h, c] += sgn * 1e-6
                O, _ = orc.attn_fwd(y["q"], y["k"], y["v"], w.scale, True)
                vals.append(float((y["do"] * O).sum()))
            fd = (vals[0] - vals[1]) / 2e-6
            grad = {"q": g["dQ"], "k": g["dK"], "v": g["dV"]}[key][b, n, h, c]
            worst = max(worst, abs(fd - grad)) if np.isfinite(grad) else np.inf
        if not worst <= 1e-7:
            fails.append("P2")
        # P3: rows of dS sum to zero
        if not np.all(np.abs(g["dS_rowsum"]) <= 1e-12):
            fails.append("P3")
        # P4: sum_j dV_j = sum_i dO_i
        if not np.allclose(g["dV"].sum(axis=1), x["do"].sum(axis=1), rtol=1e-12, atol=1e-12):
            fails.append("P4")
        # P9: torch's CPU fp64 attention with autograd
        t = {n: torch.tensor(x[n]).permute(0, 2, 1, 3).contiguous() for n in ("q", "k", "v", "do")}
        for n in ("q", "k", "v"):
            t[n].requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            t["q"], t["k"], t["v"], is_causal=True, scale=w.scale)
        o.backward(t["do"])
        O, L = orc.attn_fwd(x["q"], x["k"], x["v"], w.scale, True)
        ok = np.allclose(O, o.detach().permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-14)
        for name, key in (("dQ", "q"), ("dK", "k"), ("dV", "v")):
            ok &= np.allclose(g[name], t[key].grad.permute(0, 2, 1, 3).numpy(),
                              rtol=1e-12, atol=1e-14)
        if not ok:
            fails.append("P9")
        # P7: L is the log-sum-exp of the kept scores
        import scipy.special
        s = w.scale * np.einsum("bihc,bjhc->bhij", x["q"], x["k"])
        s = np.where(np.tril(np.ones((8, 8), dtype=bool)), s, -np.inf)
        if not np.allclose(L, scipy.special.logsumexp(s, axis=-1), rtol=1e-13, atol=1e-13):
            fails.append("P7")
    return fails


def test_unmodified_oracle_passes_battery():
    assert _battery() == []


def _orig(name):
    return getattr(orc, name)


MUTANTS = {
    "mask_excludes_diagonal": ("causal_keep",
                               lambda nq, nk: np.arange(nk)[None, :] < np.arange(nq)[:, None]),
    "mask_dropped": ("masked_scores",
                     lambda q, k, scale, causal: orc.scores(q, k, scale)),
    "mask_transposed": ("causal_keep",
                        lambda nq, nk: np.arange(nk)[None, :] >= np.arange(nq)[:, None]),
    "D_dropped": ("softmax_backward", lambda p, dp: (p * dp, (p * dp).sum(axis=1))),
    "dS_sign_flipped": ("softmax_backward",
                        lambda p, dp: (p * ((p * dp).sum(axis=1)[:, None] - dp),
                                       (p * dp).sum(axis=1))),
    "scale_dropped_in_grads": ("grad_q_k", lambda ds, q, k, scale: (ds @ k, ds.T @ q)),
    "scale_doubled_in_grads": ("grad_q_k",
                               lambda ds, q, k, scale: (2 * scale * (ds @ k), 2 * scale * (ds.T @ q))),
    "dq_dk_swapped": ("grad_q_k", lambda ds, q, k, scale: (scale * (ds.T @ q), scale * (ds @ k))),
    "dS_transposed_in_dq": ("grad_q_k", lambda ds, q, k, scale: (scale * (ds.T @ k), scale * (ds.T @ q))),
    "softmax_without_normaliser": ("softmax_rows",
                                   lambda s: (s.max(axis=1), np.exp(s - s.max(axis=1)[:, None]),
                                              np.ones(s.shape[0]))),
    "log_base_2_in_L": ("head_forward", None),
    "scale_applied_twice_in_scores": ("scores", lambda q, k, scale: scale * scale * (q @ k.T)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if name == "log_base_2_in_L":
        real = _orig("head_forward")

        def fn(q, k, v, scale, causal):
            o, lse, p = real(q, k, v, scale, causal)
            s = orc.masked_scores(q, k, scale, causal)
            m = s.max(axis=1)
            return o, m + (lse - m) / math.log(2), p
    monkeypatch.setattr(orc, attr, fn)
    assert _battery() != [], f"mutant {name} survived every pin"
