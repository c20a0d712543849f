"""Exact softmax attention, forward and backward, as a plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes, and where that is defined
-------------------------------------------
Sources are the pages' titles and sections:

* ddx issue #217, "Backward of batched attention builds a contraction over
  every pair of sequences and heads", repro script: the SQL loss (CTEs
  ``scores``, ``weights``, ``norm``, ``heads``) and the JAX loss beside it.
  Scores are the per-head dot product of a query row with a key row times a
  scale (1/2 there); a key position is kept when it is not after the query
  position (diagonal kept); the weights are exp(score minus the row max); the
  row normaliser z is their sum; the head output is the weighted sum of value
  rows divided by z.  Tensors are indexed (sequence, position, head, channel)
  in row-major order.
* ddx issue #243, "Attention's gradient: a softmax shift's backward computed
  twice, and recomputing scores instead of saving them", item 1: the gradient
  through the row max cancels because the shift cancels in w/z; item 2: the
  backward needs the scores, dP = dO V^T, and the softmax-weighted sums of dP,
  and one saved number per row, m + log z, is enough to rebuild the scores.
* ddx PR #162, "perf(ddx-ad): transpose causal attention's contractions
  without their joins", section "What changed": transpose p = w/z per score,
  then p @ v (the plan jax.grad uses).  The same section describes a mask
  that reads only grouping keys, so every row of a group passes or none does;
  ``block_keep`` is that mask with groups of MASK_BLOCK query rows by
  MASK_BLOCK key rows (a block-sparse mask), combined with the causal rule.

A row whose every key is masked has no softmax.  Its output row is 0, its
row scalar L is -inf and it adds nothing to any gradient (the limit of a row
whose kept weights all tend to 0; the pages never produce such a row, since
the causal rule keeps the diagonal).

Everything here is the textbook definition materialised at N x N per
(batch, head), in float64, so a reader can check each line against the
formulas: no tiling, no online softmax, no fusion.  The only grouping is in
``attn_bwd_sampled``, which evaluates whole rows (or whole columns) of the same
definition for a few chosen indices; rows are independent, so batching them
changes no value.

Pins (tests/test_oracle_pins.py): pair counts against the counts the pages
print, central finite differences, the shift-cancellation identity, sum rules,
metamorphic shifts, closed forms for Q = 0 and N = 1, scipy's logsumexp and
torch's CPU fp64 scaled_dot_product_attention with autograd.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "MASK_BLOCK",
    "causal_keep",
    "block_keep",
    "keep_mask",
    "scores",
    "masked_scores",
    "softmax_rows",
    "softmax_backward",
    "grad_q_k",
    "head_forward",
    "head_backward",
    "attn_fwd",
    "attn_bwd",
    "attn_bwd_sampled",
    "literal_backward_head",
    "pair_count",
    "head_bwd_bwd",
    "attn_bwd_bwd",
    "attn_bwd_bwd_sampled",
]


# --------------------------------------------------------------------------
# Forward steps (issue #217 repro: CTEs scores -> weights -> norm -> heads)
# --------------------------------------------------------------------------

def causal_keep(n_q: int, n_k: int) -> np.ndarray:
    """Boolean keep-mask: key position j is kept for query position i iff j <= i.

    Issue #217 repro: the score join keeps q.pos >= k.pos; the JAX loss uses a
    lower-triangular mask.  The diagonal is kept, so every row keeps >= 1 key.
    """
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


MASK_BLOCK = 128   # query rows and key rows per block of a block-sparse mask


def block_keep(n_q: int, n_k: int, block_mask, mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Element keep-mask of a block mask: keep[i, j] iff block_mask[i // mb, j // mb] != 0.

    PR #162, "What changed": a filter on grouping keys passes a whole group of
    rows or none of it; here a group is a mask_block x mask_block block.
    """
    bm = np.asarray(block_mask) != 0
    bi = np.arange(n_q) // mask_block
    bj = np.arange(n_k) // mask_block
    return bm[bi[:, None], bj[None, :]]


def keep_mask(n_q: int, n_k: int, causal: bool, block_mask=None,
              mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Pairs kept: the causal rule (if causal) and the block mask (if given)."""
    keep = causal_keep(n_q, n_k) if causal else np.ones((n_q, n_k), dtype=bool)
    if block_mask is not None:
        keep = keep & block_keep(n_q, n_k, block_mask, mask_block)
    return keep


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S[i, j] = scale * sum_c q[i, c] k[j, c]  (issue #217 repro, CTE ``scores``)."""
    return scale * (q @ k.T)


def masked_scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                  block_mask=None, mask_block: int = MASK_BLOCK) -> np.ndarray:
    """Scores with masked-out pairs set to -inf (absent rows in the SQL spelling)."""
    s = scores(q, k, scale)
    if causal or block_mask is not None:
        s = np.where(keep_mask(s.shape[0], s.shape[1], causal, block_mask, mask_block), s, -np.inf)
    return s


def softmax_rows(s: np.ndarray):
    """Row max m, shifted weights w = exp(s - m), normaliser z = sum_j w.

    Issue #217 repro, CTEs ``weights`` (exp of the score minus the row MAX
    window) and ``norm`` (SUM of the weights per row).  -inf scores give w = 0;
    a row of -inf scores (no kept key) has m = -inf, w = 0 and z = 0.
    """
    m = s.max(axis=1)
    m_shift = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - m_shift[:, None])
    z = w.sum(axis=1)
    return m, w, z


def _normalise(m, w, z):
    """P = w / z and L = m + log z; a row with z = 0 gets P = 0 and L = -inf."""
    live = z > 0
    p = np.divide(w, z[:, None], out=np.zeros_like(w), where=live[:, None])
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(np.where(live, z, 1.0)), -np.inf)
    return p, lse


def head_forward(q, k, v, scale: float, causal: bool, block_mask=None,
                 mask_block: int = MASK_BLOCK):
    """One (batch, head): O = (w / z) V and the saved row scalar L = m + log z.

    O follows the CTE ``heads`` of the issue #217 repro; L is the one number per
    row that issue #243 (item 2) names as enough to rebuild the scores.
    Returns O [N, d], L [N], P [N, N].
    """
    s = masked_scores(q, k, scale, causal, block_mask, mask_block)
    m, w, z = softmax_rows(s)
    p, lse = _normalise(m, w, z)
    o = p @ v
    return o, lse, p


# --------------------------------------------------------------------------
# Backward steps (PR #162 "What changed": transpose p = w/z, then p @ v)
# --------------------------------------------------------------------------

def softmax_backward(p: np.ndarray, dp: np.ndarray):
    """dS = P o (dP - D) with D_i = sum_j P_ij dP_ij.

    The cotangent of the softmax input.  There is no term for the row-max
    shift: issue #243 (item 1) notes that its gradient cancels in w/z.
    D is formed from P and dP here (the definition); that it equals
    rowsum(dO o O) is checked by the pins, not assumed.
    """
    d = (p * dp).sum(axis=1)
    ds = p * (dp - d[:, None])
    return ds, d


def grad_q_k(ds: np.ndarray, q: np.ndarray, k: np.ndarray, scale: float):
    """dQ = scale * dS K and dK = scale * dS^T Q (S = scale * Q K^T)."""
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk


def head_backward(q, k, v, do, scale: float, causal: bool, block_mask=None,
                  mask_block: int = MASK_BLOCK):
    """Exact gradient of sum(dO o O) for one (batch, head), every table materialised.

    Returns dQ, dK, dV [N, d], D [N], dS row sums [N], P [N, N], and the
    forward's O [N, d] and L [N] (``head_forward``'s, computed on the way).
    """
    o, lse, p = head_forward(q, k, v, scale, causal, block_mask, mask_block)
    dv = p.T @ do                      # p @ v transposed against the output cotangent
    dp = do @ v.T                      # dP = dO V^T (issue #243, item 2)
    ds, d = softmax_backward(p, dp)
    dq, dk = grad_q_k(ds, q, k, scale)
    return dq, dk, dv, d, ds.sum(axis=1), p, o, lse


def literal_backward_head(q, k, v, do, scale: float, causal: bool):
    """The same gradient spelled step by step as the SQL plan names its tables.

    Issue #217 repro output lists the backward steps in the order
    cotangent_2 (dO) -> contraction_0 (g = dO V^T) -> cotangent_1 (z-bar) ->
    cotangent_0 (s-bar) -> grad_0_q.  Here, with w = exp(s - m):
      g_ij    = dO_i . v_j
      zbar_i  = -sum_j w_ij g_ij / z_i^2
      wbar_ij = g_ij / z_i + zbar_i
      sbar_ij = w_ij wbar_ij            (direct path into the scores)
      mbar_i  = -sum_j sbar_ij          (path through the row max)
    Issue #243 (item 1) says mbar cancels; the pins check |mbar| ~ 0 and that
    sbar equals softmax_backward's dS.  Returns sbar [N, N] and mbar [N].
    """
    s = masked_scores(q, k, scale, causal)
    m, w, z = softmax_rows(s)
    g = do @ v.T
    zbar = -(w * g).sum(axis=1) / z ** 2
    wbar = g / z[:, None] + zbar[:, None]
    sbar = w * wbar
    mbar = -sbar.sum(axis=1)
    return sbar, mbar


# --------------------------------------------------------------------------
# Batched entry points, tensors laid out [B, N, H, d] (sequence, pos, head, c)
# --------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _head_mask(block_mask, b, h):
    """The [nb, nb] block mask of (b, h): one shared mask, or one per (b, h)."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm if bm.ndim == 2 else bm[b, h]


def attn_fwd(Q, K, V, scale: float, causal: bool = True, block_mask=None,
             mask_block: int = MASK_BLOCK):
    """O [B, N, H, d] and L [B, H, N] (natural log) for every (batch, head).

    block_mask: None, [nb, nb] (shared) or [B, H, nb, nb], nb = ceil(N / mask_block).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, N, H, _ = Q.shape
    O = np.empty_like(V)
    L = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o, lse, _ = head_forward(Q[b, :, h], K[b, :, h], V[b, :, h], scale, causal,
                                     _head_mask(block_mask, b, h), mask_block)
            O[b, :, h] = o
            L[b, h] = lse
    return O, L


def attn_bwd(Q, K, V, dO, scale: float, causal: bool = True, block_mask=None,
             mask_block: int = MASK_BLOCK):
    """dQ, dK, dV [B, N, H, d] plus diagnostics D and dS row sums [B, H, N], and
    the forward's O [B, N, H, d] and L [B, H, N] (the same values as ``attn_fwd``)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, N, H, _ = Q.shape
    dQ = np.empty_like(Q)
    dK = np.empty_like(K)
    dV = np.empty_like(V)
    O = np.empty_like(V)
    L = np.empty((B, H, N))
    D = np.empty((B, H, N))
    ds_rows = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            dq, dk, dv, d, dsr, _, o, lse = head_backward(
                Q[b, :, h], K[b, :, h], V[b, :, h], dO[b, :, h], scale, causal,
                _head_mask(block_mask, b, h), mask_block)
            dQ[b, :, h], dK[b, :, h], dV[b, :, h] = dq, dk, dv
            O[b, :, h], L[b, h] = o, lse
            D[b, h], ds_rows[b, h] = d, dsr
    return {"dQ": dQ, "dK": dK, "dV": dV, "D": D, "dS_rowsum": ds_rows, "O": O, "L": L}


def attn_bwd_sampled(Q, K, V, dO, scale: float, causal: bool, b: int, h: int,
                     rows, cols, row_block: int = 512, block_mask=None,
                     mask_block: int = MASK_BLOCK):
    """Selected outputs of one (b, h) without any N x N array.

    dQ and O are returned for the query rows ``rows``; dK and dV for the key
    rows ``cols``.  Each is the definition of ``head_backward`` evaluated for
    that row or column alone:
      * query row i needs score row i, its softmax, dP row i and D_i;
      * key row j needs column j of P and dS, hence L_i and D_i for every
        query row i; those come from full score rows evaluated ``row_block``
        rows at a time (rows are independent, so the grouping changes nothing).
    """
    q = _f64(Q[b, :, h]); k = _f64(K[b, :, h]); v = _f64(V[b, :, h]); do = _f64(dO[b, :, h])
    n = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)

    bm = _head_mask(block_mask, b, h)

    def keep_rows(r0, r1):
        # the kept pairs of query rows r0 .. r1 - 1, every key
        keep = np.ones((r1 - r0, n), dtype=bool)
        if causal:
            keep &= np.arange(n)[None, :] <= np.arange(r0, r1)[:, None]
        if bm is not None:
            keep &= (np.asarray(bm) != 0)[(np.arange(r0, r1) // mask_block)[:, None],
                                          (np.arange(n) // mask_block)[None, :]]
        return keep

    def row_stats(r0, r1):
        s = np.where(keep_rows(r0, r1), scale * (q[r0:r1] @ k.T), -np.inf)
        m, w, z = softmax_rows(s)
        p, lse = _normalise(m, w, z)
        dp = do[r0:r1] @ v.T
        d = (p * dp).sum(axis=1)
        return lse, d, p, dp

    # per-row scalars L and D for all rows
    L = np.empty(n)
    D = np.empty(n)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        L[r0:r1], D[r0:r1], _, _ = row_stats(r0, r1)

    out = {"rows": rows, "cols": cols, "L": L, "D": D}
    dq = np.empty((rows.size, q.shape[1]))
    o = np.empty((rows.size, v.shape[1]))
    for t, i in enumerate(rows):
        _, _, p, dp = row_stats(int(i), int(i) + 1)
        ds = p * (dp - D[i])
        dq[t] = scale * (ds @ k)[0]
        o[t] = (p @ v)[0]
    out["dQ"] = dq
    out["O"] = o

    dk = np.empty((cols.size, k.shape[1]))
    dv = np.empty((cols.size, v.shape[1]))
    live = np.isfinite(L)                                # rows with a kept key
    for t, j in enumerate(cols):
        s_col = scale * (q @ k[j])                       # S[:, j]
        keep = live.copy()
        if causal:
            keep &= np.arange(n) >= j
        if bm is not None:
            keep &= (np.asarray(bm) != 0)[np.arange(n) // mask_block, j // mask_block]
        # P[:, j] = exp(S - L) on kept pairs
        p_col = np.exp(np.where(keep, s_col - np.where(live, L, 0.0), -np.inf))
        dp_col = do @ v[j]                               # dP[:, j]
        ds_col = p_col * (dp_col - D)
        dv[t] = p_col @ do
        dk[t] = scale * (ds_col @ q)
    out["dK"] = dk
    out["dV"] = dv
    return out


# --------------------------------------------------------------------------
# Backward of the backward (the page "Approaching I/O-optimality for
# Approximate Attention", first abstract, FlashBoB: the exact gradient of the
# backward pass, for which a pair of per-row quantities suffices beyond the
# recomputed scores).  Given cotangents gQ, gK, gV of the
# backward's outputs dQ, dK, dV, return the gradients of
#     l2 = <gQ, dQ> + <gK, dK> + <gV, dV>
# with respect to Q, K, V and dO.  Written out from the chain rule:
#   <gV, dV> = <P, A>,   A = dO gV^T
#   <gQ, dQ> + <gK, dK> = <dS, G>,   G = scale (gQ K^T + Q gK^T)
# so l2 = sum_ij P_ij (A_ij + (dP_ij - D_i) G_ij), with D_i = sum_j P_ij dP_ij.
#   d l2 / d dP = W = P o (G - r),   r_i = sum_j P_ij G_ij
#   d l2 / d P  = A + (dP - D) o (G - r) - D r   (the last term is constant
#                 along a row and cancels in the softmax backward), so
#   d l2 / d S  = dS2 = P o (Psi - E),  Psi = A + (dP - D) o (G - r),
#                 E_i = sum_j P_ij Psi_ij
# and, with S = scale Q K^T, dP = dO V^T, A = dO gV^T and G as above:
#   hQ = scale (dS2 K + dS gK),   hK = scale (dS2^T Q + dS^T gQ),
#   hV = W^T dO,                  hdO = P gV + W V.
# r and E are the two row scalars.
# --------------------------------------------------------------------------

def head_bwd_bwd(q, k, v, do, gq, gk, gv, scale: float, causal: bool, block_mask=None,
                 mask_block: int = MASK_BLOCK):
    """One (batch, head): hQ, hK, hV, hdO [N, d] and the row scalars r, E [N]."""
    _, _, p = head_forward(q, k, v, scale, causal, block_mask, mask_block)
    dp = do @ v.T
    ds, d = softmax_backward(p, dp)
    g = scale * (gq @ k.T + q @ gk.T)
    a = do @ gv.T
    r = (p * g).sum(axis=1)
    w = p * (g - r[:, None])
    psi = a + (dp - d[:, None]) * (g - r[:, None])
    e = (p * psi).sum(axis=1)
    ds2 = p * (psi - e[:, None])
    hq = scale * (ds2 @ k + ds @ gk)
    hk = scale * (ds2.T @ q + ds.T @ gq)
    hv = w.T @ do
    hdo = p @ gv + w @ v
    return hq, hk, hv, hdo, r, e


def attn_bwd_bwd(Q, K, V, dO, gQ, gK, gV, scale: float, causal: bool = True, block_mask=None,
                 mask_block: int = MASK_BLOCK):
    """hQ, hK, hV, hdO [B, N, H, d] and r, E [B, H, N] for every (batch, head)."""
    X = [_f64(t) for t in (Q, K, V, dO, gQ, gK, gV)]
    B, N, H, _ = X[0].shape
    out = {n: np.empty_like(X[i]) for n, i in (("hQ", 0), ("hK", 1), ("hV", 2), ("hdO", 3))}
    out["r"] = np.empty((B, H, N))
    out["E"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            res = head_bwd_bwd(*(t[b, :, h] for t in X), scale, causal,
                               _head_mask(block_mask, b, h), mask_block)
            for n, x in zip(("hQ", "hK", "hV", "hdO"), res[:4]):
                out[n][b, :, h] = x
            out["r"][b, h], out["E"][b, h] = res[4], res[5]
    return out


def attn_bwd_bwd_sampled(Q, K, V, dO, gQ, gK, gV, scale: float, causal: bool, b: int, h: int,
                         rows, cols, row_block: int = 512):
    """Selected outputs of ``head_bwd_bwd`` for one (b, h) without N x N memory.

    hQ and hdO for the query rows ``rows``, hK and hV for the key rows
    ``cols``, and the row scalars for every row.  Row quantities (L, D, r, E)
    come from whole score rows evaluated ``row_block`` rows at a time; a key
    column then needs its column of P, dP, G and A, rebuilt from those
    scalars.  Each value is the same definition as ``head_bwd_bwd``.
    """
    q, k, v, do, gq, gk, gv = (_f64(t[b, :, h]) for t in (Q, K, V, dO, gQ, gK, gV))
    n = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)

    def block(r0, r1):
        s = scale * (q[r0:r1] @ k.T)
        if causal:
            s = np.where(np.arange(n)[None, :] <= np.arange(r0, r1)[:, None], s, -np.inf)
        m, w, z = softmax_rows(s)
        p, lse = _normalise(m, w, z)
        dp = do[r0:r1] @ v.T
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        g = scale * (gq[r0:r1] @ k.T + q[r0:r1] @ gk.T)
        a = do[r0:r1] @ gv.T
        r = (p * g).sum(axis=1)
        e = (p * (a + (dp - dd[:, None]) * (g - r[:, None]))).sum(axis=1)
        return lse, dd, r, e, p, dp, ds, g, a

    L, D, R, E = (np.empty(n) for _ in range(4))
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        L[r0:r1], D[r0:r1], R[r0:r1], E[r0:r1] = block(r0, r1)[:4]
    out = {"rows": rows, "cols": cols, "L": L, "D": D, "r": R, "E": E}
    hq = np.empty((rows.size, q.shape[1]))
    hdo = np.empty((rows.size, q.shape[1]))
    for t, i in enumerate(rows):
        _, dd, r, e, p, dp, ds, g, a = block(int(i), int(i) + 1)
        w = p * (g - r[:, None])
        ds2 = p * (a + (dp - dd[:, None]) * (g - r[:, None]) - e[:, None])
        hq[t] = scale * (ds2 @ k + ds @ gk)[0]
        hdo[t] = (p @ gv + w @ v)[0]
    hk = np.empty((cols.size, q.shape[1]))
    hv = np.empty((cols.size, q.shape[1]))
    live = np.isfinite(L)
    for t, j in enumerate(cols):
        keep = live.copy()
        if causal:
            keep &= np.arange(n) >= j
        s_col = scale * (q @ k[j])
        p_col = np.exp(np.where(keep, s_col - np.where(live, L, 0.0), -np.inf))
        dp_col = do @ v[j]
        g_col = scale * (gq @ k[j] + q @ gk[j])
        a_col = do @ gv[j]
        ds_col = p_col * (dp_col - D)
        w_col = p_col * (g_col - R)
        ds2_col = p_col * (a_col + (dp_col - D) * (g_col - R) - E)
        hk[t] = scale * (ds2_col @ q + ds_col @ gq)
        hv[t] = w_col @ do
    out.update(hQ=hq, hdO=hdo, hK=hk, hV=hv)
    return out


# --------------------------------------------------------------------------
# Pair count (pinned against the score-table row counts the pages print)
# --------------------------------------------------------------------------

def pair_count(B: int, H: int, N: int, causal: bool = True) -> int:
    """Number of kept (i, j) pairs: B*H*N(N+1)/2 causal (diagonal kept), else B*H*N^2.

    Counted from the mask itself, so a wrong mask shows up against the row
    counts the pages print for the score tables.
    """
    if N == 0:
        return 0
    keep = causal_keep(N, N) if causal else np.ones((N, N), dtype=bool)
    return int(B * H * int(keep.sum()))
