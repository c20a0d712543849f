"""Error measures and gates shared by the GPU parity tests (not a test module).

For a tensor laid out [B, N, H, d] (or L: [B, H, N]) and its fp64 oracle:

* ``whole`` -- relative Frobenius error over the whole tensor;
* ``head``  -- the largest relative Frobenius error of one (b, h) slice;
* ``row``   -- the largest error of one row (one position of one head),
  measured against that row's own norm, or against the root-mean-square row
  norm of its (b, h) slice where the row is smaller than that (rows whose
  exact value is zero or nearly so, e.g. dQ of a causal row 0), so a single
  wrong row shows up even in a 16,384-row head.

Gates: ``whole`` and ``head`` <= tol, ``row`` <= ROW_FACTOR * tol, with tol
1e-5 (float32 path) or 2e-2 (bf16 path).  Every measured error is printed,
and appended as a JSON line to the file named by ATTN_PARITY_REPORT if set.

A (b, h) slice whose reference is exactly zero (dQ and dK of a one-position
sequence: the only key gets the whole softmax, so dS = 0) is measured
against the caller's ``floor`` instead of its own norm: the computed value is
zero in exact arithmetic, and only float32 rounding (about 1e-7 of the dV
scale) may remain.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2}
ROW_FACTOR = 5.0


def _heads(x: np.ndarray) -> np.ndarray:
    """[B, N, H, d] -> [B, H, N, d]; [B, H, N] -> [B, H, N, 1]."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 4:
        return np.transpose(x, (0, 2, 1, 3))
    if x.ndim == 3:
        return x[..., None]
    raise ValueError(x.shape)


def errors(got, ref, floor: float = 0.0) -> dict:
    g, r = _heads(got), _heads(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    diff = g - r
    dn = np.sqrt((diff ** 2).sum(axis=(2, 3)))                       # [B, H]
    rn = np.sqrt((r ** 2).sum(axis=(2, 3)))
    rn = np.where(rn > 0, rn, max(floor, 1e-30))
    whole = float(np.sqrt((dn ** 2).sum()) / np.sqrt((rn ** 2).sum()))
    head = float((dn / rn).max())
    rms_row = rn / np.sqrt(r.shape[2])                                # [B, H]
    row_err = np.sqrt((diff ** 2).sum(axis=3))                        # [B, H, N]
    row_ref = np.maximum(np.sqrt((r ** 2).sum(axis=3)), rms_row[..., None])
    row = float((row_err / row_ref).max())
    return {"whole": whole, "head": head, "row": row}


def report(tag: str, errs: dict) -> None:
    line = {"case": tag, **{k: v for k, v in errs.items()}}
    print(f"[parity] {json.dumps(line)}", flush=True)
    sys.stdout.flush()
    path = os.environ.get("ATTN_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def check(tag: str, got: dict, ref: dict, dtype: str, names=("dQ", "dK", "dV", "O", "L"),
          floor: float = 0.0, tol: float = None) -> dict:
    """Measure, print and gate every named tensor; returns {name: errors}.
    ``tol`` overrides the dtype's tolerance (derived per case by the caller)."""
    tol = TOL[dtype] if tol is None else tol
    out = {n: errors(got[n], ref[n], floor) for n in names}
    report(tag, {n: out[n] for n in names})
    for n, e in out.items():
        assert all(np.isfinite(v) for v in e.values()), (tag, n, e)
        assert e["whole"] <= tol, (tag, n, e)
        assert e["head"] <= tol, (tag, n, e)
        assert e["row"] <= ROW_FACTOR * tol, (tag, n, e)
    return out
