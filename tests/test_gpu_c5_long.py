"""c5_long against the full fp64 oracle, head by head, for both feeds.

c5_long is the headline workload: 1 sequence x 16 heads x 16,384 tokens x
head dim 128, bf16, causal, scale 1/sqrt(128).  The GPU runs it once per
feed in the launch configuration bench.py times (the whole [1, 16384, 16, 128]
problem in one call), then each head's dQ, dK, dV, O and L is compared with
the oracle's full N x N evaluation of that head (about 2-3 s of host time
per head), gated per head and per row (``tests/gpu_check.py``, 2e-2).  The
feeds are (i) the library's own O and L and (ii) the oracle's O and L cast to
the device type.  A last test gates the whole tensors and the sum rules.
"""

import math
import sys

import numpy as np
import pytest

from exact_softmax_attention_attn_amd import workloads
from oracle import attn_oracle as orc
from tests import gpu_check

pytestmark = pytest.mark.gpu

W = workloads.get("c5_long")
_CACHE = {}


def _say(msg):
    print(f"[gpu c5_long] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_softmax_attention_attn_amd import binding
    binding.load()
    return binding


def _inputs():
    if "x" not in _CACHE:
        _say("inputs")
        _CACHE["x"] = workloads.make_inputs(W, seed=0)
    return _CACHE["x"]


def _oracle_head(h):
    """The oracle's O, L, dQ, dK, dV of head h as one-head slices [1, N, 1, d] / [1, 1, N]."""
    key = ("oracle", h)
    if key not in _CACHE:
        x = _inputs()
        _say(f"oracle head {h}")
        xs = [x[n][:, :, h:h + 1].astype(np.float64) for n in ("q", "k", "v", "do")]
        g = orc.attn_bwd(*xs, W.scale, W.causal)
        _CACHE[key] = {n: g[n] for n in ("O", "L", "dQ", "dK", "dV")}
    return _CACHE[key]


def _gpu(binding, feed):
    """The GPU's O, L, dQ, dK, dV for the whole workload (float32 host arrays)."""
    key = ("gpu", feed)
    if key not in _CACHE:
        import torch
        x = _inputs()
        q, k, v, do = (torch.from_numpy(x[n]).cuda().to(torch.bfloat16) for n in ("q", "k", "v", "do"))
        o, lse = binding.attn_fwd_lse(q, k, v, causal=W.causal, scale=W.scale)
        if feed == "oracle":
            heads = [_oracle_head(h) for h in range(W.H)]
            o_in = torch.from_numpy(np.concatenate([r["O"] for r in heads], axis=2).astype(np.float32))
            o_in = o_in.cuda().to(torch.bfloat16).contiguous()
            l_in = torch.from_numpy(np.concatenate([r["L"] for r in heads], axis=1).astype(np.float32))
            l_in = l_in.cuda().contiguous()
        else:
            o_in, l_in = o, lse
        _say(f"GPU forward + backward, feed={feed}")
        dq, dk, dv = binding.attn_bwd(q, k, v, o_in, do, l_in, causal=W.causal, scale=W.scale)
        torch.cuda.synchronize()
        _CACHE[key] = {"O": o.float().cpu().numpy(), "L": lse.cpu().numpy(),
                       "dQ": dq.float().cpu().numpy(), "dK": dk.float().cpu().numpy(),
                       "dV": dv.float().cpu().numpy()}
    return _CACHE[key]


def _head_slice(t, h):
    return t[:, :, h:h + 1] if t.ndim == 4 else t[:, h:h + 1]


def _check_head(binding, feed, h):
    ref = _oracle_head(h)
    got = {n: _head_slice(a, h) for n, a in _gpu(binding, feed).items()}
    errs = gpu_check.check(f"c5_long head {h} feed={feed}", got, ref, "bf16")
    # squared error and reference norms, for the whole-tensor gate
    _CACHE[("sq", feed, h)] = {n: (float(((got[n] - ref[n]) ** 2).sum()), float((ref[n] ** 2).sum()))
                               for n in ref}
    return errs


@pytest.mark.parametrize("h", range(W.H))
def test_c5_long_head_own_feed(B, h):
    _check_head(B, "own", h)


@pytest.mark.parametrize("h", range(W.H))
def test_c5_long_head_oracle_feed(B, h):
    _check_head(B, "oracle", h)


def test_c5_long_whole_tensors_and_sum_rules(B):
    for feed in ("own", "oracle"):
        for h in range(W.H):
            if ("sq", feed, h) not in _CACHE:
                _check_head(B, feed, h)
        whole = {}
        for n in ("O", "L", "dQ", "dK", "dV"):
            d2 = sum(_CACHE[("sq", feed, h)][n][0] for h in range(W.H))
            r2 = sum(_CACHE[("sq", feed, h)][n][1] for h in range(W.H))
            whole[n] = math.sqrt(d2 / r2)
        gpu_check.report(f"c5_long whole feed={feed}", whole)
        assert max(whole.values()) <= gpu_check.TOL["bf16"], (feed, whole)
        # sum_j dV_j = sum_i dO_i (softmax rows sum to 1); sum_j dK_j = 0 (dS rows sum to 0)
        got = _gpu(B, feed)
        x = _inputs()
        sdv = got["dV"].astype(np.float64).sum(axis=1)
        sdo = x["do"].astype(np.float64).sum(axis=1)
        assert np.linalg.norm(sdv - sdo) <= gpu_check.TOL["bf16"] * np.linalg.norm(sdo)
        dk = got["dK"].astype(np.float64)
        assert np.all(np.abs(dk.sum(axis=1)) <= gpu_check.TOL["bf16"] * np.abs(dk).sum(axis=1) + 1e-6)
