"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Every case is gated per tensor, per (b, h) and per row (``tests/gpu_check.py``):
relative Frobenius error <= 1e-5 on the float32 path and <= 2e-2 on the bf16
path, for dQ, dK, dV and the forward's O and L; every measured error is
printed.  Two feeds for the backward: (i) O and L from the library's own
forward (the user flow) and (ii) the oracle's O and L cast to the device type
(isolates the backward).
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


def _check_full(binding, x, scale, causal, dtype, tag, tol=None):
    xs = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "do")}
    ref = orc.attn_bwd(xs["q"], xs["k"], xs["v"], xs["do"], scale, causal)
    b_, n_, h_, _ = xs["q"].shape
    floor = float(np.linalg.norm(ref["dV"])) / math.sqrt(b_ * h_)
    out = {}
    for feed in ("own", "oracle"):
        _say(f"{tag} feed={feed}")
        got = _run(binding, x, scale, causal, dtype, None if feed == "own" else (ref["O"], ref["L"]))
        out[feed] = gpu_check.check(f"{tag} feed={feed}", got, ref, dtype, floor=floor, tol=tol)
    return out


def shifted_tol(dtype, scale, q_shift, k_shift):
    """Tolerance for scores lowered by scale * q_shift * k_shift.  A float32
    score carries rounding of about its own magnitude times 2^-24 (its
    products are summed in float32), and P = exp(S - L) turns that absolute
    error into a relative one; the unshifted inputs' scores reach about 8
    (natural units), so the float32 bar scales by 1 + shift / 8.  The bf16
    bar is the bf16 rounding of P and dS, which does not grow with the
    shift."""
    if dtype == "bf16":
        return TOL["bf16"]
    return TOL["f32"] * (1.0 + scale * q_shift * k_shift / 8.0)


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
# The pipelined bf16 kernels (head dim 64 and 128) on sequences shorter than
# one 64-row tile: one ragged tile per walk, and dQ walks whose unchecked
# main loop is empty.
EDGE += [(1, 2, n, d, "bf16", c) for n in (1, 7, 63) for d in (64, 128) for c in (True, False)]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_parity_edge_shapes(B, case):
    b, h, n, d, dtype, causal = case
    x = workloads.make_random(b, h, n, d, dtype, seed=n + d, qkv_std=0.5 if dtype == "bf16" else 1.0)
    _check_full(B, x, 1.0 / math.sqrt(d), causal, dtype, f"edge {case}")


def _forward_rescales(q, k, scale, causal, sub=32, threshold=8.0):
    """How often the pipelined forward's running max moves after a row's
    first key sub-tile: it moves when a sub-tile's max (log2 units) exceeds
    the running max by more than ``threshold``.  Scores from the oracle."""
    count = 0
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            s = orc.masked_scores(q[b, :, h], k[b, :, h], scale, causal) * math.log2(math.e)
            n = s.shape[1]
            m = s[:, :sub].max(axis=1)
            for j0 in range(sub, n, sub):
                mx = s[:, j0:j0 + sub].max(axis=1)
                up = mx > m + threshold
                count += int(up.sum())
                m = np.where(up, mx, m)
    return count


PEAKED = [
    # B, H, N, d, dtype, causal: keys whose norm grows along N, qkv_std 2
    (1, 2, 1000, 128, "bf16", True),
    (1, 2, 1000, 128, "bf16", False),
    (1, 2, 1100, 64, "bf16", True),
    (1, 2, 700, 64, "bf16", False),
    (1, 2, 600, 64, "f32", True),
    (1, 1, 400, 32, "f32", False),
]


@pytest.mark.parametrize("case", PEAKED, ids=lambda c: "x".join(map(str, c)))
def test_parity_peaked_softmax(B, case):
    """Sharply peaked rows whose maximum climbs along the walk: the forward
    rescales its live accumulators mid-walk (checked on the inputs)."""
    b, h, n, d, dtype, causal = case
    scale = 1.0 / math.sqrt(d)
    x = workloads.make_peaked(b, h, n, d, dtype, seed=7 + n, qkv_std=2.0, growth=3.0)
    moves = _forward_rescales(x["q"].astype(np.float64), x["k"].astype(np.float64), scale, causal)
    _say(f"peaked {case}: {moves} running-max moves after the first sub-tile")
    assert moves >= 10 * b * h
    _check_full(B, x, scale, causal, dtype, f"peaked {case}")


SHIFTED = [
    # B, H, N, d, dtype, causal, q_shift: every score of a row lowered by
    # scale * q_shift > 100 (keys share channel 0 = -1, queries have channel
    # 0 = q_shift), so L < -88 and exp(-L) overflows float32.  N is ragged, so
    # the last key tile carries padded keys.
    (1, 2, 1000, 128, "bf16", False, 1296.0),
    (1, 2, 1000, 128, "bf16", True, 1296.0),
    (1, 2, 1000, 64, "bf16", False, 900.0),
    (1, 2, 1000, 64, "f32", False, 900.0),
    (1, 2, 1000, 40, "bf16", False, 768.0),
    (1, 1, 1000, 128, "f32", False, 1296.0),
]


@pytest.mark.parametrize("case", SHIFTED, ids=lambda c: "x".join(map(str, c)))
def test_parity_shifted_scores(B, case):
    b, h, n, d, dtype, causal, q_shift = case
    scale = 1.0 / math.sqrt(d)
    assert scale * q_shift > 100.0
    x = workloads.make_shifted(b, h, n, d, dtype, seed=3 + d, q_shift=q_shift, k_shift=1.0)
    _check_full(B, x, scale, causal, dtype, f"shifted {case}",
                tol=shifted_tol(dtype, scale, q_shift, 1.0))


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


@pytest.mark.parametrize("name", ["c5_full", "c5_ragged", "c5_window", "c5_d256"])
def test_c5_variants_sampled_against_oracle(B, name):
    """16,384 (or 16,383) tokens beyond square causal: sampled rows and
    columns of two heads, evaluated one by one by the oracle.  (c5_long itself
    is compared head by head in full in test_gpu_c5_long.py.)"""
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
    for h in (0, w.H - 5):
        _say(f"{name} oracle sample head {h}")
        s = orc.attn_bwd_sampled(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal, 0, h, rows, cols,
                                 row_block=1024, block_mask=bm)
        got = {"dQ": dq[0, rows, h].float().cpu().numpy(), "O": o[0, rows, h].float().cpu().numpy(),
               "dK": dk[0, cols, h].float().cpu().numpy(), "dV": dv[0, cols, h].float().cpu().numpy(),
               "L": lse[0, h].cpu().numpy()}
        # sampled rows as one (b, h) slice [1, rows, 1, d]; L [1, 1, N]
        shape = {n: (lambda a: a[None, :, None, :]) for n in ("dQ", "O", "dK", "dV")}
        g = {n: shape[n](got[n]) for n in ("dQ", "O", "dK", "dV")}
        r = {n: shape[n](s[n]) for n in ("dQ", "O", "dK", "dV")}
        g["L"], r["L"] = got["L"][None, None, :], s["L"][None, None, :]
        gpu_check.check(f"{name} sampled head {h}", g, r, "bf16")
    # properties over the whole tensor: sum_j dV_j = sum_i dO_i; sum_j dK_j = 0
    sdv = dv.double().sum(dim=1).cpu().numpy()
    sdo = do.double().sum(dim=1).cpu().numpy()
    assert rel_fro(sdv, sdo) <= TOL["bf16"]
    sdk = dk.double().sum(dim=1).cpu().numpy()
    adk = dk.double().abs().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(sdk) <= TOL["bf16"] * adk + 1e-6)


@pytest.mark.parametrize("recipe", ["causal", "window"])
def test_longest_sequence_sampled_against_oracle(B, recipe):
    """N = 65,536 (the longest a block-masked call takes: 1,024 tiles of 64
    rows per visit list), one head of d = 64, bf16: sampled rows and columns
    against the oracle, plus the sum rules.  Under the window mask (16 blocks
    and the first block) key block 0 is kept by every query block, so its dK/dV
    walk fills the visit list to exactly its 1,024 entries."""
    import torch
    N, d = 65536, 64
    scale = 1.0 / math.sqrt(d)
    _say(f"N={N} {recipe} inputs")
    x = workloads.make_random(1, 1, N, d, "bf16", seed=17, qkv_std=0.5)
    q, k, v, do = (_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    bm = workloads.window_block_mask(N, 16, 1) if recipe == "window" else None
    _say(f"N={N} {recipe} forward + backward on the GPU")
    if bm is None:
        o, lse = B.attn_fwd_lse(q, k, v, causal=True, scale=scale)
        dq, dk, dv = B.attn_bwd(q, k, v, o, do, lse, causal=True, scale=scale)
    else:
        assert int(bm[:, 0].sum()) * 2 == 1024          # key block 0's walk: 1,024 tiles
        mask = torch.from_numpy(bm).cuda()
        o, lse = B.attn_fwd_lse_masked(q, k, v, mask, causal=True, scale=scale)
        dq, dk, dv = B.attn_bwd_masked(q, k, v, o, do, lse, mask, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 32767, 32768, N - 2, N - 1],
                                     rng.integers(0, N, 24)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 32767, 65407, N - 1],
                                     rng.integers(0, N, 24)]))
    _say(f"N={N} {recipe} oracle sample")
    s = orc.attn_bwd_sampled(x["q"], x["k"], x["v"], x["do"], scale, True, 0, 0, rows, cols,
                             row_block=1024, block_mask=bm)
    got = {"dQ": dq[0, rows, 0].float().cpu().numpy(), "O": o[0, rows, 0].float().cpu().numpy(),
           "dK": dk[0, cols, 0].float().cpu().numpy(), "dV": dv[0, cols, 0].float().cpu().numpy()}
    g = {n: a[None, :, None, :] for n, a in got.items()}
    r = {n: s[n][None, :, None, :] for n in got}
    g["L"], r["L"] = lse[0, 0].cpu().numpy()[None, None, :], s["L"][None, None, :]
    gpu_check.check(f"N={N} {recipe} sampled", g, r, "bf16")
    sdv = dv.double().sum(dim=1).cpu().numpy()
    sdo = do.double().sum(dim=1).cpu().numpy()
    assert rel_fro(sdv, sdo) <= TOL["bf16"]
    sdk = dk.double().sum(dim=1).cpu().numpy()
    adk = dk.double().abs().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(sdk) <= TOL["bf16"] * adk + 1e-6)
