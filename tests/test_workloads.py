"""Seeded generators: determinism, recipes, bf16 rounding."""

import math

import numpy as np

from exact_softmax_attention_attn_amd import workloads


def test_workloads_with_their_shapes():
    names = [w.name for w in workloads.WORKLOADS]
    assert names == ["c1_tiny", "c2_nanogpt_cpu", "c3_single_seq", "c4_batched", "c5_long",
                     "c5_full", "c5_ragged", "c5_window", "c5_bob", "c5_d256", "c5_fwd"]
    assert workloads.get("c1_tiny").shape == (3, 8, 2, 4)
    assert workloads.get("c2_nanogpt_cpu").shape == (12, 64, 4, 32)
    assert workloads.get("c3_single_seq").shape == (1, 256, 1, 64)
    assert workloads.get("c4_batched").shape == (4, 1024, 16, 64)
    assert workloads.get("c5_long").shape == (1, 16384, 16, 128)
    assert workloads.get("c5_full").shape == (1, 16384, 16, 128)
    assert not workloads.get("c5_full").causal
    assert workloads.get("c5_ragged").shape == (1, 16383, 16, 128)
    assert workloads.get("c5_d256").shape == (1, 16384, 8, 256)
    assert all(workloads.get(n).causal for n in names if n != "c5_full")
    for w in workloads.WORKLOADS:
        assert math.isclose(w.scale, 1 / math.sqrt(w.d)) or w.name == "c1_tiny"
    assert workloads.get("c1_tiny").scale == 0.5


def test_generators_are_deterministic_and_seed_dependent():
    w = workloads.get("c2_nanogpt_cpu")
    a = workloads.make_inputs(w, 0)
    b = workloads.make_inputs(w, 0)
    c = workloads.make_inputs(w, 1)
    for k in "q", "k", "v", "do":
        np.testing.assert_array_equal(a[k], b[k])
        assert not np.array_equal(a[k], c[k])
        assert a[k].dtype == np.float32 and a[k].shape == w.shape
    assert abs(a["q"].std() - 1.0) < 0.02


def test_bf16_workloads_hold_bf16_values():
    w = workloads.get("c4_batched")
    x = workloads.make_inputs(w, 0)
    for k in "q", "k", "v", "do":
        bits = x[k].view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)
    assert abs(x["q"].std() - 0.5) < 0.01 and abs(x["do"].std() - 1.0) < 0.01


def test_bf16_round_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 3.0e38],
                    dtype=np.float64)
    got = workloads.bf16_round(vals)
    assert got[0] == 1.0
    assert got[1] == 1.0
    assert got[2] == 1 + 2 ** -6          # halfway, rounds to the even mantissa
    assert got[3] == 1 + 2 ** -7
    assert got[4] == -2.5
    assert np.all(got.view(np.uint32) & 0xFFFF == 0)


def test_block_mask_generators():
    m = workloads.window_block_mask(1000, 3, 1)             # nb = 8
    assert m.shape == (8, 8) and m.dtype == np.uint8
    assert m[7].tolist() == [1, 0, 0, 0, 0, 1, 1, 1]        # sink + blocks 5..7
    assert np.all(np.triu(m, 1) == 0)
    r = workloads.make_block_mask(1000, 0.3, seed=1, heads=(2, 3), empty_rows=(2,))
    assert r.shape == (2, 3, 8, 8)
    assert np.all(r[..., 2, :] == 0)
    assert np.all(r[..., 0, 0] == 1) and np.all(r[..., 5, 5] == 1)
    np.testing.assert_array_equal(r, workloads.make_block_mask(1000, 0.3, seed=1, heads=(2, 3),
                                                               empty_rows=(2,)))
    w = workloads.get("c5_window")
    wm = workloads.workload_mask(w)
    assert wm.shape == (128, 128) and int(wm.sum(axis=1).max()) == 17   # 16 + the sink
    assert workloads.workload_mask(workloads.get("c5_long")) is None
