"""Checks of the seeded input generator (no method arithmetic lives there)."""
import numpy as np
import pytest
import torch


def test_bf16_rounding_matches_torch(synth_mod):
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.normal(size=4000).astype(np.float32),
                         rng.uniform(-1e30, 1e30, size=2000).astype(np.float32),
                         np.array([0.0, -0.0, 1.0, 65504.0, 3.3895314e38, 1e-40, -1e-42],
                                  dtype=np.float32)])
    # ties: values exactly halfway between two bf16 numbers
    ties = ((np.arange(1000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    xs = np.concatenate([xs, ties[np.isfinite(ties)]])
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([synth_mod.f32_to_bf16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_f16_rounding_matches_numpy(synth_mod):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    xs = xs[np.isfinite(xs)]
    extra = np.array([65504.0, 65519.99, 65520.0, 65536.0, 6.1e-5, 5.96e-8, 2.98e-8,
                      2.9802322e-08, 2.9802326e-08, 1e-8, -0.0, 0.0], dtype=np.float32)
    small = (rng.uniform(-1, 1, size=5000) * 2.0 ** -14).astype(np.float32)  # subnormal range
    xs = np.concatenate([xs, extra, small, rng.normal(size=5000).astype(np.float32)])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([synth_mod.f32_to_f16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_deterministic_and_sliceable(synth_mod):
    o1, l1 = synth_mod.combine_inputs("fp16_base2")
    o2, l2 = synth_mod.combine_inputs("fp16_base2")
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    o3, l3 = synth_mod.combine_inputs("fp16_base2", b_lo=17, b_hi=45)
    assert np.array_equal(o3, o1[:, 17:45])
    assert np.array_equal(l3.view(np.uint32), l1[:, 17:45].view(np.uint32))
    r1 = synth_mod.rank_inputs("packed", 3, b_lo=0, b_hi=64)
    r2 = synth_mod.rank_inputs("packed", 3, b_lo=10, b_hi=20)
    assert np.array_equal(r1[0][10:20], r2[0])
    r0 = synth_mod.rank_inputs("packed", 0, b_lo=0, b_hi=64)
    assert not np.array_equal(r0[0], r1[0])  # ranks draw independent tensors


def test_recipes(synth_mod):
    o, l = synth_mod.combine_inputs("small")
    assert o.shape == (2, 4, 8, 128) and l.shape == (2, 4, 8)
    assert np.all(np.isneginf(l[:, 3, 7]))
    f = l[np.isfinite(l)]
    assert f.min() >= -2 and f.max() < 8
    o, l = synth_mod.combine_inputs("fp16_base2")
    assert abs(np.isnan(l).mean() - 0.02) < 0.005 and abs(np.isposinf(l).mean() - 0.02) < 0.005
    vals = o.view(np.float16).astype(np.float64)
    assert abs(vals.mean()) < 0.01 and abs(vals.std() - 1) < 0.01
    o, l = synth_mod.combine_inputs("mla_decode", b_lo=0, b_hi=512)
    vals = (o.astype(np.uint32) << 16).view(np.float32)
    assert abs(vals.std() - 0.5) < 0.01
    assert abs(np.isneginf(l).mean() - 0.01) < 0.003
    f = l[np.isfinite(l)]
    assert abs(f.mean() - 10) < 0.1 and abs(f.std() - 3) < 0.1
    o, l = synth_mod.combine_inputs("large_batch", b_lo=0, b_hi=256)
    assert abs((~np.isfinite(l)).mean() - 0.005) < 0.0015
    for bad in (np.isnan(l), np.isposinf(l), np.isneginf(l)):
        assert bad.sum() > 0
    w = synth_mod.WORKLOADS["packed"]
    o, l = synth_mod.rank_inputs(w, 0, b_lo=0, b_hi=16)
    assert o.shape == (16, 64, 128) and l.shape == (16, 64)
    assert w.rows == 2048 * 8


def test_bad_ranges(synth_mod):
    with pytest.raises(ValueError):
        synth_mod.combine_inputs("small", b_lo=3, b_hi=99)
    with pytest.raises(ValueError):
        synth_mod.rank_inputs("packed", 8)
