"""Pins for the seeded input generator (no GPU)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp2(rng.integers(-40, 40, 100000))).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000],
                    dtype=np.uint32).view(np.float32)
    a = np.concatenate([a, ties])
    got = workloads.f32_to_bf16_bits(a)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert got[-4] == 0x3F80 and got[-3] == 0x3F82  # tie to even


def test_bf16_decode_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = workloads.bf16_bits_to_f32(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(workloads.f32_to_bf16_bits(vals[fin]), bits[fin])


def test_case_recipe():
    c = workloads.make_case("tiny")
    assert c["codes"].shape == (1, 256, 512) and c["codes"].dtype == np.uint8
    assert c["scales"].shape == (1, 256, 8) and c["scales"].dtype == np.uint16
    assert c["x"].shape == (1, 1, 512) and c["x"].dtype == np.float32
    assert set(np.unique(c["codes"])) == set(range(16))
    s = workloads.bf16_bits_to_f32(c["scales"]).astype(np.float64)
    b = workloads.bf16_bits_to_f32(c["biases"]).astype(np.float64)
    assert np.array_equal(b, -8.0 * s)
    assert 0.015 < s.std() < 0.025
    c2 = workloads.make_case("tiny")
    for k in ("codes", "scales", "biases", "x"):
        assert np.array_equal(c[k], c2[k])
    c3 = workloads.make_case("tiny", seed=1)
    assert not np.array_equal(c["codes"], c3["codes"])


def test_moe_scale_and_shapes():
    w = workloads.WORKLOADS["moe_down"]
    x = workloads.make_x(w["n_mat"], w["nb"], w["in_dim"], 0, w["x_scale"])
    x1 = workloads.make_x(w["n_mat"], w["nb"], w["in_dim"], 0, 1.0)
    assert np.array_equal(x, x1 * np.float32(0.5))
    assert x.shape == (8, 4, 640)


def test_weight_bytes():
    assert workloads.weight_bytes(1, 9728, 2560) == 14008320
    assert workloads.weight_bytes(1, 151936, 2560) == 218787840
    assert workloads.weight_bytes(8, 2560, 640) == 7372800


def test_routing_recipe():
    for seed in range(4):
        sel, wmap = workloads.make_routing(4, 32, 8, seed=seed)
        assert sel.dtype == np.int32 and np.all(np.diff(sel) > 0)
        assert sel.min() >= 0 and sel.max() < 32
        assert wmap.shape == (4, sel.size) and wmap.dtype == np.float32
        assert np.all((wmap > 0).sum(axis=1) == 8)
        assert np.all((wmap > 0).any(axis=0))  # every slot is some token's pick
        assert np.allclose(wmap.sum(axis=1), 1.0, atol=1e-6)
    a = workloads.make_routing(4, 32, 8, seed=1)
    b = workloads.make_routing(4, 32, 8, seed=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
