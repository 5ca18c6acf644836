"""Seeded input generator: determinism, shapes, distributions, and its 16-bit rounding
agrees with the oracle's independent encoder."""

import os

import numpy as np
import pytest

import oracle
import workloads as W


def test_shapes_and_determinism():
    w = W.custom(33, 17, 65, W.BF16, W.BF16, W.B_KN)
    a1, b1 = W.make_inputs(w)
    a2, b2 = W.make_inputs(w)
    assert a1.shape == (33, 65) and b1.shape == (65, 17)
    assert a1.dtype == np.uint16 and np.array_equal(a1, a2) and np.array_equal(b1, b2)
    w2 = W.custom(33, 17, 65, W.F16, W.F16, W.B_NK)
    a3, b3 = W.make_inputs(w2)
    assert b3.shape == (17, 65)
    assert not np.array_equal(a1, W.make_inputs(w, seed_a=7)[0])


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_rounding_matches_oracle_encoder(dtype):
    r = np.random.Generator(np.random.PCG64(0))
    x32 = (r.standard_normal(200000) * np.exp2(r.integers(-20, 10, 200000))).astype(np.float32)
    bits = W.float32_to_bits(x32, dtype)
    assert np.array_equal(bits, oracle.encode(x32.astype(np.float64), dtype))


def test_distributions():
    w = W.custom(512, 512, 512, W.F16, W.F16, W.B_NK, dist=("uniform", -1.0, 1.0))
    a, _ = W.make_inputs(w)
    v = oracle.decode(a, "f16")
    assert v.min() >= -1 and v.max() <= 1 and abs(v.mean()) < 0.01
    assert abs(v.std() - (1 / 3) ** 0.5) < 0.01
    w = W.custom(512, 512, 512, W.BF16, W.BF16, W.B_KN, dist=("normal", 0.02))
    a, _ = W.make_inputs(w)
    v = oracle.decode(a, "bf16")
    assert abs(v.std() - 0.02) < 0.001
    w = W.WORKLOADS["pallas_hopper_example"]
    assert (w.M, w.N, w.K) == (132 * 128, 4 * 128, 10 * 64)


def test_workload_table():
    t = W.WORKLOADS
    assert (t["nn_bf16_8192"].M, t["nn_bf16_8192"].b_layout) == (8192, W.B_KN)
    assert t["tn_f16_3000x5000x1000_f32out"].out_dtype == W.F32
    assert t["nn_bf16_3072x4096x4096_gelu"].epilogue == "gelu_tanh"
    assert t["nn_f16_2048x2048x1024_relu_f32out"].epilogue == "relu"


def test_pallas_example_shape_is_the_golden_one():
    # the Pallas guide's Hopper matmul example shape (tests/golden/hopper_example_shape.txt)
    golden = {}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "hopper_example_shape.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            golden[k] = int(v)
    w = W.WORKLOADS["pallas_hopper_example"]
    assert (w.M, w.N, w.K) == (golden["m"], golden["n"], golden["k"])
    assert golden["m"] == 132 * golden["tile_m"] and golden["n"] == 4 * golden["tile_n"]
    assert golden["k"] == 10 * golden["tile_k"]
    assert w.in_dtype == W.F16 and w.b_layout == W.B_KN and w.dist == ("unit",)
