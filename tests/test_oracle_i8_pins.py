"""CPU pins of the I8_S oracle (int8 weights x int8 activations) against
values fixed by hand and by the mathematics, independent of the oracle itself:
the worked examples in tests/golden/i8_linear_worked.txt, exact rounding ties,
power-of-two scale invariance, the half-step error bound, numpy's integer
matmul, and the ReLU / bias special cases.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden


def golden():
    ex = {}
    for row in read_golden("i8_linear_worked.txt"):
        ex.setdefault(row[0], {}).setdefault(row[1], []).append(row[2:])
    return ex


def bits(h):
    return np.array([int(h, 16)], np.uint32).view(np.float32)[0]


def test_worked_example_unit_scales():
    A = golden()["A"]
    x = np.array([A["x"][0]], np.float32).astype(np.float32)
    W = np.array(A["w"], np.float32)
    bias = np.array(A["bias"][0], np.float32)
    q, s = oracle.i8_quant_weights(W)
    assert s == np.float32(A["scale"][0][0])
    np.testing.assert_array_equal(q, np.array(A["q"], np.int8))
    r = oracle.i8_linear(x, q, s, bias, relu=False)
    np.testing.assert_array_equal(r["acc"][0], np.array(A["acc"][0], np.int32))
    np.testing.assert_array_equal(r["y"][0], np.array(A["y"][0], np.float32))
    r = oracle.i8_linear(x, q, s, bias, relu=True)
    np.testing.assert_array_equal(r["y"][0], np.array(A["y_relu"][0], np.float32))


def test_worked_example_scales():
    B = golden()["B"]
    x = np.array([B["x"][0]], np.float32)
    W = np.array(B["w"], np.float32)
    q, s = oracle.i8_quant_weights(W)
    assert s == bits(B["scale_bits"][0][0])
    np.testing.assert_array_equal(q[0], np.array(B["q"][0], np.int8))
    r = oracle.i8_linear(x, q, s)
    assert int(r["acc"][0, 0]) == int(B["acc"][0][0])
    assert r["y"][0, 0] == bits(B["y_bits"][0][0])
    r = oracle.i8_linear(x, q, s, np.array(B["bias"][0], np.float32))
    assert r["y"][0, 0] == bits(B["y_bias_bits"][0][0])


def test_weight_ties_round_to_even():
    # max|W| = 127 gives s = 1 exactly, so W / s = W and the ties are exact.
    W = np.array([[0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 126.5, 127.0]], np.float32)
    q, s = oracle.i8_quant_weights(W)
    assert s == np.float32(1.0)
    np.testing.assert_array_equal(q[0], np.array([0, 2, 2, -2, 4, 0, 126, 127], np.int8))


def test_weight_scale_invariance_and_bound():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((37, 96)) * 0.02).astype(np.float32)
    q, s = oracle.i8_quant_weights(W)
    # the largest |W| maps to +-127; every weight is within half a step
    i = np.unravel_index(np.argmax(np.abs(W)), W.shape)
    assert abs(int(q[i])) == 127
    err = np.abs(W.astype(np.float64) - q.astype(np.float64) * np.float64(s))
    assert err.max() <= 0.5 * float(s) * (1 + 1e-6)
    # scaling W by a power of two scales s exactly and leaves q unchanged
    for e in (-3, 4):
        q2, s2 = oracle.i8_quant_weights(W * np.float32(2.0 ** e))
        np.testing.assert_array_equal(q2, q)
        assert s2 == np.float32(s * np.float32(2.0 ** e))


def test_zero_weights():
    q, s = oracle.i8_quant_weights(np.zeros((3, 64), np.float32))
    assert s == 0 and not q.any()


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 33, 128), (4, 3, 2048)])
def test_matmul_equals_numpy(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    xq = rng.integers(-127, 128, size=(M, K), dtype=np.int16).astype(np.int8)
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int16).astype(np.int8)
    ref = xq.astype(np.int64) @ q.astype(np.int64).T
    np.testing.assert_array_equal(oracle.i8_matmul(xq, q), ref.astype(np.int32))


def test_matmul_extremes():
    K = 4096
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -127
    q = np.full((2, K), 127, np.int8)
    q[1, ::2] = -127
    acc = oracle.i8_matmul(xq, q)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K
    assert acc[0, 1] == 0 and acc[1, 1] == 0


def test_relu_and_bias_cases():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    q, s = oracle.i8_quant_weights((rng.standard_normal((40, 256)) * 0.02).astype(np.float32))
    b = (rng.standard_normal(40) * 0.1).astype(np.float32)
    plain = oracle.i8_linear(x, q, s)
    zero_b = oracle.i8_linear(x, q, s, np.zeros(40, np.float32))
    np.testing.assert_array_equal(plain["y"], zero_b["y"])
    biased = oracle.i8_linear(x, q, s, b)
    relu = oracle.i8_linear(x, q, s, b, relu=True)
    assert (relu["y"] >= 0).all()
    np.testing.assert_array_equal(relu["y"], np.where(biased["y"] > 0, biased["y"], 0))
    # a zero activation row: xq = 0, x_scale = 1, y = relu?(bias)
    x0 = np.zeros((1, 256), np.float32)
    r = oracle.i8_linear(x0, q, s, b, relu=True)
    assert r["x_scale"][0] == 1 and not r["acc"].any()
    np.testing.assert_array_equal(r["y"][0], np.maximum(b, 0))


def test_sampled_matches_full():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 384)).astype(np.float32)
    q, s = oracle.i8_quant_weights((rng.standard_normal((50, 384)) * 0.02).astype(np.float32))
    b = (rng.standard_normal(50) * 0.1).astype(np.float32)
    full = oracle.i8_linear(x, q, s, b, relu=True)
    ms = np.array([0, 3, 8, 8], np.int64)
    ns = np.array([0, 49, 7, 13], np.int64)
    acc, d, y = oracle.i8_linear_sampled(full["xq"], full["x_scale"], q, s, b, True, ms, ns)
    np.testing.assert_array_equal(acc, full["acc"][ms, ns])
    np.testing.assert_array_equal(y, full["y"][ms, ns])


def test_weight_code_is_the_ieee_quotient():
    # golden example C: the quotient W/s and the product W*fl32(1/s) fall on
    # opposite sides of 9.5; the reading is the quotient.
    C = golden()["C"]
    W = np.zeros((1, 64), np.float32)
    vals = [float.fromhex(h) for h in C["w_hex"][0]]
    W[0, :len(vals)] = vals
    q, s = oracle.i8_quant_weights(W)
    assert s == np.float32(C["scale"][0][0])
    np.testing.assert_array_equal(q[0, :2], np.array(C["q"][0], np.int8))
    assert not q[0, 2:].any()
    # the example discriminates: the reciprocal form rounds the other way
    assert np.rint(np.float32(W[0, 1]) * (np.float32(1) / s)) == 10
