"""CPU pins of the oracle's 8-bit per-row table (the decoder's embeddings and
lm_head) against values fixed by hand and by the mathematics, independent of
the oracle itself: the worked example in tests/golden/rowq_worked.txt, the
reduction of each row to the per-tensor int8 quantization (pinned on its own),
power-of-two scale invariance per row, numpy's integer matmul, the exact
rational dequantization bound, and exact fp32 products for the embedding.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import read_golden
from ternary_weight_decoder_amd import synth


def golden():
    g = {}
    for r in read_golden("rowq_worked.txt"):
        g.setdefault(r[0], []).append(r[1:])
    return g


def u32(h):
    return np.array([int(h, 16)], np.uint32).view(np.float32)[0]


def test_worked_example():
    g = golden()
    W = np.array([[float.fromhex(v) for v in r[1:]] for r in g["w_hex"]], np.float32)
    q, s = oracle.rowq_quant_weights(W)
    np.testing.assert_array_equal(q, np.array([r[1:] for r in g["q"]], np.int8))
    assert s.tobytes() == np.array([u32(h) for h in g["scale_bits"][0]], np.float32).tobytes()
    x = np.array([r[1:] for r in g["x"]], np.float32)
    out = oracle.rowq_linear(x, q, s)
    np.testing.assert_array_equal(out["acc"], np.array([r[1:] for r in g["acc"]], np.int32))
    want = np.array([[u32(h) for h in r[1:]] for r in g["y_bits"]], np.float32)
    assert out["y"].tobytes() == want.tobytes()
    e = oracle.rowq_embed(np.array(g["ids"][0], np.int32), q, s)
    want = np.array([[float.fromhex(v) for v in r[1:]] for r in g["emb_hex"]], np.float32)
    assert e.tobytes() == want.tobytes()


def test_rows_reduce_to_the_per_tensor_quantization():
    # each row alone, through the (separately pinned) per-tensor int8
    # quantization, must give that row's codes and scale
    W = synth.student_t_weights(37, 320, 11)
    W[5] = 0.0
    W[9, 17] = np.float32(-0.5)          # a row whose maximum is a negative entry
    q, s = oracle.rowq_quant_weights(W)
    for n in range(W.shape[0]):
        qn, sn = oracle.i8_quant_weights(W[n:n + 1])
        np.testing.assert_array_equal(q[n], qn[0])
        assert s[n] == sn


def test_row_scale_invariance_and_bound():
    rng = np.random.default_rng(3)
    W = synth.normal_weights(64, 256, 4)
    q, s = oracle.rowq_quant_weights(W)
    f = np.float32(2.0) ** rng.integers(-6, 7, size=(64, 1)).astype(np.float32)
    q2, s2 = oracle.rowq_quant_weights((W * f).astype(np.float32))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, (s * f[:, 0]).astype(np.float32))
    assert (np.abs(q).max(axis=1) == 127).all()
    r = W.astype(np.float64) / s[:, None].astype(np.float64)
    assert np.abs(q - r).max() <= 0.5 + 1e-4
    assert (np.sign(q) * np.sign(W) >= 0).all()


def test_lm_head_matches_integer_product_and_exact_dequant():
    W = synth.normal_weights(300, 384, 8)
    x = synth.activations(5, 384, 9)
    q, s = oracle.rowq_quant_weights(W)
    out = oracle.rowq_linear(x, q, s)
    xq, xs = oracle.quant_act(x)
    np.testing.assert_array_equal(out["xq"], xq)
    acc = xq.astype(np.int64) @ q.astype(np.int64).T
    np.testing.assert_array_equal(out["acc"], acc.astype(np.int32))
    for m, n in [(0, 0), (1, 17), (4, 299), (2, 150), (3, 64)]:
        exact = Fraction(int(acc[m, n])) * Fraction(float(s[n])) / Fraction(float(xs[m]))
        got = Fraction(float(out["y"][m, n]))
        ulp = abs(float(np.spacing(out["y"][m, n])))
        assert abs(got - exact) <= Fraction(ulp) / 2


def test_lm_head_scale_follows_the_column():
    # scaling one table row by 2 doubles that output column and no other
    W = synth.normal_weights(16, 128, 12)
    x = synth.activations(3, 128, 13)
    q, s = oracle.rowq_quant_weights(W)
    base = oracle.rowq_linear(x, q, s)["y"]
    s2 = s.copy()
    s2[7] *= np.float32(2.0)
    y2 = oracle.rowq_linear(x, q, s2)["y"]
    np.testing.assert_array_equal(y2[:, 7], base[:, 7] * np.float32(2.0))
    np.testing.assert_array_equal(np.delete(y2, 7, axis=1), np.delete(base, 7, axis=1))


def test_embedding_is_the_scaled_row():
    W = synth.normal_weights(50, 256, 14)
    q, s = oracle.rowq_quant_weights(W)
    ids = np.array([0, 49, 7, 7, -1, 50, 23], np.int32)
    e = oracle.rowq_embed(ids, q, s)
    for t, i in enumerate(ids):
        if 0 <= i < 50:
            # one IEEE fp32 product of two exact inputs
            np.testing.assert_array_equal(e[t], q[i].astype(np.float32) * s[i])
        else:
            assert not e[t].any()


def test_sampled_matches_full():
    W = synth.normal_weights(97, 256, 15)
    x = synth.activations(4, 256, 16)
    q, s = oracle.rowq_quant_weights(W)
    full = oracle.rowq_linear(x, q, s)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 4, 40)
    ns = rng.integers(0, 97, 40)
    acc, y = oracle.rowq_linear_sampled(full["xq"], full["x_scale"], q, s, ms, ns)
    np.testing.assert_array_equal(acc, full["acc"][ms, ns])
    np.testing.assert_array_equal(y, full["y"][ms, ns])


# ---- I8_S with per-channel weight scales -------------------------------------

def test_per_channel_layer_worked_example():
    g = golden()
    W = np.array([[float.fromhex(v) for v in r[1:]] for r in g["w_hex"]], np.float32)
    q, s = oracle.rowq_quant_weights(W)
    x = np.array([r[1:] for r in g["x"]], np.float32)
    b = np.array(g["bias"][0], np.float32)
    for relu, key in ((False, "yb_bits"), (True, "ybr_bits")):
        out = oracle.i8_linear_rows(x, q, s, b, relu=relu)
        np.testing.assert_array_equal(out["acc"], np.array([r[1:] for r in g["acc"]], np.int32))
        want = np.array([[u32(h) for h in r[1:]] for r in g[key]], np.float32)
        assert out["y"].tobytes() == want.tobytes(), key
    # without bias or ReLU it is the lm_head's output
    out = oracle.i8_linear_rows(x, q, s)
    want = np.array([[u32(h) for h in r[1:]] for r in g["y_bits"]], np.float32)
    assert out["y"].tobytes() == want.tobytes()


@pytest.mark.parametrize("relu", [False, True])
def test_per_channel_layer_with_equal_scales_is_the_per_tensor_layer(relu):
    # every channel scale equal to the tensor scale: the separately pinned
    # per-tensor I8_S layer, bit for bit
    W = synth.normal_weights(70, 192, 20)
    x = synth.activations(9, 192, 21)
    b = synth.normal_weights(1, 70, 22, std=0.1)[0]
    q, s = oracle.i8_quant_weights(W)
    ref = oracle.i8_linear(x, q, s, b, relu=relu)
    out = oracle.i8_linear_rows(x, q, np.full(70, s, np.float32), b, relu=relu)
    assert out["y"].tobytes() == ref["y"].tobytes()
    np.testing.assert_array_equal(out["acc"], ref["acc"])


def test_per_channel_layer_bias_and_scale_follow_the_channel():
    W = synth.normal_weights(12, 128, 23)
    x = synth.activations(4, 128, 24)
    q, s = oracle.rowq_quant_weights(W)
    base = oracle.i8_linear_rows(x, q, s)["y"]
    b = np.zeros(12, np.float32)
    b[5] = np.float32(0.75)
    y = oracle.i8_linear_rows(x, q, s, b)["y"]
    np.testing.assert_array_equal(np.delete(y, 5, axis=1), np.delete(base, 5, axis=1))
    exact = [Fraction(float(v)) + Fraction(3, 4) for v in base[:, 5]]
    assert all(abs(Fraction(float(g)) - e) <= Fraction(abs(float(np.spacing(g)))) for g, e in
               zip(y[:, 5], exact))
    s2 = s.copy()
    s2[3] *= np.float32(4.0)
    y2 = oracle.i8_linear_rows(x, q, s2)["y"]
    np.testing.assert_array_equal(y2[:, 3], base[:, 3] * np.float32(4.0))
    r = oracle.i8_linear_rows(x, q, s, relu=True)["y"]
    np.testing.assert_array_equal(r, np.maximum(base, 0))


def test_per_channel_sampled_matches_full():
    W = synth.normal_weights(40, 256, 25)
    x = synth.activations(6, 256, 26)
    b = synth.normal_weights(1, 40, 27, std=0.1)[0]
    q, s = oracle.rowq_quant_weights(W)
    full = oracle.i8_linear_rows(x, q, s, b, relu=True)
    ms = np.arange(6).repeat(40)
    ns = np.tile(np.arange(40), 6)
    acc, d, y = oracle.i8_linear_rows_sampled(full["xq"], full["x_scale"], q, s, b, True, ms, ns)
    np.testing.assert_array_equal(acc, full["acc"].ravel())
    np.testing.assert_array_equal(y, full["y"].ravel())


# ---- the table's storage layout ----------------------------------------------

def test_table_layout_golden():
    rows = read_golden("table_layout.txt")
    V = int([r for r in rows if r[0] == "V"][0][1])
    K = int([r for r in rows if r[0] == "K"][0][1])
    assert oracle.table_bytes(V, K) == int([r for r in rows if r[0] == "bytes"][0][1])
    for r in rows:
        if r[0] != "at":
            continue
        v, k, off = int(r[1]), int(r[2]), int(r[3])
        q = np.zeros((V, K), np.int8)
        q[v, k] = 7
        t = oracle.table_pack(q)
        assert np.flatnonzero(t).tolist() == [off], (v, k)


@pytest.mark.parametrize("V,K", [(1, 64), (16, 256), (37, 320), (40, 1536), (100, 768)])
def test_table_round_trip_and_padding(V, K):
    rng = np.random.default_rng(V * K)
    q = rng.integers(-127, 128, size=(V, K), dtype=np.int16).astype(np.int8)
    t = oracle.table_pack(q)
    assert t.size == ((V + 15) // 16 * 16) * ((K + 255) // 256 * 256)
    back, bad = oracle.table_unpack(t, V, K)
    assert bad == 0
    np.testing.assert_array_equal(back, q)
    # all-ones codes: the zero bytes of the table are exactly its padding, so
    # the layout is a bijection onto the other bytes
    ones = oracle.table_pack(np.ones((V, K), np.int8))
    assert np.count_nonzero(ones) == V * K
    pad = np.flatnonzero(ones == 0)
    assert pad.size == t.size - V * K
    if pad.size:
        t2 = t.copy()
        t2[pad[pad.size // 2]] = 1
        assert oracle.table_unpack(t2, V, K)[1] == 1
