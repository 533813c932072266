"""GPU parity of the decoder's 8-bit per-row table (embeddings and lm_head)
against the oracle, through the C ABI.

Table bytes (the oracle's own packing of its codes into the storage order,
zero padding included) and scales, embedding rows, int8 activations, int32
accumulators and the lm_head outputs (exactly rounded fp64 epilogue) are all
bit-exact.
Shapes cover ragged V around the 16-column block, K of one MFMA step (64),
ragged 256-input items, every M from 1 to 16, the LDS limit, zero rows on
both sides, out-of-range token ids, and the full 151,936 x 1536 table.
Outputs carry a NaN canary past their ends.
"""
import sys

import numpy as np
import pytest

import oracle
from conftest import read_golden
from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu
CANARY = 4096


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ternary_weight_decoder_amd import binding
    binding.lib()
    return binding


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def guarded(n, dtype, fill):
    import torch
    t = torch.full((n + CANARY,), fill, dtype=dtype, device="cuda:0")
    return t, t[:n]


def canary_ok(buf, n):
    tail = buf[n:].cpu().numpy()
    return np.isnan(tail).all() if tail.dtype.kind == "f" else (tail == tail[0]).all()


def gpu_table(tb, W):
    """The table in its storage order and the row scales, made on the GPU."""
    import torch
    V, K = W.shape
    nb = tb.bitnet_table_bytes(V, K)
    qb, q = guarded(nb, torch.int8, 77)
    sb, s = guarded(V, torch.float32, float("nan"))
    tb.bitnet_table_quant_into(dev(W), V, K, q, s)
    torch.cuda.synchronize()
    assert canary_ok(qb, nb) and canary_ok(sb, V)
    return q, s


def run_lm_head(tb, x, t_dev, s_dev):
    import torch
    M, K = x.shape
    N = s_dev.numel()
    yb, y = guarded(M * N, torch.float32, float("nan"))
    ab, acc = guarded(M * N, torch.int32, -7)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda:0")
    xs = torch.empty(M, dtype=torch.float32, device="cuda:0")
    tb.bitnet_lm_head_into(M, N, K, dev(x), t_dev, s_dev, y, xq, xs, acc)
    torch.cuda.synchronize()
    assert canary_ok(yb, M * N), "y canary overwritten"
    assert canary_ok(ab, M * N), "acc canary overwritten"
    return (y.view(M, N).cpu().numpy(), acc.view(M, N).cpu().numpy(), xq.cpu().numpy(),
            xs.cpu().numpy())


@pytest.mark.parametrize("N,K", [(1, 64), (200, 192), (37, 1536), (1000, 4096), (16, 8960),
                                 (21, 320)])
def test_table_quant_bit_exact(tb, N, K):
    say(f"[table quant] N={N} K={K}")
    W = synth.student_t_weights(N, K, 900 + N + K)
    if N > 5:
        W[3] = 0.0                       # zero row: scale 0, codes 0
        W[4, -1] = np.float32(-1.0)      # the row maximum at the last entry
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    t, s = gpu_table(tb, W)
    assert t.cpu().numpy().tobytes() == oracle.table_pack(q_ref).tobytes()
    assert s.cpu().numpy().tobytes() == s_ref.tobytes()


@pytest.mark.parametrize("N,K", [(3, 64), (200, 192)])
def test_row_major_quant_bit_exact(tb, N, K):
    # the per-channel I8_S weights: the same codes, plain row-major
    import torch
    W = synth.normal_weights(N, K, 950 + N)
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    q, s = tb.bitnet_i8_quant_weights_rows(torch.from_numpy(W).to("cuda:0"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    assert s.cpu().numpy().tobytes() == s_ref.tobytes()


def test_worked_example(tb):
    say("[table] worked example")
    g = {}
    for r in read_golden("rowq_worked.txt"):
        g.setdefault(r[0], []).append(r[1:])
    W = np.zeros((4, 64), np.float32)
    W[:, :4] = np.array([[float.fromhex(v) for v in r[1:]] for r in g["w_hex"]], np.float32)
    q, s = gpu_table(tb, W)
    qh, bad = oracle.table_unpack(q.cpu().numpy(), 4, 64)
    assert bad == 0
    np.testing.assert_array_equal(qh[:, :4], np.array([r[1:] for r in g["q"]], np.int8))
    assert not qh[:, 4:].any()
    want_s = np.array([int(h, 16) for h in g["scale_bits"][0]], np.uint32).view(np.float32)
    assert s.cpu().numpy().tobytes() == want_s.tobytes()
    x = np.zeros((2, 64), np.float32)
    x[:, :4] = np.array([r[1:] for r in g["x"]], np.float32)
    y, acc, _, _ = run_lm_head(tb, x, q, s)
    np.testing.assert_array_equal(acc, np.array([r[1:] for r in g["acc"]], np.int32))
    want_y = np.array([[int(h, 16) for h in r[1:]] for r in g["y_bits"]], np.uint32)
    assert y.view(np.uint32).tolist() == want_y.tolist()


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_lm_head_every_m(tb, M):
    N, K = 333, 1536
    say(f"[lm_head] M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, 910)
    W[5] = 0.0
    x = synth.activations(M, K, 911 + M)
    if M >= 3:
        x[1] = 0.0                       # zero row: x_scale 1, outputs 0
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    ref = oracle.rowq_linear(x, q_ref, s_ref)
    q, s = gpu_table(tb, W)
    y, acc, xq, xs = run_lm_head(tb, x, q, s)
    np.testing.assert_array_equal(xq, ref["xq"])
    assert xs.tobytes() == ref["x_scale"].tobytes()
    np.testing.assert_array_equal(acc, ref["acc"])
    assert y.tobytes() == ref["y"].tobytes()


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (3, 17, 64), (2, 31, 320), (5, 250, 768),
                                   (14, 129, 3968), (16, 1000, 3456), (1, 4099, 16320),
                                   (4, 70000, 192), (16, 151936 // 4, 1536)])
def test_lm_head_shapes(tb, M, N, K):
    say(f"[lm_head] M={M} N={N} K={K}")
    W = synth.student_t_weights(N, K, 920 + N)
    x = synth.activations(M, K, 921 + K)
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    ref = oracle.rowq_linear(x, q_ref, s_ref)
    y, acc, xq, xs = run_lm_head(tb, x, dev(oracle.table_pack(q_ref)), dev(s_ref))
    np.testing.assert_array_equal(xq, ref["xq"])
    np.testing.assert_array_equal(acc, ref["acc"])
    assert y.tobytes() == ref["y"].tobytes()


def test_lm_head_worst_case_magnitude(tb):
    # every product at +-127 * 127: |acc| = 16129 * K
    M, N, K = 2, 48, 4096
    say("[lm_head] worst-case magnitude")
    x = np.full((M, K), 3.0, np.float32)
    x[1] *= -1.0
    W = np.full((N, K), 0.5, np.float32)
    W[1::2] *= -1.0
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    ref = oracle.rowq_linear(x, q_ref, s_ref)
    assert abs(int(ref["acc"][0, 0])) == 127 * 127 * K
    y, acc, _, _ = run_lm_head(tb, x, dev(oracle.table_pack(q_ref)), dev(s_ref))
    np.testing.assert_array_equal(acc, ref["acc"])
    assert y.tobytes() == ref["y"].tobytes()


def test_lm_head_repeat_and_sensitivity(tb):
    M, N, K = 4, 2000, 1536
    say("[lm_head] repeat")
    W = synth.normal_weights(N, K, 930)
    x = synth.activations(M, K, 931)
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    qd, sd = dev(oracle.table_pack(q_ref)), dev(s_ref)
    y1, _, _, _ = run_lm_head(tb, x, qd, sd)
    y2, _, _, _ = run_lm_head(tb, x, qd, sd)
    assert y1.tobytes() == y2.tobytes()
    x2 = x.copy()
    x2[2, 100] += np.float32(1.0)
    y3, _, _, _ = run_lm_head(tb, x2, qd, sd)
    assert (y3[2] != y1[2]).any() and y3[[0, 1, 3]].tobytes() == y1[[0, 1, 3]].tobytes()


def test_embed_lookup(tb):
    import torch
    N, K = 300, 1536
    say("[embed] lookup")
    W = synth.normal_weights(N, K, 940)
    W[7] = 0.0
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    ids = np.array([0, 299, 7, 7, -1, 300, 123456, 42] + list(range(50, 90)), np.int32)
    ref = oracle.rowq_embed(ids, q_ref, s_ref)
    T = ids.size
    ob, out = guarded(T * K, torch.float32, float("nan"))
    table = dev(oracle.table_pack(q_ref))
    tb.bitnet_embed_lookup_into(dev(ids), T, table, dev(s_ref), N, K, out)
    torch.cuda.synchronize()
    assert canary_ok(ob, T * K)
    assert out.view(T, K).cpu().numpy().tobytes() == ref.tobytes()
    # no tokens: nothing launched, nothing written
    tb.bitnet_embed_lookup_into(dev(ids[:1]), 0, table, dev(s_ref), N, K, ob[T * K:])
    torch.cuda.synchronize()
    assert canary_ok(ob, T * K)


def test_full_table(tb):
    """The 151,936 x 1536 table: codes and scales bit-exact, the lm_head at M = 1
    against the oracle on every output and at M = 16 on sampled outputs, and
    the embedding rows of 64 ids."""
    import torch
    V, K = synth.VOCAB, synth.HIDDEN
    say(f"[table] full V={V} K={K}")
    W = synth.table_weights()
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    Wd = dev(W)
    q = torch.empty(tb.bitnet_table_bytes(V, K), dtype=torch.int8, device="cuda:0")
    s = torch.empty(V, dtype=torch.float32, device="cuda:0")
    tb.bitnet_table_quant_into(Wd, V, K, q, s)
    torch.cuda.synchronize()
    del Wd
    assert np.array_equal(q.cpu().numpy(), oracle.table_pack(q_ref))
    assert s.cpu().numpy().tobytes() == s_ref.tobytes()
    x1 = synth.activations(1, K, synth.TABLE_SEED + 2)
    ref = oracle.rowq_linear(x1, q_ref, s_ref)
    y, acc, _, _ = run_lm_head(tb, x1, q, s)
    np.testing.assert_array_equal(acc, ref["acc"])
    assert y.tobytes() == ref["y"].tobytes()
    x16 = synth.activations(16, K, synth.TABLE_SEED + 3)
    y, acc, xq, xs = run_lm_head(tb, x16, q, s)
    xq_ref, xs_ref = oracle.quant_act(x16)
    np.testing.assert_array_equal(xq, xq_ref)
    rng = np.random.default_rng(5)
    ms = rng.integers(0, 16, 4000)
    ns = np.concatenate([rng.integers(0, V, 3984), np.arange(V - 16, V)])
    acc_s, y_s = oracle.rowq_linear_sampled(xq_ref, xs_ref, q_ref, s_ref, ms, ns)
    np.testing.assert_array_equal(acc[ms, ns], acc_s)
    assert y[ms, ns].tobytes() == y_s.tobytes()
    ids = synth.token_ids(64)
    out = tb.bitnet_embed_lookup(dev(ids), q, s, K)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == oracle.rowq_embed(ids, q_ref, s_ref).tobytes()
