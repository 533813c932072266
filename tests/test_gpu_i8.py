"""GPU parity of the I8_S path (int8 weights x int8 activations) against the oracle.

Weight codes and scales are bit-exact; accumulators are bit-exact; outputs
are within the epilogue's bound 4 * 2^-24 * (|acc * w_scale / x_scale| +
|bias|), derived from its three fp32 roundings (accumulator to float, the
row factor, the product) and the bias add.  Shapes cover ragged M and N
around the 128 x 128 tile, K of one step (64) and odd step counts, bias and
ReLU on and off, a zero activation row, and both full-size encoder layers on
sampled outputs.
"""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu
TOL = 4.0 * 2.0 ** -24


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


def check_y(y, ref_y, d, bias_vals, what):
    bound = TOL * (np.abs(d) + np.abs(bias_vals)) + 1e-37
    err = np.abs(y.astype(np.float64) - ref_y.astype(np.float64))
    worst = (err / bound).max() if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the bound"


@pytest.mark.parametrize("N,K", [(128, 64), (200, 192), (2048, 512), (512, 2048), (7, 64)])
def test_i8_weight_quant_bit_exact(tb, N, K):
    import torch
    say(f"[i8] weight quantization N={N} K={K}")
    W = synth.normal_weights(N, K, 500 + N + K)
    if N == 7:
        W[-1, -1] = np.float32(-3.0)       # the maximum sits at the last element
    q_ref, s_ref = oracle.i8_quant_weights(W)
    q, s = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to("cuda:0"))
    assert s.cpu().numpy()[0] == s_ref
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_i8_weight_quant_zero_and_ties(tb):
    import torch
    q, s = tb.bitnet_i8_quant_weights(torch.zeros((64, 64), device="cuda:0"))
    assert s.item() == 0.0 and not q.any().item()
    W = np.zeros((1, 64), np.float32)
    W[0, :8] = [0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 126.5, 127.0]
    q_ref, s_ref = oracle.i8_quant_weights(W)
    q, s = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to("cuda:0"))
    assert s.item() == s_ref == 1.0
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_i8_weight_quant_golden_quotient(tb):
    # hand-worked example C of i8_linear_worked.txt: W/s and W*fl32(1/s) round
    # to different codes; the kernel must give the quotient's (9, not 10)
    import torch
    from conftest import read_golden
    say("[i8] weight quantization golden quotient")
    C = {}
    for row in read_golden("i8_linear_worked.txt"):
        if row[0] == "C":
            C[row[1]] = row[2:]
    W = np.zeros((1, 64), np.float32)
    vals = [float.fromhex(h) for h in C["w_hex"]]
    W[0, :len(vals)] = vals
    q, s = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to("cuda:0"))
    assert s.item() == float(C["scale"][0])
    qh = q.cpu().numpy()
    np.testing.assert_array_equal(qh[0, :2], np.array([int(v) for v in C["q"]], np.int8))
    assert not qh[0, 2:].any()


def run_linear(tb, M, N, K, bias_on, relu, seed, zero_row=False):
    import torch
    dev = "cuda:0"
    rng = np.random.default_rng(seed)
    x = synth.activations(M, K, seed)
    if zero_row:
        x[M // 2] = 0
    W = synth.normal_weights(N, K, seed + 1)
    b = (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)) if bias_on else None
    q, s = oracle.i8_quant_weights(W)
    ref = oracle.i8_linear(x, q, s, b, relu)
    qd = torch.from_numpy(q).to(dev)
    sd = torch.tensor([s], dtype=torch.float32, device=dev)
    bd = torch.from_numpy(b).to(dev) if b is not None else None
    xd = torch.from_numpy(x).to(dev)
    ybuf = torch.full((M * N + 64,), float("nan"), device=dev)
    y = ybuf[:M * N].view(M, N)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    tb.bitnet_i8_linear_into(M, N, K, xd, qd, sd, bd, relu, y, ws, acc)
    torch.cuda.synchronize()
    assert torch.isnan(ybuf[M * N:]).all().item(), "wrote past the end of y"
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    d = ref["acc"].astype(np.float64) * np.float64(s) / ref["x_scale"].astype(np.float64)[:, None]
    bias_vals = np.zeros(N) if b is None else np.broadcast_to(b.astype(np.float64), (M, N))
    check_y(y.cpu().numpy(), ref["y"], d, bias_vals, f"M={M} N={N} K={K}")
    if relu:
        assert (y >= 0).all().item()


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (5, 7, 64), (130, 200, 192), (257, 129, 512),
                                   (128, 128, 128), (64, 2048, 512), (300, 96, 2048)])
@pytest.mark.parametrize("bias_on,relu", [(True, True), (False, False), (True, False)])
def test_i8_linear_parity(tb, M, N, K, bias_on, relu):
    say(f"[i8] linear M={M} N={N} K={K} bias={bias_on} relu={relu}")
    run_linear(tb, M, N, K, bias_on, relu, seed=M * 7 + N * 3 + K)


def test_i8_linear_zero_row(tb):
    say("[i8] linear with a zero activation row")
    run_linear(tb, 40, 130, 256, True, True, seed=77, zero_row=True)


@pytest.mark.parametrize("name", sorted(synth.I8_LAYERS))
def test_i8_full_layer_sampled(tb, name):
    import torch
    M, K, N, relu = synth.I8_LAYERS[name]
    say(f"[i8] full layer {name}: M={M} K={K} N={N} relu={relu}")
    x, W, b = synth.i8_layer_inputs(name)
    dev = "cuda:0"
    q_ref, s_ref = oracle.i8_quant_weights(W)
    qd, sd = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to(dev))
    assert sd.item() == s_ref
    np.testing.assert_array_equal(qd.cpu().numpy(), q_ref)
    y, acc = tb.bitnet_i8_linear(torch.from_numpy(x).to(dev), qd, sd, torch.from_numpy(b).to(dev),
                                 relu, return_acc=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 24)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 48)]))
    xq, xs = oracle.quant_act(x[rows])
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    acc_ref, d, y_ref = oracle.i8_linear_sampled(xq, xs, q_ref, s_ref, b, relu, ms, ns)
    got_acc = acc.cpu().numpy()[rows][:, cols].reshape(-1)
    got_y = y.cpu().numpy()[rows][:, cols].reshape(-1)
    np.testing.assert_array_equal(got_acc, acc_ref)
    check_y(got_y, y_ref, d, b[ns].astype(np.float64), name)
    assert not np.isnan(y.cpu().numpy()).any()


def test_i8_linear_short_tiles_many_workgroups(tb):
    """M = 8192, N = 1920: 960 tiles of 128 rows, so the call uses 64-row tiles,
    1920 workgroups, more than are resident at once.  Sampled parity, and two
    runs agree bit for bit."""
    import torch
    M, N, K = 8192, 1920, 512
    say(f"[i8] linear M={M} N={N} K={K}, 64-row tiles")
    dev = "cuda:0"
    x = synth.activations(M, K, 4321)
    W = synth.normal_weights(N, K, 4322)
    b = (np.random.default_rng(4323).standard_normal(N, dtype=np.float32) * np.float32(0.1))
    q_ref, s_ref = oracle.i8_quant_weights(W)
    qd, sd = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to(dev))
    xd, bd = torch.from_numpy(x).to(dev), torch.from_numpy(b).to(dev)
    y1, acc1 = tb.bitnet_i8_linear(xd, qd, sd, bd, True, return_acc=True)
    y2 = tb.bitnet_i8_linear(xd, qd, sd, bd, True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 32)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 64)]))
    xq, xs = oracle.quant_act(x[rows])
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    acc_ref, d, y_ref = oracle.i8_linear_sampled(xq, xs, q_ref, s_ref, b, True, ms, ns)
    np.testing.assert_array_equal(acc1.cpu().numpy()[rows][:, cols].reshape(-1), acc_ref)
    check_y(y1.cpu().numpy()[rows][:, cols].reshape(-1), y_ref, d, b[ns].astype(np.float64),
            "short tiles")


@pytest.mark.parametrize("K", [64, 1024])
def test_i8_linear_tall_tiles(tb, K):
    """M = 16384, N = 4096: 4096 tiles of 128 rows, the size from which the call
    switches to 128-row tiles, with steps of 64 (K = 64) and of 128 inputs
    (K = 1024).  Sampled parity; no output left unwritten."""
    import torch
    M, N = 16384, 4096
    say(f"[i8] linear M={M} N={N} K={K}, 128-row tiles")
    dev = "cuda:0"
    x = synth.activations(M, K, 5321)
    W = synth.normal_weights(N, K, 5322)
    q_ref, s_ref = oracle.i8_quant_weights(W)
    qd, sd = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to(dev))
    y = torch.full((M, N), float("nan"), device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    tb.bitnet_i8_linear_into(M, N, K, torch.from_numpy(x).to(dev), qd, sd, None, False, y, ws, acc)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 32)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 64)]))
    xq, xs = oracle.quant_act(x[rows])
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    acc_ref, d, y_ref = oracle.i8_linear_sampled(xq, xs, q_ref, s_ref, None, False, ms, ns)
    np.testing.assert_array_equal(acc.cpu().numpy()[rows][:, cols].reshape(-1), acc_ref)
    check_y(y.cpu().numpy()[rows][:, cols].reshape(-1), y_ref, d, np.zeros(ms.size), "tall tiles")


# ---- per-channel weight scales (bitnet_i8_linear_rows) ----------------------
# Bound of the per-channel epilogue fl32(fl32(fl32(acc) * s[n]) * fl32(1 / x_scale))
# + bias: five roundings.
TOL_ROWS = 5.0 * 2.0 ** -24


def check_y_rows(y, ref_y, d, bias_vals, what):
    bound = TOL_ROWS * (np.abs(d) + np.abs(bias_vals)) + 1e-37
    err = np.abs(y.astype(np.float64) - ref_y.astype(np.float64))
    worst = (err / bound).max() if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the bound"


def run_linear_rows(tb, M, N, K, bias_on, relu, seed, zero_row=False, zero_channel=False):
    import torch
    dev = "cuda:0"
    rng = np.random.default_rng(seed)
    x = synth.activations(M, K, seed)
    if zero_row:
        x[M // 2] = 0
    W = synth.student_t_weights(N, K, seed + 1)
    if zero_channel:
        W[N // 3] = 0
    b = (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)) if bias_on else None
    q, s = oracle.rowq_quant_weights(W)
    qd, sd = tb.bitnet_i8_quant_weights_rows(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qd.cpu().numpy(), q)
    assert sd.cpu().numpy().tobytes() == s.tobytes()
    ref = oracle.i8_linear_rows(x, q, s, b, relu)
    bd = torch.from_numpy(b).to(dev) if b is not None else None
    xd = torch.from_numpy(x).to(dev)
    ybuf = torch.full((M * N + 64,), float("nan"), device=dev)
    y = ybuf[:M * N].view(M, N)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    tb.bitnet_i8_linear_rows_into(M, N, K, xd, qd, sd, bd, relu, y, ws, acc)
    torch.cuda.synchronize()
    assert torch.isnan(ybuf[M * N:]).all().item(), "wrote past the end of y"
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    d = (ref["acc"].astype(np.float64) * s.astype(np.float64)[None, :]
         / ref["x_scale"].astype(np.float64)[:, None])
    bias_vals = np.zeros((M, N)) if b is None else np.broadcast_to(b.astype(np.float64), (M, N))
    check_y_rows(y.cpu().numpy(), ref["y"], d, bias_vals, f"M={M} N={N} K={K}")
    if relu:
        assert (y >= 0).all().item()


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (5, 7, 64), (130, 200, 192), (257, 129, 512),
                                   (64, 2048, 512), (300, 96, 2048)])
@pytest.mark.parametrize("bias_on,relu", [(True, True), (False, False)])
def test_i8_linear_rows_parity(tb, M, N, K, bias_on, relu):
    say(f"[i8 rows] linear M={M} N={N} K={K} bias={bias_on} relu={relu}")
    run_linear_rows(tb, M, N, K, bias_on, relu, seed=M * 5 + N * 11 + K)


def test_i8_linear_rows_zero_row_and_channel(tb):
    say("[i8 rows] zero activation row and zero weight channel")
    run_linear_rows(tb, 40, 130, 256, True, False, seed=91, zero_row=True, zero_channel=True)


@pytest.mark.parametrize("K", [64, 1024])
def test_i8_linear_rows_tall_tiles_sampled(tb, K):
    """4096 tiles of 128 rows (the tall-tile path) with per-channel scales, with
    steps of 64 and of 128 inputs."""
    import torch
    M, N = 16384, 4096
    say(f"[i8 rows] linear M={M} N={N} K={K}, 128-row tiles")
    dev = "cuda:0"
    x = synth.activations(M, K, 6321)
    W = synth.normal_weights(N, K, 6322)
    b = (np.random.default_rng(6323).standard_normal(N, dtype=np.float32) * np.float32(0.1))
    q, s = oracle.rowq_quant_weights(W)
    y, acc = tb.bitnet_i8_linear_rows(torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev),
                                      torch.from_numpy(s).to(dev), torch.from_numpy(b).to(dev),
                                      True, return_acc=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 32)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 64)]))
    xq, xs = oracle.quant_act(x[rows])
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    acc_ref, d, y_ref = oracle.i8_linear_rows_sampled(xq, xs, q, s, b, True, ms, ns)
    np.testing.assert_array_equal(acc.cpu().numpy()[rows][:, cols].reshape(-1), acc_ref)
    check_y_rows(y.cpu().numpy()[rows][:, cols].reshape(-1), y_ref, d, b[ns].astype(np.float64),
                 "tall tiles")
    assert not torch.isnan(y).any().item()


# ---- larger ragged layers: every output against the oracle, and bit for bit
# against the same call made on slices of the rows (rows are independent, so
# any split of M must give the same bytes, whatever tiles each call uses).

def _row_slices(tb, x, q, s, b, relu, rows_fn, K, N):
    import torch
    dev = "cuda:0"
    M = x.shape[0]
    cuts = [0, 1500, M] if M < 3000 else [0, 1500, 3000, M]
    ys, accs = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        m = hi - lo
        y = torch.full((m, N), float("nan"), device=dev)
        acc = torch.empty((m, N), dtype=torch.int32, device=dev)
        ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(m, K), dtype=torch.uint8, device=dev)
        rows_fn(m, N, K, x[lo:hi], q, s, b, relu, y, ws, acc)
        ys.append(y)
        accs.append(acc)
    return torch.cat(ys), torch.cat(accs)


@pytest.mark.parametrize("M,N,K", [(2085, 300, 768), (2048, 1000, 256), (2085, 2048, 256),
                                   (4100, 72, 2048)])
@pytest.mark.parametrize("bias_on,relu", [(True, True), (False, False)])
def test_i8_linear_large_ragged_parity(tb, M, N, K, bias_on, relu):
    import torch
    say(f"[i8] large layer M={M} N={N} K={K} bias={bias_on} relu={relu}")
    dev = "cuda:0"
    seed = M + 3 * N + 5 * K
    x = synth.activations(M, K, seed)
    x[M // 3] = 0
    W = synth.normal_weights(N, K, seed + 1)
    rng = np.random.default_rng(seed)
    b = (rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)) if bias_on else None
    q, s = oracle.i8_quant_weights(W)
    ref = oracle.i8_linear(x, q, s, b, relu)
    qd = torch.from_numpy(q).to(dev)
    sd = torch.tensor([s], dtype=torch.float32, device=dev)
    bd = torch.from_numpy(b).to(dev) if b is not None else None
    xd = torch.from_numpy(x).to(dev)
    ybuf = torch.full((M * N + 64,), float("nan"), device=dev)
    y = ybuf[:M * N].view(M, N)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    tb.bitnet_i8_linear_into(M, N, K, xd, qd, sd, bd, relu, y, ws, acc)
    y2, acc2 = _row_slices(tb, xd, qd, sd, bd, relu, tb.bitnet_i8_linear_into, K, N)
    torch.cuda.synchronize()
    assert torch.isnan(ybuf[M * N:]).all().item(), "wrote past the end of y"
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    d = ref["acc"].astype(np.float64) * np.float64(s) / ref["x_scale"].astype(np.float64)[:, None]
    bias_vals = np.zeros(N) if b is None else np.broadcast_to(b.astype(np.float64), (M, N))
    check_y(y.cpu().numpy(), ref["y"], d, bias_vals, f"M={M} N={N} K={K}")
    assert torch.equal(acc, acc2)
    assert torch.equal(y, y2), "the whole call and its row slices differ"


@pytest.mark.parametrize("M,N,K", [(2085, 520, 1024), (2048, 2048, 512)])
def test_i8_linear_rows_large_ragged_parity(tb, M, N, K):
    """Per-channel scales on larger ragged layers, a zero weight channel
    included; against the oracle and against row slices of the same call."""
    import torch
    say(f"[i8 rows] large layer M={M} N={N} K={K}")
    dev = "cuda:0"
    seed = 2 * M + N + K
    x = synth.activations(M, K, seed)
    W = synth.student_t_weights(N, K, seed + 1)
    W[N // 3] = 0
    b = np.random.default_rng(seed).standard_normal(N, dtype=np.float32) * np.float32(0.1)
    q, s = oracle.rowq_quant_weights(W)
    ref = oracle.i8_linear_rows(x, q, s, b, True)
    qd, sd = torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev)
    bd, xd = torch.from_numpy(b).to(dev), torch.from_numpy(x).to(dev)
    y = torch.full((M, N), float("nan"), device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    tb.bitnet_i8_linear_rows_into(M, N, K, xd, qd, sd, bd, True, y, ws, acc)
    y2, acc2 = _row_slices(tb, xd, qd, sd, bd, True, tb.bitnet_i8_linear_rows_into, K, N)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    d = (ref["acc"].astype(np.float64) * s.astype(np.float64)[None, :]
         / ref["x_scale"].astype(np.float64)[:, None])
    check_y_rows(y.cpu().numpy(), ref["y"], d, np.broadcast_to(b.astype(np.float64), (M, N)),
                 f"M={M} N={N} K={K}")
    assert torch.equal(acc, acc2)
    assert torch.equal(y, y2), "the whole call and its row slices differ"
