"""GPU parity at the largest shapes the boundary accepts.

The size rules keep every device offset in 32 bits: M*K, N*K and M*N below
2^31, and (M + 128)*N*4 below 2^31 (the fp32 output addressed with a 128-row
tile past M).  Each test takes one of those bounds to within a few hundred
elements of 2^31 and checks the call against the oracle:
  - M*K: the whole projection (quantization + prefill GEMM) over 1,398,101 rows
    of K = 1536 (8.6 GB of fp32 activations);
  - (M + 128)*N*4: the prefill GEMM at M = 1800 with N = 278,460 columns
    (a 2 GB fp32 output);
  - N*K: ternarize + pack of an 8960-input weight with 239,674 rows (8.6 GB of
    fp32 masters), then the decode GEMV on it at M = 1 (quantization fused)
    and M = 16 (rows staged from the quantization launch).
Inputs are seeded: activations and the large masters come from torch's
generator on the GPU, the small masters from the host generators; the oracle
sees the same arrays.  Outputs are checked on sampled rows and columns (the
first and last of each among them), int8 rows, scales and int32 accumulators
bit for bit, fp32 outputs bit for bit on the decode path and within 1e-6
relative on the prefill path; every output buffer is NaN-filled with a canary
tail, and no NaN may remain.
"""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
CANARY = 4096
LIMIT = 1 << 31


@pytest.fixture(scope="module")
def tb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ternary_weight_decoder_amd import binding
    binding.lib()
    return binding


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def guarded(n, dtype):
    """n elements followed by a canary tail, all NaN (or -1 for integers)."""
    import torch
    fill = float("nan") if dtype.is_floating_point else -1
    buf = torch.full((n + CANARY,), fill, dtype=dtype, device="cuda:0")
    return buf, buf[:n]


def assert_canary(buf, n):
    import torch
    tail = buf[n:]
    ok = torch.isnan(tail).all() if tail.dtype.is_floating_point else (tail == -1).all()
    assert bool(ok), "canary overwritten"


def gpu_normal(shape, seed, scale=1.0):
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device="cuda:0")
    if scale != 1.0:
        t.mul_(scale)
    return t


def samples(size, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, size - 2, size - 1],
                                     rng.integers(0, size, count)])).astype(np.int64)


def pack_both(tb, W_host, W_dev):
    """Ternarize + pack on the GPU and in the oracle; both must agree exactly."""
    import torch
    N, K = W_host.shape
    packed = torch.empty(N * K // 4, dtype=torch.uint8, device="cuda:0")
    w_scale = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(tb.bitnet_ternarize_workspace_bytes(N), dtype=torch.uint8, device="cuda:0")
    tb.bitnet_ternarize_pack_into(W_dev, N, K, packed, w_scale, ws)
    ref_packed, ref_scale = oracle.ternarize_pack(W_host)
    torch.cuda.synchronize()
    assert w_scale.cpu().numpy()[0] == ref_scale, "w_scale differs"
    assert np.array_equal(packed.cpu().numpy(), ref_packed), "packed codes differ"
    return packed, w_scale, ref_packed, ref_scale


def run_and_check(tb, x, packed, w_scale, ref_packed, ref_scale, N, rows, cols, exact_y):
    """One bitnet_ternary_matmul call with every optional output, checked on
    rows x cols against the oracle."""
    import torch
    M, K = x.shape
    y_buf, y = guarded(M * N, torch.float32)
    a_buf, acc = guarded(M * N, torch.int32)
    s_buf, xs = guarded(M, torch.float32)
    xq = torch.full((M * K,), -128, dtype=torch.int8, device="cuda:0")
    ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    tb.bitnet_ternary_matmul_into(M, N, K, x, packed, w_scale, y, ws, xq, xs, acc)
    torch.cuda.synchronize()
    for buf, n in ((y_buf, M * N), (a_buf, M * N), (s_buf, M)):
        assert_canary(buf, n)
    assert not bool(torch.isnan(y).any()), "unwritten output"
    assert not bool((xq == -128).any()), "unwritten int8 row (or -128)"
    del ws
    r = torch.from_numpy(rows).to("cuda:0")
    x_rows = x[r].cpu().numpy()
    ref_xq, ref_xs = oracle.quant_act(x_rows)
    np.testing.assert_array_equal(xq.view(M, K)[r].cpu().numpy(), ref_xq)
    np.testing.assert_array_equal(xs[r].cpu().numpy(), ref_xs)
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    ref_acc, ref_y = oracle.matmul_sampled(ref_xq, ref_xs, ref_packed, ref_scale, N, ms, ns)
    c = torch.from_numpy(cols).to("cuda:0")
    got_acc = acc.view(M, N)[r][:, c].cpu().numpy().reshape(-1)
    got_y = y.view(M, N)[r][:, c].cpu().numpy().reshape(-1)
    np.testing.assert_array_equal(got_acc, ref_acc)
    if exact_y:
        np.testing.assert_array_equal(got_y.view(np.uint32), ref_y.view(np.uint32))
    zero = ref_y == 0
    assert (got_y[zero] == 0).all()
    rel = np.abs(got_y.astype(np.float64) - ref_y) / np.maximum(np.abs(ref_y.astype(np.float64)),
                                                                 1e-300)
    worst = float(rel[~zero].max()) if (~zero).any() else 0.0
    assert worst <= REL_TOL, f"max relative error {worst:.3e}"
    return worst


def test_max_rows_times_k(tb):
    """M*K = 2^31 - 512: 1,398,101 rows of 1536 inputs through the whole
    projection (quantization launch + prefill GEMM), N = 256."""
    import torch
    M, N, K = 1398101, 256, 1536
    say(f"[limits] M*K: M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=91)
    packed, w_scale, ref_packed, ref_scale = pack_both(tb, W, torch.from_numpy(W).to("cuda:0"))
    x = gpu_normal((M, K), seed=92)
    worst = run_and_check(tb, x, packed, w_scale, ref_packed, ref_scale, N,
                          samples(M, 60, 93), samples(N, 30, 94), exact_y=False)
    say(f"[limits] M*K ok, max relative error {worst:.2e}")


def test_max_output_bytes(tb):
    """(M + 128)*N*4 = 2^31 - 128: the prefill GEMM at M = 1800 writing a
    2 GB fp32 output (N = 278,460, a ragged last column tile)."""
    import torch
    M, N, K = 1800, 278460, 128
    say(f"[limits] output bytes: M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=95)
    packed, w_scale, ref_packed, ref_scale = pack_both(tb, W, torch.from_numpy(W).to("cuda:0"))
    x = gpu_normal((M, K), seed=96)
    cols = np.unique(np.concatenate([samples(N, 40, 97), np.arange(N - 300, N)]))
    worst = run_and_check(tb, x, packed, w_scale, ref_packed, ref_scale, N,
                          samples(M, 40, 98), cols, exact_y=False)
    say(f"[limits] output bytes ok, max relative error {worst:.2e}")


def test_max_codes_decode(tb):
    """N*K = 2^31 - 4608: an 8960-input weight with 239,674 rows ternarized
    and packed (8.6 GB of masters, 537 MB of codes), then the decode GEMV at
    M = 1 (quantization fused) and M = 16 (rows staged)."""
    import torch
    N, K = 239674, 8960
    say(f"[limits] N*K: N={N} K={K}: masters on the GPU, a host copy for the oracle")
    W_dev = gpu_normal((N, K), seed=99, scale=0.02)
    W_host = W_dev.cpu().numpy()
    packed, w_scale, ref_packed, ref_scale = pack_both(tb, W_host, W_dev)
    del W_dev, W_host
    torch.cuda.empty_cache()
    for M in (1, 16):
        x = gpu_normal((M, K), seed=100 + M)
        rows = np.arange(M, dtype=np.int64)
        run_and_check(tb, x, packed, w_scale, ref_packed, ref_scale, N, rows,
                      samples(N, 60, 101 + M), exact_y=True)
        say(f"[limits] N*K decode M={M} ok (bit-exact)")


# ---- I8_S layers and the 8-bit table at their own limits ----------------------

I8_TOL = 4.0 * 2.0 ** -24        # per-tensor epilogue: three fp32 roundings and the bias add
I8_TOL_ROWS = 5.0 * 2.0 ** -24   # per-channel epilogue: one rounding more


def check_i8(tb, x, q_dev, s_dev, q_ref, s_ref, b, per_channel, rows, cols):
    """One I8_S linear call (bias, ReLU) checked on rows x cols: accumulators
    bit-exact, outputs within the epilogue's bound, no NaN left, canary kept."""
    import torch
    M, K = x.shape
    N = q_ref.shape[0]
    y_buf, y = guarded(M * N, torch.float32)
    a_buf, acc = guarded(M * N, torch.int32)
    ws = torch.empty(tb.bitnet_i8_linear_workspace_bytes(M, K), dtype=torch.uint8,
                     device="cuda:0")
    call = tb.bitnet_i8_linear_rows_into if per_channel else tb.bitnet_i8_linear_into
    call(M, N, K, x, q_dev, s_dev, torch.from_numpy(b).to("cuda:0"), True, y, ws, acc)
    torch.cuda.synchronize()
    for buf in (y_buf, a_buf):
        assert_canary(buf, M * N)
    assert not bool(torch.isnan(y).any()), "unwritten output"
    del ws
    r = torch.from_numpy(rows).to("cuda:0")
    xq, xs = oracle.quant_act(x[r].cpu().numpy())
    ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
    ns = np.tile(cols, rows.size).astype(np.int64)
    sampled = oracle.i8_linear_rows_sampled if per_channel else oracle.i8_linear_sampled
    acc_ref, d, y_ref = sampled(xq, xs, q_ref, s_ref, b, True, ms, ns)
    c = torch.from_numpy(cols).to("cuda:0")
    np.testing.assert_array_equal(acc.view(M, N)[r][:, c].cpu().numpy().reshape(-1), acc_ref)
    got = y.view(M, N)[r][:, c].cpu().numpy().reshape(-1)
    tol = I8_TOL_ROWS if per_channel else I8_TOL
    bound = tol * (np.abs(d) + np.abs(b[ns].astype(np.float64))) + 1e-37
    worst = float((np.abs(got.astype(np.float64) - y_ref.astype(np.float64)) / bound).max())
    assert worst <= 1.0, f"error {worst:.3f} x the bound"
    assert (got >= 0).all()
    return worst


def test_i8_max_rows_times_k(tb):
    """I8_S layer (one weight scale, bias, ReLU) at M*K = 2^31 - 512:
    1,398,101 rows of 1536 inputs, N = 256."""
    import torch
    M, N, K = 1398101, 256, 1536
    say(f"[limits] I8_S M*K: M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=111)
    b = np.random.default_rng(112).standard_normal(N, dtype=np.float32) * np.float32(0.1)
    q_ref, s_ref = oracle.i8_quant_weights(W)
    q_dev, s_dev = tb.bitnet_i8_quant_weights(torch.from_numpy(W).to("cuda:0"))
    torch.cuda.synchronize()
    assert s_dev.cpu().numpy()[0] == s_ref
    np.testing.assert_array_equal(q_dev.cpu().numpy(), q_ref)
    x = gpu_normal((M, K), seed=113)
    worst = check_i8(tb, x, q_dev, s_dev, q_ref, s_ref, b, False, samples(M, 60, 114),
                     samples(N, 30, 115))
    say(f"[limits] I8_S M*K ok, worst {worst:.3f} of the bound")


def test_i8_rows_max_output_bytes(tb):
    """I8_S layer with one weight scale per output channel at
    (M + 128)*N*4 = 2^31 - 128: M = 1800, N = 278,460, K = 128."""
    import torch
    M, N, K = 1800, 278460, 128
    say(f"[limits] I8_S per-channel output bytes: M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=116)
    b = np.random.default_rng(117).standard_normal(N, dtype=np.float32) * np.float32(0.1)
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    q_dev, s_dev = tb.bitnet_i8_quant_weights_rows(torch.from_numpy(W).to("cuda:0"))
    torch.cuda.synchronize()
    assert s_dev.cpu().numpy().tobytes() == s_ref.tobytes()
    np.testing.assert_array_equal(q_dev.cpu().numpy(), q_ref)
    x = gpu_normal((M, K), seed=118)
    cols = np.unique(np.concatenate([samples(N, 40, 119), np.arange(N - 300, N)]))
    worst = check_i8(tb, x, q_dev, s_dev, q_ref, s_ref, b, True, samples(M, 40, 120), cols)
    say(f"[limits] I8_S per-channel output bytes ok, worst {worst:.3f} of the bound")


def test_table_max_bytes(tb):
    """The 8-bit table at its largest: V = 1,398,096 rows of 1536 inputs
    (2^31 - 12,288 bytes of codes from 8.6 GB of masters), codes and scales
    bit-exact, the lm_head at M = 1 and 16 on sampled columns and the
    embedding of the first and last rows, bit-exact."""
    import torch
    V, K = 1398096, 1536
    assert oracle.table_bytes(V, K) < LIMIT <= oracle.table_bytes(V + 1, K)
    say(f"[limits] table V={V} K={K}: masters on the GPU, a host copy for the oracle")
    W_dev = gpu_normal((V, K), seed=121, scale=0.02)
    table = torch.empty(tb.bitnet_table_bytes(V, K), dtype=torch.int8, device="cuda:0")
    s_dev = torch.full((V,), float("nan"), dtype=torch.float32, device="cuda:0")
    tb.bitnet_table_quant_into(W_dev, V, K, table, s_dev)
    W_host = W_dev.cpu().numpy()
    del W_dev
    q_ref, s_ref = oracle.rowq_quant_weights(W_host)
    del W_host
    torch.cuda.synchronize()
    assert s_dev.cpu().numpy().tobytes() == s_ref.tobytes()
    assert np.array_equal(table.cpu().numpy(), oracle.table_pack(q_ref))
    torch.cuda.empty_cache()
    for M in (1, 16):
        x = gpu_normal((M, K), seed=122 + M)
        y_buf, y = guarded(M * V, torch.float32)
        a_buf, acc = guarded(M * V, torch.int32)
        tb.bitnet_lm_head_into(M, V, K, x, table, s_dev, y, acc_out=acc)
        torch.cuda.synchronize()
        for buf in (y_buf, a_buf):
            assert_canary(buf, M * V)
        assert not bool(torch.isnan(y).any()), "unwritten output"
        xq, xs = oracle.quant_act(x.cpu().numpy())
        cols = np.unique(np.concatenate([samples(V, 200, 124 + M), np.arange(V - 40, V)]))
        ms = np.repeat(np.arange(M), cols.size).astype(np.int64)
        ns = np.tile(cols, M).astype(np.int64)
        acc_s, y_s = oracle.rowq_linear_sampled(xq, xs, q_ref, s_ref, ms, ns)
        c = torch.from_numpy(cols).to("cuda:0")
        np.testing.assert_array_equal(acc.view(M, V)[:, c].cpu().numpy().reshape(-1), acc_s)
        assert y.view(M, V)[:, c].cpu().numpy().reshape(-1).tobytes() == y_s.tobytes()
        say(f"[limits] table lm_head M={M} ok (bit-exact)")
    ids = np.array([0, 1, V - 2, V - 1, 700001], dtype=np.int32)
    out = tb.bitnet_embed_lookup(torch.from_numpy(ids).to("cuda:0"), table, s_dev, K)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == oracle.rowq_embed(ids, q_ref, s_ref).tobytes()
    say("[limits] table embedding ok (bit-exact)")


def test_dwconv_max_elements(tb):
    """The depthwise convolution at B*T*C = 2^29 - 1024 (the fp32 input and
    output just under 2 GB each): 2 sequences of 524,287 frames x 512
    channels, 7 taps, bias and ReLU; every output, accumulator and scale
    bit-exact against the oracle."""
    import torch
    B, T, C, k = 2, 524287, 512, 7
    assert B * T * C < LIMIT // 4 <= B * (T + 1) * C
    say(f"[limits] depthwise conv B={B} T={T} C={C} k={k}")
    x = gpu_normal((B, T, C), seed=131)
    W = np.random.default_rng(132).standard_normal((C, k), dtype=np.float32) * np.float32(0.1)
    b = np.random.default_rng(133).standard_normal(C, dtype=np.float32) * np.float32(0.1)
    q, s = tb.bitnet_i8_dwconv_quant_weights(torch.from_numpy(W).to("cuda:0"))
    y_buf, y = guarded(B * T * C, torch.float32)
    a_buf, acc = guarded(B * T * C, torch.int32)
    xs = torch.full((B, C), float("nan"), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(tb.bitnet_i8_dwconv_workspace_bytes(B, T, C), dtype=torch.uint8,
                     device="cuda:0")
    tb.bitnet_i8_dwconv_into(B, T, C, k, x, q, s, torch.from_numpy(b).to("cuda:0"), True, y, ws,
                             acc, xs)
    torch.cuda.synchronize()
    for buf in (y_buf, a_buf):
        assert_canary(buf, B * T * C)
    del ws
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    assert s.cpu().numpy().tobytes() == s_ref.tobytes()
    ref = oracle.i8_dwconv(x.cpu().numpy(), q_ref, s_ref, b, True)
    assert xs.cpu().numpy().tobytes() == ref["x_scale"].tobytes()
    assert np.array_equal(acc.cpu().numpy(), ref["acc"].reshape(-1))
    assert y.cpu().numpy().tobytes() == ref["y"].tobytes()
    say("[limits] depthwise conv ok (bit-exact)")


@pytest.mark.parametrize("M", [1, 4, 16, 200])
def test_grouped_max_count(tb, M):
    """The grouped call at its largest problem count (256 ragged projections,
    a third of them sharing inputs), every output against the oracle; at
    prefill sizes also the overlapped call at its largest chunk count (32),
    bit for bit against the grouped call."""
    import torch
    count = tb.BITNET_MAX_GROUP
    say(f"[limits] grouped call, {count} projections, M={M}")
    rng = np.random.default_rng(140 + M)
    shapes = [(int(rng.choice([16, 72, 200, 520, 1000])), int(rng.choice([128, 256, 640, 1536])))
              for _ in range(count)]
    Ws = [synth.normal_weights(N, K, seed=150000 + i) for i, (N, K) in enumerate(shapes)]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    xs_host, dx, xd = [], [], {}
    for i, (N, K) in enumerate(shapes):
        key = (i // 3, K) if i % 2 == 0 else (i, K)   # some neighbours share an input buffer
        if key not in xd:
            x = synth.activations(M, K, seed=160000 + i)
            xd[key] = (x, torch.from_numpy(x).to("cuda:0"))
        xs_host.append(xd[key][0])
        dx.append(xd[key][1])
    dp = [torch.from_numpy(p).to("cuda:0") for p, _ in packs]
    ds = [torch.tensor([s], dtype=torch.float32, device="cuda:0") for _, s in packs]
    Ns, Ks = [N for N, _ in shapes], [K for _, K in shapes]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N in Ns]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, Ns, Ks)
    plan.run()
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(shapes):
        ref = oracle.ternary_matmul(xs_host[i], packs[i][0], packs[i][1], N)["y"]
        y = ys[i].cpu().numpy()
        assert not np.isnan(y).any(), f"problem {i}: unwritten output"
        if M <= 16:
            np.testing.assert_array_equal(y.view(np.uint32), ref.view(np.uint32))
        else:
            zero = ref == 0
            assert (y[zero] == 0).all()
            rel = np.abs(y.astype(np.float64) - ref) / np.maximum(np.abs(ref.astype(np.float64)),
                                                                  1e-300)
            assert float(rel[~zero].max(initial=0.0)) <= REL_TOL, f"problem {i}"
    if M > 16:
        ys2 = [torch.full((M, N), float("nan"), device="cuda:0") for N in Ns]
        plan2 = tb.GroupedPlan(M, dx, dp, ds, ys2, Ns, Ks)
        aux = torch.cuda.Stream()
        plan2.run_overlap(aux, 32)
        torch.cuda.synchronize()
        for a, b in zip(ys2, ys):
            assert torch.equal(a, b)
    say(f"[limits] grouped call, {count} projections, M={M} ok")
