"""GPU parity: the HIP path against the CPU oracle, element by element.

Inputs come from the seeded generators; the oracle and the HIP library each
compute from them independently.  Packed bytes, scales, int8 activations and
int32 accumulators must be bit-exact; fp32 outputs must be within 1e-6
relative (exactly 0 where the accumulator is 0).  Outputs are pre-filled with a
NaN sentinel and guarded by a canary tail so that unwritten or overrun elements
show up.
"""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_decoder_amd import synth
from conftest import read_golden, ternarize_rounding_cases

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
CANARY = 4096


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


def dev_tensor(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def guarded(n, dtype, fill):
    """A device buffer of n elements + a canary tail, all set to `fill`."""
    import torch
    t = torch.full((n + CANARY,), fill, dtype=dtype, device="cuda:0")
    return t, t[:n]


def check_canary(buf, n, fill):
    tail = buf[n:].cpu().numpy()
    if np.isnan(fill):
        assert np.isnan(tail).all(), "canary overwritten"
    else:
        assert (tail == fill).all(), "canary overwritten"


def assert_y_close(y, ref):
    assert not np.isnan(y).any(), "unwritten output (NaN sentinel survived)"
    zero = ref == 0
    assert (y[zero] == 0).all()
    rel = np.abs(y.astype(np.float64) - ref.astype(np.float64)) / np.maximum(
        np.abs(ref.astype(np.float64)), 1e-300)
    worst = float(rel[~zero].max()) if (~zero).any() else 0.0
    assert worst <= REL_TOL, f"max relative error {worst:.3e}"


def assert_y_matches(y, ref, M):
    """Decode calls (M <= 16) reproduce the exactly rounded value bit for bit;
    prefill calls are held to the relative tolerance."""
    if M <= 16:
        assert not np.isnan(y).any(), "unwritten output (NaN sentinel survived)"
        np.testing.assert_array_equal(y.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    else:
        assert_y_close(y, ref)


def gpu_ternarize_pack(tb, W):
    import torch
    N, K = W.shape
    packed_buf, packed = guarded(N * K // 4, torch.uint8, 0xAB)
    ws = torch.empty(tb.bitnet_ternarize_workspace_bytes(N), dtype=torch.uint8, device="cuda:0")
    w_scale = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda:0")
    tb.bitnet_ternarize_pack_into(dev_tensor(W), N, K, packed, w_scale, ws)
    torch.cuda.synchronize()
    check_canary(packed_buf, N * K // 4, 0xAB)
    return packed.cpu().numpy(), np.float32(w_scale.cpu().numpy()[0])


def gpu_matmul(tb, x, packed, w_scale, N, K):
    import torch
    M = x.shape[0]
    ybuf, y = guarded(M * N, torch.float32, float("nan"))
    accbuf, acc = guarded(M * N, torch.int32, -12345)
    xqbuf, xq = guarded(M * K, torch.int8, 99)
    xsbuf, xs = guarded(M, torch.float32, float("nan"))
    ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    ws_scale = torch.full((1,), float(w_scale), dtype=torch.float32, device="cuda:0")
    tb.bitnet_ternary_matmul_into(M, N, K, dev_tensor(x), dev_tensor(packed), ws_scale, y, ws,
                                  xq, xs, acc)
    torch.cuda.synchronize()
    check_canary(ybuf, M * N, float("nan"))
    check_canary(accbuf, M * N, -12345)
    check_canary(xqbuf, M * K, 99)
    check_canary(xsbuf, M, float("nan"))
    return {"y": y.cpu().numpy().reshape(M, N), "acc": acc.cpu().numpy().reshape(M, N),
            "xq": xq.cpu().numpy().reshape(M, K), "x_scale": xs.cpu().numpy()}


# ---------------------------------------------------------------------------
# Ternarization + packing
# ---------------------------------------------------------------------------

TERN_CASES = {
    "q_1536x1536": lambda: synth.normal_weights(1536, 1536, 0),
    "kv_256x1536": lambda: synth.normal_weights(256, 1536, 1002),
    "gate_8960x1536": lambda: synth.normal_weights(8960, 1536, 1004),
    "down_1536x8960": lambda: synth.normal_weights(1536, 8960, 1006),
    "t3_8960x1536": lambda: synth.student_t_weights(8960, 1536, 50004),
    "ragged_37x384": lambda: synth.normal_weights(37, 384, 5),
    "tiny_1x128": lambda: synth.normal_weights(1, 128, 6),
    "zero_16x256": lambda: np.zeros((16, 256), np.float32),
}


@pytest.mark.parametrize("case", sorted(TERN_CASES))
def test_ternarize_pack_parity(tb, case):
    say(f"[ternarize_pack] {case}")
    W = TERN_CASES[case]()
    N, K = W.shape
    packed_ref, s_ref = oracle.ternarize_pack(W)
    packed, s = gpu_ternarize_pack(tb, W)
    assert s.tobytes() == s_ref.tobytes()
    np.testing.assert_array_equal(packed, packed_ref)
    _, bad = oracle.unpack(packed, N, K)
    assert bad == 0


def test_ternarize_golden_ties(tb):
    say("[ternarize_pack] golden ties")
    rows = read_golden("ternarize_ties.txt")
    # Example A: row 0 |W| = 1.0, rows 1-2 |W| = 0.25 -> m = 0.5, codes sign / 0 / 0.
    N, K = 3, 128
    A = np.array([[1.0] * K, [0.25] * K, [0.25] * K], np.float32)
    sign = np.where((np.add.outer(np.arange(N), np.arange(K)) % 3) == 0, -1, 1)
    W = (A * sign).astype(np.float32)
    packed, s = gpu_ternarize_pack(tb, W)
    assert s == np.float32(0.5)
    q, _ = oracle.unpack(packed, N, K)
    np.testing.assert_array_equal(q, np.stack([sign[0], 0 * sign[1], 0 * sign[2]]).astype(np.int8))
    assert any(r[0] == "example" for r in rows)


@pytest.mark.parametrize("ex", ternarize_rounding_cases(), ids=lambda e: e["name"])
def test_ternarize_golden_rounding_readings(tb, ex):
    # the hand-worked cases that fix the mean's single rounding and the IEEE
    # quotient W/m: the kernel must give the golden scale and codes
    say(f"[ternarize_pack] golden rounding {ex['name']}")
    N, K = ex["W"].shape
    packed, s = gpu_ternarize_pack(tb, ex["W"])
    assert float(s) == ex["scale"], (float(s).hex(), float(ex["scale"]).hex())
    q, bad = oracle.unpack(packed, N, K)
    assert bad == 0
    np.testing.assert_array_equal(q, ex["codes"])


# ---------------------------------------------------------------------------
# Activation quantization
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 1536), (4, 1536), (16, 8960), (17, 128), (256, 1536),
                                 (1800, 1536), (3, 8960), (5, 2048), (6, 2176), (2, 10240),
                                 (3, 10368), (2, 24576)])
def test_quant_act_parity(tb, M, K):
    import torch
    say(f"[quant_act] M={M} K={K}")
    x = synth.activations(M, K, seed=M * 7 + K)
    if M == 3:
        x[1] = 0.0
    xq_ref, xs_ref = oracle.quant_act(x)
    xqbuf, xq = guarded(M * K, torch.int8, 99)
    xsbuf, xs = guarded(M, torch.float32, float("nan"))
    tb.bitnet_quant_act_into(dev_tensor(x), M, K, xq, xs)
    torch.cuda.synchronize()
    check_canary(xqbuf, M * K, 99)
    check_canary(xsbuf, M, float("nan"))
    np.testing.assert_array_equal(xq.cpu().numpy().reshape(M, K), xq_ref)
    assert xs.cpu().numpy().tobytes() == xs_ref.tobytes()


def test_quant_act_golden(tb):
    import torch
    say("[quant_act] golden rows")
    rows = read_golden("quant_act_worked.txt")
    cur = {}
    cases = []
    for r in rows:
        if r[0] == "row":
            cur = {}
            cases.append(cur)
        elif r[0] == "scale":
            cur["scale"] = float(r[1])
        elif r[0] == "x":
            cur["x"] = [float(v) for v in r[1:]]
        elif r[0] == "xq":
            cur["xq"] = [int(v) for v in r[1:]]
    for c in cases:
        x = np.zeros((1, 128), np.float32)
        x[0, :len(c["x"])] = c["x"]
        xq, xs = tb.bitnet_quant_act(dev_tensor(x))
        torch.cuda.synchronize()
        assert xs.cpu().numpy()[0] == np.float32(c["scale"])
        np.testing.assert_array_equal(xq.cpu().numpy()[0, :len(c["xq"])], c["xq"])


# ---------------------------------------------------------------------------
# Projection: decode GEMV (M <= 16) and prefill GEMM (M > 16)
# ---------------------------------------------------------------------------

MATMUL_CASES = [(m, 200, 384) for m in range(1, 21)] + [
    (1, 1536, 1536), (1, 256, 1536), (1, 8960, 1536), (1, 1536, 8960), (4, 1536, 8960),
    (16, 1536, 8960), (16, 65, 128), (32, 300, 512), (64, 8960, 1536), (256, 1536, 1536),
    (257, 520, 256), (1800, 300, 1536), (129, 257, 1280), (20, 136, 10368), (40, 72, 2176),
    # 128-row tiles whose last row block holds 1..4 blocks of 32 rows
    (90, 300, 384), (200, 520, 640), (161, 264, 512), (236, 72, 1152),
    # decode rows staged through LDS in chunks of 4 units: partial chunks, ragged N
    (5, 200, 2048), (3, 72, 8960), (16, 300, 1280), (2, 520, 4608), (13, 1000, 768),
    # single-row launches with K split 2 or 4 ways across the waves of a workgroup
    (1, 300, 2048), (1, 130, 3072), (1, 72, 8960), (1, 1000, 4224),
]


@pytest.mark.parametrize("M,N,K", MATMUL_CASES)
def test_matmul_parity(tb, M, N, K):
    say(f"[matmul] M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=N + K)
    x = synth.activations(M, K, seed=1000 + M)
    packed, s = oracle.ternarize_pack(W)
    ref = oracle.ternary_matmul(x, packed, s, N)
    got = gpu_matmul(tb, x, packed, s, N, K)
    np.testing.assert_array_equal(got["xq"], ref["xq"])
    assert got["x_scale"].tobytes() == ref["x_scale"].tobytes()
    np.testing.assert_array_equal(got["acc"], ref["acc"])
    assert_y_matches(got["y"], ref["y"], M)


@pytest.mark.parametrize("M,N,K", [(300, 512, 256), (40, 768, 384), (20, 256, 1536),
                                   (129, 520, 256), (5, 300, 2048), (1, 1536, 8960)])
def test_matmul_y_only_parity(tb, M, N, K):
    """Without the optional outputs (the form the grouped and benchmark calls
    take): full 256-column prefill tiles use the transposed 16-byte stores."""
    import torch
    say(f"[matmul y only] M={M} N={N} K={K}")
    W = synth.normal_weights(N, K, seed=3 * N + K)
    x = synth.activations(M, K, seed=500 + M)
    packed, s = oracle.ternarize_pack(W)
    ref = oracle.ternary_matmul(x, packed, s, N)
    ybuf, y = guarded(M * N, torch.float32, float("nan"))
    ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    w_scale = torch.full((1,), float(s), dtype=torch.float32, device="cuda:0")
    tb.bitnet_ternary_matmul_into(M, N, K, dev_tensor(x), dev_tensor(packed), w_scale, y, ws)
    torch.cuda.synchronize()
    check_canary(ybuf, M * N, float("nan"))
    assert_y_matches(y.cpu().numpy().reshape(M, N), ref["y"], M)


@pytest.mark.parametrize("M", [1, 17])
def test_matmul_worst_case_magnitude(tb, M):
    say(f"[matmul] worst-case magnitude M={M}")
    K, N = 8960, 64
    x = np.ones((M, K), np.float32)            # absmax 1 -> xq = 127 everywhere
    W = np.full((N, K), 0.5, np.float32)
    W[1::2] = -0.5                              # codes +1 on even rows, -1 on odd rows
    packed, s = oracle.ternarize_pack(W)
    got = gpu_matmul(tb, x, packed, s, N, K)
    want = np.where(np.arange(N) % 2 == 0, 127 * K, -127 * K)
    np.testing.assert_array_equal(got["acc"], np.tile(want, (M, 1)))
    assert_y_matches(got["y"], oracle.ternary_matmul(x, packed, s, N)["y"], M)


@pytest.mark.parametrize("M", [5, 64])
def test_matmul_q8_parity(tb, M):
    import torch
    say(f"[matmul_q8] M={M}")
    N, K = 300, 1536
    W = synth.normal_weights(N, K, seed=77)
    x = synth.activations(M, K, seed=78)
    packed, s = oracle.ternarize_pack(W)
    ref = oracle.ternary_matmul(x, packed, s, N)
    y, acc = tb.bitnet_ternary_matmul_q8(dev_tensor(ref["xq"]), dev_tensor(ref["x_scale"]),
                                         dev_tensor(packed), dev_tensor(np.array([s])), N,
                                         return_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
    assert_y_matches(y.cpu().numpy(), ref["y"], M)


def test_zero_activation_row_and_zero_weights(tb):
    say("[matmul] zero row / zero tensor")
    M, N, K = 3, 64, 256
    x = synth.activations(M, K, seed=3)
    x[1] = 0.0
    W = synth.normal_weights(N, K, seed=4)
    packed, s = oracle.ternarize_pack(W)
    got = gpu_matmul(tb, x, packed, s, N, K)
    assert got["x_scale"][1] == 1.0 and not got["acc"][1].any() and not got["y"][1].any()
    Wz = np.zeros((N, K), np.float32)
    pz, sz = oracle.ternarize_pack(Wz)
    got = gpu_matmul(tb, x, pz, sz, N, K)
    assert not got["acc"].any() and not got["y"].any()


def test_deterministic_and_input_sensitive(tb):
    say("[matmul] determinism / smell test")
    M, N, K = 4, 1536, 1536
    x = synth.activations(M, K, seed=9)
    p1, s1 = oracle.ternarize_pack(synth.normal_weights(N, K, 10))
    p2, s2 = oracle.ternarize_pack(synth.normal_weights(N, K, 11))
    a = gpu_matmul(tb, x, p1, s1, N, K)
    b = gpu_matmul(tb, x, p1, s1, N, K)
    c = gpu_matmul(tb, x, p2, s2, N, K)
    assert a["y"].tobytes() == b["y"].tobytes()
    assert (a["y"] != c["y"]).mean() > 0.99


def test_misaligned_input_is_rejected_and_nothing_written(tb):
    import torch
    say("[matmul] misaligned pointer")
    M, N, K = 1, 64, 128
    flat = torch.zeros(M * K + 4, dtype=torch.float32, device="cuda:0")
    x = flat[1:1 + M * K].view(M, K)
    packed = torch.zeros(N * K // 4, dtype=torch.uint8, device="cuda:0")
    w = torch.ones(1, dtype=torch.float32, device="cuda:0")
    y = torch.full((M, N), float("nan"), device="cuda:0")
    ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(tb.BitnetError) as ei:
        tb.bitnet_ternary_matmul_into(M, N, K, x, packed, w, y, ws)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert torch.isnan(y).all()


# ---------------------------------------------------------------------------
# Grouped launches: one decoder layer, and the 196-matrix sweep
# ---------------------------------------------------------------------------

def _layer_inputs(M, problems):
    Ws = [synth.problem_weights(p) for p in problems]
    xs = [synth.problem_activations(p, M) for p in problems]
    return Ws, xs


@pytest.mark.parametrize("M", [1, 4, 16, 256])
def test_grouped_layer_parity(tb, M):
    import torch
    say(f"[grouped] one layer M={M}")
    problems = synth.layer_problems()
    Ws, xs = _layer_inputs(M, problems)
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dx = [dev_tensor(x) for x in xs]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, p.N), float("nan"), device="cuda:0") for p in problems]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, [p.N for p in problems], [p.K for p in problems])
    plan.run()
    torch.cuda.synchronize()
    for i, p in enumerate(problems):
        ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], p.N)
        assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)


@pytest.mark.parametrize("M", [1, 3, 16, 40, 64, 65, 200])
def test_grouped_many_ragged_parity(tb, M):
    """64 independent projections of mixed ragged shapes in one grouped call,
    every output checked against the oracle.  With these sizes the host deals
    whole projections to the XCDs in every regime: M = 1 (fused quantization,
    K split across waves), M = 3 (fused, several rows), M = 16 (rows staged
    through LDS), M = 40 and 64 (the prefill GEMM, 64-row tiles, plain row
    loads in the quantization launch), M = 65 (128-row tiles with the loads
    spread over each unit, a last row block of one 32-row block, non-temporal
    row loads) and M = 200 (the last row block three 32-row blocks deep)."""
    import torch
    say(f"[grouped] 64 ragged projections M={M}")
    rng = np.random.default_rng(900)
    shapes = [(int(rng.choice([72, 200, 520, 1000, 1536, 2600])),
               int(rng.choice([128, 384, 1536, 2176]))) for _ in range(64)]
    Ws = [synth.normal_weights(N, K, seed=3000 + i) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activations(M, K, seed=4000 + i) for i, (N, K) in enumerate(shapes)]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dx = [dev_tensor(x) for x in xs]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N, _ in shapes]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, [N for N, _ in shapes], [K for _, K in shapes])
    plan.run()
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(shapes):
        ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], N)
        assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)


@pytest.mark.parametrize("M", [1, 3, 5])
def test_grouped_large_ragged_parity(tb, M):
    """160 ragged projections in one grouped decode call, a launch big enough
    to fill the chip (over 1000 tiles): at M = 1 and 3 every workgroup
    quantizes its rows itself, at M = 5 (5 x 2176 > 8960) the rows are staged
    from the quantization launch.  Two calls in a row; every output against
    the oracle, bit for bit."""
    import torch
    say(f"[grouped] 160 ragged projections, M={M}")
    rng = np.random.default_rng(960 + M)
    shapes = [(int(rng.choice([72, 300, 1000, 1536, 2600, 4200])),
               int(rng.choice([128, 384, 1536, 2176]))) for _ in range(160)]
    Ws = [synth.normal_weights(N, K, seed=11000 + i) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activations(M, K, seed=12000 + i) for i, (N, K) in enumerate(shapes)]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dx = [dev_tensor(x) for x in xs]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N, _ in shapes]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, [N for N, _ in shapes], [K for _, K in shapes])
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(shapes):
        ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], N)
        assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)


@pytest.mark.parametrize("M", [2, 3, 4])
def test_grouped_staged_decode_parity(tb, M):
    """Decode calls of 2 to 4 rows whose longest projection puts M * K above
    the in-workgroup quantization limit, so every projection's rows come from
    the quantization launch and are staged through LDS: 96 ragged projections
    with K from 128 (rows shorter than one staged chunk) to 8960, two of them
    sharing an input; two calls in a row; every output against the oracle,
    bit for bit."""
    import torch
    say(f"[grouped] staged decode, 96 ragged projections, M={M}")
    rng = np.random.default_rng(970 + M)
    shapes = [(int(rng.choice([72, 200, 1000, 1536, 2600])),
               int(rng.choice([128, 384, 1536, 1664, 4608, 8960]))) for _ in range(96)]
    shapes[0] = (1536, 8960)   # M * K above the in-workgroup limit at every M here
    shapes[1] = (520, 1536)
    shapes[2] = (200, 1536)    # shares problem 1's input
    Ws = [synth.normal_weights(N, K, seed=13000 + i) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activations(M, K, seed=14000 + i) for i, (N, K) in enumerate(shapes)]
    xs[2] = xs[1]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dx = [dev_tensor(x) for x in xs]
    dx[2] = dx[1]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N, _ in shapes]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, [N for N, _ in shapes], [K for _, K in shapes])
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(shapes):
        ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], N)
        assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)


@pytest.mark.parametrize("M", [32, 64, 200])
def test_grouped_skewed_parity(tb, M):
    """A grouped GEMM launch of two long-K projections (K = 8960, sharing one
    input) among six short ones, as batched decode mixes down with gate and up:
    32-, 64- and 128-row tiles (M = 200 leaves a ragged last row block), two
    calls in a row, every output against the oracle."""
    import torch
    say(f"[grouped] skewed launch M={M}")
    shapes = [(512, 8960), (520, 8960)] + [(1024, 1536), (1000, 1536), (256, 1536),
                                           (2048, 1536), (768, 384), (200, 1536)]
    Ws = [synth.normal_weights(N, K, seed=15000 + i) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activations(M, K, seed=16000 + i) for i, (N, K) in enumerate(shapes)]
    xs[1] = xs[0]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dx = [dev_tensor(x) for x in xs]
    dx[1] = dx[0]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N, _ in shapes]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, [N for N, _ in shapes], [K for _, K in shapes])
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    for i, (N, K) in enumerate(shapes):
        ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], N)
        assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)


@pytest.mark.parametrize("M,nchunks", [(40, 2), (300, 5), (1800, 7)])
def test_grouped_overlap_matches_grouped(tb, M, nchunks):
    """The prefill grouped call with its quantization on a second stream gives
    the plain grouped call's outputs, bit for bit, twice in a row over the same
    workspace (the second call's quantization must wait for the first call's
    contraction).  Problems share inputs across chunk boundaries."""
    import torch
    say(f"[grouped overlap] M={M} chunks={nchunks}")
    rng = np.random.default_rng(930 + M)
    shapes = [(int(rng.choice([72, 520, 1536, 2600])), int(rng.choice([128, 1536, 2176])))
              for _ in range(24)]
    Ws = [synth.normal_weights(N, K, seed=7000 + i) for i, (N, K) in enumerate(shapes)]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    xd = {}
    dx = []
    for i, (N, K) in enumerate(shapes):
        key = (i // 3, K)        # neighbours with the same K read one input buffer
        if key not in xd:
            xd[key] = dev_tensor(synth.activations(M, K, seed=8000 + i))
        dx.append(xd[key])
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    Ns, Ks = [N for N, _ in shapes], [K for _, K in shapes]
    ys_ref = [torch.full((M, N), float("nan"), device="cuda:0") for N in Ns]
    tb.GroupedPlan(M, dx, dp, ds, ys_ref, Ns, Ks).run()
    torch.cuda.synchronize()
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N in Ns]
    plan = tb.GroupedPlan(M, dx, dp, ds, ys, Ns, Ks)
    aux = torch.cuda.Stream()
    for _ in range(2):
        for y in ys:
            y.fill_(float("nan"))
        plan.run_overlap(aux, nchunks)
        plan.run_overlap(aux, nchunks)
        torch.cuda.synchronize()
        for a, b in zip(ys, ys_ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("M", [1, 4, 16, 40, 200])
def test_grouped_shared_inputs_parity(tb, M):
    """One layer called the way a decoder calls it: q, k and v read one input
    buffer, gate and up another, and an extra problem reads the q input's buffer
    with K = 128 (other rows, so a quantized copy of its own).  Each shared input
    is quantized once; every output is checked against the oracle."""
    import torch
    say(f"[grouped] shared inputs M={M}")
    x_attn = synth.activations(M, 1536, seed=5100)
    x_o = synth.activations(M, 1536, seed=5101)
    x_mlp = synth.activations(M, 1536, seed=5102)
    x_down = synth.activations(M, 8960, seed=5103)
    d_attn, d_o, d_mlp, d_down = (dev_tensor(x) for x in (x_attn, x_o, x_mlp, x_down))
    reads = [(x_attn, d_attn), (x_attn, d_attn), (x_attn, d_attn), (x_o, d_o), (x_mlp, d_mlp),
             (x_mlp, d_mlp), (x_down, d_down)]
    shapes = [(N, K) for _, K, N in synth.PROJECTIONS]
    xs = [h for h, _ in reads]
    dxs = [d for _, d in reads]
    shapes.append((200, 128))
    xs.append(np.ascontiguousarray(x_attn.reshape(-1)[:M * 128].reshape(M, 128)))
    dxs.append(d_attn)
    Ws = [synth.normal_weights(N, K, seed=5200 + i) for i, (N, K) in enumerate(shapes)]
    packs = [oracle.ternarize_pack(W) for W in Ws]
    dp = [dev_tensor(p) for p, _ in packs]
    ds = [dev_tensor(np.array([s], np.float32)) for _, s in packs]
    ys = [torch.full((M, N), float("nan"), device="cuda:0") for N, _ in shapes]
    plan = tb.GroupedPlan(M, dxs, dp, ds, ys, [N for N, _ in shapes], [K for _, K in shapes])
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
        for i, (N, K) in enumerate(shapes):
            ref = oracle.ternary_matmul(xs[i], packs[i][0], packs[i][1], N)
            assert_y_matches(ys[i].cpu().numpy(), ref["y"], M)
        for y in ys:
            y.fill_(float("nan"))
