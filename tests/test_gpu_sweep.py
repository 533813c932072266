"""GPU parity at full size: all 196 projections of the 28-layer decoder, in the
grouped launches the benchmark times, checked on sampled outputs.

Two weight sets, each drawn once (seeded, on the host): the decode sweep's
0.02 N(0,1) masters (also prefill at M=256), and the long-form set of
Student-t(3) masters scaled to std 0.01 (prefill at M=1800, batched decode at
M=32 and 64).  Every matrix is ternarized and packed twice, by the oracle and
by the library, and the two packings must be bit-identical with identical
scales.  Activations are drawn on the host from each workload's own seeds.
The expected outputs use only the oracle's packing and the oracle's
quantization of the sampled rows.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
ROWS_PER_MATRIX = 4
COLS_PER_MATRIX = 24


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ternarized_set(problems, heavy_tail, what):
    import torch
    from ternary_weight_decoder_amd import binding as tb
    tb.lib()
    say(f"[{what}] ternarizing {len(problems)} matrices on the host and on the GPU")
    ws = torch.empty(tb.bitnet_ternarize_workspace_bytes(synth.INTERMEDIATE), dtype=torch.uint8,
                     device="cuda:0")
    workers = max(1, min(16, os.cpu_count() or 1))
    packs, packed_dev, scales_dev = [], [], []
    for p, W in zip(problems, synth.problem_weights_iter(problems, heavy_tail, workers)):
        ref_packed, ref_scale = oracle.ternarize_pack(W)
        pk = torch.empty(p.N * p.K // 4, dtype=torch.uint8, device="cuda:0")
        sc = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda:0")
        tb.bitnet_ternarize_pack_into(torch.from_numpy(W).to("cuda:0"), p.N, p.K, pk, sc, ws)
        torch.cuda.synchronize()
        assert sc.cpu().numpy()[0] == ref_scale, p.name
        assert np.array_equal(pk.cpu().numpy(), ref_packed), p.name
        packs.append((ref_packed, ref_scale))
        packed_dev.append(pk)
        scales_dev.append(sc)
    return {"tb": tb, "problems": problems, "packs": packs, "packed": packed_dev,
            "scales": scales_dev}


@pytest.fixture(scope="module")
def sweep():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _ternarized_set(synth.sweep_problems(), False, "sweep")


@pytest.fixture(scope="module")
def longform():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _ternarized_set(synth.longform_problems(), True, "long-form")


def gpu_activations(M, K, seed):
    """N(0,1) rows with 1% of the channels x20, drawn on the GPU (seeded)."""
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device="cuda:0")
    cols = torch.randperm(K, generator=g, device="cuda:0")[:max(1, K // 100)]
    x[:, cols] *= 20.0
    return x


def run_and_check(sweep, M, subset, host_x, lut=False, x_problems=None):
    """x_problems: problems whose activation seeds to use (same order as the
    set's), default the set's own."""
    import torch
    tb = sweep["tb"]
    idx = [i for i, p in enumerate(sweep["problems"]) if subset(p)]
    probs = [sweep["problems"][i] for i in idx]
    if host_x:
        xp = [(x_problems or sweep["problems"])[i] for i in idx]
        workers = max(1, min(16, os.cpu_count() or 1))
        xs = [torch.from_numpy(x).to("cuda:0")
              for x in synth.problem_activations_iter(xp, M, workers)]
    else:
        xs = [gpu_activations(M, p.K, 70000 + 7 * p.layer + p.proj) for p in probs]
    ys = [torch.full((M, p.N), float("nan"), device="cuda:0") for p in probs]
    args = (xs, [sweep["packed"][i] for i in idx], [sweep["scales"][i] for i in idx], ys,
            [p.N for p in probs], [p.K for p in probs])
    plan = tb.LutPlan(*args) if lut else tb.GroupedPlan(M, *args)
    plan.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    worst = 0.0
    for j, (i, p) in enumerate(zip(idx, probs)):
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, ROWS_PER_MATRIX)]))
        cols = np.unique(np.concatenate([[0, p.N - 1], rng.integers(0, p.N, COLS_PER_MATRIX)]))
        x_rows = xs[j][torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
        xq, xsc = oracle.quant_act(x_rows)
        ms = np.repeat(np.arange(rows.size), cols.size).astype(np.int64)
        ns = np.tile(cols, rows.size).astype(np.int64)
        packed, w_scale = sweep["packs"][i]
        _, yref = oracle.matmul_sampled(xq, xsc, packed, w_scale, p.N, ms, ns)
        y = ys[j].cpu().numpy()[rows][:, cols].reshape(-1)
        assert not np.isnan(ys[j].cpu().numpy()).any(), f"{p.name}: unwritten output"
        if M <= 16:
            # decode: the exactly rounded value, bit for bit
            np.testing.assert_array_equal(y.view(np.uint32), yref.view(np.uint32), p.name)
        zero = yref == 0
        assert (y[zero] == 0).all(), p.name
        rel = np.abs(y.astype(np.float64) - yref) / np.maximum(np.abs(yref.astype(np.float64)),
                                                               1e-300)
        if (~zero).any():
            worst = max(worst, float(rel[~zero].max()))
        assert worst <= REL_TOL, f"{p.name}: max relative error {worst:.3e}"
    say(f"[sweep] M={M}: {len(probs)} matrices, max relative error {worst:.2e}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_sweep_sampled(sweep, M):
    """The 196-matrix decode sweep (one grouped launch) at M = 1, 4, 16."""
    say(f"[sweep] decode M={M}")
    run_and_check(sweep, M, lambda p: True, host_x=True)


def test_lut_decode_sweep_sampled(sweep):
    """The lookup-table variant over the same 196-matrix sweep at M = 1."""
    say("[sweep] lookup-table decode M=1")
    run_and_check(sweep, 1, lambda p: True, host_x=True, lut=True)


@pytest.mark.parametrize("M", [32, 64])
def test_batched_decode_sampled(longform, M):
    """Batched decode on the 28 gate and 28 down long-form projections
    (Student-t(3) weights; activations seed 60000+7l+p)."""
    say(f"[long-form] batched decode M={M}")
    run_and_check(longform, M, lambda p: p.proj in (4, 6), host_x=True)


def test_prefill_m256_sampled(sweep):
    """Prefill at M=256 over all 196 projections in one grouped launch
    (activations seed 30000+7l+p)."""
    say("[sweep] prefill M=256")
    run_and_check(sweep, 256, lambda p: True, host_x=True, x_problems=synth.prefill_problems())


def test_prefill_m1800_longform_sampled(longform):
    """Long-form prefill at M=1800 over all 196 Student-t(3) projections in one
    grouped launch (activations seed 60000+7l+p)."""
    say("[long-form] prefill M=1800")
    run_and_check(longform, 1800, lambda p: True, host_x=True)


def test_prefill_m1800_gpu_activations_sampled(sweep):
    """Prefill at M=1800 over the sweep's weights with activations drawn on the
    GPU (a second, independent input stream)."""
    say("[sweep] prefill M=1800, GPU-drawn activations")
    run_and_check(sweep, 1800, lambda p: True, host_x=False)
