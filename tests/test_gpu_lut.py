"""GPU parity of the lookup-table decode variant (M = 1) against the oracle.

Outputs are exactly rounded, so they are compared bit for bit: ragged N, the
one-unit K, the chunk boundary of the tables (16 units) and past it, the
longest K the call accepts, several projections of different K in one
launch, and a zero activation row.
"""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu


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


def run_group(tb, shapes, seed, zero_row=False):
    import torch
    dev = "cuda:0"
    xs, pk, sc, ys, refs = [], [], [], [], []
    for i, (N, K) in enumerate(shapes):
        W = synth.normal_weights(N, K, seed + i)
        packed, s = oracle.ternarize_pack(W)
        x = np.zeros((1, K), np.float32) if zero_row else synth.activations(1, K, seed + 100 + i)
        refs.append(oracle.ternary_matmul(x, packed, s, N)["y"])
        xs.append(torch.from_numpy(x).to(dev))
        pk.append(torch.from_numpy(packed).to(dev))
        sc.append(torch.tensor([s], dtype=torch.float32, device=dev))
        # one canary past the end of every output
        ys.append(torch.full((1, N + 1), float("nan"), device=dev))
    plan = tb.LutPlan(xs, pk, sc, [y[:, :N] for y in ys], [n for n, _ in shapes],
                      [k for _, k in shapes])
    plan.run()
    torch.cuda.synchronize()
    for (N, K), y, ref in zip(shapes, ys, refs):
        got = y.cpu().numpy()
        assert np.isnan(got[0, N]), f"{N}x{K}: wrote past the end"
        np.testing.assert_array_equal(got[:, :N].view(np.uint32), ref.view(np.uint32),
                                      f"{N}x{K}")


@pytest.mark.parametrize("N,K", [(200, 128), (256, 1536), (1000, 2048), (1536, 2176),
                                 (1536, 8960), (300, 16384)])
def test_lut_single(tb, N, K):
    say(f"[lut] N={N} K={K}")
    run_group(tb, [(N, K)], seed=900)


def test_lut_group_mixed_k(tb):
    say("[lut] one layer's projections plus ragged shapes in one launch")
    shapes = [(p.N, p.K) for p in synth.layer_problems()] + [(77, 384), (513, 640)]
    run_group(tb, shapes, seed=910)


def test_lut_zero_row(tb):
    say("[lut] zero activation row")
    run_group(tb, [(384, 1536)], seed=920, zero_row=True)
