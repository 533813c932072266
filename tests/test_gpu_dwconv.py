"""GPU parity of the I8_S causal depthwise convolution against the oracle,
through the C ABI: per-channel weight codes and scales, the per-(sequence,
channel) activation scales, the int32 accumulators and the outputs are all
bit-exact.  Shapes cover one frame, kernels of 1, 3, 7 and 64 taps, ragged
frame counts around the 64-frame tile and the 128-frame chunk, several
sequences, bias and ReLU on and off, a zero input column and a zero kernel
channel, and the 8192-frame x 512-channel encoder stand-in.  Outputs carry a
NaN canary past their ends."""
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


def run_case(tb, B, T, C, k, bias_on, relu, seed, zero_col=False, zero_chan=False):
    import torch
    dev = "cuda:0"
    x = synth.activations(B * T, C, seed).reshape(B, T, C)
    if zero_col:
        x[B - 1, :, C // 2] = 0.0
    W = synth.normal_weights(C, k, seed + 1, std=0.1)
    if zero_chan:
        W[1] = 0.0
    bias = synth.normal_weights(1, C, seed + 2, std=0.1)[0] if bias_on else None
    q_ref, s_ref = oracle.rowq_quant_weights(W)
    q, s = tb.bitnet_i8_dwconv_quant_weights(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    assert s.cpu().numpy().tobytes() == s_ref.tobytes()
    ref = oracle.i8_dwconv(x, q_ref, s_ref, bias, relu)
    n = B * T * C
    ybuf = torch.full((n + 64,), float("nan"), device=dev)
    abuf = torch.full((n + 64,), -7, dtype=torch.int32, device=dev)
    xs = torch.full((B, C), float("nan"), device=dev)
    ws = torch.empty(tb.bitnet_i8_dwconv_workspace_bytes(B, T, C), dtype=torch.uint8, device=dev)
    bd = torch.from_numpy(bias).to(dev) if bias is not None else None
    tb.bitnet_i8_dwconv_into(B, T, C, k, torch.from_numpy(x).to(dev), q, s, bd, relu, ybuf[:n],
                             ws, abuf[:n], xs)
    torch.cuda.synchronize()
    assert torch.isnan(ybuf[n:]).all().item() and (abuf[n:] == -7).all().item(), "canary"
    assert xs.cpu().numpy().tobytes() == ref["x_scale"].tobytes()
    np.testing.assert_array_equal(abuf[:n].cpu().numpy().reshape(B, T, C), ref["acc"])
    assert ybuf[:n].cpu().numpy().tobytes() == ref["y"].tobytes()


@pytest.mark.parametrize("B,T,C,k", [(1, 1, 64, 1), (1, 5, 64, 7), (2, 130, 128, 7),
                                     (3, 300, 64, 3), (1, 129, 192, 64), (2, 64, 64, 7)])
@pytest.mark.parametrize("bias_on,relu", [(True, False), (False, True)])
def test_dwconv_parity(tb, B, T, C, k, bias_on, relu):
    say(f"[dwconv] B={B} T={T} C={C} k={k} bias={bias_on} relu={relu}")
    run_case(tb, B, T, C, k, bias_on, relu, seed=B * 1000 + T + C + k)


def test_dwconv_zero_column_and_channel(tb):
    say("[dwconv] zero input column and zero kernel channel")
    run_case(tb, 2, 200, 128, 7, True, False, seed=77, zero_col=True, zero_chan=True)


def test_dwconv_encoder_size(tb):
    say("[dwconv] encoder stand-in B=1 T=8192 C=512 k=7")
    run_case(tb, 1, 8192, 512, 7, True, False, seed=70100)


@pytest.mark.parametrize("B,T,C,k", [(2, 8392, 64, 3), (1, 20000, 64, 7)])
def test_dwconv_long_sequence(tb, B, T, C, k):
    """Sequences longer than 64 chunks of 128 frames: the column maxima use
    chunks of 256 (8392 frames, 33 chunks) and 512 frames (20000, 40 chunks)."""
    say(f"[dwconv] long sequence B={B} T={T} C={C} k={k}")
    run_case(tb, B, T, C, k, True, True, seed=B * 7 + T)
