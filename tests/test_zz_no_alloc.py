"""The no-allocation projection (built-in scratch) against the projection with
a caller's workspace, through the C ABI: bit-identical y, accumulators, int8
rows and scales, on two calls in a row whose second input is smaller (the
scratch keeps the first call's contents), for the decode path that stages
quantized rows (M <= 16, long K) and for the prefill GEMM (M > 16)."""
import numpy as np
import pytest

from ternary_weight_decoder_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ternary_weight_decoder_amd import binding
    binding.lib()
    return binding


def run_both(tb, M, N, K, seed):
    import torch
    dev = "cuda:0"
    W = synth.student_t_weights(N, K, seed)
    x = torch.from_numpy(synth.activations(M, K, seed + 1)).to(dev)
    packed, w_scale = tb.bitnet_ternarize_pack(torch.from_numpy(W).to(dev))
    outs = []
    for noalloc in (False, True):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        acc = torch.full((M, N), -7, dtype=torch.int32, device=dev)
        xq = torch.zeros((M, K), dtype=torch.int8, device=dev)
        xs = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
        if noalloc:
            tb.bitnet_ternary_matmul_noalloc_into(M, N, K, x, packed, w_scale, y, xq, xs, acc)
        else:
            ws = torch.empty(tb.bitnet_matmul_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
            tb.bitnet_ternary_matmul_into(M, N, K, x, packed, w_scale, y, ws, xq, xs, acc)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (y, acc, xq, xs)])
    for a, b in zip(*outs):
        assert a.tobytes() == b.tobytes()
    assert not np.isnan(outs[1][0]).any()


@pytest.mark.parametrize("first,second", [
    ((16, 1536, 8960), (3, 200, 1536)),        # decode, rows staged in the scratch
    ((1800, 1536, 8960), (40, 300, 384)),       # prefill GEMM
    ((300, 2000, 1536), (17, 64, 128)),
])
def test_noalloc_matches_workspace_call_twice(tb, first, second):
    print(f"[noalloc] {first} then {second}", flush=True)
    run_both(tb, *first, seed=1000 + first[0])
    run_both(tb, *second, seed=2000 + second[0])


def test_noalloc_rejects_beyond_the_scratch(tb):
    import torch
    M, K = 1800, 18688
    assert tb.bitnet_matmul_workspace_bytes(M, K) > tb.bitnet_scratch_bytes()
    d = torch.empty(16, dtype=torch.float32, device="cuda:0")
    with pytest.raises(tb.BitnetError) as e:
        tb.bitnet_ternary_matmul_noalloc_into(M, 64, K, d, d, d, d)
    assert e.value.status == 8
