"""GPU parity of the staged decode call: one token through dependent stages.

Per layer the stages are q,k,v (input h) | o (input y_q) | gate, up (input
y_o) | down (input y_up), and y_down is the next layer's h: every stage reads
what an earlier stage of the same launch wrote.  (The attention and the
gate-times-up product between these projections are not part of the
projection path; the chain feeds y_q and y_up through instead.)  The oracle
runs the same chain on its own outputs; decode outputs are exactly rounded,
so every stage must match bit for bit.
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


def build_chain(tb, layers):
    import torch
    problems = synth.sweep_problems(layers)
    packs = [oracle.ternarize_pack(synth.problem_weights(p)) for p in problems]
    dev = "cuda:0"
    h0 = synth.activations(1, synth.HIDDEN, seed=4242)
    h = torch.from_numpy(h0).to(dev)
    bufs, stages = {}, []
    for l in range(layers):
        P = problems[7 * l:7 * l + 7]
        y = {j: torch.full((1, P[j].N), float("nan"), device=dev) for j in range(7)}
        W = {j: (torch.from_numpy(packs[7 * l + j][0]).to(dev),
                 torch.tensor([packs[7 * l + j][1]], dtype=torch.float32, device=dev))
             for j in range(7)}

        def prob(j, x):
            return (x, W[j][0], W[j][1], y[j], P[j].N, P[j].K)
        stages.append([prob(0, h), prob(1, h), prob(2, h)])
        stages.append([prob(3, y[0])])
        stages.append([prob(4, y[3]), prob(5, y[3])])
        stages.append([prob(6, y[5])])
        bufs[l] = y
        h = y[6]
    return problems, packs, h0, stages, bufs


def oracle_chain(problems, packs, h0, layers):
    out = {}
    h = h0
    for l in range(layers):
        r = {}
        def run(j, x):
            pk, s = packs[7 * l + j]
            return oracle.ternary_matmul(x, pk, s, problems[7 * l + j].N)["y"]
        r[0], r[1], r[2] = run(0, h), run(1, h), run(2, h)
        r[3] = run(3, r[0])
        r[4], r[5] = run(4, r[3]), run(5, r[3])
        r[6] = run(6, r[5])
        out[l] = r
        h = r[6]
    return out


@pytest.mark.parametrize("layers", [2, 28])
def test_stages_chain_bit_exact(tb, layers):
    import torch
    say(f"[stages] dependent chain, {layers} layers ({4 * layers} stages)")
    problems, packs, h0, stages, bufs = build_chain(tb, layers)
    plan = tb.StagedPlan(1, stages)
    plan.run()
    torch.cuda.synchronize()
    assert not plan.timed_out() and plan.timeouts_total() == 0
    ref = oracle_chain(problems, packs, h0, layers)
    for l in range(layers):
        for j in range(7):
            got = bufs[l][j].cpu().numpy()
            assert not np.isnan(got).any(), f"layer {l} projection {j}: unwritten"
            np.testing.assert_array_equal(got.view(np.uint32), ref[l][j].view(np.uint32),
                                          f"layer {l} projection {j}")
    # A second run over the same buffers reproduces the first bit for bit.
    first = [bufs[l][j].clone() for l in range(layers) for j in range(7)]
    plan.run()
    torch.cuda.synchronize()
    assert not plan.timed_out() and plan.timeouts_total() == 0
    again = [bufs[l][j] for l in range(layers) for j in range(7)]
    assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_stages_single_stage_matches_grouped(tb):
    """One stage holding one layer's projections equals the grouped call."""
    import torch
    say("[stages] one stage vs grouped call")
    problems = synth.layer_problems()
    dev = "cuda:0"
    packs = [oracle.ternarize_pack(synth.problem_weights(p)) for p in problems]
    xs = [torch.from_numpy(synth.problem_activations(p, 1)).to(dev) for p in problems]
    dp = [torch.from_numpy(pk).to(dev) for pk, _ in packs]
    ds = [torch.tensor([s], dtype=torch.float32, device=dev) for _, s in packs]
    y1 = [torch.full((1, p.N), float("nan"), device=dev) for p in problems]
    y2 = [torch.full((1, p.N), float("nan"), device=dev) for p in problems]
    plan = tb.StagedPlan(1, [[(xs[i], dp[i], ds[i], y1[i], p.N, p.K)
                              for i, p in enumerate(problems)]])
    plan.run()
    g = tb.GroupedPlan(1, xs, dp, ds, y2, [p.N for p in problems], [p.K for p in problems])
    g.run()
    torch.cuda.synchronize()
    assert not plan.timed_out() and plan.timeouts_total() == 0
    for a, b in zip(y1, y2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("M", [1, 3, 16])
def test_stages_general_shapes_bit_exact(tb, M):
    """Several rows, ragged N, a one-unit K, two problems per stage:
    A,B <- x | C <- y_A | D <- y_C | E,F <- y_D."""
    import torch
    say(f"[stages] general chain, M={M}")
    Kc = min(1024, (8960 // M) // 128 * 128)
    shapes = {"A": (Kc, Kc), "B": (Kc, 200), "C": (Kc, 128), "D": (128, Kc),
              "E": (Kc, 77), "F": (Kc, Kc)}
    src = {"A": "x", "B": "x", "C": "A", "D": "C", "E": "D", "F": "D"}
    order = [["A", "B"], ["C"], ["D"], ["E", "F"]]
    dev = "cuda:0"
    packs, W = {}, {}
    for i, (name, (K, N)) in enumerate(shapes.items()):
        pk, s = oracle.ternarize_pack(synth.normal_weights(N, K, 700 + i))
        packs[name] = (pk, s)
        W[name] = (torch.from_numpy(pk).to(dev), torch.tensor([s], dtype=torch.float32, device=dev))
    x0 = synth.activations(M, Kc, seed=701)
    xd = torch.from_numpy(x0).to(dev)
    ys = {n: torch.full((M, shapes[n][1]), float("nan"), device=dev) for n in shapes}
    stages = [[(xd if src[n] == "x" else ys[src[n]], W[n][0], W[n][1], ys[n], shapes[n][1],
                shapes[n][0]) for n in st] for st in order]
    plan = tb.StagedPlan(M, stages)
    plan.run()
    torch.cuda.synchronize()
    assert not plan.timed_out() and plan.timeouts_total() == 0
    ref = {}
    for st in order:
        for n in st:
            xin = x0 if src[n] == "x" else ref[src[n]]
            pk, s = packs[n]
            ref[n] = oracle.ternary_matmul(xin, pk, s, shapes[n][1])["y"]
    for n in shapes:
        got = ys[n].cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint32), ref[n].view(np.uint32), n)


@pytest.mark.parametrize("M", [1, 4])
def test_stages_max_stages_bit_exact(tb, M):
    """The staged call at its largest sizes: 256 stages of one problem each
    (N = K = 128), every stage reading the previous stage's output.  Each
    stage's master is a seeded N(0,1) matrix times a power of two picked on
    the host so that the chain's outputs stay near 1 (the codes do not depend
    on that factor); every output bit for bit against the oracle's own chain."""
    import torch
    n = tb.BITNET_MAX_GROUP
    say(f"[stages] {n} single-problem stages, M={M}")
    dev = "cuda:0"
    x = synth.activations(M, 128, seed=910)
    xd = torch.from_numpy(x).to(dev)
    refs, stages, ys = [], [], []
    prev, prev_d = x, xd
    for s in range(n):
        W0 = synth.normal_weights(128, 128, seed=920 + s, std=1.0)
        pk, sc = oracle.ternarize_pack(W0)
        a = float(np.abs(oracle.ternary_matmul(prev, pk, sc, 128)["y"]).max())
        c = np.float32(2.0 ** -round(np.log2(a))) if a > 0 else np.float32(1.0)
        pk, sc = oracle.ternarize_pack(W0 * c)
        ref = oracle.ternary_matmul(prev, pk, sc, 128)["y"]
        y = torch.full((M, 128), float("nan"), device=dev)
        stages.append([(prev_d, torch.from_numpy(pk).to(dev),
                        torch.tensor([sc], dtype=torch.float32, device=dev), y, 128, 128)])
        refs.append(ref)
        ys.append(y)
        prev, prev_d = ref, y
    assert 0.1 < float(np.abs(refs[-1]).max()) < 10.0
    plan = tb.StagedPlan(M, stages)
    for _ in range(2):
        for y in ys:
            y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert not plan.timed_out() and plan.timeouts_total() == 0
        for s in range(n):
            np.testing.assert_array_equal(ys[s].cpu().numpy().view(np.uint32),
                                          refs[s].view(np.uint32), f"stage {s}")
