"""Seeded synthetic inputs for the ternary projection workloads.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no ternarization, packing, quantization or matmul), so the
CPU oracle and the HIP path can both consume its arrays without sharing any
code that computes a result.

Shapes: the LM decoder is a Qwen2.5-1.5B-style stack of 28 layers with hidden
size 1536 (the audio features handed to the decoder are 1536 wide, ONNX model
card "multimodalart/VibeVoice-ASR-BitNet-ONNX", Layout table) and 7 ternary
projections per layer, 196 matrices in all (same card, Quantization table, row
"LM projections").  Weights are stored out x in, i.e. W[N, K] row-major, and a
projection maps x[M, K] to y[M, N].

Token counts: 24 kHz audio is cut into 3200-sample frames, one speech token per
frame (same card, Layout table), so 30 s of audio gives 225 frames; with a
31-token prompt that is M = 256.  Four minutes at 7.5 frames/s gives M = 1800.

Random streams: numpy ``default_rng(seed)`` (PCG64).  Normal draws are made
directly in float32; Student-t draws are made in float64 and cast.
"""
from __future__ import annotations

import math
import multiprocessing
from dataclasses import dataclass

import numpy as np

HIDDEN = 1536
INTERMEDIATE = 8960
N_LAYERS = 28
UNIT = 128  # codes per packing unit

# (name, K, N) for the 7 projections of one layer, in layer order.
PROJECTIONS = (
    ("q", HIDDEN, HIDDEN),
    ("k", HIDDEN, 256),
    ("v", HIDDEN, 256),
    ("o", HIDDEN, HIDDEN),
    ("gate", HIDDEN, INTERMEDIATE),
    ("up", HIDDEN, INTERMEDIATE),
    ("down", INTERMEDIATE, HIDDEN),
)

PREFILL_M_30S = 225 + 31      # 30 s of 24 kHz audio in 3200-sample frames + prompt
PREFILL_M_LONG = 1800         # 240 s at 7.5 frames/s


@dataclass(frozen=True)
class Problem:
    """One projection instance: which layer/projection and its seeds."""
    layer: int
    proj: int
    K: int
    N: int
    w_seed: int
    x_seed: int

    @property
    def name(self) -> str:
        return f"L{self.layer}.{PROJECTIONS[self.proj][0]}"


def normal_weights(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """fp32 master weights ~ N(0, std^2), shape [N, K]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)


def student_t_weights(N: int, K: int, seed: int, df: float = 3.0,
                      std: float = 0.01) -> np.ndarray:
    """fp32 master weights from a Student-t(df) rescaled to standard deviation std."""
    rng = np.random.default_rng(seed)
    t = rng.standard_t(df, size=(N, K))
    return (t * (std / math.sqrt(df / (df - 2.0)))).astype(np.float32)


def outlier_columns(K: int, rng: np.random.Generator, frac: float = 0.01) -> np.ndarray:
    """round(frac*K) distinct channel indices, the same for every row."""
    n_out = int(round(frac * K))
    return np.sort(rng.choice(K, size=n_out, replace=False))


def activations(M: int, K: int, seed: int, outliers: bool = True,
                outlier_gain: float = 20.0) -> np.ndarray:
    """fp32 activations ~ N(0,1), shape [M, K]; optionally 1% of channels x20."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        cols = outlier_columns(K, rng)
        x[:, cols] *= np.float32(outlier_gain)
    return x


# ---------------------------------------------------------------------------
# Workloads.  Each returns plain numpy arrays; nothing here depends on torch.
# ---------------------------------------------------------------------------

def single_gemv(seed: int = 0, N: int = HIDDEN, K: int = HIDDEN, M: int = 1):
    """Single 1536x1536 GEMV at M=1: W drawn first, then x, from one stream."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return W, x


def layer_problems() -> list[Problem]:
    """One decoder layer's 7 projections (weights seed 1000+p, x seed 2000+p)."""
    return [Problem(0, p, K, N, 1000 + p, 2000 + p)
            for p, (_, K, N) in enumerate(PROJECTIONS)]


def sweep_problems(n_layers: int = N_LAYERS, w_base: int = 10000,
                   x_base: int = 20000) -> list[Problem]:
    """All 7 x n_layers projections with independent seeds base+7*layer+proj."""
    out = []
    for layer in range(n_layers):
        for p, (_, K, N) in enumerate(PROJECTIONS):
            out.append(Problem(layer, p, K, N, w_base + 7 * layer + p,
                               x_base + 7 * layer + p))
    return out


def prefill_problems(n_layers: int = N_LAYERS) -> list[Problem]:
    """Prefill at M=256 on the sweep's weights; activations seed 30000+7l+p."""
    return sweep_problems(n_layers, w_base=10000, x_base=30000)


def longform_problems(n_layers: int = N_LAYERS) -> list[Problem]:
    """Long-form prefill M=1800 with Student-t(3) weights (std 0.01)."""
    return sweep_problems(n_layers, w_base=50000, x_base=60000)


def problem_weights(p: Problem, heavy_tail: bool = False) -> np.ndarray:
    if heavy_tail:
        return student_t_weights(p.N, p.K, p.w_seed)
    return normal_weights(p.N, p.K, p.w_seed)


def problem_activations(p: Problem, M: int, outliers: bool = True) -> np.ndarray:
    return activations(M, p.K, p.x_seed, outliers=outliers)


def random_codes(N: int, K: int, seed: int, p_zero: float = 0.34) -> np.ndarray:
    """Ternary codes in {-1,0,+1} (int8) with the given zero fraction, for tests."""
    rng = np.random.default_rng(seed)
    u = rng.random((N, K))
    q = np.where(u < p_zero, 0, np.where(rng.random((N, K)) < 0.5, -1, 1))
    return q.astype(np.int8)


def random_int8(M: int, K: int, seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 values in [lo, hi], for tests of the integer contraction."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(M, K), dtype=np.int16).astype(np.int8)


# ---- I8_S audio-encoder layers ----------------------------------------------
# The pages name the encoders' format (int8 weights and activations, ReLU for
# GELU, fused matmul + bias + ReLU) and describe a ConvNeXt-style tokenizer
# whose activations outweigh its weights, but give no layer sizes.  The two
# layers below are the pointwise pair of one such block over 8192 frames:
# 512 -> 2048 channels with bias and ReLU, then 2048 -> 512 with bias.  In the
# first, the fp32 activations (16 MB) outweigh the int8 weights (1 MB) 16:1.
I8_FRAMES = 8192
I8_LAYERS = {
    # name: (M, K, N, relu)
    "pw1": (I8_FRAMES, 512, 2048, True),
    "pw2": (I8_FRAMES, 2048, 512, False),
}


def i8_layer_inputs(name: str, seed: int = 70000):
    """(x [M,K], W [N,K], bias [N]) for one I8_S layer: x as `activations`
    (N(0,1), 1% of channels x20), W ~ N(0, 0.02^2), bias ~ N(0, 0.1^2)."""
    M, K, N, _ = I8_LAYERS[name]
    off = sorted(I8_LAYERS).index(name)
    x = activations(M, K, seed + 10 * off)
    W = normal_weights(N, K, seed + 10 * off + 1)
    bias = np.random.default_rng(seed + 10 * off + 2).standard_normal(N, dtype=np.float32)
    return x, W, (bias * np.float32(0.1)).astype(np.float32)


# ---- the decoder's 8-bit table: embeddings and lm_head ----------------------
# [V, K] = [151936, 1536]: the prompt's token ids reach 151648 (<|speech_pad|>)
# and V*K int8 plus one fp32 scale per row is the model card's 234 MB of
# embeddings.  The table's master weights are drawn ~ N(0, 0.02^2) like the
# projections' (no trained weights are used); the lm_head input is a hidden
# state, N(0,1) with 1% of channels x20 like every other projection input.
VOCAB = 151936
TABLE_SEED = 80000


def table_weights(V: int = VOCAB, K: int = HIDDEN, seed: int = TABLE_SEED) -> np.ndarray:
    """fp32 master weights of the embedding / lm_head table, shape [V, K]."""
    return normal_weights(V, K, seed)


def token_ids(T: int, V: int = VOCAB, seed: int = TABLE_SEED + 1) -> np.ndarray:
    """T token ids drawn uniformly from [0, V), int32."""
    return np.random.default_rng(seed).integers(0, V, size=T, dtype=np.int64).astype(np.int32)


# ---- generation in worker processes -------------------------------------------
# The workloads' arrays are drawn with numpy on the host, one seeded stream per
# matrix; drawing the 196 Student-t masters of the long-form workload takes
# over a minute on one core, so the benchmark spreads the matrices over worker
# processes (spawned, so that they never touch the GPU).  Results arrive in
# the order of the problems, identical to drawing them one by one.

def _weights_job(args):
    N, K, seed, heavy = args
    return student_t_weights(N, K, seed) if heavy else normal_weights(N, K, seed)


def _activations_job(args):
    M, K, seed = args
    return activations(M, K, seed)


def _parallel(job, jobs, workers):
    if workers <= 1:
        yield from map(job, jobs)
        return
    ctx = multiprocessing.get_context("spawn")
    with ctx.Pool(workers) as pool:
        yield from pool.imap(job, jobs, chunksize=1)


def problem_weights_iter(problems, heavy_tail: bool = False, workers: int = 1):
    """problem_weights(p, heavy_tail) for each problem, in order."""
    yield from _parallel(_weights_job, [(p.N, p.K, p.w_seed, heavy_tail) for p in problems],
                         workers)


def problem_activations_iter(problems, M: int, workers: int = 1):
    """problem_activations(p, M) for each problem, in order."""
    yield from _parallel(_activations_job, [(M, p.K, p.x_seed) for p in problems], workers)
