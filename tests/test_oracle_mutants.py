"""The pins must catch plausible mistakes in the oracle.

Each case compiles a copy of the oracle with one deliberate slip (on the CPU,
into a temporary directory) and runs the pin suite against it in a subprocess;
the suite has to fail.  This guards the pins themselves.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    # rounding ties away from zero instead of to even
    "round_half_away": ("float t = rintf(r);", "float t = roundf(r);"),
    # absmax instead of absmean as the tensor scale
    "absmax_scale": ("row += fabs((double)W[n * K + k]);",
                     "row = fmax(row, fabs((double)W[n * K + k]) * (double)(N * K));"),
    # 64-code units
    "unit_64": ("#define ORACLE_UNIT 128", "#define ORACLE_UNIT 64"),
    # fields placed by r/16 instead of r/32
    "field_shift": ("static int packed_shift(int64_t k) { return 2 * (int)((k % ORACLE_UNIT) / 32); }",
                    "static int packed_shift(int64_t k) { return 2 * (int)((k % ORACLE_UNIT) / 16) % 8; }"),
    # the minus-one codes added instead of subtracted
    "sign_dropped": ("acc[m * N + n] = plus - minus;", "acc[m * N + n] = plus + minus;"),
    # activation scale applied as a divide in the epilogue's place
    "dequant_inverted": ("(double)acc[m * N + n] * (double)w_scale /\n                                   (double)x_scale[m]",
                         "(double)acc[m * N + n] * (double)w_scale *\n                                   (double)x_scale[m]"),
    # activation rounding half away from zero
    "act_round": ("float t = rintf(p);          /* half to even */", "float t = roundf(p);"),
    # transposed operand: row n of codes read with the activation row index
    "transposed": ("int8_t c = q[n * K + k];", "int8_t c = q[(m % N) * K + k];"),
    # code from W times the rounded reciprocal of m instead of the quotient W/m
    "code_by_reciprocal": ("float r = w / m;", "float r = w * (1.0f / m);"),
    # mean rounded twice: fp64 sum rounded to fp32, then an fp32 division
    "mean_rounded_twice": ("return (float)(total / (double)(N * K));",
                           "return (float)total / (float)(N * K);"),
}

# Slips in the I8_S functions, caught by the I8_S pins.
I8_MUTANTS = {
    "i8_round_half_away": ("float t = rintf(W[i] / s);", "float t = roundf(W[i] / s);"),
    # weight code from W times the rounded reciprocal of s instead of W/s
    "i8_code_by_reciprocal": ("float t = rintf(W[i] / s);", "float t = rintf(W[i] * (1.0f / s));"),
    "i8_scale_128": ("float s = a / 127.0f;                 /* fp32, correctly rounded */",
                     "float s = a / 128.0f;"),
    "i8_transposed": ("s += (int64_t)xq[m * K + k] * (int64_t)q[n * K + k];",
                      "s += (int64_t)xq[m * K + k] * (int64_t)q[(m % N) * K + k];"),
    "i8_bias_dropped": ("if (bias) v += (double)bias[n];", ""),
    "i8_relu_inverted": ("if (relu && !(v > 0.0)) v = 0.0;", "if (relu && (v > 0.0)) v = 0.0;"),
    "i8_dequant_inverted": ("(double)acc[m * N + n] * (double)w_scale / (double)xs[m];",
                            "(double)acc[m * N + n] * (double)w_scale * (double)xs[m];"),
}


# Slips in the 8-bit per-row table (embeddings and lm_head), caught by its pins.
ROWQ_MUTANTS = {
    # one scale for the whole table instead of one per row
    "rowq_per_tensor": ("for (int64_t k = 0; k < K; ++k) a = fabsf(row[k]) > a ? fabsf(row[k]) : a;",
                        "for (int64_t k = 0; k < N * K; ++k) a = fabsf(W[k]) > a ? fabsf(W[k]) : a;"),
    "rowq_round_half_away": ("float t = rintf(row[k] / s);", "float t = roundf(row[k] / s);"),
    "rowq_code_by_reciprocal": ("float t = rintf(row[k] / s);",
                                "float t = rintf(row[k] * (1.0f / s));"),
    "rowq_scale_127_5": ("float s = a / 127.0f;                 /* row scale: fp32, correctly rounded */",
                         "float s = a / 127.5f;"),
    # the lm_head output scaled by the activation row's index into the table scales
    "rowq_scale_index": ("(double)acc[m * N + n] * (double)w_scale[n] /",
                         "(double)acc[m * N + n] * (double)w_scale[m % N] /"),
    # embedding scaled by the neighbouring row's scale
    "rowq_embed_scale_row": ("(float)((double)q[id * K + k] * (double)w_scale[id])",
                             "(float)((double)q[id * K + k] * (double)w_scale[(id + 1) % N])"),
    # per-channel layer: the bias of the activation row's index
    "rows_bias_index": ("if (bias) v += (double)bias[n];          /* channel bias */",
                        "if (bias) v += (double)bias[m % N];"),
    # per-channel layer: ReLU keeps the negative part
    "rows_relu_inverted": ("if (relu && v <= 0.0) v = 0.0;\n            y[m * N + n] = (float)v;",
                           "if (relu && v > 0.0) v = 0.0;\n            y[m * N + n] = (float)v;"),
    # per-channel layer: one channel's scale for all
    "rows_scale_first": ("double v = (double)acc[m * N + n] * (double)w_scale[n] / (double)xs[m];",
                         "double v = (double)acc[m * N + n] * (double)w_scale[0] / (double)xs[m];"),
    # table layout: the 16-input groups and the 64-input steps swapped
    "table_h_j_swapped": ("return tile * 4096 + j * 1024 + h * 256 + (v % 16) * 16 + e;",
                          "return tile * 4096 + h * 1024 + j * 256 + (v % 16) * 16 + e;"),
    # table layout: tiles ordered by input chunk first
    "table_chunk_major": ("int64_t tile = (v / 16) * chunks + k / 256;",
                          "int64_t tile = (k / 256) * 16 + v / 16;"),
    # embedding rows read transposed
    "rowq_embed_transposed": ("(float)((double)q[id * K + k] * (double)w_scale[id])",
                              "(float)((double)q[(k % N) * K + id % K] * (double)w_scale[id])"),
}


# Slips in the I8_S depthwise convolution, caught by its pins.
DWCONV_MUTANTS = {
    # anti-causal: later frames instead of earlier ones
    "dw_anticausal": ("int64_t src = t - (k - 1) + j;   /* causal: earlier frames only */",
                      "int64_t src = t + j;"),
    # kernel taps read in reverse
    "dw_taps_reversed": ("acc += (int32_t)xq[(b * T + src) * C + c] * (int32_t)q[c * k + j];",
                         "acc += (int32_t)xq[(b * T + src) * C + c] * (int32_t)q[c * k + (k - 1 - j)];"),
    # one activation scale per channel shared by all sequences
    "dw_scale_ignores_sequence": ("double v = (double)acc * (double)w_scale[c] / (double)xs[b * C + c];",
                                  "double v = (double)acc * (double)w_scale[c] / (double)xs[c];"),
    # activation column absmax over the first frame only
    "dw_colmax_first_frame": ("for (int64_t t = 0; t < T; ++t) {\n                float v = fabsf(col[t * C]);",
                              "for (int64_t t = 0; t < 1; ++t) {\n                float v = fabsf(col[t * C]);"),
    # bias of the wrong channel
    "dw_bias_index": ("if (bias) v += (double)bias[c];\n                if (relu && v <= 0.0) v = 0.0;\n                y[o] = (float)v;",
                      "if (bias) v += (double)bias[(c + 1) % C];\n                if (relu && v <= 0.0) v = 0.0;\n                y[o] = (float)v;"),
}


def run_pins_on_mutant(tmp_path, old, new, pin_file):
    src = open(os.path.join(ROOT, "oracle", "bitnet_oracle.c")).read()
    assert old in src, "mutation site not found"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mut), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, BITNET_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pin_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    r = run_pins_on_mutant(tmp_path, old, new, "test_oracle_pins.py")
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(I8_MUTANTS))
def test_i8_pins_reject_mutant(name, tmp_path):
    old, new = I8_MUTANTS[name]
    r = run_pins_on_mutant(tmp_path, old, new, "test_oracle_i8_pins.py")
    assert r.returncode != 0, f"I8_S pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(ROWQ_MUTANTS))
def test_rowq_pins_reject_mutant(name, tmp_path):
    old, new = ROWQ_MUTANTS[name]
    r = run_pins_on_mutant(tmp_path, old, new, "test_oracle_rowq_pins.py")
    assert r.returncode != 0, f"per-row table pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(DWCONV_MUTANTS))
def test_dwconv_pins_reject_mutant(name, tmp_path):
    old, new = DWCONV_MUTANTS[name]
    r = run_pins_on_mutant(tmp_path, old, new, "test_oracle_dwconv_pins.py")
    assert r.returncode != 0, f"depthwise-conv pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
