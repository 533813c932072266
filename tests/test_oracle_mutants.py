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
}

# Slips in the I8_S functions, caught by the I8_S pins.
I8_MUTANTS = {
    "i8_round_half_away": ("float t = rintf(W[i] / s);", "float t = roundf(W[i] / s);"),
    "i8_scale_128": ("float s = a / 127.0f;                 /* fp32, correctly rounded */",
                     "float s = a / 128.0f;"),
    "i8_transposed": ("s += (int64_t)xq[m * K + k] * (int64_t)q[n * K + k];",
                      "s += (int64_t)xq[m * K + k] * (int64_t)q[(m % N) * K + k];"),
    "i8_bias_dropped": ("if (bias) v += (double)bias[n];", ""),
    "i8_relu_inverted": ("if (relu && !(v > 0.0)) v = 0.0;", "if (relu && (v > 0.0)) v = 0.0;"),
    "i8_dequant_inverted": ("(double)acc[m * N + n] * (double)w_scale / (double)xs[m];",
                            "(double)acc[m * N + n] * (double)w_scale * (double)xs[m];"),
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
