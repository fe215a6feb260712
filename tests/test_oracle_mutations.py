"""Planted mistakes: every plausible slip in the oracle must fail at least one of its pins.

Each case below copies oracle/ssd_oracle.c, changes one expression (a dropped term, a wrong
sign or index, a swapped operand, another rounding rule), compiles the copy with the oracle's
own flags into a temporary library, and runs the pin files against it in a fresh interpreter
(the oracle loads the library named by SSD_ORACLE_LIB).  The pins pass on the real oracle
(the rest of the suite); here each mutant must make pytest report a failing test.  All of this
runs on the CPU; the HIP library is not involved."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssd_oracle.c")
PINS = {
    "rec": ["tests/test_oracle_recurrence.py"],
    "quant": ["tests/test_oracle_quantizer.py"],
    "f16": ["tests/test_oracle_state_f16.py"],
    "i8": ["tests/test_oracle_state_i8.py"],
    "fe": ["tests/test_oracle_frontend.py"],
    "corr": ["tests/test_oracle_correction.py"],
    "pn": ["tests/test_oracle_per_state.py"],
    "pc": ["tests/test_oracle_per_channel.py"],
}

# (name, pin files, text in ssd_oracle.c, replacement)
MUTANTS = [
    ("readout by B instead of C", "rec", "acc += Cv[n] * Sp[n];", "acc += Bv[n] * Sp[n];"),
    ("D x dropped", "rec", "y_out[t * P + p] = acc + Dh * xv[p] + mu;", "y_out[t * P + p] = acc + mu;"),
    ("correction indexed (p, h)", "corr", "ycorr[(int64_t)h * P + p]", "ycorr[(int64_t)p * H + h]"),
    ("correction subtracted", "corr", "acc + Dh * xv[p] + mu;", "acc + Dh * xv[p] - mu;"),
    ("unquantized readout by B", "corr", "acc += Cr[n] * Sp[n];", "acc += Br[n] * Sp[n];"),
    ("unquantized x dropped", "corr", "const double u = d * xr[p];", "const double u = d;"),
    ("unquantized decay sign", "corr", "const double a = exp(d * Ah);\n    const double* xr",
     "const double a = exp(-d * Ah);\n    const double* xr"),
    ("decay exponent sign", "rec", "const double a = exp(d * Ah);\n    for (int32_t p = 0; p < P; ++p)   /*",
     "const double a = exp(-d * Ah);\n    for (int32_t p = 0; p < P; ++p)   /*"),
    ("group map h % G", "rec", "const int32_t g = h / (H / G);\n  const int bc_per_state = scale_flags & 1, x_per_channel = (scale_flags >> 1) & 1;\n  double* S",
     "const int32_t g = h % G;\n  const int bc_per_state = scale_flags & 1, x_per_channel = (scale_flags >> 1) & 1;\n  double* S"),
    ("unquantized group map h % G", "corr", "const int32_t g = h / (H / G);\n  double* S = (double*)calloc((size_t)P * N, sizeof(double));\n  if (h0)",
     "const int32_t g = h % G;\n  double* S = (double*)calloc((size_t)P * N, sizeof(double));\n  if (h0)"),
    ("x dropped from the input term", "rec", "const double u = d * xv[p];", "const double u = d;"),
    ("dt dropped from the input term", "rec", "const double u = d * xv[p];", "const double u = xv[p];"),
    ("y read before the update", "rec", "Sp[n] = a * Sp[n] + u * Bv[n];\n        acc += Cv[n] * Sp[n];",
     "acc += Cv[n] * Sp[n];\n        Sp[n] = a * Sp[n] + u * Bv[n];"),
    ("per-head x scale ignored", "rec", "xv[p] = (double)sx[x_per_channel ? (int64_t)h * P + p : h] *",
     "xv[p] = (double)sx[x_per_channel ? (int64_t)h * P + p : 0] *"),
    ("per-channel x scale indexed (p, h)", "pc", "xv[p] = (double)sx[x_per_channel ? (int64_t)h * P + p : h] *",
     "xv[p] = (double)sx[x_per_channel ? (int64_t)p * H + h : h] *"),
    ("per-channel x scale taken per head", "pc", "xv[p] = (double)sx[x_per_channel ? (int64_t)h * P + p : h] *",
     "xv[p] = (double)sx[x_per_channel ? (int64_t)h * P : h] *"),
    ("per-channel x scale dropped from the chunk state", "pc",
     "const double xw = w * (double)sx[x_per_channel ? (int64_t)h * P + p : h] *",
     "const double xw = w * (double)sx[h] *"),
    ("dt dropped from the chunk state", "rec", "const double w = exp(last - acs[c * chunk + j]) * (double)dt[row * H + h];",
     "const double w = exp(last - acs[c * chunk + j]);"),
    ("chunk cumsum restarts wrong", "rec", "for (int32_t j = 0; j < chunk && c * chunk + j < L; ++j) {\n      acc +=",
     "for (int32_t j = 0; j < chunk && c * chunk + j < L; ++j) {\n      acc = 0.0;\n      acc +="),
    ("per-state scale indexed (n, g)", "pn", "const int32_t k = bc_per_state ? g * N + n : g;",
     "const int32_t k = bc_per_state ? n * G + g : g;"),
    ("per-state B scale dropped from the chunk state", "pn", "(double)sB[bc_per_state ? g * N + n : g]", "(double)sB[g]"),
    ("per-channel quantizer indexed by k only", "pn", "quantize_one(x[e], scale[(int64_t)k * inner + i])",
     "quantize_one(x[e], scale[k])"),
    ("quantizer ties away from zero", "quant", "float r = rintf(t);", "float r = roundf(t);"),
    ("quantizer by reciprocal multiply", "quant", "volatile float t = v / scale;",
     "volatile float t = v * (1.0f / scale);"),
    ("quantizer allows -128", "quant", "if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;"),
    ("binary16 ties away from zero", "f16", "const double r = nearbyint(a / quantum) * quantum;",
     "const double r = round(a / quantum) * quantum;"),
    ("binary16 spacing one binade off", "f16", "quantum = ldexp(1.0, e2 - 1 - 10);", "quantum = ldexp(1.0, e2 - 10);"),
    ("8-bit state ties away from zero", "i8", "c = nearbyint(row[n] / (double)s);", "c = round(row[n] / (double)s);"),
    ("8-bit state scale max/128", "i8", "float s = (float)(m / 127.0);", "float s = (float)(m / 128.0);"),
    ("SiLU sign", "fe", "const double a = v / (1.0 + exp(-v));", "const double a = v / (1.0 + exp(v));"),
    ("convolution taps reversed", "fe", "const int64_t src = t - dconv + 1 + k;", "const int64_t src = t - k;"),
    ("softplus sign", "fe", "fmax(v, 0.0) + log1p(exp(-fabs(v)))", "fmax(v, 0.0) + log1p(exp(fabs(v)))"),
]


@pytest.mark.parametrize("name,pins,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, pins, old, new, tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"{name}: the expression to change must occur exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.compile_library(str(src), str(tmp_path / "libmutant.so"))
    env = dict(os.environ, SSD_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS[pins]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    # pytest's exit status 1: tests ran and at least one failed (2-5: interrupted, internal or
    # usage errors, no tests collected -- none of which would say anything about the mutant)
    assert r.returncode == 1, f"{name}: no pin failed (exit {r.returncode})\n{r.stdout[-2000:]}"
