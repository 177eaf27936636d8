"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU),
builds it, and runs the pin suite against that build in a child process; the
suite has to fail.  The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tri_oracle.c")

MUTANTS = [
    ("pack2 radix", "power *= 4;", "power *= 3;"),
    ("pack16 radix", "value = value * 3 +", "value = value * 4 +"),
    ("pack16 digit order", "for (int j = 4; j >= 0; --j)", "for (int j = 0; j <= 4; ++j)"),
    ("digit of -1", "if (w < 0) return 0;", "if (w < 0) return 2;"),
    ("padding trit", "if (k >= K) return 0;", "if (k >= K) return 1;"),
    ("2-bit decode sign", "int t = (code == 3) ? 0 : code - 1;", "int t = (code == 3) ? 0 : 1 - code;"),
    ("2-bit code 3", "int t = (code == 3) ? 0 : code - 1;", "int t = code - 1;"),
    ("1.6-bit digit", "int x = rest % 3;", "int x = rest % 4;"),
    ("1.6-bit digit offset", "W[n * K + k] = (int8_t)(x - 1);", "W[n * K + k] = (int8_t)(1 - x);"),
    ("2-bit row bytes", "16 * ((K + 63) / 64)", "16 * (K / 64 + 1)"),
    ("1.6-bit row bytes", "16 * ((K + 79) / 80)", "16 * ((K + 63) / 64)"),
    ("dropped first term", "for (int64_t k = 0; k < K; ++k)\n                sum +=",
     "for (int64_t k = 1; k < K; ++k)\n                sum +="),
    ("transposed weights", "(double)W[n * K + k]", "(double)W[k * N + n]"),
    ("activation row ignored", "oracle_half_to_double(X[m * K + k])", "oracle_half_to_double(X[k])"),
    ("scale dropped", "Y[m * N + n] = scale * sum;", "Y[m * N + n] = sum;"),
    ("float accumulator", "double sum = 0.0;", "float sum = 0.0f;"),
    ("fp16 exponent bias", "exponent - 25", "exponent - 24"),
    ("fp16 subnormal scale", "ldexp((double)mantissa, -24)", "ldexp((double)mantissa, -25)"),
    ("fp16 sign dropped", "return sign ? -v : v;", "return v;"),
    ("quantise without abs", "row += fabs((double)W[n * K + k]);", "row += (double)W[n * K + k];"),
    ("quantise ties away from zero", "q = rint((double)W[i] / (double)s);", "q = round((double)W[i] / (double)s);"),
    ("quantise not clipped", "if (q > 1.0) q = 1.0;", ";"),
    ("quantise mean over K only", "(double)N * (double)K", "(double)K"),
    ("quantise sign flipped", "T[i] = (int8_t)q;", "T[i] = (int8_t)-q;"),
    ("silu as sigmoid", "out[i] = a[i] / (1.0 + exp(-a[i])) * b[i];", "out[i] = 1.0 / (1.0 + exp(-a[i])) * b[i];"),
    ("silu gate without the up layer", "out[i] = a[i] / (1.0 + exp(-a[i])) * b[i];", "out[i] = a[i] / (1.0 + exp(-a[i]));"),
    ("fused: eps dropped", "double r = sqrt(sq / (double)K + eps);", "double r = sqrt(sq / (double)K);"),
    ("fused: mean over K-1", "double r = sqrt(sq / (double)K + eps);", "double r = sqrt(sq / (double)(K - 1) + eps);"),
    ("fused: gain ignored", "x[k] = x[k] * (gain ? oracle_half_to_double(gain[k]) : 1.0) / r;", "x[k] = x[k] / r;"),
    ("fused: residual dropped", "Y[m * N + n] = (residual ? oracle_half_to_double(residual[m * N + n]) : 0.0) + scale * sum;",
     "Y[m * N + n] = scale * sum;"),
    ("quantise threshold at the scale", "q = rint((double)W[i] / (double)s);", "q = rint((double)W[i] / (double)s / 2.0);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, "mutation anchor not found: %r" % old
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", str(mutant), "-o", str(lib), "-lm"])
    env = dict(os.environ, TRI_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "planted mistake '%s' was not caught:\n%s" % (name, r.stdout[-2000:])
