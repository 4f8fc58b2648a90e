"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Each mutant is one textual edit of ``oracle/oracle.c`` (which must match exactly once),
compiled with gcc into a temporary library; the pin suite then runs against it in a
subprocess (``MOE_ORACLE_LIB``) and must fail.  The real oracle is never touched.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

MUTANTS = [
    ("router bias dropped", "if (b_r) acc += (double)b_r[e];", "if (b_r) acc += 0.0;"),
    ("router operand transposed", "(double)w_r[(size_t)e * H + h]", "(double)w_r[(size_t)h * E + e]"),
    ("ties to the higher index", "  return ea < eb;\n}", "  return ea > eb;\n}"),
    ("NaN ranked first", "if (na != nb) return nb;", "if (na != nb) return na;"),
    ("renormalisation flag inverted", "    if (renormalize) {", "    if (!renormalize) {"),
    ("weights not normalised by the top logit",
     "w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]] - top) / denom;",
     "w[(size_t)t * k + j] = exp((double)l[ids[(size_t)t * k + j]]) / denom;"),
    ("padding off by one", "int32_t padded = (counts[e] + BM - 1) / BM * BM;",
     "int32_t padded = (counts[e] + BM) / BM * BM;"),
    ("alignment order not stable", "    for (int64_t i = 0; i < n; ++i)\n      if (ids[i] == e)",
     "    for (int64_t i = n - 1; i >= 0; --i)\n      if (ids[i] == e)"),
    ("wrong sentinel", "for (int64_t p = 0; p < cap; ++p) sorted[p] = (int32_t)n;",
     "for (int64_t p = 0; p < cap; ++p) sorted[p] = -1;"),
    ("block map shifted", "block_expert[p / BM] = e;", "block_expert[p / BM] = e + 1;"),
    ("capacity ignores padding", "int64_t c = n + touched * (BM - 1);", "int64_t c = n + touched;"),
    ("silu sign flipped", "return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    ("gate reads the up rows", "g += xa[h] * weight(w_gu, sgu, wtype, (size_t)r, (size_t)h, (size_t)H);",
     "g += xa[h] * weight(w_gu, sgu, wtype, (size_t)(I + r), (size_t)h, (size_t)H);"),
    ("down operand transposed", "acc += hbuf[r] * weight(w_d, sd, wtype, (size_t)o, (size_t)r, (size_t)I);",
     "acc += hbuf[r] * weight(w_d, sd, wtype, (size_t)r, (size_t)o, (size_t)H);"),
    ("fp8 down scale dropped", "if (wtype == 1 || wtype == 2) acc *= (double)s_d[o];",
     "if (wtype == 1 || wtype == 2) acc *= 1.0;"),
    ("fp8 up scale from the gate row", "u *= (double)s_gu[I + r];", "u *= (double)s_gu[r];"),
    ("combine weight dropped", "acc[o] += wj * y[o];", "acc[o] += y[o];"),
    ("shared gate dropped", "acc[o] += gamma * y[o];", "acc[o] += y[o];"),
    ("shared gate sign", "static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }",
     "static double sigmoid(double z) { return 1.0 / (1.0 + exp(z)); }"),
    ("bf16 rounds toward zero", "double q = nearbyint(a / quantum); /* ties to even",
     "double q = floor(a / quantum); /* ties to even"),
    ("fp8 exponent bias", "else mag = ldexp(1.0 + (double)m / 8.0, E - 7);",
     "else mag = ldexp(1.0 + (double)m / 8.0, E - 8);"),
    ("fp8 subnormal scale", "if (E == 0) mag = ldexp((double)m / 8.0, -6);",
     "if (E == 0) mag = ldexp((double)m / 8.0, -7);"),
    ("fp8 encoder truncates", "int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);",
     "int m = (int)floor((ldexp(a, -e) - 1.0) * 8.0);"),
    ("fp8 encoder subnormal step", "nearbyint(a * 512.0)", "nearbyint(a * 256.0)"),
    ("fp8 encoder saturates low", "if (a >= 448.0) return", "if (a >= 416.0) return"),
    ("activation scale one binade high", "e = f <= 0.875 ? ex - 9 : ex - 8;", "e = f < 0.875 ? ex - 9 : ex - 8;"),
    ("activation scale threshold wrong", "e = f <= 0.875 ? ex - 9 : ex - 8;", "e = f <= 0.75 ? ex - 9 : ex - 8;"),
    ("token scale dropped from the gate sums", "      g *= sx;\n", "      g *= 1.0;\n"),
    ("h scale dropped", "if (wtype == 2) acc *= sh;", "if (wtype == 2) acc *= 1.0;"),
    ("token not quantised", "    for (int h = 0; h < H; ++h) xa[h] = oracle_fp8_value(q[h]);\n",
     "    for (int h = 0; h < H; ++h) xa[h] = xa[h] / sx;\n"),
    ("h not quantised", "    for (int r = 0; r < I; ++r) hbuf[r] = oracle_fp8_value(q[r]);\n",
     "    for (int r = 0; r < I; ++r) hbuf[r] = hbuf[r] / sh;\n"),
    ("fp4 nibble order swapped", "(col & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15)",
     "(col & 1) ? (uint8_t)(b & 15) : (uint8_t)(b >> 4)"),
    ("fp4 subnormal step", "double mag = E == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);",
     "double mag = E == 0 ? 1.0 * m : ldexp(1.0 + 0.5 * m, E - 1);"),
    ("e8m0 bias", "ldexp(1.0, (int)X - 127)", "ldexp(1.0, (int)X - 126)"),
    ("mxfp4 scale block of the wrong row", "((const uint8_t *)sc)[row * (cols / 32) + col / 32]",
     "((const uint8_t *)sc)[col / 32]"),
    ("h not rounded", "hbuf[r] = rounding ? oracle_bf16_rounded(a) : a;", "hbuf[r] = a;"),
    ("expert output not rounded", "y[o] = rounding ? oracle_bf16_rounded(acc) : acc;", "y[o] = acc;"),
]


def _run_mutant(mutant, workdir):
    name, old, new = mutant
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant '{name}': pattern must occur exactly once"
    tag = "".join(c if c.isalnum() else "_" for c in name)
    csrc = os.path.join(workdir, f"{tag}.c")
    lib = os.path.join(workdir, f"lib{tag}.so")
    with open(csrc, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", csrc, "-o", lib, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, MOE_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda m: _run_mutant(m, d), MUTANTS))
    survived = [name for name, rc in results if rc == 0]
    assert not survived, f"mutants not caught by the pins: {survived}"


def test_unmutated_copy_passes():
    with tempfile.TemporaryDirectory() as d:
        name, rc = _run_mutant(("identity", "static double silu", "static double silu"), d)
    assert rc == 0
