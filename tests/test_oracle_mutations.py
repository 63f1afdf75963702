"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of oracle/swin_oracle.c (a
reversed shift or unshift, a flipped relative index, a dropped or wrong
scale, mask, bias, residual or epsilon, a transposed operand or index map, a
wrong rounding rule, a backward term from the wrong matrix, ...), builds
it with gcc, and runs tests/test_oracle.py against the mutant
(SWIN_ORACLE_LIB names the build): the pins must fail.  The mistakes are planted on the CPU only; the
oracle itself is untouched.  Each snippet must occur exactly once in the
oracle source, so a change of the oracle that moves a snippet fails here
loudly instead of testing nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "swin_oracle.c")

MUTATIONS = {
    "shift rolled the wrong way":
        ("oracle_roll(x, B, H, W, (int)C3, -s, -s, xr);",
         "oracle_roll(x, B, H, W, (int)C3, s, s, xr);"),
    "relative index key minus query":
        ("int dy = i / M - j / M, dx = i % M - j % M;",
         "int dy = j / M - i / M, dx = j % M - i % M;"),
    "score scale dropped":
        ("        double sc = dot * scale;\n", "        double sc = dot;\n"),
    "bias table read head-major":
        ("          sc += (double)J->table[(long)J->rel[i * N + j] * nh + h];",
         "          sc += (double)J->table[(long)h * (2 * M - 1) * (2 * M - 1) + J->rel[i * N + j]];"),
    "shift mask dropped in the forward":
        ("          if (mk) sc += mk[i * N + j];\n        }\n        S[i * Np + j] = sc;",
         "        }\n        S[i * Np + j] = sc;"),
    "mask value -10":
        ("? 0.0 : -100.0;", "? 0.0 : -10.0;"),
    "region band boundary off by one":
        ("  if (p < L - M) return 0;", "  if (p < L - M + 1) return 0;"),
    "weights transposed in the value product":
        ("for (int j = 0; j < Np; ++j) acc += P[i * Np + j] * v[j * d + e];",
         "for (int j = 0; j < Np; ++j) acc += P[j * Np + i] * v[j * d + e];"),
    "window tokens in column-major order":
        ("            long n = (b * nWy + wy) * nWx + wx, t = ty * M + tx;\n"
         "            const double* src = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;",
         "            long n = (b * nWy + wy) * nWx + wx, t = tx * M + ty;\n"
         "            const double* src = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;"),
    "linear bias dropped":
        ("      if (J->bias) acc += (double)J->bias[j];\n", ""),
    "layer norm variance over C + 1":
        ("    var /= C;\n", "    var /= C + 1;\n"),
    "int8 query scale used for the key":
        ("out[i] = (double)codes[i] * (double)scales[part];",
         "out[i] = (double)codes[i] * (double)scales[part == 1 ? 0 : part];"),
    "int8 rounding half away from zero":
        ("float q = nearbyintf(fmaf((float)a, scale, shift));",
         "float q = roundf(fmaf((float)a, scale, shift));"),
    "int8 codes clamped to -128":
        ("q < -127.0f ? -127.0f : q;", "q < -128.0f ? -128.0f : q;"),
    "backward dK without the scale":
        ("dx[(long)t * 3 * C + C + h * d + e] = ak * scale;",
         "dx[(long)t * 3 * C + C + h * d + e] = ak;"),
    "backward dS with the sign flipped":
        ("dP[i * N + j] = S[i * N + j] * (dP[i * N + j] - Dr[i]);",
         "dP[i * N + j] = S[i * N + j] * (Dr[i] - dP[i * N + j]);"),
    "unshift rolled the same way as the shift":
        ("oracle_roll(o, B, H, W, (int)C, s, s, out);", "oracle_roll(o, B, H, W, (int)C, -s, -s, out);"),
    "window reverse in column-major order":
        ("            long n = (b * nWy + wy) * nWx + wx, t = ty * M + tx;\n"
         "            double* dst = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;",
         "            long n = (b * nWy + wy) * nWx + wx, t = tx * M + ty;\n"
         "            double* dst = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;"),
    "score scale 1/d instead of 1/sqrt(d)":
        ("  const double scale = 1.0 / sqrt((double)d);\n  const double* base",
         "  const double scale = 1.0 / (double)d;\n  const double* base"),
    "padded keys scored 0 instead of -inf":
        ("          S[i * Np + j] = -INFINITY;", "          S[i * Np + j] = 0.0;"),
    "region label axes swapped":
        ("3 * band(y, H, M, s) + band(x, W, M, s)", "3 * band(x, W, M, s) + band(y, H, M, s)"),
    "linear residual dropped":
        ("      if (J->r) acc += load_elem(J->r, J->rdtype, t * J->N + j);\n", ""),
    "layer norm without eps":
        ("    const double r = 1.0 / sqrt(var + eps);", "    const double r = 1.0 / sqrt(var);"),
    "layer norm without beta":
        (" * (double)gamma[c] + (double)beta[c];", " * (double)gamma[c];"),
    "backward dV from P untransposed":
        ("            av += S[u * N + t] * G_(u, e);", "            av += S[t * N + u] * G_(u, e);"),
    "backward D without P":
        ("          Di += S[i * N + j] * acc;", "          Di += acc;"),
    "backward dQ without the scale":
        ("          dx[(long)t * 3 * C + h * d + e] = aq * scale;",
         "          dx[(long)t * 3 * C + h * d + e] = aq;"),
    "backward bias gradient from P instead of dS":
        ("          J->dtable[(long)J->rel[i * N + j] * nh + h] += dP[i * N + j];",
         "          J->dtable[(long)J->rel[i * N + j] * nh + h] += S[i * N + j];"),
    "int8 linear bias not divided by the output scale":
        ("const float shift = (J->bias ? J->bias[j] : 0.0f) / J->so[j];",
         "const float shift = (J->bias ? J->bias[j] : 0.0f);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"snippet of '{name}' not found exactly once in the oracle"
    mutant = tmp_path / "swin_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libswinoracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-I", os.path.join(ROOT, "oracle"),
                    "-o", str(lib), str(mutant), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, SWIN_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-1500:]
    assert res.returncode == 1 and " failed" in res.stdout, f"'{name}' was not caught:\n{tail}"
