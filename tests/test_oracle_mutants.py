"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible slip in a private copy of oracle.c (a dropped
term, a wrong sign, constant, rounding, index, bit order or code), builds it
into a temporary library, and runs the pin suite against it in a child
process.  The pin suite must fail for every mutant: a pin set that let one of
them through would not be pinning the oracle.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")
sys.path.insert(0, ROOT)
from oracle.build import CFLAGS  # noqa: E402

# (name, original text, replacement) -- each original must occur in oracle.c
MUTANTS = [
    ("gamma_drops_abs", "v[i] = fabs((double)W[i]);", "v[i] = ((double)W[i]);"),
    ("gamma_pairwise_drops_left", "v[i] += v[i + h];", "v[i] = v[i + h];"),
    ("gamma_skips_last_term", "v[i] = fabs((double)W[i]);",
     "v[i] = i + 1 < n ? fabs((double)W[i]) : 0.0;"),
    ("gamma_sequential_sum", "const double total = v[0];",
     "double total = 0.0;\n    for (int64_t i = 0; i < n; ++i) total += fabs((double)W[i]);"),
    ("gamma_rows_first",
     "    for (int64_t h = 1; h < n; h *= 2) {\n#pragma omp parallel for schedule(static)\n"
     "        for (int64_t i = 0; i < n - h; i += 2 * h)\n            v[i] += v[i + h];\n    }\n",
     "    for (int64_t r = 0; r < N; ++r)\n        for (int64_t h = 1; h < K; h *= 2)\n"
     "            for (int64_t i = 0; i < K - h; i += 2 * h)\n"
     "                v[r * K + i] += v[r * K + i + h];\n"
     "    for (int64_t h = 1; h < N; h *= 2)\n        for (int64_t i = 0; i < N - h; i += 2 * h)\n"
     "            v[i * K] += v[(i + h) * K];\n"),
    ("gamma_wrong_n", "total / (double)n", "total / (double)(n + 1)"),
    ("round_ties_away", "Wq[i] = (int8_t)nearbyint(t);", "Wq[i] = (int8_t)round(t);"),
    ("no_clamp", "if (t > 1.0) t = 1.0;", ""),
    ("code_minus_one", "if (q == -1) return 2;", "if (q == -1) return 3;"),
    ("bit_order_msb_first", "<< (2 * j));", "<< (2 * (3 - j)));"),
    ("decode_swapped", "if (code == 1) return 1;\n    if (code == 2) return -1;",
     "if (code == 2) return 1;\n    if (code == 1) return -1;"),
    ("t5_floor_encoding", "(256 * v + 242) / 243", "(256 * v) / 243"),
    ("t5_pad_digit_zero", "k < K ? Wq[n * K + k] + 1 : 1;", "k < K ? Wq[n * K + k] + 1 : 0;"),
    ("t5_digit_order_reversed", "pow3[4 - (int)(k % 5)]", "pow3[(int)(k % 5)]"),
    ("t5_decode_rounds_up", "(243 * q) / 256", "(243 * q + 255) / 256"),
    ("t5_rows_unpadded", "((K + 4) / 5 + 15) / 16 * 16", "(K + 4) / 5"),
    ("bf16_shift", "(uint32_t)src[i] << 16;", "(uint32_t)src[i] << 15;"),
    ("act_128", "float s = 127.0f / a;", "float s = 128.0f / a;"),
    ("act_trunc", "float r = nearbyintf(p);", "float r = truncf(p);"),
    ("act_scale_inverted", "d[m] = a / 127.0f;", "d[m] = 127.0f / a;"),
    ("act_absmax_no_abs", "float ax = fabsf(x[k]);", "float ax = x[k];"),
    ("acc_sub_as_add", "c -= Xq[m * K + k];", "c += Xq[m * K + k];"),
    ("acc_wrong_index", "c += Xq[m * K + k];", "c += Xq[m * K + (k ^ 1)];"),
    ("dequant_wrong_row_scale", "* (double)gamma * (double)d[m];", "* (double)gamma * (double)d[0];"),
    ("ffn_drops_gate", "float h = Wu ? r2 * U[m * F + f] : r2;", "float h = r2;"),
    ("ffn_relu_is_abs", "float r = G[m * F + f] > 0.0f ? G[m * F + f] : 0.0f;",
     "float r = fabsf(G[m * F + f]);"),
    ("ffn_rms_multiplies", "(double)dh[m] / rms[m] : 0.0;", "(double)dh[m] * rms[m] : 0.0;"),
    ("ffn_rms_no_mean", "sqrt(ss / (double)F + (double)eps)", "sqrt(ss + (double)eps)"),
    ("ffn_gain_dropped", "float z = norm_w ? h * norm_w[f] : h;", "float z = h;"),
    ("ffn_y32_scale_order", "float c = gamma_d * dz32;", "float c = gamma_d * (float)dh[m];"),
    ("act4_8_levels", "float s = 7.0f / a;", "float s = 8.0f / a;"),
    ("act4_clamp_6", "if (r > 7.0f) r = 7.0f;", "if (r > 6.0f) r = 6.0f;"),
    ("act4_scale_wrong", "d[m] = a / 7.0f;", "d[m] = a / 8.0f;"),
    ("act4_trunc", "            float r = nearbyintf(p);\n            if (r > 7.0f)",
     "            float r = truncf(p);\n            if (r > 7.0f)"),
    ("act4_nibble_order", "P[m * (K / 2) + b] = (uint8_t)(lo | (hi << 4));",
     "P[m * (K / 2) + b] = (uint8_t)(hi | (lo << 4));"),
    ("act4_unsigned_nibble", "return (int8_t)(v < 8 ? v : (int)v - 16);", "return (int8_t)v;"),
]


def _run_mutant(name, old, new, src_text, tmpdir):
    assert src_text.count(old) >= 1, f"{name}: pattern not found"
    mut_c = os.path.join(tmpdir, f"{name}.c")
    mut_so = os.path.join(tmpdir, f"{name}.so")
    with open(mut_c, "w") as f:
        f.write(src_text.replace(old, new, 1))
    flags = [f for f in CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, mut_c, "-o", mut_so, "-lm"], check=True,
                   capture_output=True)
    env = dict(os.environ, BITLINEAR_ORACLE_LIB=mut_so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py"),
                        os.path.join(HERE, "test_oracle_stack.py"),
                        os.path.join(HERE, "test_oracle_a4.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_mutant_is_caught():
    with open(SRC) as f:
        src_text = f.read()
    with tempfile.TemporaryDirectory() as tmpdir:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_mutant(*m, src_text, tmpdir), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"
    broken = [(n, rc) for n, rc, _ in results if rc not in (1,)]
    assert not broken, f"mutant runs ended abnormally (not a test failure): {broken}"
