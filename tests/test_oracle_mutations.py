"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of ``oracle/bq8_oracle.c`` (on the
CPU, in a temporary directory), points a child pytest at that copy and runs
the oracle pin tests that should notice it.  The case passes only if the
child run FAILS: a pin that still passes with the mistake in place would not
be pinning anything.  The real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bq8_oracle.c")

# name: (original text, planted mistake, pin files expected to catch it)
MUTATIONS = {
    "q4_0_drops_minus8": (
        "int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);\n"
        "                    double wv = dw * (double)(nib - 8);",
        "int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);\n"
        "                    double wv = dw * (double)(nib);",
        ["test_oracle_q4_0.py"]),
    "q4_0_nibbles_swapped": (
        "int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);\n"
        "                    double wv = dw * (double)(nib - 8);",
        "int nib = (j < 16) ? (wb[2 + j] >> 4) : (wb[2 + j - 16] & 0x0F);\n"
        "                    double wv = dw * (double)(nib - 8);",
        ["test_oracle_q4_0.py"]),
    "q8_1_rounds_half_even": (
        "double a = floor(fabs((double)t) + 0.5); /* exact in binary64 */",
        "double a = nearbyint(fabs((double)t));",
        ["test_oracle_q8_1.py"]),
    "q8_1_divides_by_128": (
        "float d = amax / 127.0f;",
        "float d = amax / 128.0f;",
        ["test_oracle_q8_1.py"]),
    "q8_1_s_without_d": (
        "float s = d * (float)sum;",
        "float s = (float)sum;",
        ["test_oracle_q8_1.py"]),
    "q6k_qh_bits_reversed": (
        "int hi = (qh[32 * h + l] >> (2 * c)) & 3;",
        "int hi = (qh[32 * h + l] >> (2 * (3 - c))) & 3;",
        ["test_oracle_q6k.py"]),
    "q6k_subscale_index_per_32": (
        "double wv = dw * (double)SC[pack_sc_at(n, k / 16, N, K)] *",
        "double wv = dw * (double)SC[pack_sc_at(n, k / 32, N, K)] *",
        ["test_oracle_q6k.py"]),
    "q6k_compact_qh_piece_stride": (
        "return N * (K / 2) + n0 * (K / 4) + ((4 * s + i / 16) * rows_t + r) * 16 + i % 16;",
        "return N * (K / 2) + n0 * (K / 4) + ((4 * s + i / 16) * rows_t + r) * 16 + (i * 5) % 16;",
        ["test_oracle_q6k_compact.py"]),
    "q6k_compact_ql_tile_base": (
        "return n0 * (K / 2) + ((8 * s + i / 16) * rows_t + r) * 16 + i % 16;",
        "return n0 * (K / 2) + ((8 * s + i / 16) + r * 8 * (K / QK_K)) * 16 + i % 16;",
        ["test_oracle_q6k_compact.py"]),
    "q4_0_packed_nibble_choice": (
        "*hi = (jj >= 8);",
        "*hi = (jj % 2);",
        ["test_oracle_q4_0_packed.py"]),
    "q4_0_packed_scale_parity": (
        "return n0 * nb + ((b / 16) * 2 + b % 2) * rows_t * 8 + r * 8 + (b % 16) / 2;",
        "return n0 * nb + ((b / 16) * 2 + (b / 2) % 2) * rows_t * 8 + r * 8 + (b % 16) / 2;",
        ["test_oracle_q4_0_packed.py"]),
    "pack_tile_row_major": (
        "return n0 * K + ((k / 16) * rows_t + r) * 16 + k % 16;",
        "return n0 * K + r * K + k;",
        ["test_oracle_q6k.py"]),
    "top1_last_of_ties": (
        "if (best < 0 || v > bv) {",
        "if (best < 0 || v >= bv) {",
        ["test_oracle_top1.py"]),
    "rms_mean_over_k_minus_1": (
        "double inv = 1.0 / sqrt(ss / (double)K + eps);",
        "double inv = 1.0 / sqrt(ss / (double)(K - 1) + eps);",
        ["test_oracle_stages.py"]),
    "q8_1_amax_signed": (
        "float a = fabsf(xb[j]);",
        "float a = xb[j];",
        ["test_oracle_q8_1.py"]),
    "q4_0_dot_drops_dx": (
        "int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);\n"
        "                    double wv = dw * (double)(nib - 8);\n"
        "                    double xv = dx * (double)(int8_t)xb[4 + j];",
        "int nib = (j < 16) ? (wb[2 + j] & 0x0F) : (wb[2 + j - 16] >> 4);\n"
        "                    double wv = dw * (double)(nib - 8);\n"
        "                    double xv = (double)(int8_t)xb[4 + j];",
        ["test_oracle_q4_0.py"]),
    "silu_sign": (
        "h[i] = gv / (1.0 + exp(-gv)) * (double)u[i];",
        "h[i] = gv / (1.0 + exp(gv)) * (double)u[i];",
        ["test_oracle_stages.py"]),
    "q6k_compact_subscale_pairs_swapped": (
        "return N * (K / 2) + N * (K / 4) + pack_sc_at(n, 16 * s + i, N, K);",
        "return N * (K / 2) + N * (K / 4) + pack_sc_at(n, 16 * s + (i ^ 1), N, K);",
        ["test_oracle_q6k_compact.py"]),
    "q6k_compact_scale_superblocks_swapped": (
        "return N * (K / 2) + N * (K / 4) + N * (K / 16) + 2 * pack_d_at(n, s, N, K);",
        "return N * (K / 2) + N * (K / 4) + N * (K / 16) + 2 * pack_d_at(n, s ^ 1, N, K);",
        ["test_oracle_q6k_compact.py"]),
    "f16_truncates": (
        "double m = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */",
        "double m = floor(ldexp(a, 10 - e));",
        ["test_oracle_fp16.py"]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    original, planted, files = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(original) == 1, f"{name}: the oracle text to mutate is gone or ambiguous"
    mut = tmp_path / "oracle"
    mut.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), mut / "__init__.py")
    (mut / "bq8_oracle.c").write_text(src.replace(original, planted))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in files]]
    r = subprocess.run(cmd, env=env, cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=300)
    tail = "\n".join(r.stdout.strip().splitlines()[-3:])
    # The child must have loaded the planted copy, and a pin must have failed.
    assert (mut / "libbq8_oracle.so").exists(), f"{name}: child did not build the copy\n{tail}"
    assert r.returncode == 1, f"{name}: pins did not catch the planted mistake\n{tail}"


def test_unmodified_copy_passes(tmp_path):
    """Control: the same harness on an unmodified copy passes every pin file,
    so the failures above come from the planted mistakes."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    mut = tmp_path / "oracle"
    mut.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), mut / "__init__.py")
    shutil.copy(SRC, mut / "bq8_oracle.c")
    files = sorted({f for _, _, fs in MUTATIONS.values() for f in fs})
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in files]]
    r = subprocess.run(cmd, env=env, cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=300)
    assert (mut / "libbq8_oracle.so").exists()
    assert r.returncode == 0, "\n".join(r.stdout.strip().splitlines()[-5:])
