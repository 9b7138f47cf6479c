"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c, plants one plausible mistake (a dropped term, a
wrong sign, an ignored stride, a transposed operand, reduced precision, ...),
compiles the copy with gcc and runs the pins of tests/oracle_pins.py against it
in a child process. The case passes when at least one pin fails (or the child
crashes). The mistakes are planted in the oracle, on the CPU; nothing here runs
on a GPU.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (name, text in oracle.c, replacement). Each text must occur exactly once.
MUTANTS = [
    ("gemm_drops_last_k", "for (int64_t k = 0; k < jb->K; ++k)",
     "for (int64_t k = 0; k < jb->K - 1; ++k)"),
    ("gemm_skips_first_k", "for (int64_t k = 0; k < jb->K; ++k)",
     "for (int64_t k = 1; k < jb->K; ++k)"),
    ("gemm_subtracts", "c[j] += p;", "c[j] -= p;"),
    ("gemm_transposed_b", "const double p = a * (double)brow[j];",
     "const double p = a * (double)jb->B[(j % jb->K) * jb->ldb + (k % jb->N)];"),
    ("gemm_ignores_lda", "jb->A[i * jb->lda + k]", "jb->A[i * jb->K + k]"),
    ("gemm_ignores_ldb", "jb->B + k * jb->ldb", "jb->B + k * jb->N"),
    ("gemm_fp32_products", "const double p = a * (double)brow[j];",
     "const double p = (float)(a * (double)brow[j]);"),
    ("gemm_magnitude_without_abs", "if (s) s[j] += fabs(p);", "if (s) s[j] += p;"),
    ("gemm_no_zero_init", "c[j] = 0.0;", "(void)c;"),
    ("gemm_drops_last_column",
     "for (int64_t j = 0; j < jb->N; ++j) {\n                const double p",
     "for (int64_t j = 0; j < jb->N - 1; ++j) {\n                const double p"),
    ("gemm_ignores_row_list", "const int64_t i = jb->rows ? jb->rows[r] : r;",
     "const int64_t i = r;"),
    ("gemm_thread_split_skips_rows",
     "nrows * t / threads, nrows * (t + 1) / threads};",
     "nrows * t / threads + (t > 0), nrows * (t + 1) / threads};"),
    ("gemv_fp32_accumulator", "double acc = 0.0, mag = 0.0;", "float acc = 0.0f; double mag = 0.0;"),
    ("gemv_drops_last_j",
     "for (int64_t j = 0; j < jb->N; ++j) {\n            const double p = (double)arow[j]",
     "for (int64_t j = 0; j < jb->N - 1; ++j) {\n            const double p = (double)arow[j]"),
    ("gemv_reversed_x", "(double)jb->x[j];", "(double)jb->x[jb->N - 1 - j];"),
    ("gemv_row_stride_n", "const float *arow = jb->A + i * jb->lda;",
     "const float *arow = jb->A + i * jb->N;"),
    ("gemv_subtracts", "acc += p;", "acc -= p;"),
    ("conv_no_low_padding_check", "const int inside = h >= 0 && h < jb->H && v >= 0 && v < jb->W;",
     "const int inside = h >= 0 && h < jb->H && v < jb->W;"),
    ("conv_skips_padded_taps",
     "const double xv = inside ? (double)xn[(c * jb->H + h) * jb->W + v] : 0.0;",
     "if (!inside) continue;\n                            const double xv = (double)xn[(c * jb->H + h) * jb->W + v];"),
    ("conv_ignores_stride", "const int64_t h = p * jb->sh + r * jb->dh - jb->ph;",
     "const int64_t h = p + r * jb->dh - jb->ph;"),
    ("conv_ignores_dilation", "const int64_t v = q * jb->sw + s * jb->dw - jb->pw;",
     "const int64_t v = q * jb->sw + s - jb->pw;"),
    ("conv_swaps_filter_axes", "(double)wk[(c * jb->R + r) * jb->S + s];",
     "(double)wk[(c * jb->S + s) * jb->R + r];"),
    ("conv_fp32_accumulator", "double acc = 0.0; /* the output, in fp64 */", "float acc = 0.0f;"),
    ("conv_drops_last_channel", "for (int64_t c = 0; c < jb->C; ++c)\n                    for (int64_t r",
     "for (int64_t c = 0; c < jb->C - 1; ++c)\n                    for (int64_t r"),
]

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
failed = []
for pin in oracle_pins.CHEAP_PINS:
    try:
        pin(orc)
    except Exception as e:  # AssertionError, or an error from a broken library
        failed.append(pin.__name__)
print("caught by:", ", ".join(failed) if failed else "NOTHING")
sys.exit(0 if failed else 3)
"""


def test_mutation_texts_are_unique():
    src = open(oracle_build.SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"{name}: planted text occurs {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1
    mutant_src = tmp_path / f"oracle_{name}.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle_build.build(src=str(mutant_src), out=str(tmp_path / f"lib{name}.so"))
    child = CHILD.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=300)
    assert r.returncode != 3, f"planted mistake {name} passed every pin:\n{r.stdout}{r.stderr}"
