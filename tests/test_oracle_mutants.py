"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c to a temporary directory, plants one plausible
mistake (transposed operand, dropped beta term, wrong sign, a dropped last k
step -- the "forgotten epilogue tile" of page "GPU-Kernel pipelinen", common
pitfalls -- a wrong fp16 exponent bias, a wrong bf16 shift, an unsigned int8
read), builds it with gcc and runs a battery of the same kinds of pins used in
test_oracle_pins.py.  The unmodified source must pass the battery and every
mutant must fail it.  The oracle's row sums (Python) get the same treatment.
Nothing here touches a GPU.
"""
import itertools
import os
import random
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "transposed_B": ("load_elem(B, k * ldb + j, kind)", "load_elem(B, j * ldb + k, kind)"),
    "dropped_beta": ("if (beta != 0.0) v += beta * (double)C0[i * ldc + j];", ";"),
    "wrong_sign": ("acc[j] += a * load_elem(B, k * ldb + j, kind);", "acc[j] -= a * load_elem(B, k * ldb + j, kind);"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; ++k) {\n            double a", "for (int64_t k = 0; k + 1 < K; ++k) {\n            double a"),
    "f16_bias": ("v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    "bf16_shift": ("uint32_t u = ((uint32_t)h) << 16;", "uint32_t u = ((uint32_t)h) << 15;"),
    "int8_unsigned": ("const int64_t a = (int64_t)A[i * lda + k];",
                      "const int64_t a = (int64_t)(uint8_t)A[i * lda + k];"),
}


def _build(tmp_path, name, patch):
    text = open(SRC).read()
    if patch is not None:
        old, new = patch
        assert text.count(old) == 1, "mutation anchor not found exactly once: %s" % name
        text = text.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    src = d / "oracle.c"
    src.write_text(text)
    so = d / "liboracle.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    str(src), "-o", str(so), "-lm"], check=True)
    return oracle._bind(str(so))


def _enc(dtype, vals):
    vals = np.asarray(vals, np.float64)
    if dtype == "f32":
        return vals.astype(np.float32)
    if dtype == "f16":
        return vals.astype(np.float16).view(np.uint16)
    return torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def battery(lib):
    """True when every pin holds for this compiled oracle.  Shapes keep N <= K so that a
    transposed-B mutant still reads inside its arrays."""
    rng = random.Random(5)
    # exact brute force, float kinds
    for dtype in ("f32", "f16", "bf16"):
        for M, N, K in [(1, 1, 1), (2, 2, 3), (3, 2, 4), (4, 3, 3), (3, 3, 5)]:
            Av = [[rng.randint(-32, 32) / 8 for _ in range(K)] for _ in range(M)]
            Bv = [[rng.randint(-32, 32) / 8 for _ in range(N)] for _ in range(K)]
            C0v = [[rng.randint(-64, 64) / 16 for _ in range(N)] for _ in range(M)]
            got = oracle.gemm(dtype, M, N, K, 1.0, _enc(dtype, Av), _enc(dtype, Bv), -0.5,
                              np.array(C0v, np.float32), lib=lib)
            for i, j in itertools.product(range(M), range(N)):
                ref = sum(Fraction(Av[i][k]) * Fraction(Bv[k][j]) for k in range(K)) - Fraction(C0v[i][j]) / 2
                if Fraction(float(got[i, j])) != ref:
                    return False
    # int8 brute force
    for M, N, K in [(2, 2, 3), (3, 1, 5)]:
        Av = [[rng.randint(-128, 127) for _ in range(K)] for _ in range(M)]
        Bv = [[rng.randint(-128, 127) for _ in range(N)] for _ in range(K)]
        got = oracle.gemm("i8", M, N, K, 1, np.array(Av, np.int8), np.array(Bv, np.int8), lib=lib)
        for i, j in itertools.product(range(M), range(N)):
            if int(got[i, j]) != sum(Av[i][k] * Bv[k][j] for k in range(K)):
                return False
    # decoders (sampled patterns)
    for b in list(range(0, 65536, 257)) + [0x0001, 0x03FF, 0x3C00, 0x7BFF, 0x8001]:
        ref = np.array([b], np.uint16).view(np.float16).astype(np.float64)[0]
        got = lib.oracle_decode_f16(b)
        if not (np.isnan(ref) and np.isnan(got)) and ref != got:
            return False
        refb = torch.tensor([b], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).item()
        gotb = lib.oracle_decode_bf16(b)
        if not (np.isnan(refb) and np.isnan(gotb)) and refb != gotb:
            return False
    return True


def test_unmodified_oracle_passes_battery(tmp_path):
    assert battery(_build(tmp_path, "original", None))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    assert not battery(_build(tmp_path, name, MUTANTS[name])), "pins missed mutant %s" % name


# ---------------------------------------------------------------- row sums
# Planted mistakes in oracle.row_sums (the hazard demonstrator's reduction):
# a dropped last column, padding summed in, saturation in place of the int32
# wrap, the row stride taken from cols instead of ldx.
ROW_SUM_MUTANTS = {
    "drop_last_column": ("flat[r * ldx:r * ldx + cols]", "flat[r * ldx:r * ldx + cols - 1]"),
    "padding_summed": ("flat[r * ldx:r * ldx + cols]", "flat[r * ldx:r * ldx + ldx]"),
    "saturating": ("out[r] = (s + 2 ** 31) % 2 ** 32 - 2 ** 31", "out[r] = max(min(s, 2 ** 31 - 1), -2 ** 31)"),
    "stride_from_cols": ("flat[r * ldx:r * ldx + cols]", "flat[r * cols:r * cols + cols]"),
}


def _row_sums_from(patch):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "__init__.py")).read()
    if patch is not None:
        old, new = patch
        assert src.count(old) == 1, "mutation anchor not found exactly once: %s" % (old,)
        src = src.replace(old, new)
    ns = {"__name__": "oracle_mutant", "__file__": oracle.__file__}
    exec(compile(src, "oracle_mutant", "exec"), ns)
    return ns["row_sums"]


def row_sum_battery(row_sums):
    """The same kinds of pins as test_oracle_pins.py: closed forms, unbounded
    integers modulo 2^32 with padding, and the wrap of two int32 maxima."""
    rows, cols = 5, 40
    X = (np.arange(rows, dtype=np.int64)[:, None] * cols + np.arange(cols)).astype(np.int32)
    if row_sums(X, rows, cols).tolist() != [r * cols * cols + cols * (cols - 1) // 2 for r in range(rows)]:
        return False
    rng = random.Random(3)
    for rows, cols, ldx in [(3, 5, 5), (4, 9, 13), (2, 64, 70)]:
        vals = [[rng.randint(-2 ** 31, 2 ** 31 - 1) for _ in range(ldx)] for _ in range(rows)]
        got = row_sums(np.array(vals, np.int64).astype(np.int32), rows, cols, ldx)
        for r in range(rows):
            if int(got[r]) != (sum(vals[r][:cols]) + 2 ** 31) % 2 ** 32 - 2 ** 31:
                return False
    return row_sums(np.array([[2 ** 31 - 1, 2 ** 31 - 1, 7]], np.int32), 1, 2, 3).tolist() == [-2]


def test_unmodified_row_sums_pass_battery():
    assert row_sum_battery(_row_sums_from(None))


@pytest.mark.parametrize("name", sorted(ROW_SUM_MUTANTS))
def test_planted_row_sum_mistake_is_caught(name):
    assert not row_sum_battery(_row_sums_from(ROW_SUM_MUTANTS[name])), "pins missed mutant %s" % name
