"""Seeded synthetic operands shared by the tests, the benchmark and the oracle.

This module only draws random numbers and lays them out in memory; it holds no
GEMM arithmetic, so both the HIP library and the oracle can be fed from it
without sharing any of the method's code.

Distributions follow the measured workloads of the pages (square 4096^3 GEMMs
on synthetic data; page "Double Buffering: Software Pipelining the K-Loop",
section "Mechanics", and page "GPU-Kernel pipelinen", step 2) and the five
benchmark configurations of this library:

  fp32    A, B (and C0 when beta != 0) i.i.d. uniform[-1, 1)  (2*U[0,1) - 1)
  fp16/bf16 A, B i.i.d. normal(0, 1) rounded to the dtype (round-to-nearest-even)
  int8    A, B i.i.d. uniform over the integers [-128, 127]

The hazard demonstrator (page "Software pipelines and asynchronous copies",
section "Practice": randomized input to a copy-and-reduce over a 4096 x 4096
array) takes int32 i.i.d. uniform over [-32768, 32767], with any padding
columns set to POISON_I32 so that a read past the columns is caught.

When beta == 0, C is pre-filled with a poison value (NaN for float, 0x7F7F7F7F
for int32) so a kernel that reads C when it must not is caught.

Every generator is a CPU ``torch.Generator`` seeded explicitly; seeds are
``1000 + 10*family + variant`` with the family of each workload in
``SEED_FAMILY``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = ("f32", "f16", "bf16", "i8")
TORCH_IN = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}
TORCH_OUT = {"f32": torch.float32, "f16": torch.float32, "bf16": torch.float32, "i8": torch.int32}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}
POISON_I32 = 0x7F7F7F7F


# Seed family of each workload: its seeds are 1000 + 10 * family + variant.
SEED_FAMILY = {"fp32_256": 0, "fp32_4096": 1, "int8_4096": 2, "half_4096": 3, "bf16_k_sweep": 4, "hazard": 7}


def seed_for(workload: str, variant: int = 0) -> int:
    return 1000 + 10 * SEED_FAMILY[workload] + variant


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw(dtype: str, rows: int, cols: int, seed: int, dist: str | None = None) -> torch.Tensor:
    """A rows x cols CPU tensor of input dtype ``dtype``."""
    g = _gen(seed)
    if dist is None:
        dist = {"f32": "uniform", "f16": "normal", "bf16": "normal", "i8": "int8"}[dtype]
    if dist == "uniform":
        t = torch.rand((rows, cols), generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        t = torch.randn((rows, cols), generator=g, dtype=torch.float32)
    elif dist == "int8":
        return torch.randint(-128, 128, (rows, cols), generator=g, dtype=torch.int8)
    elif dist == "smallint":  # small integers: every product and sum exact in fp32
        t = torch.randint(-4, 5, (rows, cols), generator=g).to(torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    if dtype == "i8":
        return t.round().clamp(-128, 127).to(torch.int8)
    return t.to(TORCH_IN[dtype])


@dataclass
class Operands:
    dtype: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    alpha: float
    beta: float
    A: torch.Tensor            # M x lda (CPU)
    B: torch.Tensor            # K x ldb (CPU)
    C: torch.Tensor            # M x ldc (CPU): C0 when beta != 0, poison otherwise
    seeds: dict = field(default_factory=dict)

    def numpy_views(self):
        """Raw numpy views for the oracle (16-bit types as uint16 bit patterns)."""
        def raw(t):
            if t.dtype in (torch.float16, torch.bfloat16):
                return t.contiguous().view(torch.int16).numpy().view(np.uint16)
            return t.contiguous().numpy()
        return raw(self.A), raw(self.B), raw(self.C)


def make_operands(dtype: str, M: int, N: int, K: int, seed: int, alpha=1.0, beta=0.0,
                  lda=None, ldb=None, ldc=None, dist=None, c_dist=None) -> Operands:
    """Seeded operands with optional padded leading dimensions.

    Padding columns (k >= K in A, n >= N in B and C) are filled with NaN
    (float) or 0x7F (int8) so that any read of them shows up in the result.
    """
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    sa, sb, sc = seed, seed + 1, seed + 2
    A = torch.empty((max(M, 1), max(lda, 1)), dtype=TORCH_IN[dtype])[:M]
    B = torch.empty((max(K, 1), max(ldb, 1)), dtype=TORCH_IN[dtype])[:K]
    pad_in = 0x7F if dtype == "i8" else float("nan")
    A.fill_(pad_in)
    B.fill_(pad_in)
    if M and K:
        A[:, :K] = draw(dtype, M, K, sa, dist)
    if K and N:
        B[:, :N] = draw(dtype, K, N, sb, dist)
    out_t = TORCH_OUT[dtype]
    C = torch.empty((max(M, 1), max(ldc, 1)), dtype=out_t)[:M]
    if dtype == "i8":
        C.fill_(POISON_I32)
    else:
        C.fill_(float("nan"))
    if beta != 0 and M and N:
        if dtype == "i8":
            C[:, :N] = torch.randint(-1000, 1001, (M, N), generator=_gen(sc), dtype=torch.int32)
        else:
            C[:, :N] = draw("f32", M, N, sc, c_dist or "uniform")
    return Operands(dtype, M, N, K, lda, ldb, ldc, alpha, beta, A.contiguous() if M else A,
                    B.contiguous() if K else B, C.contiguous() if M else C,
                    seeds={"A": sa, "B": sb, "C": sc})


# The five benchmark configurations (sizes and value distributions).
RAGGED = dict(dtype="bf16", M=4000, N=3968, K=4001, lda=4001, ldb=3968, ldc=3968)


def make_hazard_input(rows: int, cols: int, seed: int, ldx: int | None = None) -> torch.Tensor:
    """A rows x ldx int32 CPU tensor: columns < cols uniform over [-32768, 32767], the rest POISON_I32."""
    ldx = cols if ldx is None else ldx
    X = torch.full((rows, ldx), POISON_I32, dtype=torch.int32)
    X[:, :cols] = torch.randint(-32768, 32768, (rows, cols), generator=_gen(seed), dtype=torch.int32)
    return X
