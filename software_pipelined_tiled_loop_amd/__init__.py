"""Software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libpgemm.so`` built from ``csrc/`` and
declared in ``include/pgemm.h``.  ``binding`` wraps its C ABI with ctypes
(argument marshalling only); importing it fails loudly when the library has
not been built.  ``inputs`` holds the seeded synthetic operand generators.

The binding is imported lazily so that ``inputs`` and the build helpers work on
machines without the compiled library.
"""
from __future__ import annotations

import importlib

__all__ = ["binding", "inputs", "build", "pgemm_gemm", "pgemm_gemm_ex", "pgemm_plan",
           "pgemm_strerror", "gemm"]


def __getattr__(name):
    if name in ("binding", "inputs", "build"):
        return importlib.import_module("." + name, __name__)
    if name in ("pgemm_gemm", "pgemm_gemm_ex", "pgemm_plan", "pgemm_strerror", "gemm",
                "pgemm_num_variants", "pgemm_variant_info", "PgemmError"):
        mod = importlib.import_module(".binding", __name__)
        return getattr(mod, name)
    raise AttributeError(name)
