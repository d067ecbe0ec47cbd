"""Host emulation of the kernel's LDS data path for every compiled tile class.

tests/layout_emulator.cpp includes the kernel header and runs its own index
functions on the CPU: producer placement into an LDS stage (each byte written
exactly once), the fragment reads with the probed lane semantics of
ds_read_b128 / ds_read_b64_tr_b16 / ds_read_b64_tr_b8 / ds_read_b32 (every read
inside its region), and the MFMA lane layouts, compared with a naive GEMM of
the tile.  It also checks by brute force the generic producer's choice of
whole 16-byte loads (every admitted read inside its matrix, none of A past K),
the DIRECT producer's K tail (LDS-DMA of whole chunks plus the element-wise
patch gives the zero-padded tile)
and the hazard demonstrator's indexing (every read, LDS, row-sum and timeline
index inside its buffer; each stage chunk produced and consumed exactly once).
No GPU is used; hipcc only compiles host code here.
"""
import os
import re
import shutil
import subprocess

import pytest

from software_pipelined_tiled_loop_amd import binding as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "layout_emulator.cpp")
DT = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}


def test_emulated_data_path_matches_naive_gemm(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "lemu")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-Wno-inline-asm", "--offload-arch=gfx950", "-x", "hip", SRC,
                    "-o", exe], check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=600).stdout
    assert out.strip().splitlines()[-1].startswith("OK"), out[-2000:]
    assert re.search(r"^chunk_fits \d+ cases$", out, re.M), out[-2000:]
    assert re.search(r"^work_split \d+ cases$", out, re.M), out[-2000:]
    assert re.search(r"^whole_loads \d+ cases$", out, re.M), out[-2000:]
    assert re.search(r"^dma_tail \d+ cases$", out, re.M), out[-2000:]
    assert re.search(r"^hazard \d+ cases$", out, re.M), out[-2000:]
    emulated = set(tuple(int(x) for x in m) for m in re.findall(r"^class (\d+) (\d+) (\d+) (\d+) (\d+) (\d+)$", out, re.M))
    # every tile class the library compiles is emulated
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        key = (DT[v["dtype"]], v["tile_m"], v["tile_n"], v["tile_k"], v["waves_m"], v["waves_n"])
        assert key in emulated, "tile class %s not emulated" % (key,)
