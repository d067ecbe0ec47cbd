"""ctypes binding of the C ABI in include/pgemm.h (argument marshalling only).

Every entry point keeps its C name and argument order.  Pointer arguments
accept either an integer device address or a torch tensor (its data_ptr());
``stream`` accepts an integer hipStream_t, a torch stream, or None for torch's
current stream on the current device.  The functions return the C status code;
``gemm`` is a convenience wrapper that raises PgemmError on a nonzero status.

Importing this module loads libpgemm.so and raises ImportError when the HIP
library has not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libpgemm.so is not built (run __graft_entry__.build() or "
                      "python -m software_pipelined_tiled_loop_amd.build); there is no fallback")

# torch ships its own HIP and HSA runtimes under the same sonames as the ROCm
# install the library is linked against.  Whichever is loaded first is the one
# the other binds to; loading libpgemm.so first would leave two HIP runtimes in
# the process, and the library's would find no device.  So torch, when
# present, is loaded first and the library shares its runtime, its device
# memory and its streams.
try:
    import torch  # noqa: F401
except ImportError:  # a caller without torch uses the ROCm runtime directly
    pass

_lib = ctypes.CDLL(LIB_PATH)

PGEMM_F32, PGEMM_F16, PGEMM_BF16, PGEMM_I8 = 0, 1, 2, 3
DTYPE_CODE = {"f32": PGEMM_F32, "f16": PGEMM_F16, "bf16": PGEMM_BF16, "i8": PGEMM_I8}
PRODUCER = {"auto": 0, "direct": 1, "register": 2, "generic": 3, "staged_a": 4, "staged_b": 5}
# pgemm_aligned: which operands meet the chunk rule (rows of whole 16-byte chunks)
ALIGNED_NONE, ALIGNED_BOTH, ALIGNED_A, ALIGNED_B = 0, 1, 2, 3
PRODUCER_NAME = {v: k for k, v in PRODUCER.items()}
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED_DTYPE", -3: "BAD_STAGES", -4: "INFEASIBLE_PLAN",
          -5: "NONINTEGRAL_SCALAR", -6: "HIP", -7: "TOO_LARGE"}


class pgemm_opts(ctypes.Structure):
    _fields_ = [("producer", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("tile_k", ctypes.c_int), ("skew", ctypes.c_int), ("workgroups", ctypes.c_int),
                ("waves", ctypes.c_int), ("reserved", ctypes.c_int * 1)]


class pgemm_plan_info(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("stages", ctypes.c_int), ("stages_eff", ctypes.c_int), ("num_k_tiles", ctypes.c_int),
                ("producer", ctypes.c_int), ("threads", ctypes.c_int), ("waves_m", ctypes.c_int),
                ("waves_n", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("wg_per_cu", ctypes.c_int),
                ("grid", ctypes.c_int), ("variant", ctypes.c_int), ("est_uncovered_cycles", ctypes.c_double)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["producer"] = PRODUCER_NAME.get(d["producer"], d["producer"])
        return d


_i64, _dbl, _vp, _int = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
_lib.pgemm_gemm.argtypes = [_i64, _i64, _i64, _dbl, _vp, _i64, _vp, _i64, _dbl, _vp, _i64, _int, _int, _vp]
_lib.pgemm_gemm.restype = _int
_lib.pgemm_gemm_ex.argtypes = [_i64, _i64, _i64, _dbl, _vp, _i64, _vp, _i64, _dbl, _vp, _i64, _int, _int,
                               ctypes.POINTER(pgemm_opts), _vp]
_lib.pgemm_gemm_ex.restype = _int
_lib.pgemm_plan.argtypes = [_i64, _i64, _i64, _int, _int, _int, ctypes.POINTER(pgemm_opts),
                            ctypes.POINTER(pgemm_plan_info)]
_lib.pgemm_plan.restype = _int
_lib.pgemm_strerror.argtypes = [_int]
_lib.pgemm_strerror.restype = ctypes.c_char_p
_lib.pgemm_num_variants.argtypes = []
_lib.pgemm_num_variants.restype = _int
_lib.pgemm_variant_info.argtypes = [_int, ctypes.POINTER(pgemm_plan_info), ctypes.POINTER(_int)]
_lib.pgemm_variant_info.restype = _int
_lib.pgemm_version.restype = _int
_lib.pgemm_model_uncovered_cycles.argtypes = [_dbl, _dbl, _int]
_lib.pgemm_model_uncovered_cycles.restype = _dbl
_lib.pgemm_model_lds_bytes.argtypes = [_int, _int, _int, _int, _int, _int]
_lib.pgemm_model_lds_bytes.restype = _i64
_lib.pgemm_model_global_loads_per_output.argtypes = [_int, _int, _i64]
_lib.pgemm_model_global_loads_per_output.restype = _dbl
_lib.pgemm_model_compute_load_ratio.argtypes = [_int, _int, _int, _int]
_lib.pgemm_model_compute_load_ratio.restype = _dbl
_lib.pgemm_hazard_copy_reduce.argtypes = [_vp, _i64, _i64, _i64, _vp, _int, _int, _int, _vp, _i64, _int, _vp]
_lib.pgemm_hazard_copy_reduce.restype = _int
_lib.pgemm_diag_mfma_ceiling.argtypes = [_int, _int, _int, _int, _int, _int, ctypes.c_uint32, _vp, ctypes.POINTER(_i64),
                                         _vp, _vp]
_lib.pgemm_diag_mfma_ceiling.restype = _int
_lib.pgemm_diag_lds_stream.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _int, _int, _int, _int,
                                       ctypes.POINTER(_i64), _vp]
_lib.pgemm_diag_lds_stream.restype = _int
_lib.pgemm_diag_wait_profile.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _int, _int,
                                         _int, _vp, _i64, _vp]
_lib.pgemm_diag_wait_profile.restype = _int
_lib.pgemm_diag_parts.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _int, _int, _int,
                                  _int, _vp, _i64, _vp]
_lib.pgemm_diag_parts.restype = _int

# Steady-state parts of a parts-ladder build (enum pgemm_part).
PART_DMA, PART_BARRIER, PART_AREADS, PART_BREADS, PART_ALL = 1, 2, 4, 8, 15

EXPORTED = ("pgemm_gemm", "pgemm_gemm_ex", "pgemm_plan", "pgemm_strerror", "pgemm_num_variants",
            "pgemm_variant_info", "pgemm_version", "pgemm_model_uncovered_cycles", "pgemm_model_lds_bytes",
            "pgemm_model_global_loads_per_output", "pgemm_model_compute_load_ratio", "pgemm_hazard_copy_reduce",
            "pgemm_diag_mfma_ceiling", "pgemm_diag_lds_stream", "pgemm_diag_wait_profile", "pgemm_diag_parts")


class PgemmError(RuntimeError):
    def __init__(self, status):
        super().__init__("pgemm status %d (%s): %s" % (status, STATUS.get(status, "?"), pgemm_strerror(status)))
        self.status = status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _opts(producer=None, tile=None, skew=0, workgroups=0, waves=0):
    if producer is None and tile is None and not skew and not workgroups and not waves:
        return None
    o = pgemm_opts()
    o.producer = PRODUCER[producer] if isinstance(producer, str) else int(producer or 0)
    if tile is not None:
        o.tile_m, o.tile_n, o.tile_k = (int(v) for v in tile)
    o.skew = int(skew)
    o.workgroups = int(workgroups)
    o.waves = int(waves)
    return o


def _opts_from(d):
    return _opts(d.get("producer"), d.get("tile"), d.get("skew", 0), d.get("workgroups", 0), d.get("waves", 0))


def pgemm_gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stages, stream=None):
    return _lib.pgemm_gemm(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                           DTYPE_CODE.get(dtype, dtype), stages, _stream(stream))


def pgemm_gemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stages, opts=None, stream=None):
    if isinstance(opts, dict):
        opts = _opts_from(opts)
    p = ctypes.byref(opts) if opts is not None else None
    return _lib.pgemm_gemm_ex(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                              DTYPE_CODE.get(dtype, dtype), stages, p, _stream(stream))


def pgemm_plan(M, N, K, dtype, stages=0, aligned=1, opts=None):
    """Returns (status, plan dict or None)."""
    if isinstance(opts, dict):
        opts = _opts_from(opts)
    info = pgemm_plan_info()
    r = _lib.pgemm_plan(M, N, K, DTYPE_CODE.get(dtype, dtype), stages, int(aligned),
                        ctypes.byref(opts) if opts is not None else None, ctypes.byref(info))
    return r, (info.as_dict() if r == 0 else None)


def pgemm_strerror(status):
    return _lib.pgemm_strerror(int(status)).decode()


def pgemm_num_variants():
    return _lib.pgemm_num_variants()


def pgemm_variant_info(index):
    info = pgemm_plan_info()
    dt = _int(0)
    r = _lib.pgemm_variant_info(index, ctypes.byref(info), ctypes.byref(dt))
    if r != 0:
        raise PgemmError(r)
    d = info.as_dict()
    d["dtype"] = {v: k for k, v in DTYPE_CODE.items()}[dt.value]
    return d


def pgemm_version():
    return _lib.pgemm_version()


def pgemm_model_uncovered_cycles(latency, compute, stages):
    return _lib.pgemm_model_uncovered_cycles(float(latency), float(compute), int(stages))


def pgemm_model_lds_bytes(bm, bn, bk, stages, elem_bytes, a_pad=0):
    return _lib.pgemm_model_lds_bytes(bm, bn, bk, stages, elem_bytes, a_pad)


def pgemm_model_global_loads_per_output(bm, bn, K):
    return _lib.pgemm_model_global_loads_per_output(bm, bn, K)


def pgemm_model_compute_load_ratio(bm, bn, bk, elem_bytes):
    return _lib.pgemm_model_compute_load_ratio(bm, bn, bk, elem_bytes)


def _regions_overlap(X, xr, xc, Y, yr, yc):
    """Whether the first xr rows x xc columns of 2-D tensor X share a byte
    with the first yr x yc of Y (rows at each tensor's row stride).  Exact
    when both row strides in bytes are equal (slices of one matrix); with
    different strides, any overlap of the two byte ranges counts."""
    if not (xr and xc and yr and yc):
        return False
    sx, sy = X.stride(0) * X.element_size(), Y.stride(0) * Y.element_size()
    wx, wy = xc * X.element_size(), yc * Y.element_size()
    x0, y0 = X.data_ptr(), Y.data_ptr()
    if x0 >= y0 + (yr - 1) * sy + wy or y0 >= x0 + (xr - 1) * sx + wx:
        return False
    if sx != sy or sx == 0:
        return True
    # row i of X and row j of Y meet iff -wy < d + (j - i) * s < wx, d = y0 - x0
    d = y0 - x0
    t0 = -d // sx
    for t in range(t0 - 1, t0 + 3):
        if -(xr - 1) <= t <= yr - 1 and -wy < d + t * sx < wx:
            return True
    return False


def gemm(A, B, C, alpha=1.0, beta=0.0, stages=0, producer=None, tile=None, M=None, N=None, K=None,
         stream=None):
    """C = alpha*A@B + beta*C on torch tensors (2-D, row-major, unit column stride).

    dtype is taken from A: float32 -> f32, float16 -> f16, bfloat16 -> bf16, int8 -> i8.
    B must have A's dtype; C is float32 (int32 for int8).  Sizes default to the
    logical shapes and must fit inside the tensors; leading dimensions are the
    row strides.  All three tensors must live on one GPU, and C must not
    overlap A or B; the call runs on that GPU (torch's current stream there
    unless `stream` is given).  Every check runs
    before anything reaches the library, so a bad call raises ValueError and
    launches nothing.
    """
    import torch
    in_dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.int8: "i8"}
    if A.dtype not in in_dt:
        raise ValueError("A has unsupported dtype %s" % A.dtype)
    dt = in_dt[A.dtype]
    out_dt = torch.int32 if dt == "i8" else torch.float32
    if B.dtype != A.dtype:
        raise ValueError("B must have A's dtype %s, got %s" % (A.dtype, B.dtype))
    if C.dtype != out_dt:
        raise ValueError("C must be %s for %s inputs, got %s" % (out_dt, A.dtype, C.dtype))
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError("%s must be a 2-D row-major tensor with unit column stride" % name)
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    for name, t, rows, cols in (("A", A, M, K), ("B", B, K, N), ("C", C, M, N)):
        if rows < 0 or cols < 0 or (rows and cols and (t.shape[0] < rows or t.shape[1] < cols)):
            raise ValueError("%s is %s, the call needs %d x %d" % (name, tuple(t.shape), rows, cols))
    for name, t, rows, cols in (("A", A, M, K), ("B", B, K, N)):
        if t.device == C.device and _regions_overlap(t, rows, cols, C, M, N):
            raise ValueError("C overlaps %s: the output must not share memory with an input" % name)
    devs = {t.device for t in (A, B, C)}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError("A, B and C must be GPU tensors on one device, got %s" % sorted(str(d) for d in devs))
    # the library launches on the current device: make it the tensors' one
    with torch.cuda.device(C.device):
        r = pgemm_gemm_ex(M, N, K, alpha, A, max(A.stride(0), 1), B, max(B.stride(0), 1), beta, C,
                          max(C.stride(0), 1), dt, stages, _opts(producer, tile), stream)
    if r != 0:
        raise PgemmError(r)
    return C


def pgemm_hazard_copy_reduce(X, rows, cols, ldx, row_sums, reuse_wait, delay_wave=-1, delay_cycles=0, trace=None,
                             trace_len=0, trace_wg=0, stream=None):
    return _lib.pgemm_hazard_copy_reduce(_ptr(X), rows, cols, ldx, _ptr(row_sums), int(reuse_wait), int(delay_wave),
                                         int(delay_cycles), _ptr(trace), int(trace_len), int(trace_wg),
                                         _stream(stream))


def pgemm_diag_mfma_ceiling(dtype, zero_operands, iters, grid, seed, out, clock=None, stream=None, waves_per_simd=2,
                            block=16):
    """Returns (status, flops of the launch)."""
    fl = _i64(0)
    r = _lib.pgemm_diag_mfma_ceiling(DTYPE_CODE.get(dtype, dtype), int(zero_operands), int(waves_per_simd), int(block),
                                     int(iters), int(grid), int(seed) & 0xFFFFFFFF, _ptr(out), ctypes.byref(fl),
                                     _ptr(clock), _stream(stream))
    return r, fl.value


def pgemm_diag_lds_stream(M, N, K, A, lda, B, ldb, dtype, tile, stages, stream=None):
    """Returns (status, LDS bytes the launch fills)."""
    nb = _i64(0)
    r = _lib.pgemm_diag_lds_stream(M, N, K, _ptr(A), lda, _ptr(B), ldb, DTYPE_CODE.get(dtype, dtype),
                                   int(tile[0]), int(tile[1]), int(tile[2]), int(stages), ctypes.byref(nb),
                                   _stream(stream))
    return r, nb.value


def pgemm_diag_wait_profile(M, N, K, A, lda, B, ldb, C, ldc, dtype, tile, stages, out, out_len, stream=None):
    return _lib.pgemm_diag_wait_profile(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, DTYPE_CODE.get(dtype, dtype),
                                        int(tile[0]), int(tile[1]), int(tile[2]), int(stages), _ptr(out),
                                        int(out_len), _stream(stream))


def pgemm_diag_parts(M, N, K, A, lda, B, ldb, C, ldc, dtype, tile, stages, parts, clock, clock_len, stream=None):
    return _lib.pgemm_diag_parts(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, DTYPE_CODE.get(dtype, dtype),
                                 int(tile[0]), int(tile[1]), int(tile[2]), int(stages), int(parts), _ptr(clock),
                                 int(clock_len), _stream(stream))
