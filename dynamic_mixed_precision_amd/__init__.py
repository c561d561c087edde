"""Python binding of libdmpq, the gfx950 hot path of 6Bit-Diffusion's dynamic
mixed-precision quantized linear layer.

Argument marshalling only: each function passes torch tensors' device
pointers, sizes and the current HIP stream to the C entry point of the same
name (``dmpq_<name>``) and raises :class:`DmpqError` on a non-OK status.  All
arithmetic runs in the library's HIP kernels; there is no fallback.  Output
tensors are allocated by the caller, as the C ABI requires.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmpq.so")

OK = 0
ROUTE_NVFP4, ROUTE_INT8, ROUTE_BF16 = 0, 1, 2
OUT_F32, OUT_BF16, OUT_I32 = 0, 1, 2
NO_HADAMARD, AMAX_GIVEN = 1, 2
EPI_GELU, EPI_NVFP4_AMAX = 1, 2
CODEC_E4M3, CODEC_E2M1 = 0, 1
W8_FROM_NVFP4, W8_DIRECT = 0, 1
TDC_SKIP, TDC_REFRESH = 0, 1
FP4_BF16_DEQUANT = 0
FP4_SCALED_MFMA = 1
OP_GAMMA, OP_QUANT_NVFP4, OP_TDC, OP_PREP_WEIGHT, OP_OUTLIER, OP_GEMM_AMAX, OP_GEMM = 0, 1, 2, 3, 4, 5, 6
OP_GEMM_W4 = 7

EXPORTS = ("dmpq_last_error", "dmpq_version", "dmpq_workspace_bytes", "dmpq_gamma_sums",
           "dmpq_gate_and_route", "dmpq_hadamard_quant_int8", "dmpq_hadamard_quant_nvfp4",
           "dmpq_qgemm_int8", "dmpq_qgemm_nvfp4", "dmpq_tdc_init", "dmpq_tdc_decide",
           "dmpq_tdc_step", "dmpq_tdc_commit", "dmpq_prep_weight", "dmpq_weight_int8_from_nvfp4",
           "dmpq_outlier_count", "dmpq_pdr_decide", "dmpq_gemm_bf16", "dmpq_qgemm_int8_ex",
           "dmpq_qgemm_nvfp4_ex", "dmpq_gemm_bf16_ex", "dmpq_selftest_codec",
           "dmpq_hadamard_quant_nvfp4_noalloc", "dmpq_qgemm_int8_from_nvfp4",
           "dmpq_hadamard_quant_int8_w8")


class DmpqError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> status {status}: {msg}")
        self.status = status


class TdcState(C.Structure):
    """Mirror of dmpq_tdc_state."""
    _fields_ = [("n_refresh", C.c_int64), ("d", C.c_double), ("acc", C.c_double),
                ("delta_valid", C.c_int32), ("gamma_valid", C.c_int32), ("gamma", C.c_double)]


class TdcParams(C.Structure):
    """Mirror of dmpq_tdc_params."""
    _fields_ = [("eps_sim", C.c_double), ("delta_acc", C.c_double)]


_lib = None


def lib():
    """Load libdmpq.so (built in-tree by dynamic_mixed_precision_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m "
                              "dynamic_mixed_precision_amd.build (needs hipcc)")
        _lib = _declare(C.CDLL(LIB_PATH))
    return _lib


def _declare(L):
    vp, i64, i32, f64 = C.c_void_p, C.c_int64, C.c_int, C.c_double
    pd = C.POINTER(C.c_double)
    sig = {
        "dmpq_last_error": (C.c_char_p, []),
        "dmpq_version": (C.c_char_p, []),
        "dmpq_workspace_bytes": (C.c_size_t, [i32, i64, i64]),
        "dmpq_gamma_sums": (i32, [vp, vp, vp, i64, vp, vp, C.c_size_t]),
        "dmpq_gate_and_route": (i32, [vp, i32, vp, vp, f64, vp, vp, vp]),
        "dmpq_hadamard_quant_int8": (i32, [vp, vp, i64, i64, i32, vp, vp]),
        "dmpq_hadamard_quant_nvfp4": (i32, [vp, vp, i64, i64, i32, vp, vp, vp, vp, C.c_size_t]),
        "dmpq_qgemm_int8": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]),
        "dmpq_qgemm_nvfp4": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32]),
        "dmpq_tdc_init": (i32, [C.POINTER(TdcState)]),
        "dmpq_tdc_decide": (i32, [C.POINTER(TdcState), C.POINTER(TdcParams), C.POINTER(C.c_int)]),
        "dmpq_tdc_step": (i32, [vp, i32, vp, vp, vp, i64, i32, vp, vp, C.c_size_t]),
        "dmpq_tdc_commit": (i32, [C.POINTER(TdcState), i32, pd]),
        "dmpq_prep_weight": (i32, [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, vp, C.c_size_t]),
        "dmpq_weight_int8_from_nvfp4": (i32, [vp, vp, vp, vp, i64, i64, vp, vp]),
        "dmpq_hadamard_quant_int8_w8": (i32, [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, i64, vp, vp]),
        "dmpq_outlier_count": (i32, [vp, vp, i64, i64, f64, vp, vp, C.c_size_t]),
        "dmpq_pdr_decide": (i32, [f64, i64, f64, C.POINTER(C.c_int)]),
        "dmpq_gemm_bf16": (i32, [vp, vp, vp, i64, i64, i64, i32, vp]),
        "dmpq_qgemm_int8_ex": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, vp, C.c_size_t]),
        "dmpq_qgemm_nvfp4_ex": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, vp,
                                      C.c_size_t]),
        "dmpq_gemm_bf16_ex": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, i32, vp, C.c_size_t]),
        "dmpq_selftest_codec": (i32, [vp, i32, C.c_uint32, C.c_uint32, vp]),
        "dmpq_hadamard_quant_nvfp4_noalloc": (i32, [vp, vp, i64, i64, i32, vp, vp, vp]),
        "dmpq_qgemm_int8_from_nvfp4": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, vp,
                                             C.c_size_t]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _check(status: int, fn: str) -> None:
    if status != OK:
        raise DmpqError(status, fn, lib().dmpq_last_error().decode())


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdmpq device arguments must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("libdmpq tensors must be contiguous")
    return t.data_ptr()


_OUT_BYTES = {OUT_F32: 4, OUT_BF16: 2, OUT_I32: 4}


def _need(t, name: str, nbytes: int, esize: int | None = None) -> None:
    """The C entry points take bare device pointers, so the sizes they will
    read and write are checked here: raise ValueError unless tensor ``t`` holds
    at least ``nbytes`` bytes (and, with ``esize``, has elements of that size)."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if esize is not None and t.element_size() != esize:
        raise ValueError(f"{name} has {t.element_size()}-byte elements, needs {esize}-byte ones")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, needs {nbytes}")


def _need_out(y, M: int, N: int, out_dtype: int) -> None:
    if out_dtype in _OUT_BYTES:  # an unknown type is the library's error to report
        _need(y, "y", M * N * _OUT_BYTES[out_dtype], _OUT_BYTES[out_dtype])


def _need_nvfp4(codes, scales, g, rows: int, K: int, what: str) -> None:
    """An NVFP4 operand of `rows` x K: K/2 code bytes and K/16 scale bytes per
    row, one fp32 tensor scale."""
    _need(codes, f"{what} codes", rows * K // 2, 1)
    _need(scales, f"{what} scales", rows * K // 16, 1)
    _need(g, f"{what} tensor scale", 4, 4)


def _need_k(w, K: int, what: str) -> None:
    if len(w.shape) != 2 or w.shape[1] != K:
        raise ValueError(f"{what} has shape {tuple(w.shape)}, needs {K} per row")


def last_error() -> str:
    return lib().dmpq_last_error().decode()


def version() -> str:
    return lib().dmpq_version().decode()


def workspace_bytes(op: int, M: int = 0, K: int = 0) -> int:
    return int(lib().dmpq_workspace_bytes(op, M, K))


def new_workspace(op: int, device="cuda", M: int = 0, K: int = 0):
    """Zero-filled workspace tensor for ``op`` (sizes M, K for OP_GEMM_AMAX)."""
    import torch
    return torch.zeros(workspace_bytes(op, M, K), dtype=torch.uint8, device=device)


def gamma_sums(x_in, x_out, sums, ws, stream=None) -> None:
    n = x_in.numel()
    _need(x_in, "x_in", 2 * n, 2)
    _need(x_out, "x_out", 2 * n, 2)
    _need(sums, "sums", 16, 8)
    _check(lib().dmpq_gamma_sums(_stream(stream), _ptr(x_in), _ptr(x_out), x_in.numel(),
                                 _ptr(sums), _ptr(ws), ws.numel()), "dmpq_gamma_sums")


def gate_and_route(sums2, alpha, beta, tau: float):
    """Host router.  sums2: 2 floats or None (Gamma missing).
    Returns (gamma, errors[n_lin], routes[n_lin]).  Runs between the step's
    device->host copy and its first launch, so it passes raw addresses (a
    ctypes pointer cast costs tens of microseconds)."""
    a = np.ascontiguousarray(alpha, np.float64)
    b = np.ascontiguousarray(beta, np.float64)
    n = len(a)
    s = None if sums2 is None else np.ascontiguousarray(sums2, np.float64)
    out = np.empty(1 + n, np.float64)  # gamma, then the errors
    r = np.empty(n, np.uint8)
    _check(lib().dmpq_gate_and_route(
        None if s is None else s.ctypes.data, n, a.ctypes.data, b.ctypes.data, tau,
        out.ctypes.data, out.ctypes.data + 8, r.ctypes.data), "dmpq_gate_and_route")
    return float(out[0]), out[1:], r


def hadamard_quant_int8(x, q, s_row, flags: int = 0, stream=None) -> None:
    M, K = x.shape
    _need(x, "x", 2 * M * K, 2)
    _need(q, "q", M * K, 1)
    _need(s_row, "s_row", 4 * M, 4)
    _check(lib().dmpq_hadamard_quant_int8(_stream(stream), _ptr(x), M, K, flags, _ptr(q),
                                          _ptr(s_row)), "dmpq_hadamard_quant_int8")


def hadamard_quant_nvfp4(x, codes, scales, g, ws, flags: int = 0, stream=None) -> None:
    M, K = x.shape
    _need(x, "x", 2 * M * K, 2)
    _need_nvfp4(codes, scales, g, M, K, "output")
    _check(lib().dmpq_hadamard_quant_nvfp4(_stream(stream), _ptr(x), M, K, flags, _ptr(codes),
                                           _ptr(scales), _ptr(g), _ptr(ws), ws.numel()),
           "dmpq_hadamard_quant_nvfp4")


def hadamard_quant_nvfp4_noalloc(x, codes, scales, g, flags: int = 0, stream=None) -> None:
    """hadamard_quant_nvfp4 without a workspace (the library's static scratch)."""
    M, K = x.shape
    _need(x, "x", 2 * M * K, 2)
    _need_nvfp4(codes, scales, g, M, K, "output")
    _check(lib().dmpq_hadamard_quant_nvfp4_noalloc(_stream(stream), _ptr(x), M, K, flags,
                                                   _ptr(codes), _ptr(scales), _ptr(g)),
           "dmpq_hadamard_quant_nvfp4_noalloc")


def _need_int8_gemm(qa, sa, qw, sw, y, out_dtype):
    M, K = qa.shape
    N = qw.shape[0]
    _need(qa, "qa", M * K, 1)
    _need(sa, "sa", 4 * M, 4)
    _need_k(qw, K, "qw")
    _need(qw, "qw", N * K, 1)
    _need(sw, "sw", 4 * N, 4)
    _need_out(y, M, N, out_dtype)
    return M, N, K


def _need_nvfp4_gemm(ca, sa, ga, cw, sw, gw, y, out_dtype):
    M, K = ca.shape[0], 2 * ca.shape[1]
    N = cw.shape[0]
    _need_nvfp4(ca, sa, ga, M, K, "activation")
    _need_k(cw, K // 2, "cw")
    _need_nvfp4(cw, sw, gw, N, K, "weight")
    _need_out(y, M, N, out_dtype)
    return M, N, K


def _need_bf16_gemm(x, w, y, out_dtype):
    M, K = x.shape
    N = w.shape[0]
    _need(x, "x", 2 * M * K, 2)
    _need_k(w, K, "w")
    _need(w, "w", 2 * N * K, 2)
    _need_out(y, M, N, out_dtype)
    return M, N, K


def qgemm_int8(qa, sa, qw, sw, y, out_dtype: int = OUT_F32, stream=None) -> None:
    M, N, K = _need_int8_gemm(qa, sa, qw, sw, y, out_dtype)
    _check(lib().dmpq_qgemm_int8(_stream(stream), _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                                 out_dtype, _ptr(y)), "dmpq_qgemm_int8")


def qgemm_nvfp4(ca, sa, ga, cw, sw, gw, y, out_dtype: int = OUT_F32,
                variant: int = FP4_BF16_DEQUANT, stream=None) -> None:
    M, N, K = _need_nvfp4_gemm(ca, sa, ga, cw, sw, gw, y, out_dtype)
    _check(lib().dmpq_qgemm_nvfp4(_stream(stream), _ptr(ca), _ptr(sa), _ptr(ga), _ptr(cw),
                                  _ptr(sw), _ptr(gw), M, N, K, out_dtype, _ptr(y), variant),
           "dmpq_qgemm_nvfp4")


def tdc_init() -> TdcState:
    st = TdcState()
    _check(lib().dmpq_tdc_init(C.byref(st)), "dmpq_tdc_init")
    return st


def tdc_decide(st: TdcState, eps_sim: float, delta_acc: float) -> bool:
    p = TdcParams(eps_sim, delta_acc)
    out = C.c_int(0)
    _check(lib().dmpq_tdc_decide(C.byref(st), C.byref(p), C.byref(out)), "dmpq_tdc_decide")
    return bool(out.value)


def tdc_step(mode: int, x_in, x_out, delta, delta_valid: bool, sums=None, ws=None,
             stream=None) -> None:
    n = x_in.numel()
    for t, name in ((x_in, "x_in"), (x_out, "x_out"), (delta, "delta")):
        _need(t, name, 2 * n, 2)
    if mode == TDC_REFRESH:
        _need(sums, "sums", 32, 8)
    _check(lib().dmpq_tdc_step(_stream(stream), mode, _ptr(x_in), _ptr(x_out), _ptr(delta),
                               x_in.numel(), int(delta_valid), _ptr(sums), _ptr(ws),
                               0 if ws is None else ws.numel()), "dmpq_tdc_step")


def tdc_commit(st: TdcState, mode: int, sums4=None) -> None:
    s = None if sums4 is None else np.ascontiguousarray(sums4, np.float64)
    _check(lib().dmpq_tdc_commit(C.byref(st), mode,
                                 None if s is None else s.ctypes.data_as(C.POINTER(C.c_double))),
           "dmpq_tdc_commit")


def prep_weight(w, cw, sw, gw, qw, sw_row, ws, int8_mode: int = W8_FROM_NVFP4,
                stream=None) -> None:
    N, K = w.shape
    _need(w, "w", 2 * N * K, 2)
    _need_nvfp4(cw, sw, gw, N, K, "weight")
    _need(qw, "qw", N * K, 1)
    _need(sw_row, "sw_row", 4 * N, 4)
    _check(lib().dmpq_prep_weight(_stream(stream), _ptr(w), N, K, int8_mode, _ptr(cw), _ptr(sw),
                                  _ptr(gw), _ptr(qw), _ptr(sw_row), _ptr(ws), ws.numel()),
           "dmpq_prep_weight")


def weight_int8_from_nvfp4(cw, sw, gw, qw, sw_row, stream=None) -> None:
    """INT8 weight (qw, sw_row) from the NVFP4 weight (cw, sw, gw)."""
    N, K = cw.shape[0], 2 * cw.shape[1]
    _need_nvfp4(cw, sw, gw, N, K, "weight")
    _need(qw, "qw", N * K, 1)
    _need(sw_row, "sw_row", 4 * N, 4)
    _check(lib().dmpq_weight_int8_from_nvfp4(_stream(stream), _ptr(cw), _ptr(sw), _ptr(gw), N, K,
                                             _ptr(qw), _ptr(sw_row)), "dmpq_weight_int8_from_nvfp4")


def hadamard_quant_int8_w8(x, q, s_row, cw, sw, gw, qw, sw_row, flags: int = 0, stream=None) -> None:
    """hadamard_quant_int8(x, q, s_row) and weight_int8_from_nvfp4(cw, sw, gw,
    qw, sw_row) in one launch (x and the weight share K)."""
    M, K = x.shape
    N = cw.shape[0]
    _need(x, "x", 2 * M * K, 2)
    _need(q, "q", M * K, 1)
    _need(s_row, "s_row", 4 * M, 4)
    _need_k(cw, K // 2, "cw")
    _need_nvfp4(cw, sw, gw, N, K, "weight")
    _need(qw, "qw", N * K, 1)
    _need(sw_row, "sw_row", 4 * N, 4)
    _check(lib().dmpq_hadamard_quant_int8_w8(_stream(stream), _ptr(x), M, K, flags, _ptr(q), _ptr(s_row),
                                             _ptr(cw), _ptr(sw), _ptr(gw), N, _ptr(qw), _ptr(sw_row)),
           "dmpq_hadamard_quant_int8_w8")


def qgemm_int8_from_nvfp4(qa, sa, cw, sw, gw, y, ws, epilogue: int = 0, out_dtype: int = OUT_BF16,
                          stream=None) -> None:
    """INT8 linear against the NVFP4 weight (cw, sw, gw), converted inside the
    GEMM; ws: an OP_GEMM_W4 workspace for (M, N)."""
    M, K = qa.shape
    N = cw.shape[0]
    _need(qa, "qa", M * K, 1)
    _need(sa, "sa", 4 * M, 4)
    _need_k(cw, K // 2, "cw")
    _need_nvfp4(cw, sw, gw, N, K, "weight")
    _need_out(y, M, N, out_dtype)
    _check(lib().dmpq_qgemm_int8_from_nvfp4(_stream(stream), _ptr(qa), _ptr(sa), _ptr(cw), _ptr(sw),
                                            _ptr(gw), M, N, K, out_dtype, _ptr(y), epilogue, *_ws(ws)),
           "dmpq_qgemm_int8_from_nvfp4")


def outlier_count(x, kappa: float, count, ws, stream=None) -> None:
    """PDR outlier count of x [M x K] bf16 (as int16 bits) into count (fp64[1])."""
    M, K = x.shape
    _need(x, "x", 2 * M * K, 2)
    _need(count, "count", 8, 8)
    _check(lib().dmpq_outlier_count(_stream(stream), _ptr(x), M, K, float(kappa), _ptr(count),
                                    _ptr(ws), ws.numel()), "dmpq_outlier_count")


def pdr_decide(count: float, n: int, rho: float) -> bool:
    force = C.c_int(0)
    _check(lib().dmpq_pdr_decide(float(count), int(n), float(rho), C.byref(force)), "dmpq_pdr_decide")
    return bool(force.value)


def gemm_bf16(x, w, y, out_dtype: int = OUT_F32, stream=None) -> None:
    """Full-precision linear y = x w^T over bf16 operands (fp32 accumulation)."""
    M, N, K = _need_bf16_gemm(x, w, y, out_dtype)
    _check(lib().dmpq_gemm_bf16(_stream(stream), _ptr(x), _ptr(w), M, N, K, out_dtype, _ptr(y)),
           "dmpq_gemm_bf16")


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel())


def qgemm_int8_ex(qa, sa, qw, sw, y, epilogue: int = 0, ws=None, out_dtype: int = OUT_BF16,
                  stream=None) -> None:
    """qgemm_int8 with a producer epilogue (EPI_GELU, EPI_NVFP4_AMAX); with an
    OP_GEMM workspace the last partial wave of tiles is split along K."""
    M, N, K = _need_int8_gemm(qa, sa, qw, sw, y, out_dtype)
    _check(lib().dmpq_qgemm_int8_ex(_stream(stream), _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N,
                                    K, out_dtype, _ptr(y), epilogue, *_ws(ws)),
           "dmpq_qgemm_int8_ex")


def qgemm_nvfp4_ex(ca, sa, ga, cw, sw, gw, y, epilogue: int = 0, ws=None, out_dtype: int = OUT_BF16,
                   stream=None) -> None:
    """qgemm_nvfp4 (BF16-dequant variant) with a producer epilogue and the
    optional tail split."""
    M, N, K = _need_nvfp4_gemm(ca, sa, ga, cw, sw, gw, y, out_dtype)
    _check(lib().dmpq_qgemm_nvfp4_ex(_stream(stream), _ptr(ca), _ptr(sa), _ptr(ga), _ptr(cw),
                                     _ptr(sw), _ptr(gw), M, N, K, out_dtype, _ptr(y), epilogue,
                                     *_ws(ws)),
           "dmpq_qgemm_nvfp4_ex")


def gemm_bf16_ex(x, w, y, epilogue: int = 0, ws=None, out_dtype: int = OUT_BF16,
                 stream=None) -> None:
    """gemm_bf16 with a producer epilogue and the optional tail split."""
    M, N, K = _need_bf16_gemm(x, w, y, out_dtype)
    _check(lib().dmpq_gemm_bf16_ex(_stream(stream), _ptr(x), _ptr(w), M, N, K, out_dtype, _ptr(y),
                                   epilogue, *_ws(ws)),
           "dmpq_gemm_bf16_ex")


def selftest_codec(codec: int, lo: int, hi: int, stats, stream=None) -> None:
    """Per-code (lowest, highest, count) of the fp32 patterns [lo, hi) through
    a device converter (CODEC_E4M3 or CODEC_E2M1); stats: uint32/int32 tensor
    of 3 words per code (128 codes for E4M3, 16 for E2M1)."""
    if codec in (CODEC_E4M3, CODEC_E2M1):  # an unknown codec is the library's error to report
        _need(stats, "stats", 12 * (128 if codec == CODEC_E4M3 else 16), 4)
    _check(lib().dmpq_selftest_codec(_stream(stream), codec, lo, hi, _ptr(stats)),
           "dmpq_selftest_codec")
