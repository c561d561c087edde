"""CPU oracle for the dynamic mixed-precision quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports
this package and shares no source with it.

The arithmetic lives in ``oracle.c`` (plain C, fp32 steps with IEEE RNE and
no contraction, fp64 reductions); this module only marshals numpy arrays.
bf16 tensors are numpy ``uint16`` arrays of bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "oracle.c")]

NO_HADAMARD = 1
W8_FROM_NVFP4 = 0
W8_DIRECT = 1
ROUTE_NVFP4 = 0
ROUTE_INT8 = 1


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (IEEE fp32, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB_PATH + ".tmp", *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _declare(C.CDLL(LIB_PATH))
    return _lib


class TdcState(C.Structure):
    _fields_ = [("n_refresh", C.c_int64), ("d", C.c_double), ("acc", C.c_double),
                ("delta_valid", C.c_int32), ("gamma_valid", C.c_int32),
                ("gamma", C.c_double)]


def _p(t):
    return C.POINTER(t)


def _declare(L):
    u8, u16, i8, i32, i64 = C.c_uint8, C.c_uint16, C.c_int8, C.c_int32, C.c_int64
    f32, f64 = C.c_float, C.c_double
    sig = {
        "orc_max_threads": (C.c_int, []),
        "orc_set_threads": (None, [C.c_int]),
        "orc_bf16_round": (u16, [f32]),
        "orc_bf16_value": (f32, [u16]),
        "orc_e2m1_value": (f32, [u8]),
        "orc_e2m1_encode": (u8, [f32]),
        "orc_e4m3_value": (f32, [u8]),
        "orc_e4m3_encode": (u8, [f32]),
        "orc_fwht16": (None, [_p(f32), _p(f32)]),
        "orc_quant_int8": (C.c_int, [_p(u16), i64, i64, C.c_int, _p(i8), _p(f32)]),
        "orc_quant_nvfp4": (C.c_int, [_p(u16), i64, i64, C.c_int, _p(u8), _p(u8), _p(f32)]),
        "orc_prep_weight": (C.c_int, [_p(u16), i64, i64, C.c_int, _p(u8), _p(u8), _p(f32),
                                      _p(i8), _p(f32)]),
        "orc_w8_from_nvfp4": (C.c_int, [_p(u8), _p(u8), _p(f32), i64, i64, _p(i8), _p(f32)]),
        "orc_outlier_count": (i64, [_p(u16), i64, i64, C.c_double]),
        "orc_outlier_count_band": (None, [_p(u16), i64, i64, C.c_double, C.c_double, _p(i64), _p(i64)]),
        "orc_pdr_force": (C.c_int, [i64, i64, C.c_double]),
        "orc_gelu": (C.c_double, [C.c_double]),
        "orc_gemm_bf16": (C.c_int, [_p(u16), _p(u16), i64, i64, i64, _p(i64), i64, _p(f64), _p(f64)]),
        "orc_gemm_int8": (C.c_int, [_p(i8), _p(f32), _p(i8), _p(f32), i64, i64, i64,
                                    _p(i64), i64, _p(i32), _p(f32)]),
        "orc_gemm_nvfp4": (C.c_int, [_p(u8), _p(u8), f32, _p(u8), _p(u8), f32, i64, i64, i64,
                                     _p(i64), i64, _p(f64), _p(f64)]),
        "orc_gamma_sums": (None, [_p(u16), _p(u16), i64, _p(f64)]),
        "orc_gamma": (f64, [_p(f64)]),
        "orc_route": (None, [_p(f64), C.c_int, _p(f64), _p(f64), f64, _p(f64), _p(f64), _p(u8)]),
        "orc_tdc_init": (None, [_p(TdcState)]),
        "orc_tdc_decide": (C.c_int, [_p(TdcState), f64, f64]),
        "orc_tdc_skip": (None, [_p(u16), _p(u16), i64, _p(u16)]),
        "orc_tdc_refresh": (None, [_p(u16), _p(u16), _p(u16), i64, C.c_int, _p(f64)]),
        "orc_tdc_commit_skip": (None, [_p(TdcState)]),
        "orc_tdc_commit_refresh": (None, [_p(TdcState), _p(f64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.POINTER(ctype))


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 tensors travel as uint16 bit patterns"
    return x


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops from now on."""
    lib().orc_set_threads(int(n))


# ---- codecs -------------------------------------------------------------

def bf16_round(f: float) -> int:
    return int(lib().orc_bf16_round(f))


def bf16_value(b: int) -> float:
    return float(lib().orc_bf16_value(b))


def e2m1_value(c: int) -> float:
    return float(lib().orc_e2m1_value(c))


def e2m1_encode(v: float) -> int:
    return int(lib().orc_e2m1_encode(v))


def e4m3_value(c: int) -> float:
    return float(lib().orc_e4m3_value(c))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(v))


def fwht16(v) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float32).reshape(16)
    out = np.empty(16, np.float32)
    lib().orc_fwht16(_ptr(a, C.c_float), _ptr(out, C.c_float))
    return out


# ---- quantizers -----------------------------------------------------------

def quant_int8(x: np.ndarray, flags: int = 0):
    x = _u16(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    rc = lib().orc_quant_int8(_ptr(x, C.c_uint16), M, K, flags, _ptr(q, C.c_int8), _ptr(s, C.c_float))
    if rc != 0:
        raise ValueError(f"orc_quant_int8: bad shape {x.shape}")
    return q, s


def quant_nvfp4(x: np.ndarray, flags: int = 0):
    x = _u16(x)
    M, K = x.shape
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    g = np.zeros(1, np.float32)
    rc = lib().orc_quant_nvfp4(_ptr(x, C.c_uint16), M, K, flags, _ptr(codes, C.c_uint8),
                               _ptr(scales, C.c_uint8), _ptr(g, C.c_float))
    if rc != 0:
        raise ValueError(f"orc_quant_nvfp4: bad shape {x.shape}")
    return codes, scales, float(g[0])


def prep_weight(w: np.ndarray, int8_mode: int = W8_FROM_NVFP4):
    w = _u16(w)
    N, K = w.shape
    cw = np.empty((N, K // 2), np.uint8)
    sw = np.empty((N, K // 16), np.uint8)
    gw = np.zeros(1, np.float32)
    qw = np.empty((N, K), np.int8)
    swr = np.empty(N, np.float32)
    rc = lib().orc_prep_weight(_ptr(w, C.c_uint16), N, K, int8_mode, _ptr(cw, C.c_uint8),
                               _ptr(sw, C.c_uint8), _ptr(gw, C.c_float), _ptr(qw, C.c_int8),
                               _ptr(swr, C.c_float))
    if rc != 0:
        raise ValueError(f"orc_prep_weight: bad shape/mode {w.shape} {int8_mode}")
    return dict(cw=cw, sw=sw, gw=float(gw[0]), qw=qw, sw_row=swr)


def w8_from_nvfp4(cw: np.ndarray, sw: np.ndarray, gw: float):
    """INT8 weight (qw [N x K], sw_row [N]) derived from an NVFP4 weight."""
    cw = np.ascontiguousarray(cw, np.uint8)
    sw = np.ascontiguousarray(sw, np.uint8)
    N, K = cw.shape[0], 2 * cw.shape[1]
    assert sw.shape == (N, K // 16)
    g = np.array([gw], np.float32)
    qw = np.empty((N, K), np.int8)
    swr = np.empty(N, np.float32)
    rc = lib().orc_w8_from_nvfp4(_ptr(cw, C.c_uint8), _ptr(sw, C.c_uint8), _ptr(g, C.c_float),
                                 N, K, _ptr(qw, C.c_int8), _ptr(swr, C.c_float))
    if rc != 0:
        raise ValueError(f"orc_w8_from_nvfp4: bad shape {N} x {K}")
    return qw, swr


# ---- GEMMs ----------------------------------------------------------------

def _rows(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, len(r)


def gemm_int8(qa, sa, qw, sw, rows=None):
    qa = np.ascontiguousarray(qa, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    sw = np.ascontiguousarray(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    r, R = _rows(rows, M)
    acc = np.empty((R, N), np.int32)
    y = np.empty((R, N), np.float32)
    rc = lib().orc_gemm_int8(_ptr(qa, C.c_int8), _ptr(sa, C.c_float), _ptr(qw, C.c_int8),
                             _ptr(sw, C.c_float), M, N, K, _ptr(r, C.c_int64), R,
                             _ptr(acc, C.c_int32), _ptr(y, C.c_float))
    if rc != 0:
        raise ValueError("orc_gemm_int8 failed (row index or int32 range)")
    return acc, y


def gemm_nvfp4(ca, sa, ga, cw, sw, gw, rows=None):
    ca = np.ascontiguousarray(ca, np.uint8)
    cw = np.ascontiguousarray(cw, np.uint8)
    sa = np.ascontiguousarray(sa, np.uint8)
    sw = np.ascontiguousarray(sw, np.uint8)
    M, K2 = ca.shape
    K = 2 * K2
    N = cw.shape[0]
    r, R = _rows(rows, M)
    y = np.empty((R, N), np.float64)
    b = np.empty((R, N), np.float64)
    rc = lib().orc_gemm_nvfp4(_ptr(ca, C.c_uint8), _ptr(sa, C.c_uint8), ga, _ptr(cw, C.c_uint8),
                              _ptr(sw, C.c_uint8), gw, M, N, K, _ptr(r, C.c_int64), R,
                              _ptr(y, C.c_double), _ptr(b, C.c_double))
    if rc != 0:
        raise ValueError("orc_gemm_nvfp4 failed")
    return y, b


# ---- Gamma, routing, TDC --------------------------------------------------

def gamma_sums(x_in, x_out) -> np.ndarray:
    x_in, x_out = _u16(x_in), _u16(x_out)
    assert x_in.size == x_out.size
    s = np.zeros(2, np.float64)
    lib().orc_gamma_sums(_ptr(x_in, C.c_uint16), _ptr(x_out, C.c_uint16), x_in.size,
                         _ptr(s, C.c_double))
    return s


def gamma(sums) -> float:
    s = np.ascontiguousarray(sums, np.float64)
    return float(lib().orc_gamma(_ptr(s, C.c_double)))


def route(sums, alpha, beta, tau):
    alpha = np.ascontiguousarray(alpha, np.float64)
    beta = np.ascontiguousarray(beta, np.float64)
    n = len(alpha)
    s = None if sums is None else np.ascontiguousarray(sums, np.float64)
    g = np.zeros(1, np.float64)
    e = np.zeros(n, np.float64)
    r = np.zeros(n, np.uint8)
    lib().orc_route(_ptr(s, C.c_double), n, _ptr(alpha, C.c_double), _ptr(beta, C.c_double),
                    tau, _ptr(g, C.c_double), _ptr(e, C.c_double), _ptr(r, C.c_uint8))
    return float(g[0]), e, r


def tdc_new() -> TdcState:
    st = TdcState()
    lib().orc_tdc_init(C.byref(st))
    return st


def tdc_decide(st: TdcState, eps_sim: float, delta_acc: float) -> bool:
    return bool(lib().orc_tdc_decide(C.byref(st), eps_sim, delta_acc))


def tdc_skip(x_in, delta) -> np.ndarray:
    x_in, delta = _u16(x_in), _u16(delta)
    out = np.empty_like(x_in)
    lib().orc_tdc_skip(_ptr(x_in, C.c_uint16), _ptr(delta, C.c_uint16), x_in.size,
                       _ptr(out, C.c_uint16))
    return out


def tdc_refresh(x_in, x_out, delta, delta_valid: bool) -> np.ndarray:
    """Updates ``delta`` in place to the new bf16 delta; returns S1..S4."""
    x_in, x_out = _u16(x_in), _u16(x_out)
    assert delta.dtype == np.uint16 and delta.flags["C_CONTIGUOUS"]
    s = np.zeros(4, np.float64)
    lib().orc_tdc_refresh(_ptr(x_in, C.c_uint16), _ptr(x_out, C.c_uint16),
                          _ptr(delta, C.c_uint16), x_in.size, int(delta_valid),
                          _ptr(s, C.c_double))
    return s


def tdc_commit_skip(st: TdcState) -> None:
    lib().orc_tdc_commit_skip(C.byref(st))


def tdc_commit_refresh(st: TdcState, sums) -> None:
    s = np.ascontiguousarray(sums, np.float64)
    lib().orc_tdc_commit_refresh(C.byref(st), _ptr(s, C.c_double))


def nibbles(codes: np.ndarray) -> np.ndarray:
    """Unpack [R, K/2] packed E2M1 codes into [R, K] 4-bit codes (layout only)."""
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


# ---- Purified Delta Refresh and the BF16 route ------------------------------

def outlier_count(x, kappa: float) -> int:
    """Elements with x^2 * K > kappa^2 * (sum of the row's squares)."""
    x = _u16(x)
    M, K = x.shape
    return int(lib().orc_outlier_count(_ptr(x, C.c_uint16), M, K, float(kappa)))


def outlier_count_band(x, kappa: float, rel: float):
    x = _u16(x)
    M, K = x.shape
    lo, hi = np.zeros(1, np.int64), np.zeros(1, np.int64)
    lib().orc_outlier_count_band(_ptr(x, C.c_uint16), M, K, float(kappa), float(rel),
                                 _ptr(lo, C.c_int64), _ptr(hi, C.c_int64))
    return int(lo[0]), int(hi[0])


def pdr_force(count: int, n: int, rho: float) -> bool:
    return bool(lib().orc_pdr_force(int(count), int(n), float(rho)))


def gemm_bf16(x, w, rows=None):
    """fp64 reference y = x w^T over bf16 operands, and the bound sum |x w|."""
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    r, R = _rows(rows, M)
    y = np.empty((R, N), np.float64)
    b = np.empty((R, N), np.float64)
    rc = lib().orc_gemm_bf16(_ptr(x, C.c_uint16), _ptr(w, C.c_uint16), M, N, K, _ptr(r, C.c_int64), R,
                             _ptr(y, C.c_double), _ptr(b, C.c_double))
    if rc != 0:
        raise ValueError("orc_gemm_bf16: bad shape or row")
    return y, b


def gelu(x):
    """Exact-erf GELU in fp64, elementwise over an array (or a scalar)."""
    f = lib().orc_gelu
    a = np.asarray(x, np.float64)
    return np.vectorize(f, otypes=[np.float64])(a) if a.ndim else float(f(float(a)))
