"""CPU oracle for the MXFP8 quantiser, the fused Gemma RMSNorm quantiser and the
MXFP8 block-scaled GEMM with BF16 output.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does. The
arithmetic lives in ``mxfp8_oracle.c`` (plain C, fp64, written from the format
definitions); this module only marshals numpy arrays through ctypes.

Arrays: BF16 tensors travel as their uint16 bit patterns, E4M3 data and UE8M0
scales as uint8. Scale layouts: 0 = linear [rows, k/32], 1 = 128x4 swizzled.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

LINEAR = 0
SWIZZLED = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    c_dp = ctypes.POINTER(ctypes.c_double)
    c_fp = ctypes.POINTER(ctypes.c_float)
    i64 = ctypes.c_int64
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_ue8m0_value.restype = ctypes.c_double
    lib.oracle_ue8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_scale_exponent.restype = ctypes.c_int
    lib.oracle_scale_exponent.argtypes = [ctypes.c_double]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    lib.oracle_swizzle_offset.restype = i64
    lib.oracle_swizzle_offset.argtypes = [i64, i64, i64]
    lib.oracle_scale_bytes.restype = i64
    lib.oracle_scale_bytes.argtypes = [i64, i64, ctypes.c_int]
    lib.oracle_add_rmsnorm_quant_mxfp8.restype = ctypes.c_int
    lib.oracle_add_rmsnorm_quant_mxfp8.argtypes = [c_u16p, c_u16p, c_u16p, i64, i64, i64, i64, ctypes.c_double,
                                                   c_u8p, c_u8p, c_u8p, c_u16p, ctypes.POINTER(ctypes.c_float)]
    lib.oracle_gemm_silu_mul_quant.restype = ctypes.c_int
    lib.oracle_gemm_silu_mul_quant.argtypes = [c_u8p, c_u8p, ctypes.c_int, c_u8p, c_u8p, ctypes.c_int, i64, i64, i64,
                                               ctypes.POINTER(ctypes.c_int64), i64, c_u8p, c_u8p,
                                               ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    lib.oracle_swizzle_scales.restype = ctypes.c_int
    lib.oracle_swizzle_scales.argtypes = [c_u8p, i64, i64, c_u8p]
    lib.oracle_mxfp8_quantize.restype = ctypes.c_int
    lib.oracle_mxfp8_quantize.argtypes = [c_u16p, i64, i64, i64, c_u8p, c_u8p, c_u8p]
    lib.oracle_rmsnorm_quant_mxfp8.restype = ctypes.c_int
    lib.oracle_rmsnorm_quant_mxfp8.argtypes = [c_u16p, c_u16p, i64, i64, i64, ctypes.c_double,
                                               c_u8p, c_u8p, c_u8p, c_fp]
    lib.oracle_mxfp8_gemm_bf16out.restype = ctypes.c_int
    lib.oracle_mxfp8_gemm_bf16out.argtypes = [c_u8p, c_u8p, ctypes.c_int, c_u8p, c_u8p, ctypes.c_int,
                                              i64, i64, i64, c_u16p, i64, c_dp]
    lib.oracle_mxfp8_gemm_sampled.restype = ctypes.c_int
    lib.oracle_mxfp8_gemm_sampled.argtypes = [c_u8p, c_u8p, ctypes.c_int, c_u8p, c_u8p, ctypes.c_int,
                                              i64, i64, i64, c_i64p, c_i64p, i64, c_u16p, c_dp]
    lib.oracle_gemm_accum_terms.restype = ctypes.c_int
    lib.oracle_gemm_accum_terms.argtypes = [c_u8p, c_u8p, ctypes.c_int, c_u8p, c_u8p, ctypes.c_int, i64, i64, i64,
                                            c_i64p, c_i64p, i64, ctypes.c_int, c_dp, c_dp]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(arr, ctype):
    if arr is None:
        return None
    assert arr.flags["C_CONTIGUOUS"]
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> int:
    """Threads for later oracle calls; returns the previous count."""
    return _load().oracle_set_num_threads(int(n))


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def e4m3_values() -> np.ndarray:
    """Values of all 256 E4M3 codes (float64; NaN for 0x7F and 0xFF)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)


def ue8m0_value(code: int) -> float:
    return _load().oracle_ue8m0_value(int(code))


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 codes (RNE, satfinite) of fp64 values."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.oracle_e4m3_encode(float(x)) for x in v], dtype=np.uint8).reshape(np.shape(values))


def scale_exponent(amax: float) -> int:
    return _load().oracle_scale_exponent(float(amax))


def bf16_from_double(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([lib.oracle_bf16_from_double(float(x)) for x in v], dtype=np.uint16).reshape(np.shape(values))


def swizzle_offset(r: int, c: int, nblk: int) -> int:
    return _load().oracle_swizzle_offset(r, c, nblk)


def scale_bytes(rows: int, k: int, layout: int) -> int:
    return _load().oracle_scale_bytes(rows, k, layout)


def gemm_silu_mul_quant(a, a_scales, a_layout, w, w_scales, w_layout, rows=None, want_gu=False):
    """Fused dense GEMM1: ``y = silu(A W_gate^T) * (A W_up^T)`` quantised per 32 along the
    intermediate dimension. ``w`` is E4M3 ``[2*inter, k]`` (gate rows, then up rows).

    ``rows`` (default: all) selects rows of ``a``; returns ``(q [nrows, inter] u8,
    s_lin [nrows, inter/32] u8, y32 [nrows, inter] f32)`` plus the fp64 ``[nrows, 2*inter]``
    gate/up values when ``want_gu``.
    """
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    sa = np.ascontiguousarray(a_scales, dtype=np.uint8)
    sw = np.ascontiguousarray(w_scales, dtype=np.uint8)
    m, k = a.shape
    inter = w.shape[0] // 2
    r = np.arange(m, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    q = np.empty((r.size, inter), dtype=np.uint8)
    s_lin = np.empty((r.size, inter // 32), dtype=np.uint8)
    y = np.empty((r.size, inter), dtype=np.float32)
    gu = np.empty((r.size, 2 * inter), dtype=np.float64) if want_gu else None
    _check(lib.oracle_gemm_silu_mul_quant(
        _ptr(a, ctypes.c_uint8), _ptr(sa, ctypes.c_uint8), int(a_layout), _ptr(w, ctypes.c_uint8),
        _ptr(sw, ctypes.c_uint8), int(w_layout), m, inter, k, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        r.size, _ptr(q, ctypes.c_uint8), _ptr(s_lin, ctypes.c_uint8), y.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
        None if gu is None else gu.ctypes.data_as(ctypes.POINTER(ctypes.c_double))), "oracle_gemm_silu_mul_quant")
    return (q, s_lin, y, gu) if want_gu else (q, s_lin, y)


def swizzle_scales(s_lin: np.ndarray) -> np.ndarray:
    """Linear scales [rows, k/32] u8 -> flat swizzled buffer (pad bytes 0)."""
    lib = _load()
    s = np.ascontiguousarray(s_lin, dtype=np.uint8)
    rows, nblk = s.shape
    out = np.empty(scale_bytes(rows, 32 * nblk, SWIZZLED), dtype=np.uint8)
    if rows:
        _check(lib.oracle_swizzle_scales(_ptr(s, ctypes.c_uint8), rows, 32 * nblk, _ptr(out, ctypes.c_uint8)),
               "oracle_swizzle_scales")
    return out


def quantize(x_bits: np.ndarray, k: int = None):
    """BF16 bits [rows, ldx] -> (codes [rows,k] u8, linear scales [rows,k/32] u8, swizzled scales u8).

    ``k`` (default: the row length) quantises only the first k columns of each row.
    """
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, ldx = x.shape
    k = ldx if k is None else int(k)
    q = np.empty((rows, k), dtype=np.uint8)
    s_lin = np.empty((rows, k // 32), dtype=np.uint8)
    s_swz = np.empty(scale_bytes(rows, k, SWIZZLED), dtype=np.uint8)
    _check(lib.oracle_mxfp8_quantize(_ptr(x, ctypes.c_uint16), rows, k, ldx, _ptr(q, ctypes.c_uint8),
                                     _ptr(s_lin, ctypes.c_uint8), _ptr(s_swz, ctypes.c_uint8)), "quantize")
    return q, s_lin, s_swz


def rmsnorm_quant(x_bits: np.ndarray, w_bits: np.ndarray, eps: float):
    """Gemma RMSNorm + MXFP8 quantisation. Returns (codes, linear scales, swizzled scales, y fp32)."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, h = x.shape
    assert w.shape == (h,)
    q = np.empty((rows, h), dtype=np.uint8)
    s_lin = np.empty((rows, h // 32), dtype=np.uint8)
    s_swz = np.empty(scale_bytes(rows, h, SWIZZLED), dtype=np.uint8)
    y = np.empty((rows, h), dtype=np.float32)
    _check(lib.oracle_rmsnorm_quant_mxfp8(_ptr(x, ctypes.c_uint16), _ptr(w, ctypes.c_uint16), rows, h, h,
                                          float(eps), _ptr(q, ctypes.c_uint8), _ptr(s_lin, ctypes.c_uint8),
                                          _ptr(s_swz, ctypes.c_uint8), _ptr(y, ctypes.c_float)), "rmsnorm_quant")
    return q, s_lin, s_swz, y


def add_rmsnorm_quant(x_bits: np.ndarray, r_bits: np.ndarray, w_bits: np.ndarray, eps: float):
    """Residual add h = BF16(x + r), then Gemma RMSNorm + MXFP8 quantisation of h.
    Returns (codes, linear scales, swizzled scales, h BF16 bits, y fp32)."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    r = np.ascontiguousarray(r_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, h = x.shape
    assert r.shape == x.shape and w.shape == (h,)
    q = np.empty((rows, h), dtype=np.uint8)
    s_lin = np.empty((rows, h // 32), dtype=np.uint8)
    s_swz = np.empty(scale_bytes(rows, h, SWIZZLED), dtype=np.uint8)
    hb = np.empty((rows, h), dtype=np.uint16)
    y = np.empty((rows, h), dtype=np.float32)
    _check(lib.oracle_add_rmsnorm_quant_mxfp8(_ptr(x, ctypes.c_uint16), _ptr(r, ctypes.c_uint16),
                                              _ptr(w, ctypes.c_uint16), rows, h, h, h, float(eps),
                                              _ptr(q, ctypes.c_uint8), _ptr(s_lin, ctypes.c_uint8),
                                              _ptr(s_swz, ctypes.c_uint8), _ptr(hb, ctypes.c_uint16),
                                              _ptr(y, ctypes.c_float)), "add_rmsnorm_quant")
    return q, s_lin, s_swz, hb, y


def gemm(a, a_scales, a_layout, b, b_scales, b_layout, want_f64=False):
    """C = A B^T with block scales. a [m,k] u8, b [n,k] u8. Returns BF16 bits [m,n] (and fp64 values)."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    as_ = np.ascontiguousarray(a_scales, dtype=np.uint8)
    bs_ = np.ascontiguousarray(b_scales, dtype=np.uint8)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    c = np.empty((m, n), dtype=np.uint16)
    f = np.empty((m, n), dtype=np.float64) if want_f64 else None
    _check(lib.oracle_mxfp8_gemm_bf16out(_ptr(a, ctypes.c_uint8), _ptr(as_, ctypes.c_uint8), a_layout,
                                         _ptr(b, ctypes.c_uint8), _ptr(bs_, ctypes.c_uint8), b_layout,
                                         m, n, k, _ptr(c, ctypes.c_uint16), n, _ptr(f, ctypes.c_double)), "gemm")
    return (c, f) if want_f64 else c


def gemm_sampled(a, a_scales, a_layout, b, b_scales, b_layout, rows, cols):
    """Selected elements C[rows[t], cols[t]]. Returns (BF16 bits [t], fp64 values [t])."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    as_ = np.ascontiguousarray(a_scales, dtype=np.uint8)
    bs_ = np.ascontiguousarray(b_scales, dtype=np.uint8)
    m, k = a.shape
    n = b.shape[0]
    r = np.ascontiguousarray(rows, dtype=np.int64)
    cc = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(r.shape[0], dtype=np.uint16)
    f = np.empty(r.shape[0], dtype=np.float64)
    _check(lib.oracle_mxfp8_gemm_sampled(_ptr(a, ctypes.c_uint8), _ptr(as_, ctypes.c_uint8), a_layout,
                                         _ptr(b, ctypes.c_uint8), _ptr(bs_, ctypes.c_uint8), b_layout,
                                         m, n, k, _ptr(r, ctypes.c_int64), _ptr(cc, ctypes.c_int64), r.shape[0],
                                         _ptr(out, ctypes.c_uint16), _ptr(f, ctypes.c_double)), "gemm_sampled")
    return out, f


def gemm_accum_terms(a, a_scales, a_layout, b, b_scales, b_layout, rows=None, cols=None, trunc_bits=13):
    """Error-budget terms of a hardware accumulation of C = A B^T (``accum_bound.c``): for each
    element (rows[t], cols[t]) (default: every element, row-major) the truncation loss T of
    aligning each group of 8 products to its largest and keeping ``trunc_bits`` bits below the
    leading one, and the absolute mass S = sum_k |A_mk B_nk| (scales included). Returns (T, S)
    as fp64 arrays, shaped [m, n] when every element is requested."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    as_ = np.ascontiguousarray(a_scales, dtype=np.uint8)
    bs_ = np.ascontiguousarray(b_scales, dtype=np.uint8)
    m, k = a.shape
    n = b.shape[0]
    full = rows is None
    if full:
        r = np.repeat(np.arange(m, dtype=np.int64), n)
        cc = np.tile(np.arange(n, dtype=np.int64), m)
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        cc = np.ascontiguousarray(cols, dtype=np.int64)
    t = np.empty(r.shape[0], dtype=np.float64)
    s = np.empty(r.shape[0], dtype=np.float64)
    _check(lib.oracle_gemm_accum_terms(_ptr(a, ctypes.c_uint8), _ptr(as_, ctypes.c_uint8), a_layout,
                                       _ptr(b, ctypes.c_uint8), _ptr(bs_, ctypes.c_uint8), b_layout, m, n, k,
                                       _ptr(r, ctypes.c_int64), _ptr(cc, ctypes.c_int64), r.shape[0],
                                       int(trunc_bits), _ptr(t, ctypes.c_double), _ptr(s, ctypes.c_double)),
           "gemm_accum_terms")
    return (t.reshape(m, n), s.reshape(m, n)) if full else (t, s)
