"""MI355X (gfx950) MXFP8 quantiser, fused Gemma RMSNorm quantiser, scale swizzle and block-scaled GEMM.

A thin ctypes binding over ``libmxfp8_amd.so`` (C ABI: ``include/mxfp8.h``). Every step of
the computation runs in the library's HIP kernels; this module only checks tensor
placement, allocates outputs with torch and passes raw device pointers together with
torch's current HIP stream. There is no CPU fallback: without the built library (or
without a GPU) every call raises.

Data conventions (vLLM PR #64659 "Details: GEMM-RS with a quantized input", PR #65496
"Details"): E4M3 data travels as ``torch.uint8`` tensors, UE8M0 scales as ``torch.uint8``
(linear ``[rows, k/32]`` or the flat 128x4-swizzled buffer), BF16 as ``torch.bfloat16``.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp8_amd.so")

LINEAR = 0
SWIZZLED = 1

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4

_lib = None


class MXFP8Error(RuntimeError):
    """A call into libmxfp8_amd returned a non-zero status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load_library():
    """Load libmxfp8_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quant_mxfp8_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.mxfp8_scale_bytes.restype = i64
    lib.mxfp8_scale_bytes.argtypes = [i64, i64, i32]
    lib.mxfp8_status_string.restype = ctypes.c_char_p
    lib.mxfp8_status_string.argtypes = [i32]
    lib.mxfp8_quantize.restype = i32
    lib.mxfp8_quantize.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    lib.mxfp8_quantize_check.restype = i32
    lib.mxfp8_quantize_check.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.rmsnorm_quant_mxfp8.restype = i32
    lib.rmsnorm_quant_mxfp8.argtypes = [vp, vp, i64, i64, i64, f32, vp, vp, vp, vp]
    lib.rmsnorm_quant_mxfp8_check.restype = i32
    lib.rmsnorm_quant_mxfp8_check.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
    lib.add_rmsnorm_quant_mxfp8.restype = i32
    lib.add_rmsnorm_quant_mxfp8.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, vp, vp, vp, vp]
    lib.add_rmsnorm_quant_mxfp8_check.restype = i32
    lib.add_rmsnorm_quant_mxfp8_check.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.mxfp8_swizzle_scales.restype = i32
    lib.mxfp8_swizzle_scales.argtypes = [vp, i64, i64, vp, vp]
    lib.mxfp8_swizzle_scales_check.restype = i32
    lib.mxfp8_swizzle_scales_check.argtypes = [vp, i64, i64, vp]
    lib.mxfp8_gemm_bf16out.restype = i32
    lib.mxfp8_gemm_bf16out.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, i64, i32, i32, vp, vp]
    lib.mxfp8_gemm_bf16out_check.restype = i32
    lib.mxfp8_gemm_bf16out_check.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, i64, i32, i32]
    lib.mxfp8_gemm_silu_mul_quant.restype = i32
    lib.mxfp8_gemm_silu_mul_quant.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp]
    lib.mxfp8_gemm_silu_mul_quant_check.restype = i32
    lib.mxfp8_gemm_silu_mul_quant_check.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, vp, vp]
    lib.mxfp8_gemm_tiles_per_chunk.restype = i64
    lib.mxfp8_gemm_tiles_per_chunk.argtypes = [i64, i64, i32, i32, i32]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mxfp8_status_string(int(status)).decode()


def scale_bytes(rows: int, k: int, layout: int) -> int:
    n = load_library().mxfp8_scale_bytes(int(rows), int(k), int(layout))
    if n < 0:
        raise MXFP8Error("mxfp8_scale_bytes", EINVAL)
    return n


def gemm_tiles_per_chunk(m: int, n: int, num_chunks: int, a_layout: int, b_layout: int) -> int:
    """Output tiles per chunk of ``gemm`` with these scale layouts (the final ``chunk_done`` value)."""
    t = load_library().mxfp8_gemm_tiles_per_chunk(int(m), int(n), int(num_chunks), int(a_layout), int(b_layout))
    if t < 0:
        raise MXFP8Error("mxfp8_gemm_tiles_per_chunk", EINVAL)
    return t


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _same_device(ref: torch.Tensor, **tensors):
    """Every tensor (None skipped) is a GPU tensor on ref's device."""
    _dev(ref, "input")
    for name, t in tensors.items():
        if t is not None and _dev(t, name).device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {ref.device}")


def _u8_buffer(t, name: str, numel: int = None, shape=None):
    """A contiguous uint8 tensor of the given shape, or of at least numel bytes. The library
    cannot see buffer sizes, so an undersized buffer is rejected here rather than becoming an
    out-of-bounds device access."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} bytes, {numel} are needed")
    return t


def _quant_outputs(out, rows: int, k: int, linear: bool, swizzled: bool, like: torch.Tensor):
    """Checked caller-provided (q, scales_linear, scales_swizzled), or new ones on like's device."""
    if out is None:
        q = torch.empty((rows, k), dtype=torch.uint8, device=like.device)
        s_lin = torch.empty((rows, k // 32), dtype=torch.uint8, device=like.device) if linear else None
        s_swz = torch.empty(scale_bytes(rows, k, SWIZZLED), dtype=torch.uint8, device=like.device) if swizzled else None
        return q, s_lin, s_swz
    q, s_lin, s_swz = out
    _u8_buffer(q, "q", shape=(rows, k))
    if s_lin is not None:
        _u8_buffer(s_lin, "scales_linear", shape=(rows, k // 32))
    if s_swz is not None:
        _u8_buffer(s_swz, "scales_swizzled", numel=scale_bytes(rows, k, SWIZZLED))
    if s_lin is None and s_swz is None:
        raise ValueError("at least one scale layout must be requested")
    return q, s_lin, s_swz


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows_view(x: torch.Tensor, name: str, dtype):
    if not isinstance(x, torch.Tensor) or x.dtype != dtype or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D {dtype} tensor with unit column stride")
    return x


def quantize(x: torch.Tensor, linear: bool = True, swizzled: bool = True, out=None):
    """BF16 ``x [rows, k]`` (row stride may exceed k) -> ``(q [rows,k] u8, scales_linear, scales_swizzled)``.

    ``out`` may pass preallocated ``(q, s_lin, s_swz)``; a scale layout not requested is None.
    """
    _rows_view(x, "x", torch.bfloat16)
    rows, k = x.shape
    if k % 32 != 0:
        raise ValueError("k must be a multiple of 32")
    q, s_lin, s_swz = _quant_outputs(out, rows, k, linear, swizzled, x)
    _same_device(x, q=q, scales_linear=s_lin, scales_swizzled=s_swz)
    st = load_library().mxfp8_quantize(_ptr(x), rows, k, x.stride(0), _ptr(q), _ptr(s_lin), _ptr(s_swz), _stream(x))
    if st != OK:
        raise MXFP8Error("mxfp8_quantize", st)
    return q, s_lin, s_swz


def rmsnorm_quant(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, linear: bool = True,
                  swizzled: bool = True, out=None):
    """Gemma RMSNorm ``x / sqrt(mean(x^2) + eps) * (1 + w)`` quantised to MXFP8 in one pass.

    Returns ``(q [rows, hidden] u8, scales_linear, scales_swizzled)``.
    """
    _rows_view(x, "x", torch.bfloat16)
    rows, h = x.shape
    if h % 32 != 0:
        raise ValueError("hidden must be a multiple of 32")
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or tuple(w.shape) != (h,) or not w.is_contiguous():
        raise ValueError("w must be a contiguous bfloat16 [hidden] tensor")
    q, s_lin, s_swz = _quant_outputs(out, rows, h, linear, swizzled, x)
    _same_device(x, w=w, q=q, scales_linear=s_lin, scales_swizzled=s_swz)
    st = load_library().rmsnorm_quant_mxfp8(_ptr(x), _ptr(w), rows, h, x.stride(0), float(eps), _ptr(q),
                                            _ptr(s_lin), _ptr(s_swz), _stream(x))
    if st != OK:
        raise MXFP8Error("rmsnorm_quant_mxfp8", st)
    return q, s_lin, s_swz


def add_rmsnorm_quant(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                      linear: bool = True, swizzled: bool = True, out=None):
    """Residual add then Gemma RMSNorm quantised to MXFP8: ``residual <- BF16(x + residual)`` (in
    place), then the norm quantiser of the updated residual. Returns ``(q, scales_linear,
    scales_swizzled)``."""
    _rows_view(x, "x", torch.bfloat16)
    _rows_view(residual, "residual", torch.bfloat16)
    rows, h = x.shape
    if h % 32 != 0:
        raise ValueError("hidden must be a multiple of 32")
    if residual.shape != x.shape:
        raise ValueError("residual must have the shape of x")
    if not isinstance(w, torch.Tensor) or w.dtype != torch.bfloat16 or tuple(w.shape) != (h,) or not w.is_contiguous():
        raise ValueError("w must be a contiguous bfloat16 [hidden] tensor")
    q, s_lin, s_swz = _quant_outputs(out, rows, h, linear, swizzled, x)
    _same_device(x, residual=residual, w=w, q=q, scales_linear=s_lin, scales_swizzled=s_swz)
    st = load_library().add_rmsnorm_quant_mxfp8(_ptr(x), _ptr(residual), _ptr(w), rows, h, x.stride(0),
                                                residual.stride(0), float(eps), _ptr(q), _ptr(s_lin), _ptr(s_swz),
                                                _stream(x))
    if st != OK:
        raise MXFP8Error("add_rmsnorm_quant_mxfp8", st)
    return q, s_lin, s_swz


def swizzle_scales(scales_linear: torch.Tensor, k: int = None, out: torch.Tensor = None) -> torch.Tensor:
    """Linear UE8M0 scales ``[rows, k/32]`` u8 -> the flat 128x4-swizzled buffer (pad bytes 0),
    the step after gathering MXFP8 activations by rows. ``k`` defaults to 32 x the column count."""
    if not isinstance(scales_linear, torch.Tensor) or scales_linear.dim() != 2:
        raise ValueError("scales_linear must be a contiguous 2-D uint8 tensor")
    _u8_buffer(scales_linear, "scales_linear")
    rows, nblk = scales_linear.shape
    k = 32 * nblk if k is None else int(k)
    if k != 32 * nblk or nblk == 0:
        raise ValueError("k must be 32 x the number of scale columns")
    if out is None:
        out = torch.empty(scale_bytes(rows, k, SWIZZLED), dtype=torch.uint8, device=scales_linear.device)
    _u8_buffer(out, "out", numel=scale_bytes(rows, k, SWIZZLED))
    _same_device(scales_linear, out=out)
    st = load_library().mxfp8_swizzle_scales(_ptr(scales_linear), rows, k, _ptr(out), _stream(scales_linear))
    if st != OK:
        raise MXFP8Error("mxfp8_swizzle_scales", st)
    return out


def gemm(a: torch.Tensor, a_scales: torch.Tensor, a_layout: int, b: torch.Tensor, b_scales: torch.Tensor,
         b_layout: int, out: torch.Tensor = None, num_chunks: int = 1, first_chunk: int = 0,
         chunk_done: torch.Tensor = None) -> torch.Tensor:
    """``C[m,n] = sum_k A[m,k] B[n,k]`` with UE8M0 block scales, BF16 out.

    ``a`` E4M3 ``[m,k]`` u8 and ``b`` E4M3 ``[n,k]`` u8 (both contiguous); scales in the given
    layouts. ``out`` (BF16 ``[m, >=n]``, unit column stride) is allocated when None. The output is
    produced as ``num_chunks`` row chunks starting with ``first_chunk``; ``chunk_done`` (int32
    ``[num_chunks]``, zeroed by the caller) counts finished tiles per chunk.
    """
    for t, nm in ((a, "a"), (b, "b")):
        _u8_buffer(t, nm)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a must be [m, k] and b [n, k]")
    m, k = a.shape
    n = b.shape[0]
    if k % 32 != 0 or int(a_layout) not in (LINEAR, SWIZZLED) or int(b_layout) not in (LINEAR, SWIZZLED):
        raise ValueError("k must be a multiple of 32 and the scale layouts LINEAR or SWIZZLED")
    _u8_buffer(a_scales, "a_scales", numel=scale_bytes(m, k, a_layout))
    _u8_buffer(b_scales, "b_scales", numel=scale_bytes(n, k, b_layout))
    if out is None:
        ldc = (n + 3) // 4 * 4  # the kernels store 4 columns at a time: keep rows 8-byte aligned
        out = torch.empty((m, ldc), dtype=torch.bfloat16, device=a.device)[:, :n]
    _rows_view(out, "out", torch.bfloat16)
    if out.shape[0] != m or out.shape[1] < n:
        raise ValueError("out must be [m, >=n]")
    if chunk_done is not None:
        if not isinstance(chunk_done, torch.Tensor) or chunk_done.dtype != torch.int32 or \
                chunk_done.numel() < num_chunks or not chunk_done.is_contiguous():
            raise ValueError("chunk_done must be a contiguous int32 tensor with num_chunks entries")
    _same_device(a, b=b, a_scales=a_scales, b_scales=b_scales, out=out, chunk_done=chunk_done)
    st = load_library().mxfp8_gemm_bf16out(_ptr(a), _ptr(a_scales), int(a_layout), _ptr(b), _ptr(b_scales),
                                           int(b_layout), m, n, k, _ptr(out), out.stride(0), int(num_chunks),
                                           int(first_chunk), _ptr(chunk_done), _stream(a))
    if st != OK:
        raise MXFP8Error("mxfp8_gemm_bf16out", st)
    return out


def gemm_silu_mul_quant(a: torch.Tensor, a_scales: torch.Tensor, a_layout: int, w: torch.Tensor,
                        w_scales: torch.Tensor, w_layout: int, linear: bool = False, swizzled: bool = True,
                        out=None):
    """Fused dense GEMM1: ``y = SiLU(A W_gate^T) * (A W_up^T)`` quantised to MXFP8.

    ``a`` E4M3 ``[m, k]`` u8, ``w`` E4M3 ``[2*inter, k]`` u8 (gate rows, then up rows), both
    contiguous, scales in the given layouts. Returns ``(q [m, inter] u8, scales_linear,
    scales_swizzled)``; ``out`` may pass them preallocated.
    """
    for t, nm in ((a, "a"), (w, "w")):
        _u8_buffer(t, nm)
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1] or w.shape[0] % 2 != 0:
        raise ValueError("a must be [m, k] and w [2*inter, k]")
    m, k = a.shape
    inter = w.shape[0] // 2
    if k % 32 != 0 or inter % 32 != 0 or int(a_layout) not in (LINEAR, SWIZZLED) or \
            int(w_layout) not in (LINEAR, SWIZZLED):
        raise ValueError("k and inter must be multiples of 32 and the scale layouts LINEAR or SWIZZLED")
    _u8_buffer(a_scales, "a_scales", numel=scale_bytes(m, k, a_layout))
    _u8_buffer(w_scales, "w_scales", numel=scale_bytes(2 * inter, k, w_layout))
    q, s_lin, s_swz = _quant_outputs(out, m, inter, linear, swizzled, a)
    _same_device(a, w=w, a_scales=a_scales, w_scales=w_scales, q=q, scales_linear=s_lin, scales_swizzled=s_swz)
    st = load_library().mxfp8_gemm_silu_mul_quant(_ptr(a), _ptr(a_scales), int(a_layout), _ptr(w), _ptr(w_scales),
                                                  int(w_layout), m, inter, k, _ptr(q), _ptr(s_lin), _ptr(s_swz),
                                                  _stream(a))
    if st != OK:
        raise MXFP8Error("mxfp8_gemm_silu_mul_quant", st)
    return q, s_lin, s_swz
