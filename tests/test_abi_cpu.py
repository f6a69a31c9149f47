"""The C ABI on the host (no GPU): the library loads, exports every function that
include/*.h declares, and its argument checks return the documented status codes
without touching the GPU."""
import ctypes
import glob
import os
import re

import pytest

import quant_mxfp8_gemm_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EALIGN, EUNSUP = mx.OK, mx.EINVAL, mx.EALIGN, mx.EUNSUPPORTED


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        import quant_mxfp8_gemm_amd.build as b
        b.build()
    return mx.load_library()


def test_header_declares_the_three_operations():
    names = _declared_functions()
    for f in ("mxfp8_quantize", "rmsnorm_quant_mxfp8", "mxfp8_gemm_bf16out", "mxfp8_swizzle_scales",
              "mxfp8_gemm_silu_mul_quant", "add_rmsnorm_quant_mxfp8", "mxfp8_scale_bytes",
              "mxfp8_status_string"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    for name in sorted(_declared_functions()):
        assert hasattr(lib, name), name


def test_scale_bytes(lib):
    assert mx.scale_bytes(128, 128, mx.LINEAR) == 128 * 4
    assert mx.scale_bytes(1024, 6144, mx.SWIZZLED) == 1024 * 192
    assert mx.scale_bytes(200, 96, mx.SWIZZLED) == 256 * 4
    assert mx.scale_bytes(1, 32, mx.SWIZZLED) == 512
    assert lib.mxfp8_scale_bytes(10, 33, 0) == -1
    assert lib.mxfp8_scale_bytes(10, 64, 7) == -1
    assert lib.mxfp8_scale_bytes(-1, 64, 0) == -1


def test_status_strings(lib):
    for st in (OK, EINVAL, EALIGN, EUNSUP, mx.EHIP):
        assert mx.status_string(st) and mx.status_string(st) != "unknown status"
    assert mx.status_string(12345) == "unknown status"


P = 1 << 20  # a fake 1 MiB-aligned address: the checks never dereference pointers


def test_quantize_check(lib):
    c = lib.mxfp8_quantize_check
    assert c(P, 128, 2048, 2048, P, P, P) == OK
    assert c(P, 128, 2048, 2048, P, None, P) == OK
    assert c(P, 0, 2048, 2048, P, P, None) == OK
    assert c(None, 0, 2048, 2048, None, None, None) == OK  # rows == 0: nothing is touched
    assert c(P, 128, 2047, 2048, P, P, P) == EINVAL      # k % 32
    assert c(P, 128, 2048, 2040, P, P, P) == EINVAL      # ldx < k
    assert c(P, -1, 2048, 2048, P, P, P) == EINVAL
    assert c(P, 128, 2048, 2048, P, None, None) == EINVAL
    assert c(None, 128, 2048, 2048, P, P, P) == EINVAL
    assert c(P + 8, 128, 2048, 2048, P, P, P) == EALIGN   # x not 16-byte aligned
    assert c(P, 128, 2048, 2052, P, P, P) == EALIGN       # ldx % 8
    assert c(P, 128, 2048, 2048, P + 4, P, P) == EALIGN   # q not 8-byte aligned


def test_rmsnorm_check(lib):
    c = lib.rmsnorm_quant_mxfp8_check
    assert c(P, P, 1024, 6144, 6144, P, P, P) == OK
    assert c(P, P, 1024, 6144, 6144, P, None, None) == EINVAL
    assert c(P, None, 1024, 6144, 6144, P, P, P) == EINVAL
    assert c(P, P, 1024, 6150, 6150, P, P, P) == EINVAL
    assert c(P, P, 1024, 32768, 32768, P, P, P) == EUNSUP
    assert c(P, P + 2, 1024, 6144, 6144, P, P, P) == EALIGN


def test_add_rmsnorm_check(lib):
    c = lib.add_rmsnorm_quant_mxfp8_check
    R = P + (64 << 20)   # a residual buffer well clear of x
    assert c(P, R, P, 1024, 6144, 6144, 6144, P, P, P) == OK
    assert c(None, None, None, 0, 6144, 6144, 6144, None, None, None) == OK
    assert c(P, None, P, 1024, 6144, 6144, 6144, P, P, P) == EINVAL     # no residual
    assert c(P, R, P, 1024, 6144, 6144, 6000, P, P, P) == EINVAL        # ldr < hidden
    assert c(P, R + 8, P, 1024, 6144, 6144, 6144, P, P, P) == EALIGN    # residual alignment
    assert c(P, R, P, 1024, 6144, 6144, 6148, P, P, P) == EALIGN        # ldr % 8
    assert c(P, P + 4096, P, 1024, 6144, 6144, 6144, P, P, P) == EINVAL  # overlaps x
    assert c(P, R, P, 1024, 6150, 6150, 6150, P, P, P) == EINVAL        # hidden % 32


def test_swizzle_check(lib):
    c = lib.mxfp8_swizzle_scales_check
    assert c(P, 1024, 6144, P) == OK
    assert c(P + 1, 1024, 6144, P) == OK          # linear scales may sit at any byte
    assert c(None, 0, 6144, None) == OK           # rows == 0: nothing is touched
    assert c(P, 1024, 6150, P) == EINVAL          # k % 32
    assert c(P, -1, 6144, P) == EINVAL
    assert c(None, 1024, 6144, P) == EINVAL
    assert c(P, 1024, 6144, None) == EINVAL
    assert c(P, 1024, 6144, P + 8) == EALIGN      # output not 16-byte aligned


def test_gemm_check(lib):
    c = lib.mxfp8_gemm_bf16out_check
    good = dict(a=P, sa=P, la=0, b=P, sb=P, lb=1, m=4096, n=6144, k=3072, c=P, ldc=6144, nc=4, fc=0)

    def call(**kw):
        d = dict(good)
        d.update(kw)
        return c(d["a"], d["sa"], d["la"], d["b"], d["sb"], d["lb"], d["m"], d["n"], d["k"], d["c"], d["ldc"],
                 d["nc"], d["fc"])

    assert call() == OK
    assert call(m=0) == EINVAL
    assert call(k=3000) == EINVAL          # k % 32
    assert call(k=3040) == EUNSUP          # k % 128
    assert call(la=2) == EINVAL
    assert call(ldc=6000) == EINVAL
    assert call(nc=3) == EINVAL            # 4096 % 3
    assert call(fc=4) == EINVAL
    assert call(fc=-1) == EINVAL
    assert call(nc=0) == EINVAL
    assert call(sb=None) == EINVAL
    assert call(a=P + 8) == EALIGN
    assert call(sa=P + 2) == EALIGN
    assert call(c=P + 4) == EALIGN
    assert call(ldc=6146) == EALIGN
    assert call(m=1 << 20, k=3072) == EUNSUP   # operand beyond 2 GiB


def test_gemm_silu_mul_quant_check(lib):
    c = lib.mxfp8_gemm_silu_mul_quant_check
    good = dict(a=P, sa=P, la=1, w=P, sw=P, lw=1, m=32768, i=3072, k=6144, q=P, sl=None, sz=P)

    def call(**kw):
        d = dict(good)
        d.update(kw)
        return c(d["a"], d["sa"], d["la"], d["w"], d["sw"], d["lw"], d["m"], d["i"], d["k"], d["q"], d["sl"], d["sz"])

    assert call() == OK
    assert call(sl=P, sz=None) == OK
    assert call(sl=None, sz=None) == EINVAL     # no scale output
    assert call(m=0) == EINVAL
    assert call(i=3000) == EINVAL              # inter % 32
    assert call(i=0) == EINVAL
    assert call(k=6150) == EINVAL              # k % 32
    assert call(k=6176) == EUNSUP              # k % 128
    assert call(la=3) == EINVAL
    assert call(w=None) == EINVAL
    assert call(q=P + 8) == EALIGN             # codes 16-byte aligned
    assert call(a=P + 4) == EALIGN
    assert call(sw=P + 2) == EALIGN
    assert call(m=1 << 20, k=6144) == EUNSUP   # A beyond 2 GiB


def test_tiles_per_chunk(lib):
    """Tile counts per chunk (linear scales unless stated): the tile follows m, n, the chunking
    and, where the two-group kernel applies, the scale layouts."""
    t = mx.gemm_tiles_per_chunk(32768, 6144, 4, 0, 0)
    assert t > 0 and t * 4 * 256 * 256 >= 32768 * 6144
    assert lib.mxfp8_gemm_tiles_per_chunk(10, 10, 3, 0, 0) == -1
    assert lib.mxfp8_gemm_tiles_per_chunk(32, 32, 1, 2, 0) == -1   # no such scale layout
    # the tile shrinks when a 256 x 256 tiling leaves the compute units idle
    assert mx.gemm_tiles_per_chunk(32768, 6144, 4, 0, 0) == 32 * 24    # 256 x 256
    assert mx.gemm_tiles_per_chunk(1024, 6144, 4, 0, 0) == 2 * 32      # 128 x 192: one full round
    assert mx.gemm_tiles_per_chunk(512, 6144, 4, 0, 0) == 1 * 48       # 128 x 128
    assert mx.gemm_tiles_per_chunk(128, 6144, 1, 0, 0) == 4 * 48       # 32 x 128
    assert mx.gemm_tiles_per_chunk(128, 6144, 4, 0, 0) == 1 * 48       # 32 x 128
    assert mx.gemm_tiles_per_chunk(33, 6144, 1, 0, 0) == 2 * 48
    assert mx.gemm_tiles_per_chunk(32, 6144, 1, 0, 0) == 192           # 32 x 32, register-loaded
    assert mx.gemm_tiles_per_chunk(1, 6144, 1, 0, 0) == 192
    assert mx.gemm_tiles_per_chunk(32, 6144, 2, 0, 0) == 48            # 32 x 128 (two chunks)
    assert mx.gemm_tiles_per_chunk(4096, 6144, 4, 0, 0) == 4 * 32      # 256 x 192: two full rounds
    assert mx.gemm_tiles_per_chunk(3072, 6144, 4, 0, 0) == 4 * 32      # 192 x 192: 768 rows per chunk, no empty rows
    assert mx.gemm_tiles_per_chunk(3000, 6144, 4, 0, 0) == 4 * 32      # 192 x 192 (256 x 192 would give 3 x 32)
    assert mx.gemm_tiles_per_chunk(700, 6144, 4, 0, 0) == 2 * 32       # 96 x 192 for 175 rows (128 x 128 would give 2 x 48)
    assert mx.gemm_tiles_per_chunk(256, 6144, 1, 0, 0) == 4 * 48       # 64 x 128
    assert mx.gemm_tiles_per_chunk(128, 6144, 1, 0, 0) == 4 * 48       # 32 x 128
    # both scales swizzled, chunks on 64-row boundaries: the two-group 256 x 192 tile replaces
    # the staged 192 x 192 one once a chunk has 256 rows
    assert mx.gemm_tiles_per_chunk(3072, 6144, 4, 1, 1) == 3 * 32    # 256 x 192
    assert mx.gemm_tiles_per_chunk(3072, 6144, 4, 0, 1) == 4 * 32    # 192 x 192 (one linear)
    assert mx.gemm_tiles_per_chunk(1536, 6144, 4, 1, 1) == 2 * 32    # 256 x 192 over 384 rows
    assert mx.gemm_tiles_per_chunk(3000, 6144, 4, 1, 1) == 4 * 32    # 750-row chunks: staged
    assert mx.gemm_tiles_per_chunk(32768, 6144, 4, 1, 1) == 32 * 24  # 256 x 256 either way
    assert mx.gemm_tiles_per_chunk(1024, 6144, 4, 1, 1) == 2 * 32    # 128 x 192 either way


# ---- the Python binding's own buffer checks (the C ABI cannot see buffer sizes)

def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_rejects_undersized_or_mislabelled_gemm_scales(lib):
    import torch
    m, n, k = 200, 64, 256
    a = torch.zeros((m, k), dtype=torch.uint8)
    b = torch.zeros((n, k), dtype=torch.uint8)
    sa_lin = torch.zeros((m, k // 32), dtype=torch.uint8)
    sb_swz = torch.zeros(mx.scale_bytes(n, k, mx.SWIZZLED), dtype=torch.uint8)
    # linear [m, k/32] scales labelled swizzled: m % 128 != 0, so the buffer is too small
    _raises(lambda: mx.gemm(a, sa_lin, mx.SWIZZLED, b, sb_swz, mx.SWIZZLED), "a_scales holds")
    _raises(lambda: mx.gemm(a, sa_lin[:100], mx.LINEAR, b, sb_swz, mx.SWIZZLED), "a_scales holds")
    _raises(lambda: mx.gemm(a, sa_lin, mx.LINEAR, b, sb_swz[:-1], mx.SWIZZLED), "b_scales holds")
    _raises(lambda: mx.gemm(a, sa_lin, mx.LINEAR, b, sb_swz, 3), "scale layouts")
    _raises(lambda: mx.gemm(a, sa_lin.float(), mx.LINEAR, b, sb_swz, mx.SWIZZLED), "contiguous uint8")
    out = torch.zeros((m, n - 1), dtype=torch.bfloat16)
    _raises(lambda: mx.gemm(a, sa_lin, mx.LINEAR, b, sb_swz, mx.SWIZZLED, out=out), r"out must be \[m, >=n\]")
    bad_done = torch.zeros(2, dtype=torch.int32)
    _raises(lambda: mx.gemm(a, sa_lin, mx.LINEAR, b, sb_swz, mx.SWIZZLED, num_chunks=4, chunk_done=bad_done),
            "chunk_done")
    # well-formed host tensors get as far as the placement check
    _raises(lambda: mx.gemm(a, sa_lin, mx.LINEAR, b, sb_swz, mx.SWIZZLED), "GPU tensor")


def test_binding_rejects_bad_quantiser_outputs(lib):
    import torch
    rows, k = 130, 256
    x = torch.zeros((rows, k), dtype=torch.bfloat16)
    w = torch.zeros(k, dtype=torch.bfloat16)
    q = torch.zeros((rows, k), dtype=torch.uint8)
    sl = torch.zeros((rows, k // 32), dtype=torch.uint8)
    ss = torch.zeros(mx.scale_bytes(rows, k, mx.SWIZZLED), dtype=torch.uint8)
    for call in (lambda out: mx.quantize(x, out=out), lambda out: mx.rmsnorm_quant(x, w, out=out),
                 lambda out: mx.add_rmsnorm_quant(x, x.clone(), w, out=out)):
        _raises(lambda: call((q[:-1], sl, ss)), "q must have shape")
        _raises(lambda: call((q, sl[:-1], ss)), "scales_linear must have shape")
        _raises(lambda: call((q, sl, ss[:-16])), "scales_swizzled holds")
        _raises(lambda: call((q.t(), sl, ss)), "contiguous uint8")
        _raises(lambda: call((q, None, None)), "at least one scale layout")
        _raises(lambda: call((q, sl, ss)), "GPU tensor")
    _raises(lambda: mx.quantize(torch.zeros((4, 48), dtype=torch.bfloat16)), "multiple of 32")


def test_binding_rejects_bad_fused_gemm1_and_swizzle_buffers(lib):
    import torch
    m, inter, k = 64, 96, 256
    a = torch.zeros((m, k), dtype=torch.uint8)
    w = torch.zeros((2 * inter, k), dtype=torch.uint8)
    sa = torch.zeros((m, k // 32), dtype=torch.uint8)
    sw = torch.zeros(mx.scale_bytes(2 * inter, k, mx.SWIZZLED), dtype=torch.uint8)
    _raises(lambda: mx.gemm_silu_mul_quant(a, sa, mx.SWIZZLED, w, sw, mx.SWIZZLED), "a_scales holds")
    _raises(lambda: mx.gemm_silu_mul_quant(a, sa, mx.LINEAR, w, sw[:100], mx.SWIZZLED), "w_scales holds")
    q = torch.zeros((m, inter), dtype=torch.uint8)
    _raises(lambda: mx.gemm_silu_mul_quant(a, sa, mx.LINEAR, w, sw, mx.SWIZZLED,
                                           out=(q, None, torch.zeros(10, dtype=torch.uint8))), "scales_swizzled holds")
    _raises(lambda: mx.gemm_silu_mul_quant(a, sa, mx.LINEAR, w, sw, mx.SWIZZLED), "GPU tensor")
    s_lin = torch.zeros((300, 6), dtype=torch.uint8)
    _raises(lambda: mx.swizzle_scales(s_lin, out=torch.zeros(100, dtype=torch.uint8)), "out holds")
    _raises(lambda: mx.swizzle_scales(s_lin), "GPU tensor")
