"""Pins of the CPU oracle to facts outside itself (CPU only).

Each check compares the oracle with something it does not contain: hand-worked
values in tests/golden/ (format definitions of OCP OFP8 E4M3 and OCP MX E8M0,
the formats the pages name for MXFP8 data and scales), torch's own float8/bfloat16
casts (independent library routines), brute force over every code, closed
forms of special inputs, and invariants of round-to-nearest. A plausible
mistake in the oracle (a wrong bias, tie rule, scale direction, swizzle index,
dropped (1+w) term, transposed GEMM operand) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


def _torch_e4m3_codes(values_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ----------------------------------------------------------------- E4M3 decode

def test_decode_golden():
    for line in _golden("e4m3_decode.txt"):
        code_s, val_s = line.split()[:2]
        got = oracle.e4m3_value(int(code_s, 16))
        if val_s == "nan":
            assert math.isnan(got), code_s
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code_s, got, want)


def test_decode_all_codes_match_torch():
    ours = oracle.e4m3_values()
    ref = _torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_ue8m0_values():
    assert oracle.ue8m0_value(127) == 1.0
    assert oracle.ue8m0_value(0) == 2.0 ** -127
    assert oracle.ue8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.ue8m0_value(255))


# ----------------------------------------------------------------- E4M3 encode

def test_encode_golden():
    for line in _golden("e4m3_encode.txt"):
        parts = line.split()
        v, code = float(parts[0]), int(parts[1], 16)
        assert int(oracle.e4m3_encode([v])[0]) == code, (v, hex(int(oracle.e4m3_encode([v])[0])), hex(code))


def test_encode_every_bf16_value_matches_torch():
    bits = np.arange(65536, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 464.0)
    vals = vals[keep]
    ours = oracle.e4m3_encode(vals.astype(np.float64))
    ref = _torch_e4m3_codes(vals)
    assert np.array_equal(ours, ref)


def test_encode_midpoints_and_neighbours_match_torch():
    mags = oracle.e4m3_values()[:127]
    mids = (mags[:-1] + mags[1:]) / 2.0          # exact in fp32
    pts = np.concatenate([mids, mags])
    f = pts.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), pts)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(0))
    allv = np.concatenate([f, up, dn, -f, -up, -dn])
    allv = allv[np.abs(allv) <= 464.0]
    assert np.array_equal(oracle.e4m3_encode(allv.astype(np.float64)), _torch_e4m3_codes(allv))


def test_encode_brute_force_nearest_even():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-12, 8.9, 4000))
    v = mag * rng.choice([-1.0, 1.0], mag.size)
    codes = oracle.e4m3_encode(v)
    table = oracle.e4m3_values()
    finite = np.array([c for c in range(256) if not math.isnan(table[c])])
    for x, c in zip(v, codes):
        d = np.abs(table[finite] - x)
        best = d.min()
        mine = abs(table[c] - x)
        assert mine == best, (x, c)
        ties = finite[d == best]
        ties_vals = set(abs(table[t]) for t in ties)
        if len(ties_vals) > 1:  # a true tie between two magnitudes: even mantissa wins
            assert c % 2 == 0, (x, c)
        assert (c & 0x80) == (0x80 if x < 0 else 0)


def test_encode_saturates_beyond_torch_range():
    for v in (464.0, 479.9, 480.0, 1e4, 1e30):
        assert int(oracle.e4m3_encode([v])[0]) == 0x7E
        assert int(oracle.e4m3_encode([-v])[0]) == 0xFE


# ------------------------------------------------------------------ UE8M0 rule

def test_scale_golden():
    for line in _golden("ue8m0_scale.txt"):
        amax_s, code_s, qmax_s = line.split()[:3]
        amax, code = float(amax_s), int(code_s)
        e = oracle.scale_exponent(amax)
        assert e + 127 == code, (amax, e + 127, code)
        if qmax_s != "-":
            assert int(oracle.e4m3_encode([math.ldexp(amax, -e)])[0]) == int(qmax_s, 16)


def test_scale_is_smallest_power_of_two_cover():
    rng = np.random.default_rng(3)
    for amax in np.exp2(rng.uniform(-100, 100, 3000)):
        e = oracle.scale_exponent(float(amax))
        assert amax <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
        assert 224.0 < amax * 2.0 ** -e <= 448.0


def test_scale_exact_powers_keep_exponent():
    for e in range(-120, 120, 7):
        assert oracle.scale_exponent(448.0 * 2.0 ** e) == e
        assert oracle.scale_exponent(np.nextafter(448.0 * 2.0 ** e, np.inf)) == e + 1


# --------------------------------------------------------------- BF16 rounding

def test_bf16_golden():
    for line in _golden("bf16_round.txt"):
        expr, bits_s = line.rsplit(None, 1)
        v = eval(expr, {"__builtins__": {}}, {})
        assert int(oracle.bf16_from_double([v])[0]) == int(bits_s, 16), (expr, hex(int(oracle.bf16_from_double([v])[0])))


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(11)
    mant = rng.integers(0, 1 << 23, 20000, dtype=np.uint32)
    expo = rng.integers(1, 254, 20000, dtype=np.uint32)
    sign = rng.integers(0, 2, 20000, dtype=np.uint32)
    f = ((sign << 31) | (expo << 23) | mant).view(np.float32)
    ties = ((np.arange(2000, dtype=np.uint32) * 65536 + 0x3F808000) & 0x7FFFFFFF).view(np.float32)
    f = np.concatenate([f, ties])
    ours = oracle.bf16_from_double(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------- swizzled layout

def _swizzle_by_reshape(s_lin: np.ndarray) -> np.ndarray:
    rows, nblk = s_lin.shape
    rp = -(-rows // 128) * 128
    cp = -(-nblk // 4) * 4
    pad = np.zeros((rp, cp), dtype=np.uint8)
    pad[:rows, :nblk] = s_lin
    # (row tile, 32-row group, row in group, col tile, col) -> (row tile, col tile, row in group, group, col)
    return pad.reshape(rp // 128, 4, 32, cp // 4, 4).transpose(0, 3, 2, 1, 4).reshape(-1)


def test_swizzle_golden():
    for line in _golden("swizzle_offsets.txt"):
        r, c, nblk, off = map(int, line.split())
        assert oracle.swizzle_offset(r, c, nblk) == off, line


@pytest.mark.parametrize("rows,nblk", [(128, 4), (256, 64), (200, 6), (1, 1), (129, 96)])
def test_swizzle_is_tiled_bijection(rows, nblk):
    total = oracle.scale_bytes(rows, nblk * 32, oracle.SWIZZLED)
    offs = np.array([oracle.swizzle_offset(r, c, nblk) for r in range(rows) for c in range(nblk)])
    assert len(set(offs.tolist())) == offs.size
    assert offs.min() >= 0 and offs.max() < total
    assert total == -(-rows // 128) * 128 * (-(-nblk // 4) * 4)
    # each (128 rows x 4 blocks) tile is one contiguous 512-byte run
    for r in range(0, rows, 37):
        for c in range(0, nblk, 3):
            t0 = oracle.swizzle_offset((r // 128) * 128, (c // 4) * 4, nblk)
            assert t0 % 512 == 0 and t0 <= oracle.swizzle_offset(r, c, nblk) < t0 + 512


def test_swizzle_rows_do_not_concatenate():
    """Swizzled scales of two 64-row shards are not the rows-concatenation of their swizzles."""
    rng = np.random.default_rng(5)
    s = rng.integers(100, 140, (128, 8), dtype=np.uint8)
    whole = _swizzle_by_reshape(s)
    parts = np.concatenate([_swizzle_by_reshape(s[:64]), _swizzle_by_reshape(s[64:])])
    assert whole.size != parts.size or not np.array_equal(whole, parts)
    # while the unswizzled scales concatenate trivially
    assert np.array_equal(np.concatenate([s[:64], s[64:]]), s)


# ------------------------------------------------------------------ quantiser

def _bf16_bits_from_f64(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_quantize_worked_block_ones():
    x = _bf16_bits_from_f64(np.ones((1, 32)))
    q, s_lin, s_swz = oracle.quantize(x)
    assert s_lin[0, 0] == 119 and np.all(q == 0x78)
    x = _bf16_bits_from_f64(-np.ones((1, 32)))
    q, s_lin, _ = oracle.quantize(x)
    assert s_lin[0, 0] == 119 and np.all(q == 0xF8)


def test_quantize_zero_block():
    x = _bf16_bits_from_f64(np.array([[0.0] * 16 + [-0.0] * 16]))
    q, s_lin, _ = oracle.quantize(x)
    assert s_lin[0, 0] == 0
    assert np.all(q[0, :16] == 0x00) and np.all(q[0, 16:] == 0x80)


def test_quantize_round_trips_representable_blocks():
    """Blocks whose values are E4M3 values times 2^e (amax in (224, 448] * 2^e) come back exactly."""
    rng = np.random.default_rng(9)
    table = oracle.e4m3_values()
    rows, k = 64, 256
    codes = rng.integers(0, 256, (rows, k)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    codes[:, ::32] = rng.integers(0x77, 0x7F, (rows, k // 32)).astype(np.uint8)  # amax in (224, 448]
    e = rng.integers(-30, 30, (rows, k // 32))
    vals = table[codes] * np.exp2(np.repeat(e, 32, axis=1))
    x = _bf16_bits_from_f64(vals)
    assert np.array_equal(_bits_to_f64(x), vals)
    q, s_lin, _ = oracle.quantize(x)
    assert np.array_equal(s_lin.astype(int), e + 127)
    assert np.array_equal(q, codes)


def test_quantize_matches_torch_cast_and_error_bound():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((96, 512)) * np.exp2(rng.integers(-8, 8, (96, 1)))
    v[5, 40:72] = 0.0
    x = _bf16_bits_from_f64(v)
    xf = _bits_to_f64(x)
    q, s_lin, _ = oracle.quantize(x)
    e = s_lin.astype(np.int64) - 127
    scaled = xf * np.exp2(-np.repeat(e, 32, axis=1))
    assert np.all(np.abs(scaled) <= 448.0)
    assert np.array_equal(q, _torch_e4m3_codes(scaled.astype(np.float32)))
    deq = oracle.e4m3_values()[q] * np.exp2(np.repeat(e, 32, axis=1))
    # round-to-nearest error bound: half a spacing (2^-4 relative for normals, 2^-10 * 2^e below)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.exp2(np.repeat(e, 32, axis=1)) * 2.0 ** -10)
    assert np.all(np.abs(deq - xf) <= bound)


@pytest.mark.parametrize("rows,k", [(128, 128), (200, 96), (1, 32), (300, 2048)])
def test_quantize_swizzled_equals_reshaped_linear(rows, k):
    x = _bf16_bits_from_f64(np.random.default_rng(rows).standard_normal((rows, k)))
    q, s_lin, s_swz = oracle.quantize(x)
    assert np.array_equal(s_swz, _swizzle_by_reshape(s_lin))


@pytest.mark.parametrize("rows,nblk", [(1, 1), (127, 5), (128, 4), (300, 96), (129, 64)])
def test_swizzle_scales_equals_reshape(rows, nblk):
    """oracle.swizzle_scales against the independent pad/reshape/transpose construction,
    including pad rows, pad blocks and a buffer that starts non-zero."""
    s = np.random.default_rng(rows * 7 + nblk).integers(1, 255, (rows, nblk), dtype=np.uint8)
    assert np.array_equal(oracle.swizzle_scales(s), _swizzle_by_reshape(s))


def test_swizzle_after_gather_equals_whole():
    """Gathering linear scale shards by rows and swizzling once gives the swizzled scales of
    the whole operand (the reason the gathered path carries linear scales)."""
    x = _bf16_bits_from_f64(np.random.default_rng(11).standard_normal((320, 256)))
    _, s_lin_whole, s_swz_whole = oracle.quantize(x)
    shards = [oracle.quantize(x[i:i + 80])[1] for i in range(0, 320, 80)]
    assert np.array_equal(oracle.swizzle_scales(np.concatenate(shards)), s_swz_whole)


def test_quantize_row_stride():
    x = _bf16_bits_from_f64(np.random.default_rng(4).standard_normal((40, 160)))
    q_full, s_full, _ = oracle.quantize(np.ascontiguousarray(x[:, :96]))
    q, s, _ = oracle.quantize(x, k=96)
    assert np.array_equal(q, q_full) and np.array_equal(s, s_full)


# ------------------------------------------------------------------- RMSNorm

EPS = float(np.float32(1e-6))


def test_rmsnorm_constant_row_closed_form():
    for c in (0.5, -3.0, 1e-3, 40.0):
        x = _bf16_bits_from_f64(np.full((2, 64), c))
        w = _bf16_bits_from_f64(np.zeros(64))
        cb = float(_bits_to_f64(x)[0, 0])
        _, _, _, y = oracle.rmsnorm_quant(x, w, EPS)
        want = np.float32(cb / math.sqrt(cb * cb + EPS))
        assert np.all(y == want)


def test_rmsnorm_plus_minus_one_row():
    sgn = np.where(np.random.default_rng(1).random(6144) < 0.5, -1.0, 1.0)
    x = _bf16_bits_from_f64(sgn[None, :])
    w = _bf16_bits_from_f64(np.zeros(6144))
    q, s_lin, s_swz, y = oracle.rmsnorm_quant(x, w, EPS)
    assert np.all(s_lin == 119)
    assert np.array_equal(q[0], np.where(sgn > 0, 0x78, 0xF8).astype(np.uint8))


def test_rmsnorm_weight_minus_one_zeroes_output():
    rng = np.random.default_rng(8)
    x = _bf16_bits_from_f64(rng.standard_normal((3, 256)))
    w = _bf16_bits_from_f64(-np.ones(256))
    q, s_lin, _, _ = oracle.rmsnorm_quant(x, w, EPS)
    assert np.all(s_lin == 0)
    neg = _bits_to_f64(x) < 0
    assert np.array_equal(q, np.where(neg, 0x80, 0x00).astype(np.uint8))


def test_rmsnorm_one_plus_w_doubles():
    rng = np.random.default_rng(10)
    x = _bf16_bits_from_f64(rng.standard_normal((4, 512)))
    q0, s0, _, y0 = oracle.rmsnorm_quant(x, _bf16_bits_from_f64(np.zeros(512)), EPS)
    q1, s1, _, y1 = oracle.rmsnorm_quant(x, _bf16_bits_from_f64(np.ones(512)), EPS)
    assert np.array_equal(y1, 2 * y0)
    assert np.array_equal(q1, q0) and np.array_equal(s1.astype(int), s0.astype(int) + 1)


def test_rmsnorm_scale_invariance_without_eps():
    rng = np.random.default_rng(12)
    xv = rng.standard_normal((4, 256))
    w = _bf16_bits_from_f64(rng.standard_normal(256) * 0.1)
    q0, s0, _, y0 = oracle.rmsnorm_quant(_bf16_bits_from_f64(xv), w, 0.0)
    q1, s1, _, y1 = oracle.rmsnorm_quant(_bf16_bits_from_f64(xv * 8), w, 0.0)
    assert np.array_equal(y0, y1) and np.array_equal(q0, q1) and np.array_equal(s0, s1)


def test_rmsnorm_two_nonzero_entries():
    """x = (3, 4, 0, ...) over 32 columns: mean(x^2) = 25/32, so y = x / sqrt(25/32 + eps)."""
    xv = np.zeros((1, 32))
    xv[0, 0], xv[0, 1] = 3.0, 4.0
    _, _, _, y = oracle.rmsnorm_quant(_bf16_bits_from_f64(xv), _bf16_bits_from_f64(np.zeros(32)), EPS)
    r = 1.0 / math.sqrt(25.0 / 32.0 + EPS)
    assert y[0, 0] == np.float32(3 * r) and y[0, 1] == np.float32(4 * r) and np.all(y[0, 2:] == 0)


# ----------------------------------------------------------------------- GEMM

def test_gemm_all_ones_gives_k():
    for k, bits in ((2048, 0x4500), (3072, 0x4540)):
        a = np.full((4, k), 0x38, np.uint8)
        b = np.full((6, k), 0x38, np.uint8)
        sa = np.full((4, k // 32), 127, np.uint8)
        sb = np.full((6, k // 32), 127, np.uint8)
        c = oracle.gemm(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR)
        assert np.all(c == bits)


def test_gemm_scales_only_closed_form():
    rng = np.random.default_rng(13)
    m, n, k = 5, 7, 256
    a = np.full((m, k), 0x38, np.uint8)
    b = np.full((n, k), 0x38, np.uint8)
    sa = rng.integers(110, 140, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (n, k // 32)).astype(np.uint8)
    _, f = oracle.gemm(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR, want_f64=True)
    want = 32.0 * np.exp2(sa.astype(np.int64)[:, None, :] + sb.astype(np.int64)[None, :, :] - 254).sum(-1)
    assert np.array_equal(f, want)


def test_gemm_one_hot_rows_pick_scaled_b_columns():
    rng = np.random.default_rng(14)
    m, n, k = 6, 9, 128
    table = _torch_e4m3_values()
    b = rng.integers(0, 256, (n, k)).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x40
    sa = rng.integers(120, 135, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, (n, k // 32)).astype(np.uint8)
    a = np.zeros((m, k), np.uint8)
    k0 = rng.integers(0, k, m)
    a[np.arange(m), k0] = 0x38
    _, f = oracle.gemm(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR, want_f64=True)
    for i in range(m):
        kb = k0[i] // 32
        want = table[b[:, k0[i]]] * np.exp2(int(sa[i, kb]) + sb[:, kb].astype(np.int64) - 254)
        assert np.array_equal(f[i], want)


@pytest.mark.parametrize("m,n,k", [(3, 5, 32), (8, 4, 64), (7, 8, 128), (1, 1, 32)])
def test_gemm_brute_force_vs_dequantized_matmul(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    table = _torch_e4m3_values()
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    b = rng.integers(0, 256, (n, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    b[(b & 0x7F) == 0x7F] = 0xB1
    sa = rng.integers(115, 140, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(115, 140, (n, k // 32)).astype(np.uint8)
    a_deq = table[a] * np.exp2(np.repeat(sa.astype(np.int64) - 127, 32, axis=1))
    b_deq = table[b] * np.exp2(np.repeat(sb.astype(np.int64) - 127, 32, axis=1))
    want = np.matmul(a_deq, b_deq.T)
    c, f = oracle.gemm(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR, want_f64=True)
    assert np.allclose(f, want, rtol=1e-12, atol=1e-300 + 1e-12 * np.abs(want).max())
    ref_bf16 = torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # fp64 -> fp32 -> bf16 may double-round; only differences of one unit in the last place are allowed
    assert np.all(np.abs(c.astype(np.int64) - ref_bf16.astype(np.int64)) <= 1)


def test_gemm_swizzled_scales_and_sampling_agree():
    rng = np.random.default_rng(15)
    m, n, k = 200, 140, 192
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    b = rng.integers(0, 0x7E, (n, k)).astype(np.uint8)
    sa = rng.integers(118, 136, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(118, 136, (n, k // 32)).astype(np.uint8)
    c_lin = oracle.gemm(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR)
    c_swz = oracle.gemm(a, _swizzle_by_reshape(sa), oracle.SWIZZLED, b, _swizzle_by_reshape(sb), oracle.SWIZZLED)
    assert np.array_equal(c_lin, c_swz)
    rows = rng.integers(0, m, 300)
    cols = rng.integers(0, n, 300)
    s_bf16, _ = oracle.gemm_sampled(a, sa, oracle.LINEAR, b, sb, oracle.LINEAR, rows, cols)
    assert np.array_equal(s_bf16, c_lin[rows, cols])


# ----------------------------------------- fused dense GEMM1: gate_up, SiLU-and-mul, quantiser

def _scale_exp(amax: float) -> int:
    """Smallest e in [-127, 127] with amax <= 448 * 2^e, by exact power-of-two comparisons."""
    if amax == 0.0:
        return -127
    e = math.ceil(math.log2(amax / 448.0))
    while e < 127 and amax > math.ldexp(448.0, e):
        e += 1
    while e > -127 and amax <= math.ldexp(448.0, e - 1):
        e -= 1
    return max(-127, min(127, e))


def _quantize_f32_rows(y32: np.ndarray):
    """Independent per-32 quantisation of fp32 rows: python scale rule + torch's E4M3 cast."""
    rows, n = y32.shape
    s = np.empty((rows, n // 32), dtype=np.uint8)
    q = np.empty((rows, n), dtype=np.uint8)
    for r in range(rows):
        for b in range(n // 32):
            blk = y32[r, 32 * b:32 * b + 32].astype(np.float64)
            e = _scale_exp(float(np.max(np.abs(blk))))
            s[r, b] = e + 127
            q[r, 32 * b:32 * b + 32] = _torch_e4m3_codes((blk * 2.0 ** -e).astype(np.float32))
    return q, s


def _silu_mul_f32(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    gt = torch.from_numpy(g.astype(np.float64))
    return (torch.nn.functional.silu(gt) * torch.from_numpy(u.astype(np.float64))).to(torch.float32).numpy()


def test_silu_mul_quant_closed_form():
    """A = ones, so gate and up are k times one weight value each; y against torch's silu."""
    inter, k = 64, 64
    table = _torch_e4m3_values()
    a = np.full((2, k), 0x38, np.uint8)                         # 1.0
    sa = np.full((2, k // 32), 127, np.uint8)
    rng = np.random.default_rng(21)
    gate_codes = rng.integers(0, 0x7E, inter).astype(np.uint8) | (rng.integers(0, 2, inter) * 0x80).astype(np.uint8)
    up_codes = rng.integers(0, 0x7E, inter).astype(np.uint8) | (rng.integers(0, 2, inter) * 0x80).astype(np.uint8)
    w = np.concatenate([np.repeat(gate_codes[:, None], k, 1), np.repeat(up_codes[:, None], k, 1)])
    sw = np.full((2 * inter, k // 32), 125, np.uint8)          # 2^-2
    q, s_lin, y, gu = oracle.gemm_silu_mul_quant(a, sa, oracle.LINEAR, w, sw, oracle.LINEAR, want_gu=True)
    g = k * table[gate_codes] * 0.25
    u = k * table[up_codes] * 0.25
    assert np.array_equal(gu[0, :inter], g) and np.array_equal(gu[0, inter:], u)
    want_y = _silu_mul_f32(g, u)
    assert np.array_equal(y[0], want_y) and np.array_equal(y[1], want_y)
    want_q, want_s = _quantize_f32_rows(want_y[None, :])
    assert np.array_equal(q[0], want_q[0]) and np.array_equal(s_lin[0], want_s[0])


def test_silu_mul_quant_brute_force():
    """Random codes and scales: decode, matmul, silu and quantise outside the oracle."""
    m, inter, k = 6, 96, 128
    rng = np.random.default_rng(22)
    table = _torch_e4m3_values()
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    w = rng.integers(0, 0x7E, (2 * inter, k)).astype(np.uint8) | (rng.integers(0, 2, (2 * inter, k)) * 0x80).astype(np.uint8)
    sa = rng.integers(118, 130, (m, k // 32)).astype(np.uint8)
    sw = rng.integers(118, 130, (2 * inter, k // 32)).astype(np.uint8)
    a_deq = table[a] * np.exp2(np.repeat(sa.astype(np.int64) - 127, 32, axis=1))
    w_deq = table[w] * np.exp2(np.repeat(sw.astype(np.int64) - 127, 32, axis=1))
    c = np.matmul(a_deq, w_deq.T)
    want_y = _silu_mul_f32(c[:, :inter], c[:, inter:])
    q, s_lin, y = oracle.gemm_silu_mul_quant(a, _swizzle_by_reshape(sa), oracle.SWIZZLED, w, sw, oracle.LINEAR)
    # the matmul sums in another order: fp32 y may differ by one unit in the last place
    yi, wi = y.view(np.int32).astype(np.int64), want_y.view(np.int32).astype(np.int64)
    assert np.all(np.abs(yi - wi) <= 1)
    same = yi == wi
    assert same.mean() > 0.9
    want_q, want_s = _quantize_f32_rows(y)
    assert np.array_equal(q, want_q) and np.array_equal(s_lin, want_s)
    q2, s2 = _quantize_f32_rows(want_y)
    assert np.array_equal(q[same], q2[same])


def test_silu_mul_quant_special_rows_and_selection():
    """Zero gate gives zero output (code 0 scales); a huge negative gate gives SiLU ~ 0;
    selecting rows returns exactly those rows of the full result."""
    inter, k = 32, 32
    a = np.full((3, k), 0x38, np.uint8)
    sa = np.full((3, 1), 127, np.uint8)
    sa[2, 0] = 127 + 8                                          # row 2: A = 256
    w = np.zeros((2 * inter, k), np.uint8)
    w[inter:] = 0x38                                            # up = k * a
    sw = np.full((2 * inter, 1), 127, np.uint8)
    q, s_lin, y = oracle.gemm_silu_mul_quant(a, sa, oracle.LINEAR, w, sw, oracle.LINEAR)
    assert np.all(y == 0) and np.all(s_lin == 0) and np.all((q & 0x7F) == 0)
    w[:inter] = 0xFE                                            # gate weight -448: gate = -448 k a
    q, s_lin, y = oracle.gemm_silu_mul_quant(a, sa, oracle.LINEAR, w, sw, oracle.LINEAR)
    g = -448.0 * k * np.array([1.0, 1.0, 256.0])
    want = _silu_mul_f32(np.repeat(g[:, None], inter, 1), np.repeat((k * np.array([1.0, 1.0, 256.0]))[:, None], inter, 1))
    assert np.array_equal(y, want) and np.all(y <= 0)
    qs, ss, ys = oracle.gemm_silu_mul_quant(a, sa, oracle.LINEAR, w, sw, oracle.LINEAR, rows=[2, 0])
    assert np.array_equal(qs, q[[2, 0]]) and np.array_equal(ss, s_lin[[2, 0]]) and np.array_equal(ys, y[[2, 0]])


# ------------------------------------------------- residual add + Gemma RMSNorm + quantiser

def _add_inputs(rows, h, seed):
    rng = np.random.default_rng(seed)
    x = _bf16_bits_from_f64(rng.standard_normal((rows, h)) * np.exp2(rng.integers(-6, 6, (rows, 1))))
    r = _bf16_bits_from_f64(rng.standard_normal((rows, h)) * 4.0)
    w = _bf16_bits_from_f64(rng.standard_normal(h) * 0.1)
    return x, r, w


def test_add_rmsnorm_residual_matches_torch_bf16_add():
    """h = BF16(x + r) against torch's fp32 add rounded to BF16 (exact sum, one rounding)."""
    x, r, w = _add_inputs(40, 256, 41)
    _, _, _, h, _ = oracle.add_rmsnorm_quant(x, r, w, EPS)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    rt = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).float()
    want = (xt + rt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, want)


def test_add_rmsnorm_is_norm_of_the_sum():
    """The quantised output is the plain norm quantiser applied to h; with r = 0 it is the
    norm quantiser applied to x."""
    x, r, w = _add_inputs(24, 512, 42)
    q, sl, ss, h, y = oracle.add_rmsnorm_quant(x, r, w, EPS)
    q2, sl2, ss2, y2 = oracle.rmsnorm_quant(h, w, EPS)
    assert np.array_equal(q, q2) and np.array_equal(sl, sl2) and np.array_equal(ss, ss2)
    assert np.array_equal(y, y2)
    zero = np.zeros_like(r)
    q3, sl3, ss3, h3, _ = oracle.add_rmsnorm_quant(x, zero, w, EPS)
    q4, sl4, ss4, _ = oracle.rmsnorm_quant(x, w, EPS)
    assert np.array_equal(q3, q4) and np.array_equal(sl3, sl4) and np.array_equal(ss3, ss4)
    assert np.array_equal(_bits_to_f64(h3), _bits_to_f64(x))


def test_add_rmsnorm_cancelling_residual_gives_zero():
    """r = -x: h = 0, y = 0, every code and scale is zero."""
    x, _, w = _add_inputs(3, 64, 43)
    r = x ^ np.uint16(0x8000)
    q, sl, _, h, y = oracle.add_rmsnorm_quant(x, r, w, EPS)
    assert np.all(_bits_to_f64(h) == 0) and np.all(y == 0)
    assert np.all(sl == 0) and np.all((q & 0x7F) == 0)
