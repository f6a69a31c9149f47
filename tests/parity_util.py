"""Helpers shared by the GPU parity tests: host/device conversions, guard bands around
outputs (out-of-bounds write detector) and the comparison rules of the parity bar."""
import numpy as np
import torch

SENTINEL_U8 = 0xA5


def bits16(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a BF16 tensor (any device)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def guarded_u8(numel: int, guard: int = 4096):
    """A uint8 device buffer of `numel` bytes with sentinel guard bands on both sides."""
    buf = torch.full((numel + 2 * guard,), SENTINEL_U8, dtype=torch.uint8, device="cuda")
    return buf, buf[guard:guard + numel]


def guard_intact(buf: torch.Tensor, guard: int = 4096) -> bool:
    h = buf.cpu().numpy()
    return bool(np.all(h[:guard] == SENTINEL_U8) and np.all(h[-guard:] == SENTINEL_U8))


def e4m3_step_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in E4M3 code steps (same sign required; +0 and -0 count as equal)."""
    a = a.astype(np.int64)
    b = b.astype(np.int64)
    ma, mb = a & 0x7F, b & 0x7F
    same_sign = ((a & 0x80) == (b & 0x80)) | ((ma == 0) & (mb == 0))
    d = np.abs(ma - mb)
    return np.where(same_sign, d, 1 << 20)


def gemm_rel_error(c_bits: np.ndarray, ref_bits: np.ndarray, abs_sum: np.ndarray):
    """Parity measure of the GEMM.

    rel_i = |c_i - r_i| / max(|r_i|, 1e-3 * S_i), where r is the oracle's BF16 output and
    S_i = sum_k |A_mk B_nk| (scales included) is the absolute mass of the dot product behind
    element i: where the dot product cancels below a thousandth of its own mass the error is
    measured against that mass, the quantity that bounds any summation error. Returns
    (max rel_i, normwise max|c-r| / max|r|, max |c-r| / S)."""
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(ref_bits)
    s = np.asarray(abs_sum, dtype=np.float64)
    if r.size == 0:
        return 0.0, 0.0, 0.0
    err = np.abs(c - r)
    floor = np.maximum(1e-3 * s, 1e-300)
    rel = err / np.maximum(np.abs(r), floor)
    rmax = float(np.max(np.abs(r)))
    return float(rel.max()), float(err.max() / max(rmax, 1e-300)), float(np.max(err / np.maximum(s, 1e-300)))


GEMM_REL_TOL = 2e-2


def gemm_rel_error_max_floor(c_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    """The tolerance reading that takes the floor from the whole output: max_i |c_i - r_i| /
    max(|r_i|, 1e-3 max_j |r_j|). Reported beside gemm_rel_error on every workload shape."""
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(ref_bits)
    if r.size == 0:
        return 0.0
    tau = max(1e-3 * float(np.max(np.abs(r))), 1e-300)
    return float(np.max(np.abs(c - r) / np.maximum(np.abs(r), tau)))


# Accumulation model of the scaled MFMA (measured on the hardware with in-bounds probes): each
# group of 8 consecutive K products is aligned to its largest product and truncated toward zero
# TRUNC_BITS bits below that product's leading one; the group sums are added in fp32.
TRUNC_BITS = 13
FP32_U = 2.0 ** -24


def accum_error_bound(trunc_loss: np.ndarray, abs_sum: np.ndarray, k: int) -> np.ndarray:
    """Worst-case |fp32 result - exact sum| under the accumulation model, per element: the
    exact truncation loss T of every group (oracle.gemm_accum_terms) plus the bound of n = k/8
    fp32 additions in any order, gamma_n * S with gamma_n = n u / (1 - n u), plus one flushed
    fp32 denormal per addition."""
    n = max(k // 8, 1)
    gamma = n * FP32_U / (1.0 - n * FP32_U)
    return np.asarray(trunc_loss, dtype=np.float64) + gamma * np.asarray(abs_sum, dtype=np.float64) + n * 2.0 ** -126


def _bf16_spacing(x: np.ndarray) -> np.ndarray:
    """BF16 spacing (8 significant bits) in the binade of |x|; the smallest subnormal step at 0."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, np.exp2(np.maximum(e, -126.0) - 7), 2.0 ** -133)


def gemm_accum_bound_ratio(c_bits: np.ndarray, ref_bits: np.ndarray, exact: np.ndarray, bound: np.ndarray) -> float:
    """Largest |c - r| / (bound + BF16 spacing) over the elements: c the kernel's BF16 output,
    r the oracle's BF16 rounding of the exact sum, bound the per-element accumulation bound
    (accum_error_bound). The kernel's fp32 sum lies within `bound` of the exact one and each
    side's BF16 rounding moves it by at most half a spacing (taken at the larger of |exact| +
    bound and |c|), so a correct kernel gives a ratio <= 1 whatever the cancellation, while a
    misapplied block scale or operand gives an error of the order of the dot product's mass."""
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(ref_bits)
    if r.size == 0:
        return 0.0
    b = np.asarray(bound, dtype=np.float64)
    x = np.maximum(np.abs(np.asarray(exact, dtype=np.float64)) + b, np.abs(c))
    return float(np.max(np.abs(c - r) / (b + _bf16_spacing(x))))


def accum_budget_used(c_bits: np.ndarray, exact: np.ndarray, bound: np.ndarray) -> float:
    """Largest (|c - exact| - half a BF16 spacing of c) / bound: the share of the accumulation
    bound the kernel's own sum used once its final rounding is taken out (reported beside
    gemm_accum_bound_ratio, whose 1-spacing allowance makes any rounding flip read close to 1)."""
    c = bf16_bits_to_f64(c_bits)
    b = np.maximum(np.asarray(bound, dtype=np.float64), 1e-300)
    if c.size == 0:
        return 0.0
    used = np.abs(c - np.asarray(exact, dtype=np.float64)) - 0.5 * _bf16_spacing(np.abs(c))
    return float(np.max(np.maximum(used, 0.0) / b))


def _scale_exp(amax: np.ndarray) -> np.ndarray:
    """Elementwise smallest e in [-127, 127] with amax <= 448 * 2^e (amax 0 -> -127)."""
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(a > 0, a, 1.0) / 448.0))
    e = np.clip(e, -127, 127)
    e = np.where(a > np.ldexp(448.0, e.astype(np.int64)), e + 1, e)
    e = np.where((e > -127) & (a <= np.ldexp(448.0, (e - 1).astype(np.int64))), e - 1, e)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def silu_mul_quant_check(q, s_lin, gu, gu_err, inter):
    """Check a fused GEMM1 output (codes q [r, inter], scales s_lin [r, inter/32]) against the
    oracle's exact gate/up values gu [r, 2*inter] and the accumulation bound gu_err of each of
    them (accum_error_bound, same shape).

    The kernel's gate and up carry the MFMA accumulation error (at most gu_err), so
    y = SiLU(g) * u is known to within dy. Every scale must be one the quantiser could pick
    for a block whose amax lies within dy of the exact one, and every dequantised code must be
    the round-to-nearest result of some value within dy of the exact y (half a spacing of E4M3
    at that magnitude, plus dy). Returns the fraction of blocks whose scale and of elements whose
    value differ from the exact decision, for the caller to bound."""
    g, u = gu[:, :inter], gu[:, inter:]
    dg = gu_err[:, :inter]
    du = gu_err[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    y = silu * u
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))  # |SiLU'(g)| <= 1.1
    dy = dsilu * np.abs(u) * dg + (np.abs(silu) + 1.1 * dg) * du + 0.5 * dg * dg * np.abs(u) \
        + 2.0 ** -20 * np.abs(y) + 1e-30
    rows = y.shape[0]
    blk = lambda v: v.reshape(rows, inter // 32, 32)
    e_gpu = s_lin.astype(np.int64) - 127
    e_lo = _scale_exp(np.max(np.maximum(blk(np.abs(y) - dy), 0.0), axis=2))
    e_hi = _scale_exp(np.max(blk(np.abs(y) + dy), axis=2))
    e_ref = _scale_exp(np.max(blk(np.abs(y)), axis=2))
    assert np.all((e_gpu >= e_lo) & (e_gpu <= e_hi)), "scale outside the reachable range"
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    eg = np.repeat(e_gpu, 32, axis=1).astype(np.float64)
    val = table[q] * np.exp2(eg)
    w_hi = (np.abs(y) + dy) * np.exp2(-eg)  # largest magnitude in the scaled domain
    with np.errstate(divide="ignore"):
        spacing = np.where(w_hi < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(w_hi, 2.0 ** -6))) - 3))
    bound = dy + 0.5 * spacing * np.exp2(eg)
    err = np.abs(val - y)
    bad = err > bound * (1 + 1e-12)
    assert not bad.any(), f"{int(bad.sum())} codes off by more than the bound, worst {float((err / bound).max()):.3f}"
    ref_val = None
    er = np.repeat(e_ref, 32, axis=1).astype(np.float64)
    scaled = y * np.exp2(-er)
    ref_codes = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref_val = ref_codes * np.exp2(er)
    return float(np.mean(e_gpu != e_ref)), float(np.mean(val != ref_val))


def near_scale_boundary(y_ref: np.ndarray) -> np.ndarray:
    """Per 32-block of y_ref [rows, h]: is the block's amax within 2^-20 (relative) of a scale
    boundary 448 * 2^e, where an fp32 evaluation of the norm in another order may pick the next
    UE8M0 code?"""
    rows, h = y_ref.shape
    amax = np.abs(y_ref.astype(np.float64)).reshape(rows, h // 32, 32).max(-1)
    with np.errstate(divide="ignore"):
        e = np.round(np.log2(np.where(amax > 0, amax, 1.0) / 448.0))
    edge = np.ldexp(448.0, e.astype(np.int64))
    return (amax > 0) & (np.abs(amax - edge) <= 2.0 ** -20 * edge)


def norm_quant_check(q, s_lin, s_swz, q_ref, s_lin_ref, s_swz_ref, y_ref, requantize):
    """The norm quantiser's bar. q, s_lin, s_swz: the kernel's codes [rows, h], linear scales
    [rows, h/32] (or None) and swizzled scales (or None); *_ref: the oracle's; y_ref: the
    oracle's fp32 y; requantize(values) -> E4M3 codes of fp64 values (the oracle's encoder).

    - A UE8M0 scale may differ from the oracle's only by one step and only in a block whose amax
      lies within 2^-20 of a boundary 448 * 2^e (near_scale_boundary); such blocks are counted.
    - Every code is compared with the oracle's y re-quantised at the kernel's scale of its
      block (the oracle's own codes wherever the scales agree) and may differ by at most one
      E4M3 step; differing codes are counted.
    - The swizzled scales hold the same bytes as the linear ones at the 128x4 positions (or,
      alone, the oracle's except in counted blocks), and every pad byte is 0.
    Returns (scale differences, code differences)."""
    rows, h = q.shape
    nblk = h // 32
    near = near_scale_boundary(y_ref)
    col_tiles = (nblk + 3) // 4
    r_idx = np.arange(rows)[:, None]
    c_idx = np.arange(nblk)[None, :]
    swz_pos = ((r_idx // 128) * col_tiles + c_idx // 4) * 512 + (r_idx % 32) * 16 + ((r_idx % 128) // 32) * 4 + c_idx % 4
    if s_lin is not None:
        s = s_lin.astype(np.int64)
    else:
        s = s_swz[swz_pos].astype(np.int64)
    sdiff = s - s_lin_ref.astype(np.int64)
    assert np.all(sdiff[~near] == 0), f"{int(np.sum(sdiff[~near] != 0))} scales differ away from a boundary"
    assert np.all(np.abs(sdiff) <= 1), "a scale differs by more than one step"
    if s_swz is not None:
        if s_lin is not None:
            assert np.array_equal(s_swz[swz_pos], s_lin), "swizzled and linear scales disagree"
        pad = np.ones(s_swz.shape[0], dtype=bool)
        pad[swz_pos.ravel()] = False
        assert np.all(s_swz[pad] == 0), "a swizzle pad byte is not 0"
        assert np.array_equal(s_swz[pad], s_swz_ref[pad])
    want = q_ref.copy()
    rb, cb = np.nonzero(sdiff)
    for r, b in zip(rb, cb):  # blocks where the kernel took the neighbouring scale
        vals = y_ref[r, 32 * b:32 * b + 32].astype(np.float64) * np.ldexp(1.0, 127 - int(s[r, b]))
        want[r, 32 * b:32 * b + 32] = requantize(vals)
    steps = e4m3_step_diff(q, want)
    assert np.all(steps <= 1), "a code differs by more than one step"
    return int(np.count_nonzero(sdiff)), int(np.count_nonzero(steps))
