"""The comparison rules the GPU parity tests use, exercised on the CPU with oracle outputs:
they accept the oracle's own result and reject planted mistakes (no GPU involved)."""
import numpy as np
import pytest

import oracle
from parity_util import TRUNC_BITS, accum_error_bound, gemm_accum_bound_ratio, silu_mul_quant_check


def _case():
    rng = np.random.default_rng(31)
    m, inter, k = 8, 64, 256
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    w = rng.integers(0, 0x70, (2 * inter, k)).astype(np.uint8) | (rng.integers(0, 2, (2 * inter, k)) * 0x80).astype(np.uint8)
    sa = rng.integers(120, 128, (m, k // 32)).astype(np.uint8)
    sw = rng.integers(118, 124, (2 * inter, k // 32)).astype(np.uint8)
    q, s, y, gu = oracle.gemm_silu_mul_quant(a, sa, 0, w, sw, 0, want_gu=True)
    t, mass = oracle.gemm_accum_terms(a, sa, 0, w, sw, 0)
    return q, s, gu, accum_error_bound(t, mass, k), inter


def test_check_accepts_the_oracle_result():
    q, s, gu, mass, inter = _case()
    s_diff, v_diff = silu_mul_quant_check(q, s, gu, mass, inter)
    assert s_diff == 0.0 and v_diff == 0.0


def test_check_rejects_swapped_gate_and_up():
    q, s, gu, mass, inter = _case()
    swapped = np.concatenate([gu[:, inter:], gu[:, :inter]], axis=1)
    with pytest.raises(AssertionError):
        silu_mul_quant_check(q, s, swapped, mass, inter)


def test_check_rejects_a_wrong_scale():
    q, s, gu, mass, inter = _case()
    s2 = s.copy()
    s2[3, 1] += 1
    with pytest.raises(AssertionError):
        silu_mul_quant_check(q, s2, gu, mass, inter)


def test_check_rejects_a_code_two_steps_off():
    q, s, gu, mass, inter = _case()
    q2 = q.copy()
    i = np.argmax((q & 0x7F) > 0x40)
    r, c = divmod(int(i), q.shape[1])
    q2[r, c] = q2[r, c] + 2
    with pytest.raises(AssertionError):
        silu_mul_quant_check(q2, s, gu, mass, inter)



def _wide_gemm_case():
    """Quantised-style codes with per-block scales spread over the UE8M0 range."""
    rng = np.random.default_rng(7)
    m, n, k = 16, 24, 256
    nblk = k // 32
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    b = rng.integers(0, 0x7E, (n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) * 0x80).astype(np.uint8)
    base = rng.integers(10, 245, nblk)
    sa = np.clip(base[None, :] + rng.integers(-8, 9, (m, nblk)), 2, 252).astype(np.uint8)
    sb = np.clip(254 - base[None, :] + rng.integers(-8, 9, (n, nblk)), 2, 252).astype(np.uint8)
    ref, exact = oracle.gemm(a, sa, 0, b, sb, 0, want_f64=True)
    t, mass = oracle.gemm_accum_terms(a, sa, 0, b, sb, 0)
    return a, sa, b, sb, ref, exact, accum_error_bound(t, mass, k)


def test_accum_bound_accepts_the_oracle_and_its_bf16_neighbour():
    a, sa, b, sb, ref, exact, bound = _wide_gemm_case()
    assert gemm_accum_bound_ratio(ref, ref, exact, bound) == 0.0
    # one BF16 step away (a rounding that landed on the other side of a midpoint) is allowed
    assert gemm_accum_bound_ratio(ref + 1, ref, exact, bound) <= 1.0


def test_accum_bound_rejects_a_block_scale_off_by_one():
    a, sa, b, sb, ref, exact, bound = _wide_gemm_case()
    sa2 = sa.copy()
    sa2[:, 3] += 1  # one block of every A row scaled twice too much
    wrong = oracle.gemm(a, sa2, 0, b, sb, 0)
    assert gemm_accum_bound_ratio(wrong, ref, exact, bound) > 1.0


def test_accum_bound_rejects_swapped_blocks():
    a, sa, b, sb, ref, exact, bound = _wide_gemm_case()
    a2 = a.copy()
    a2[:, 0:32], a2[:, 32:64] = a[:, 32:64], a[:, 0:32]  # data of blocks 0 and 1 exchanged
    wrong = oracle.gemm(a2, sa, 0, b, sb, 0)
    assert gemm_accum_bound_ratio(wrong, ref, exact, bound) > 1.0


def test_accum_bound_rejects_a_transposed_operand():
    rng = np.random.default_rng(3)
    m = n = 32
    k = 512
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    b = rng.integers(0, 0x7E, (n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) * 0x80).astype(np.uint8)
    s = rng.integers(118, 128, (m, k // 32)).astype(np.uint8)
    ref, exact = oracle.gemm(a, s, 0, b, s, 0, want_f64=True)
    t, mass = oracle.gemm_accum_terms(a, s, 0, b, s, 0)
    bound = accum_error_bound(t, mass, k)
    assert gemm_accum_bound_ratio(ref.T.copy(), ref, exact, bound) > 1.0


def _emulate_model(a, sa, b, sb, trunc_bits, order):
    """Brute-force emulation of the accumulation model on the decoded operands: per group of 8
    consecutive K products, truncate each toward zero below 2^(E - trunc_bits) (E the exponent
    of the group's largest product), sum the group exactly, scale it, and add the group sums
    into an fp32 accumulator in the given order."""
    dec = oracle.e4m3_values()
    m, k = a.shape
    n = b.shape[0]
    out = np.zeros((m, n), dtype=np.float32)
    for i in range(m):
        for j in range(n):
            p = dec[a[i]] * dec[b[j]]
            sums = []
            for g in range(k // 8):
                pg = p[8 * g:8 * g + 8]
                pmax = np.max(np.abs(pg))
                if pmax > 0:
                    unit = 2.0 ** (np.floor(np.log2(pmax)) - trunc_bits)
                    pg = np.sign(pg) * np.floor(np.abs(pg) / unit) * unit
                kb = g // 4
                sums.append(float(np.sum(pg)) * 2.0 ** (int(sa[i, kb]) + int(sb[j, kb]) - 254))
            acc = np.float32(0.0)
            for g in order(len(sums)):
                acc = np.float32(acc + np.float32(sums[g]))
            out[i, j] = acc
    return out


@pytest.mark.parametrize("order", [lambda n: range(n), lambda n: range(n - 1, -1, -1)])
def test_accum_bound_covers_an_emulated_accumulation(order):
    """The bound holds for an fp32 accumulation that truncates as the model says, summed forward
    or backward, on data chosen to make the truncation bite: each group mixes products near the
    top of its range with products 2^8..2^12 smaller."""
    rng = np.random.default_rng(11)
    m, n, k = 6, 5, 256
    big = rng.integers(0x60, 0x7E, (m, k)).astype(np.uint8)
    small = rng.integers(0x08, 0x30, (m, k)).astype(np.uint8)
    a = np.where(rng.random((m, k)) < 0.5, big, small) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    b = rng.integers(0x30, 0x7E, (n, k)).astype(np.uint8) | (rng.integers(0, 2, (n, k)) * 0x80).astype(np.uint8)
    sa = rng.integers(110, 140, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (n, k // 32)).astype(np.uint8)
    _, exact = oracle.gemm(a, sa, 0, b, sb, 0, want_f64=True)
    t, mass = oracle.gemm_accum_terms(a, sa, 0, b, sb, 0, trunc_bits=TRUNC_BITS)
    bound = accum_error_bound(t, mass, k)
    emu = _emulate_model(a, sa, b, sb, TRUNC_BITS, order).astype(np.float64)
    assert np.all(t > 0), "the data must make the truncation lose something"
    assert np.all(np.abs(emu - exact) <= bound)
    # and the truncation term is what carries it: without T the emulation falls outside
    assert np.any(np.abs(emu - exact) > bound - t)


def test_accum_terms_mass_is_the_gemm_of_magnitudes():
    """S equals the oracle's GEMM of the code magnitudes (an independent evaluation)."""
    rng = np.random.default_rng(5)
    a = rng.integers(0, 256, (9, 128)).astype(np.uint8)
    b = rng.integers(0, 256, (7, 128)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x10  # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x22
    s = rng.integers(100, 150, (9, 4)).astype(np.uint8)
    t = rng.integers(100, 150, (7, 4)).astype(np.uint8)
    _, mass_ref = oracle.gemm(a & 0x7F, s, 0, b & 0x7F, t, 0, want_f64=True)
    trunc, mass = oracle.gemm_accum_terms(a, s, 0, b, t, 0)
    assert np.allclose(mass, mass_ref, rtol=1e-12, atol=0)  # fp64 sums in another order
    assert np.all(trunc >= 0) and np.all(trunc <= mass * 2.0 ** -TRUNC_BITS * 8)


def _norm_case():
    import synth
    from parity_util import bits16
    x, w = synth.norm_inputs_bf16(40, 256)
    q, sl, ss, y = oracle.rmsnorm_quant(bits16(x), bits16(w), float(np.float32(1e-6)))
    return q, sl, ss, y


def test_norm_check_accepts_the_oracle_result():
    from parity_util import norm_quant_check
    q, sl, ss, y = _norm_case()
    assert norm_quant_check(q, sl, ss, q, sl, ss, y, oracle.e4m3_encode) == (0, 0)
    assert norm_quant_check(q, None, ss, q, sl, ss, y, oracle.e4m3_encode) == (0, 0)
    assert norm_quant_check(q, sl, None, q, sl, ss, y, oracle.e4m3_encode) == (0, 0)


def test_norm_check_rejects_a_scale_off_away_from_a_boundary():
    from parity_util import norm_quant_check, near_scale_boundary
    q, sl, ss, y = _norm_case()
    near = near_scale_boundary(y)
    r, b = np.argwhere(~near)[0]
    sl2 = sl.copy()
    sl2[r, b] += 1
    with pytest.raises(AssertionError):
        norm_quant_check(q, sl2, None, q, sl, ss, y, oracle.e4m3_encode)


def test_norm_check_rejects_a_code_two_steps_off_and_a_bad_swizzle():
    from parity_util import norm_quant_check
    q, sl, ss, y = _norm_case()
    q2 = q.copy()
    i = int(np.argmax((q & 0x7F) > 0x40))
    q2.flat[i] += 2
    with pytest.raises(AssertionError):
        norm_quant_check(q2, sl, ss, q, sl, ss, y, oracle.e4m3_encode)
    ss2 = ss.copy()
    ss2[5] ^= 1
    with pytest.raises(AssertionError):
        norm_quant_check(q, sl, ss2, q, sl, ss, y, oracle.e4m3_encode)


def test_norm_check_allows_the_next_scale_only_at_a_boundary():
    """A block whose amax sits exactly on 448 * 2^e: a kernel that took the next scale (as a
    sum in another order could) passes with its codes re-quantised at that scale, and is
    counted; the same step with codes left at the old scale fails."""
    from parity_util import norm_quant_check, near_scale_boundary
    q, sl, ss, y = _norm_case()
    y = y.copy()
    y[3, 32:64] *= np.float32(448.0 / np.max(np.abs(y[3, 32:64])))  # amax exactly 448 * 2^0
    q_ref = q.copy()
    q_ref[3, 32:64] = oracle.e4m3_encode(y[3, 32:64].astype(np.float64))
    sl_ref = sl.copy()
    sl_ref[3, 1] = 127
    assert near_scale_boundary(y)[3, 1]
    sl_gpu = sl_ref.copy()
    sl_gpu[3, 1] = 128
    q_gpu = q_ref.copy()
    q_gpu[3, 32:64] = oracle.e4m3_encode(y[3, 32:64].astype(np.float64) / 2.0)
    n_scale, n_code = norm_quant_check(q_gpu, sl_gpu, None, q_ref, sl_ref, None, y, oracle.e4m3_encode)
    assert n_scale == 1 and n_code == 0
    with pytest.raises(AssertionError):
        norm_quant_check(q_ref, sl_gpu, None, q_ref, sl_ref, None, y, oracle.e4m3_encode)
