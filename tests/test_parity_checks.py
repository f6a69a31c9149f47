"""The comparison rules the GPU parity tests use, exercised on the CPU with oracle outputs:
they accept the oracle's own result and reject planted mistakes (no GPU involved)."""
import numpy as np
import pytest

import oracle
from parity_util import gemm_mass_bound_ratio, silu_mul_quant_check


def _case():
    rng = np.random.default_rng(31)
    m, inter, k = 8, 64, 256
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)) * 0x80).astype(np.uint8)
    w = rng.integers(0, 0x70, (2 * inter, k)).astype(np.uint8) | (rng.integers(0, 2, (2 * inter, k)) * 0x80).astype(np.uint8)
    sa = rng.integers(120, 128, (m, k // 32)).astype(np.uint8)
    sw = rng.integers(118, 124, (2 * inter, k // 32)).astype(np.uint8)
    q, s, y, gu = oracle.gemm_silu_mul_quant(a, sa, 0, w, sw, 0, want_gu=True)
    ri = np.repeat(np.arange(m, dtype=np.int64), 2 * inter)
    ci = np.tile(np.arange(2 * inter, dtype=np.int64), m)
    _, mass = oracle.gemm_sampled(a & 0x7F, sa, 0, w & 0x7F, sw, 0, ri, ci)
    return q, s, gu, mass.reshape(m, 2 * inter), inter


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
    _, mass = oracle.gemm(a & 0x7F, sa, 0, b & 0x7F, sb, 0, want_f64=True)
    return a, sa, b, sb, ref, exact, mass


def test_mass_bound_accepts_the_oracle_and_its_bf16_neighbour():
    a, sa, b, sb, ref, exact, mass = _wide_gemm_case()
    assert gemm_mass_bound_ratio(ref, ref, exact, mass) == 0.0
    # one BF16 step away (a rounding that landed on the other side of a midpoint) is allowed
    assert gemm_mass_bound_ratio(ref + 1, ref, exact, mass) <= 1.0


def test_mass_bound_rejects_a_block_scale_off_by_one():
    a, sa, b, sb, ref, exact, mass = _wide_gemm_case()
    sa2 = sa.copy()
    sa2[:, 3] += 1  # one block of every A row scaled twice too much
    wrong = oracle.gemm(a, sa2, 0, b, sb, 0)
    assert gemm_mass_bound_ratio(wrong, ref, exact, mass) > 1.0


def test_mass_bound_rejects_swapped_blocks():
    a, sa, b, sb, ref, exact, mass = _wide_gemm_case()
    a2 = a.copy()
    a2[:, 0:32], a2[:, 32:64] = a[:, 32:64], a[:, 0:32]  # data of blocks 0 and 1 exchanged
    wrong = oracle.gemm(a2, sa, 0, b, sb, 0)
    assert gemm_mass_bound_ratio(wrong, ref, exact, mass) > 1.0
