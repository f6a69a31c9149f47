"""The comparison rules the GPU parity tests use, exercised on the CPU with oracle outputs:
they accept the oracle's own result and reject planted mistakes (no GPU involved)."""
import numpy as np
import pytest

import oracle
from parity_util import silu_mul_quant_check


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
