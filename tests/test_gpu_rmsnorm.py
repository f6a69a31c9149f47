"""GPU parity of rmsnorm_quant_mxfp8 against the CPU oracle.

Bar: UE8M0 scales identical except in blocks whose oracle amax lies within 2^-20
(relative) of a power-of-two boundary 448 * 2^e, where one step is allowed and counted;
E4M3 codes identical except at most one code step where the RMSNorm arithmetic can
differ. Both sides take the quantisation decisions on fp32 y; the kernel forms y in fp64
and rounds once, so the expected number of differences is zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quant_mxfp8_gemm_amd as mx
import synth
from parity_util import bits16, e4m3_step_diff, guard_intact, guarded_u8

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-6))


def _near_boundary(y_ref: np.ndarray) -> np.ndarray:
    """Per block: is amax within 2^-20 relative of 448 * 2^e for some integer e?"""
    rows, h = y_ref.shape
    amax = np.abs(y_ref.astype(np.float64)).reshape(rows, h // 32, 32).max(-1)
    with np.errstate(divide="ignore"):
        t = np.log2(np.where(amax > 0, amax, 1.0) / 448.0)
    frac = np.abs(t - np.round(t))
    return (amax > 0) & (frac < 2.0 ** -20 / math.log(2) * 2)


def _check(x: torch.Tensor, w: torch.Tensor, x_dev=None, linear=True, swizzled=True):
    rows, h = x.shape
    q_ref, sl_ref, ss_ref, y_ref = oracle.rmsnorm_quant(bits16(x), bits16(w), EPS)
    if x_dev is None:
        x_dev = x.cuda()
    qb, q = guarded_u8(rows * h)
    lb, sl = guarded_u8(rows * (h // 32))
    sb, ss = guarded_u8(mx.scale_bytes(rows, h, mx.SWIZZLED))
    mx.rmsnorm_quant(x_dev, w.cuda(), EPS, out=(q.view(rows, h), sl.view(rows, h // 32) if linear else None,
                                               ss if swizzled else None))
    torch.cuda.synchronize()
    for b in (qb, lb, sb):
        assert guard_intact(b)
    q = q.view(rows, h).cpu().numpy()
    near = _near_boundary(y_ref)
    if linear:
        sl = sl.view(rows, h // 32).cpu().numpy()
        sdiff = np.abs(sl.astype(int) - sl_ref.astype(int))
        assert np.all(sdiff[~near] == 0), f"{np.sum(sdiff[~near] != 0)} scales differ away from a boundary"
        assert np.all(sdiff <= 1)
        n_scale = int(np.sum(sdiff != 0))
    else:
        n_scale = 0
    if swizzled:
        ssv = ss.cpu().numpy()
        sw_diff = np.abs(ssv.astype(int) - ss_ref.astype(int))
        assert np.all(sw_diff <= 1)
        if linear:
            assert int(np.sum(sw_diff != 0)) == n_scale
        else:
            n_scale = int(np.sum(sw_diff != 0))
            assert n_scale <= int(near.sum())
    steps = e4m3_step_diff(q, q_ref)
    if n_scale == 0:
        assert np.all(steps <= 1), "a code differs by more than one step"
    n_code = int(np.sum(steps != 0))
    print(f"rmsnorm rows={rows} hidden={h}: scale diffs {n_scale}, code diffs {n_code}, "
          f"near-boundary blocks {int(near.sum())}", flush=True)
    return n_scale, n_code


def test_rmsnorm_workload_1024x6144():
    """1024 tokens x hidden 6144, x ~ N(0,1) with 1% outliers x50, w ~ N(0, 0.1^2)."""
    x, w = synth.norm_inputs_bf16(1024, 6144)
    n_scale, n_code = _check(x, w)
    assert n_scale <= 2 and n_code <= 64


@pytest.mark.parametrize("rows,h,ldx", [(37, 96, 128), (5, 32, 32), (64, 16384, 16384), (300, 2048, 2056),
                                        (130, 6144, 6144)])
def test_rmsnorm_shapes(rows, h, ldx):
    print(f"rmsnorm rows={rows} hidden={h} ldx={ldx}", flush=True)
    full, _ = synth.norm_inputs_bf16(rows, ldx, seed_x=rows)
    w = synth.normal_bf16((h,), 0.1, seed=h)
    x_dev = full.cuda()[:, :h]
    n_scale, n_code = _check(full[:, :h].contiguous(), w, x_dev=x_dev)
    assert n_scale <= 1 and n_code <= 8


def test_rmsnorm_weight_minus_one_gives_zero_codes():
    x = synth.activations_bf16(16, 256, seed=3)
    w = torch.full((256,), -1.0, dtype=torch.bfloat16)
    q, sl, ss = mx.rmsnorm_quant(x.cuda(), w.cuda(), EPS)
    torch.cuda.synchronize()
    neg = x.float().numpy() < 0
    assert np.array_equal(q.cpu().numpy(), np.where(neg, 0x80, 0x00).astype(np.uint8))
    assert np.all(sl.cpu().numpy() == 0)


@pytest.mark.parametrize("linear,swizzled", [(True, False), (False, True)])
def test_rmsnorm_single_layout(linear, swizzled):
    x, w = synth.norm_inputs_bf16(64, 512)
    _check(x, w, linear=linear, swizzled=swizzled)


@pytest.mark.parametrize("rows,h", [(1024, 6144), (37, 4096), (5, 96)])
def test_add_rmsnorm_matches_oracle(rows, h):
    """Residual add + norm quantiser: the updated residual is bit-exact and the codes and scales
    meet the same bar as the plain norm quantiser."""
    print(f"add_rmsnorm rows={rows} hidden={h}", flush=True)
    x, w = synth.norm_inputs_bf16(rows, h)
    r = synth.normal_bf16((rows, h), seed=9, sigma=2.0)
    q_ref, sl_ref, ss_ref, h_ref, y_ref = oracle.add_rmsnorm_quant(bits16(x), bits16(r), bits16(w), EPS)
    rd = r.cuda().clone()
    q, sl, ss = mx.add_rmsnorm_quant(x.cuda(), rd, w.cuda(), EPS)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(rd), h_ref), "residual stream"
    near = _near_boundary(y_ref)
    sdiff = np.abs(sl.cpu().numpy().astype(int) - sl_ref.astype(int))
    assert np.all(sdiff[~near] == 0) and np.all(sdiff <= 1)
    steps = e4m3_step_diff(q.cpu().numpy(), q_ref)
    if int(sdiff.sum()) == 0:
        assert np.array_equal(ss.cpu().numpy(), ss_ref)
        assert np.all(steps <= 1)
    print(f"  scale diffs {int((sdiff != 0).sum())}, code diffs {int((steps != 0).sum())}", flush=True)
