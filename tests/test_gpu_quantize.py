"""GPU parity of mxfp8_quantize against the CPU oracle: codes and both scale layouts
bit-exact (BF16 inputs make every step exact), pad bytes zero, nothing written outside
the outputs."""
import numpy as np
import pytest
import torch

import oracle
import quant_mxfp8_gemm_amd as mx
import synth
from parity_util import bits16, dev_u8, guard_intact, guarded_u8

pytestmark = pytest.mark.gpu


def _run_gpu(x_dev: torch.Tensor, linear=True, swizzled=True):
    rows, k = x_dev.shape
    qb, q = guarded_u8(rows * k)
    lb, sl = guarded_u8(rows * (k // 32)) if linear else (None, None)
    sb, ss = guarded_u8(mx.scale_bytes(rows, k, mx.SWIZZLED)) if swizzled else (None, None)
    mx.quantize(x_dev, out=(q.view(rows, k), sl.view(rows, k // 32) if linear else None, ss))
    torch.cuda.synchronize()
    assert guard_intact(qb)
    if linear:
        assert guard_intact(lb)
    if swizzled:
        assert guard_intact(sb)
    return (q.view(rows, k).cpu().numpy(), sl.view(rows, k // 32).cpu().numpy() if linear else None,
            ss.cpu().numpy() if swizzled else None)


def _check(x_cpu_bf16: torch.Tensor, x_dev=None, linear=True, swizzled=True):
    bits = bits16(x_cpu_bf16)
    q_ref, sl_ref, ss_ref = oracle.quantize(bits)
    if x_dev is None:
        x_dev = x_cpu_bf16.cuda()
    q, sl, ss = _run_gpu(x_dev, linear, swizzled)
    assert np.array_equal(q, q_ref), f"{np.sum(q != q_ref)} codes differ"
    if linear:
        assert np.array_equal(sl, sl_ref), f"{np.sum(sl != sl_ref)} linear scales differ"
    if swizzled:
        assert np.array_equal(ss, ss_ref), f"{np.sum(ss != ss_ref)} swizzled scale bytes differ"


@pytest.mark.parametrize("rows,k,kind", [
    (128, 2048, "act"),        # o_proj activation, M=128
    (6144, 2048, "weight"),    # o_proj weight [N, K]
    (6144, 3072, "weight"),    # down_proj weight [N, K]
    (1024, 3072, "gated"),     # down_proj activation silu(g)*u
    (4096, 2048, "act"),
])
def test_quantize_workload_shapes(rows, k, kind):
    print(f"quantize rows={rows} k={k} kind={kind}", flush=True)
    if kind == "act":
        x = synth.activations_bf16(rows, k, seed=0)
    elif kind == "gated":
        x = synth.gated_activations_bf16(rows, k, seed=0)
    else:
        x = synth.weights_bf16(rows, k, seed=1)
    _check(x)


@pytest.mark.parametrize("k", [3072, 2048])
def test_quantize_full_chain_input(k):
    """The per-rank chain input, BF16 [32768, k] ~ N(0,1), compared in full."""
    print(f"quantize full rows=32768 k={k}", flush=True)
    _check(synth.activations_bf16(32768, k, seed=0))


@pytest.mark.parametrize("rows,k,ldx", [(200, 96, 128), (1, 32, 32), (129, 160, 200), (37, 2048, 2056)])
def test_quantize_ragged_and_strided(rows, k, ldx):
    print(f"quantize ragged rows={rows} k={k} ldx={ldx}", flush=True)
    full = synth.activations_bf16(rows, ldx, seed=rows)
    x_dev = full.cuda()[:, :k]
    assert x_dev.stride(0) == ldx
    _check(full[:, :k].contiguous(), x_dev=x_dev)


@pytest.mark.parametrize("linear,swizzled", [(True, False), (False, True)])
def test_quantize_single_layout(linear, swizzled):
    print(f"quantize layout linear={linear} swizzled={swizzled}", flush=True)
    _check(synth.activations_bf16(300, 256, seed=4), linear=linear, swizzled=swizzled)


def test_quantize_edge_values():
    """Zero and negative-zero blocks, amax exactly on and just above 448 * 2^e, huge and tiny
    exponents, BF16 subnormals and the largest finite BF16."""
    rng = np.random.default_rng(21)
    rows, k = 64, 512
    v = rng.standard_normal((rows, k))
    v[0, :32] = 0.0
    v[0, 32:64] = -0.0
    for i, e in enumerate(range(-30, 30, 4)):
        v[1 + i, :32] *= 0.5
        v[1 + i, 5] = 448.0 * 2.0 ** e           # exactly on the boundary
        v[1 + i, 32:64] *= 0.5
        v[1 + i, 40] = 450.0 * 2.0 ** e          # just above it
    v[20] = rng.standard_normal(k) * 1e37
    v[21] = rng.standard_normal(k) * 1e-37
    v[22, :32] = 3.3895313892515355e38           # largest finite BF16
    v[23] = rng.standard_normal(k) * 2.0 ** -130  # BF16 subnormals
    v[24, :32] = rng.standard_normal(32) * 2.0 ** -133
    v[25] = np.where(rng.random(k) < 0.5, -1.0, 1.0) * 2.0 ** rng.integers(-60, 60, k)
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    _check(x)


def test_quantize_zero_rows_is_a_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, sl, ss = mx.quantize(x)
    torch.cuda.synchronize()
    assert q.numel() == 0 and sl.numel() == 0 and ss.numel() == 0
