"""GPU parity of the fused dense GEMM1 (mxfp8_gemm_silu_mul_quant: gate_up MXFP8 GEMM, SiLU(gate)
* up, per-32 MXFP8 quantisation) against the oracle.

Inputs are quantised by the oracle on the CPU. The kernel forms gate and up in the MFMA's fp32
accumulators, whose error is bounded per element by the worst case of the MFMA's accumulation
(parity_util.accum_error_bound: each group's truncation loss plus the fp32 summation bound), so
its quantisation decisions may differ from the oracle's exact ones only within that bound: every
scale must be reachable from an amax within the bound, every dequantised code must be a correct
rounding of a value within the bound, and the share of decisions that differ must stay small.
The oracle's own codes and scales are compared exactly where the comparison is decided. Small
shapes (one per tile configuration, ragged rows and columns) are checked in full; the workload
(M = 32768 tokens, inter = 3072 per rank, hidden K = 6144) on whole sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import quant_mxfp8_gemm_amd as mx
import synth
from parity_util import accum_error_bound, bits16, dev_u8, guard_intact, guarded_u8, silu_mul_quant_check

pytestmark = pytest.mark.gpu


def _operands(m, inter, k, seed_a=0, seed_w=1):
    a = synth.activations_bf16(m, k, seed=seed_a)
    w = synth.weights_bf16(2 * inter, k, seed=seed_w)
    qa, sa_lin, sa_swz = oracle.quantize(bits16(a))
    qw, sw_lin, sw_swz = oracle.quantize(bits16(w))
    return qa, {mx.LINEAR: sa_lin, mx.SWIZZLED: sa_swz}, qw, {mx.LINEAR: sw_lin, mx.SWIZZLED: sw_swz}


def _run(qa, sa, la, qw, sw, lw):
    m = qa.shape[0]
    inter = qw.shape[0] // 2
    qbuf, q = guarded_u8(m * inter)
    lbuf, s_lin = guarded_u8(m * (inter // 32))
    zbuf, s_swz = guarded_u8(mx.scale_bytes(m, inter, mx.SWIZZLED))
    mx.gemm_silu_mul_quant(dev_u8(qa), dev_u8(sa), la, dev_u8(qw), dev_u8(sw), lw,
                           out=(q.view(m, inter), s_lin.view(m, inter // 32), s_swz))
    torch.cuda.synchronize()
    assert guard_intact(qbuf) and guard_intact(lbuf) and guard_intact(zbuf), "write outside an output"
    return q.view(m, inter).cpu().numpy(), s_lin.view(m, inter // 32).cpu().numpy(), s_swz.cpu().numpy()


def _mass(qa, sa, la, qw, sw, lw, rows):
    """The accumulation bound of every gate_up element of the listed rows (gate columns, then up)."""
    n = qw.shape[0]
    ri = np.repeat(np.asarray(rows, dtype=np.int64), n)
    ci = np.tile(np.arange(n, dtype=np.int64), len(rows))
    trunc, mass = oracle.gemm_accum_terms(qa, sa, la, qw, sw, lw, ri, ci)
    return accum_error_bound(trunc, mass, qa.shape[1]).reshape(len(rows), n)


# (m, inter, k, tile_m): one case per tile configuration (256 x 256, 256 x 192, 192 x 192,
# 128 x 192, 96 x 192, 128 x 128, 64 x 128, 32 x 128), with ragged rows and columns
CASES = [(2048, 4096, 128, 256), (2048, 3072, 256, 256), (1500, 3072, 256, 192), (1024, 3072, 256, 128),
         (768, 3072, 256, 96), (1000, 1536, 256, 128),
         (100, 6112, 256, 64), (40, 1056, 256, 32)]


@pytest.mark.parametrize("la,lw", [(1, 1), (0, 1)])
@pytest.mark.parametrize("m,inter,k,tile_m", CASES)
def test_gemm_silu_mul_quant_full(m, inter, k, tile_m, la, lw):
    print(f"gemm_silu_mul_quant m={m} inter={inter} k={k} tile_m={tile_m} layouts={la}{lw}", flush=True)
    qa, sa, qw, sw = _operands(m, inter, k, seed_a=m, seed_w=inter)
    q, s_lin, s_swz = _run(qa, sa[la], la, qw, sw[lw], lw)
    q_ref, s_ref, _, gu = oracle.gemm_silu_mul_quant(qa, sa[la], la, qw, sw[lw], lw, want_gu=True)
    mass = _mass(qa, sa[la], la, qw, sw[lw], lw, range(m))
    s_diff, v_diff = silu_mul_quant_check(q, s_lin, gu, mass, inter)
    print(f"  scales differing {s_diff:.2e}, values differing {v_diff:.2e}", flush=True)
    assert s_diff <= 0.01 and v_diff <= 0.01
    # both layouts carry the same scales; pad bytes are zero
    assert np.array_equal(s_swz, oracle.swizzle_scales(s_lin))
    # where the kernel's scale agrees with the oracle's, most codes are the oracle's codes
    assert np.mean(q == q_ref) > 0.99 and np.mean(s_lin == s_ref) > 0.99


@pytest.mark.parametrize("m,inter,k", [(1, 32, 128), (3, 96, 384)])
def test_gemm_silu_mul_quant_minimal(m, inter, k):
    """The smallest shapes: one row, one 32-block of the intermediate dimension."""
    qa, sa, qw, sw = _operands(m, inter, k, seed_a=5, seed_w=6)
    q, s_lin, s_swz = _run(qa, sa[0], 0, qw, sw[0], 0)
    q_ref, s_ref, _, gu = oracle.gemm_silu_mul_quant(qa, sa[0], 0, qw, sw[0], 0, want_gu=True)
    mass = _mass(qa, sa[0], 0, qw, sw[0], 0, range(m))
    silu_mul_quant_check(q, s_lin, gu, mass, inter)
    assert np.array_equal(s_swz, oracle.swizzle_scales(s_lin))


def test_gemm_silu_mul_quant_workload_rows():
    """M = 32768, inter = 3072, K = 6144 (the dense MLP per TP4 rank feeding down_proj K = 3072)."""
    m, inter, k = 32768, 3072, 6144
    print(f"gemm_silu_mul_quant workload m={m} inter={inter} k={k}", flush=True)
    qa, sa, qw, sw = _operands(m, inter, k)
    q, s_lin, s_swz = _run(qa, sa[1], 1, qw, sw[1], 1)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 8191, 8192, 16384, 32767],
                                     rng.integers(0, m, 30)])).astype(np.int64)
    q_ref, s_ref, _, gu = oracle.gemm_silu_mul_quant(qa, sa[1], 1, qw, sw[1], 1, rows=rows, want_gu=True)
    mass = _mass(qa, sa[1], 1, qw, sw[1], 1, rows)
    s_diff, v_diff = silu_mul_quant_check(q[rows], s_lin[rows], gu, mass, inter)
    print(f"  scales differing {s_diff:.2e}, values differing {v_diff:.2e}", flush=True)
    assert s_diff <= 0.01 and v_diff <= 0.01
    assert np.mean(q[rows] == q_ref) > 0.99
    # the swizzled scales of the sampled rows sit where the 128x4 layout puts them
    nblk = inter // 32
    for r in rows[:8]:
        offs = [oracle.swizzle_offset(int(r), c, nblk) for c in range(nblk)]
        assert np.array_equal(s_swz[offs], s_lin[r])


@pytest.mark.parametrize("m,inter,k,tile_n", [(2048, 3072, 640, 192), (2048, 6144, 384, 192), (8192, 3072, 384, 256)])
def test_gemm_silu_mul_quant_split_ring_matches_staged(m, inter, k, tile_n):
    """With swizzled, 16-byte aligned scales the 256 x 192 and 256 x 256 tiles run as two wave
    groups (B three stages deep, the scales in registers; 512 and 768 tiles in the last two
    cases, so workgroups take two or three); scale buffers 4 bytes off that alignment take the
    staged kernel. Both form the same fp32 sums, so codes and scales agree bit for bit (and with
    the oracle's within the accumulation bound, checked on the first case)."""
    assert mx.gemm_tiles_per_chunk(m, 2 * inter, 1, 1, 1) == ((m + 255) // 256) * (2 * inter // tile_n)
    print(f"fused GEMM1 two-group vs staged m={m} inter={inter} k={k}", flush=True)
    qa, sa, qw, sw = _operands(m, inter, k, seed_a=11, seed_w=12)
    outs = []
    for off in (0, 4):
        bufs = []
        for arr in (sa[1], sw[1]):
            buf = torch.zeros(arr.size + 16, dtype=torch.uint8, device="cuda")
            view = buf[off:off + arr.size]
            view.copy_(dev_u8(arr).view(-1))
            bufs.append(view)
        assert (bufs[0].data_ptr() % 16 == 0) == (off == 0)
        q, s_lin, s_swz = mx.gemm_silu_mul_quant(dev_u8(qa), bufs[0], 1, dev_u8(qw), bufs[1], 1, linear=True,
                                                 swizzled=True)
        outs.append((q.cpu().numpy(), s_lin.cpu().numpy(), s_swz.cpu().numpy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)
    if (m, inter) != (2048, 3072):
        return
    q_ref, s_ref, _, gu = oracle.gemm_silu_mul_quant(qa, sa[1], 1, qw, sw[1], 1, want_gu=True)
    mass = _mass(qa, sa[1], 1, qw, sw[1], 1, range(m))
    s_diff, v_diff = silu_mul_quant_check(outs[0][0], outs[0][1], gu, mass, inter)
    assert s_diff <= 0.01 and v_diff <= 0.01


def test_gemm_silu_mul_quant_feeds_down_proj():
    """The fused output is a valid down_proj operand: the GEMM on it equals the GEMM on the
    same codes with scales rebuilt from the linear copy."""
    m, inter, k = 512, 1024, 512
    qa, sa, qw, sw = _operands(m, inter, k)
    q, s_lin, s_swz = mx.gemm_silu_mul_quant(dev_u8(qa), dev_u8(sa[1]), 1, dev_u8(qw), dev_u8(sw[1]), 1,
                                             linear=True, swizzled=True)
    wd, _, wds = mx.quantize(synth.weights_bf16(768, inter, seed=3).cuda(), linear=False)
    c1 = mx.gemm(q, s_swz, mx.SWIZZLED, wd, wds, mx.SWIZZLED, num_chunks=4)
    c2 = mx.gemm(q, s_lin, mx.LINEAR, wd, wds, mx.SWIZZLED, num_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("seed", range(8))
def test_gemm_silu_mul_quant_random_shapes(seed):
    """Seeded random shapes (M 1-1500, inter a multiple of 32 up to 1888, K 128-896, either scale
    layout on either side) in full, with the same decision bounds as the fixed cases."""
    rng = np.random.default_rng(5000 + seed)
    m, inter, k = int(rng.integers(1, 1500)), int(rng.integers(1, 60)) * 32, int(rng.integers(1, 8)) * 128
    la, lw = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    print(f"gemm_silu_mul_quant random seed={seed}: m={m} inter={inter} k={k} layouts={la}{lw}", flush=True)
    qa, sa, qw, sw = _operands(m, inter, k, seed_a=6000 + seed, seed_w=7000 + seed)
    q, s_lin, s_swz = _run(qa, sa[la], la, qw, sw[lw], lw)
    q_ref, s_ref, _, gu = oracle.gemm_silu_mul_quant(qa, sa[la], la, qw, sw[lw], lw, want_gu=True)
    s_diff, v_diff = silu_mul_quant_check(q, s_lin, gu, _mass(qa, sa[la], la, qw, sw[lw], lw, range(m)), inter)
    assert s_diff <= 0.01 and v_diff <= 0.01
    assert np.array_equal(s_swz, oracle.swizzle_scales(s_lin))
