"""GPU parity of mxfp8_swizzle_scales (linear -> 128x4 swizzled scales) against the oracle,
bit-exact over the whole output buffer including pad bytes, and the gather path it serves:
quantise row shards with linear scales, concatenate, swizzle once, then run the GEMM."""
import numpy as np
import pytest
import torch

import oracle
import quant_mxfp8_gemm_amd as mx
import synth
from parity_util import bits16, dev_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,k", [(1, 32), (127, 160), (128, 128), (300, 2048), (1024, 6144),
                                    (4096, 3072), (32768, 3072), (200, 224)])
@pytest.mark.parametrize("offset", [0, 1])
def test_swizzle_scales_matches_oracle(rows, k, offset):
    print(f"swizzle rows={rows} k={k} offset={offset}", flush=True)
    nblk = k // 32
    s = np.random.default_rng(rows + k).integers(0, 256, (rows, nblk), dtype=np.uint8)
    ref = oracle.swizzle_scales(s)
    # linear scales at a byte offset inside a larger buffer (offset 1: unaligned byte path)
    base = torch.zeros(rows * nblk + 16, dtype=torch.uint8, device="cuda")
    lin = base[offset:offset + rows * nblk].view(rows, nblk)
    lin.copy_(torch.from_numpy(s).cuda())
    total = mx.scale_bytes(rows, k, mx.SWIZZLED)
    guard = 256
    out = torch.full((total + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    mx.swizzle_scales(lin, out=out[:total])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:total], ref)
    assert np.all(got[total:] == 0xA5), "write past the swizzled buffer"


def test_swizzle_scales_zero_rows_is_noop():
    s = torch.empty((0, 4), dtype=torch.uint8, device="cuda")
    out = mx.swizzle_scales(s)
    assert out.numel() == 0


def test_gather_then_swizzle_feeds_gemm():
    """Four row shards of the norm input are quantised with linear scales only (one per rank),
    gathered by concatenation, swizzled once, and multiplied; the result equals the GEMM on the
    unsharded operand quantised with swizzled scales directly."""
    x, w = synth.norm_inputs_bf16(1024, 6144)
    xd, wd = x.cuda(), w.cuda()
    shards = [mx.rmsnorm_quant(xd[i:i + 256], wd, 1e-6, linear=True, swizzled=False) for i in range(0, 1024, 256)]
    q = torch.cat([sh[0] for sh in shards])
    s_lin = torch.cat([sh[1] for sh in shards])
    s_swz = mx.swizzle_scales(s_lin)
    q_whole, _, s_whole = mx.rmsnorm_quant(xd, wd, 1e-6, linear=False, swizzled=True)
    torch.cuda.synchronize()
    assert torch.equal(q, q_whole) and torch.equal(s_swz, s_whole)
    # the gathered operand against the oracle's swizzle of the same linear scales
    assert np.array_equal(s_swz.cpu().numpy(), oracle.swizzle_scales(s_lin.cpu().numpy()))
    wq, _, ws = mx.quantize(synth.weights_bf16(512, 6144, seed=1).cuda(), linear=False)
    c1 = mx.gemm(q, s_swz, mx.SWIZZLED, wq, ws, mx.SWIZZLED, num_chunks=4)
    c2 = mx.gemm(q_whole, s_whole, mx.SWIZZLED, wq, ws, mx.SWIZZLED, num_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
