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
