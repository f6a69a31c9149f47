// quantize.hip - BF16 -> MXFP8 (E4M3 data + UE8M0 scale per 32 elements along K).
//
// The activation quantisation of the GEMM-RS path (vLLM PR #64659, "Details: GEMM-RS with a
// quantized input") and of qkv_proj after the all-gather (PR #65496, "Overview").
//
// HBM streaming kernel: every lane owns 16-byte pieces (8 BF16) of the input, four neighbouring
// lanes form one 32-element block, and two DPP lane swaps give the block amax. The amax is taken
// on the BF16 magnitude bits as integers (order-preserving for non-negative floats), the UE8M0
// exponent comes straight from those bits, and the scaled values (exact power-of-two products)
// go through the hardware fp32 -> E4M3 conversion, which rounds to nearest even.
// Each lane keeps QU pieces in flight before converting any of them. The input is read and the
// codes are written with streaming (non-temporal) accesses: each byte is touched once here
// (non-temporal loads measured 2-3% faster at [32768, 3072] and [32768, 2048]).
#include "device_common.h"
#include "kernels.h"

namespace mxfp8 {
namespace {

constexpr int QT = 256;  // threads per workgroup
constexpr int QU = 2;    // 16-byte pieces per lane

template <typename Idx, bool LIN, bool SWZ>
__global__ __launch_bounds__(QT) void quantize_kernel(const uint16_t* __restrict__ x, Idx rows, Idx k,
                                                      Idx ldx, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ s_lin,
                                                      uint8_t* __restrict__ s_swz) {
  const Idx cpr = k >> 3;  // pieces per row (a multiple of 4)
  const Idx total = rows * cpr;
  const Idx nblk = k >> 5;
  const Idx col_tiles = (nblk + 3) >> 2;
  const Idx base = (Idx)blockIdx.x * (QT * QU) + threadIdx.x;

  uint4 v[QU];
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const Idx p = base + (Idx)(u * QT);
    if (p < total) {
      const Idx r = p / cpr;
      const Idx c8 = p - r * cpr;
      v[u] = load16_stream(x + r * ldx + c8 * 8);
    } else {
      v[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

#pragma unroll
  for (int u = 0; u < QU; ++u) {
    const Idx p = base + (Idx)(u * QT);
    const uint4 t = v[u];
    uint32_t m = max(max(t.x & 0x7FFFu, (t.x >> 16) & 0x7FFFu), max(t.y & 0x7FFFu, (t.y >> 16) & 0x7FFFu));
    m = max(m, max(max(t.z & 0x7FFFu, (t.z >> 16) & 0x7FFFu), max(t.w & 0x7FFFu, (t.w >> 16) & 0x7FFFu)));
    // the four lanes of a block are all in range or all out of range (total % 4 == 0)
    m = max(m, dpp_u32<DPP_XOR1>(m));
    m = max(m, dpp_u32<DPP_XOR2>(m));
    const uint32_t s = ue8m0_from_amax_bf16_bits(m);
    const float f = inv_scale_from_ue8m0(s);
    const uint32_t lo = cvt_e4m3x4(bf16_lo(t.x) * f, bf16_hi(t.x) * f, bf16_lo(t.y) * f, bf16_hi(t.y) * f);
    const uint32_t hi = cvt_e4m3x4(bf16_lo(t.z) * f, bf16_hi(t.z) * f, bf16_lo(t.w) * f, bf16_hi(t.w) * f);
    if (p < total) {
      const Idx r = p / cpr;
      const Idx c8 = p - r * cpr;
      __builtin_nontemporal_store(((uint64_t)hi << 32) | lo, (uint64_t*)(q + r * k + c8 * 8));
      if ((threadIdx.x & 3) == 0) {
        const Idx b = c8 >> 2;
        if (LIN) s_lin[r * nblk + b] = (uint8_t)s;
        if (SWZ) s_swz[swizzled_offset(r, b, col_tiles)] = (uint8_t)s;
      }
    }
  }
}

// Writes 0 to every pad byte (row >= rows or block >= nblk) of a swizzled scale buffer.
__global__ __launch_bounds__(256) void swizzle_pad_kernel(uint8_t* __restrict__ s_swz, int64_t rows,
                                                          int64_t nblk, int64_t total) {
  const int64_t col_tiles = (nblk + 3) >> 2;
  for (int64_t off = (int64_t)blockIdx.x * 256 + threadIdx.x; off < total; off += (int64_t)gridDim.x * 256) {
    const int64_t tile = off >> 9;
    const int64_t in = off & 511;
    const int64_t r = (tile / col_tiles) * 128 + ((in >> 2) & 3) * 32 + (in >> 4);
    const int64_t c = (tile % col_tiles) * 4 + (in & 3);
    if (r >= rows || c >= nblk) s_swz[off] = 0;
  }
}

template <typename Idx>
hipError_t launch_q(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q, uint8_t* s_lin,
                    uint8_t* s_swz, hipStream_t stream) {
  const int64_t pieces = rows * (k / 8);
  const int64_t grid = (pieces + QT * QU - 1) / (QT * QU);
  if (s_lin && s_swz)
    quantize_kernel<Idx, true, true><<<dim3((unsigned)grid), dim3(QT), 0, stream>>>(x, (Idx)rows, (Idx)k, (Idx)ldx, q, s_lin, s_swz);
  else if (s_lin)
    quantize_kernel<Idx, true, false><<<dim3((unsigned)grid), dim3(QT), 0, stream>>>(x, (Idx)rows, (Idx)k, (Idx)ldx, q, s_lin, s_swz);
  else
    quantize_kernel<Idx, false, true><<<dim3((unsigned)grid), dim3(QT), 0, stream>>>(x, (Idx)rows, (Idx)k, (Idx)ldx, q, s_lin, s_swz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swizzle_pad_zero(uint8_t* s_swz, int64_t rows, int64_t k, hipStream_t stream) {
  const int64_t nblk = k / 32;
  if (rows % 128 == 0 && nblk % 4 == 0) return hipSuccess;
  const int64_t total = ((rows + 127) / 128) * 128 * ((nblk + 3) / 4) * 4;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  swizzle_pad_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(s_swz, rows, nblk, total);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                           uint8_t* s_lin, uint8_t* s_swz, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipError_t e;
  // 32-bit index arithmetic whenever every offset fits
  if (rows * ldx < (int64_t)1 << 31 && rows * (k / 8) + QT * QU < (int64_t)1 << 31)
    e = launch_q<uint32_t>(x, rows, k, ldx, q, s_lin, s_swz, stream);
  else
    e = launch_q<int64_t>(x, rows, k, ldx, q, s_lin, s_swz, stream);
  if (e != hipSuccess) return e;
  if (s_swz) e = launch_swizzle_pad_zero(s_swz, rows, k, stream);
  return e;
}

}  // namespace mxfp8
