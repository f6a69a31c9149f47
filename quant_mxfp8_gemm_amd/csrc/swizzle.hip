// swizzle.hip - linear UE8M0 scales [rows, nblk] -> the 128x4 swizzled layout.
//
// Swizzled scales of several row blocks cannot be concatenated into the swizzled scales of
// the whole (vLLM PR #65496, "Tradeoff"): a 512-byte tile mixes 128 rows. A gathered MXFP8
// activation therefore carries linear scales, which concatenate by rows, and is swizzled
// once after the gather, before the GEMM (PR #65496, "Details"; PR #64659, "Details").
//
// One thread writes one 16-byte unit of the output: unit d of tile (a, e) holds rows
// 128a + 32b + d for b = 0..3, each with blocks 4e..4e+3 (byte 4b + f = block 4e + f).
// Consecutive threads write consecutive units, so the stores are full lines; the four
// 4-byte reads per thread come from rows nblk bytes apart and are served by L2.
#include "device_common.h"
#include "kernels.h"

namespace mxfp8 {
namespace {

constexpr int ST = 256;

template <bool DWORDS>
__global__ __launch_bounds__(ST) void swizzle_scales_kernel(const uint8_t* __restrict__ lin, int64_t rows,
                                                            int64_t nblk, int64_t col_tiles, int64_t units,
                                                            uint8_t* __restrict__ swz) {
  for (int64_t u = (int64_t)blockIdx.x * ST + threadIdx.x; u < units; u += (int64_t)gridDim.x * ST) {
    const int64_t tile = u >> 5;
    const int64_t d = u & 31;
    const int64_t r0 = (tile / col_tiles) * 128 + d;
    const int64_t c0 = (tile % col_tiles) * 4;
    uint32_t w[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t r = r0 + 32 * b;
      if (r >= rows) {
        w[b] = 0;
      } else if (DWORDS) {
        // nblk % 4 == 0 and a 4-byte aligned base: the four blocks are one aligned dword
        w[b] = *(const uint32_t*)(lin + r * nblk + c0);
      } else {
        uint32_t v = 0;
        for (int f = 0; f < 4; ++f)
          if (c0 + f < nblk) v |= (uint32_t)lin[r * nblk + c0 + f] << (8 * f);
        w[b] = v;
      }
    }
    *(uint4*)(swz + u * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_swizzle_scales(const uint8_t* lin, int64_t rows, int64_t k, uint8_t* swz, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t nblk = k / 32;
  const int64_t col_tiles = (nblk + 3) / 4;
  const int64_t units = ((rows + 127) / 128) * col_tiles * 32;
  int64_t grid = (units + ST - 1) / ST;
  if (grid > 65536) grid = 65536;
  if (nblk % 4 == 0 && (uintptr_t)lin % 4 == 0)
    swizzle_scales_kernel<true><<<dim3((unsigned)grid), dim3(ST), 0, stream>>>(lin, rows, nblk, col_tiles, units, swz);
  else
    swizzle_scales_kernel<false><<<dim3((unsigned)grid), dim3(ST), 0, stream>>>(lin, rows, nblk, col_tiles, units, swz);
  return hipGetLastError();
}

}  // namespace mxfp8
