// rmsnorm_quant.hip - Gemma-style RMSNorm fused with MXFP8 quantisation.
//
// y = x / sqrt(mean(x^2) + eps) * (1 + w), quantised per 32 elements to E4M3 + UE8M0 and written
// with linear and/or 128x4-swizzled scales in the same pass: the norm that hands qkv_proj a
// QuantizedActivation (vLLM PR #65496, "Details") and the Gemma norm + MXFP8 quant fusion of
// PR #64111 ("Claims"), without the all-reduce. PR #65496 ("Tradeoff") is why both scale
// layouts can be emitted: swizzled scales cannot be concatenated by rows after a gather.
//
// One workgroup per row; the row stays in registers (CPT 16-byte pieces per lane). The sum of
// squares and y itself are formed in fp64 and y is rounded once to fp32, so the fp32 value that
// decides each scale and code is the correctly rounded y; the kernel is bound by HBM traffic,
// which hides the extra arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace mxfp8 {
namespace {

constexpr int RT = 256;  // threads per workgroup (4 waves)

// Sum over the 64 lanes, in every lane: four DPP steps inside each row of 16 lanes, then two
// cross-row exchanges.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<DPP_XOR1>(v);
  v += dpp_f64<DPP_XOR2>(v);
  v += dpp_f64<DPP_HALF_MIRROR>(v);
  v += dpp_f64<DPP_MIRROR>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Two BF16 pairs added and rounded back to BF16 (nearest even). The fp32 sum of two BF16
// values rounded to BF16 equals their exact sum rounded once: fp32 carries more than twice
// BF16's precision plus two bits, so the intermediate rounding cannot move the result.
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  return pack_bf16x2(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b));
}

// RES: the row is first replaced by h = BF16(x + res) (written back to res, the residual
// stream) and the norm is taken of h.
template <int CPT, bool LIN, bool SWZ, bool RES>
__global__ __launch_bounds__(RT) void rmsnorm_quant_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w, int hidden,
                                                           int64_t ldx, double eps,
                                                           uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ s_lin,
                                                           uint8_t* __restrict__ s_swz,
                                                           uint16_t* __restrict__ res, int64_t ldr) {
  __shared__ double partial[RT / 64];
  const int64_t row = blockIdx.x;
  const int cpr = hidden >> 3;
  const int nblk = hidden >> 5;
  const int col_tiles = (nblk + 3) >> 2;
  const uint16_t* xr = x + row * ldx;

  uint4 v[CPT], wv[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {  // the weight row is loaded with x, not after the reduction
    const int c8 = u * RT + (int)threadIdx.x;
    wv[u] = c8 < cpr ? *(const uint4*)(w + c8 * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  // every load of the row is in flight before the first one is used
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c8 = u * RT + (int)threadIdx.x;
    v[u] = c8 < cpr ? *(const uint4*)(xr + c8 * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (RES) {
    uint4 rv[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c8 = u * RT + (int)threadIdx.x;
      rv[u] = c8 < cpr ? *(const uint4*)(res + row * ldr + c8 * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
    // all sums before the first store: a load waited for after a store would wait for it too
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      v[u] = make_uint4(add_bf16x2(v[u].x, rv[u].x), add_bf16x2(v[u].y, rv[u].y), add_bf16x2(v[u].z, rv[u].z),
                        add_bf16x2(v[u].w, rv[u].w));
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c8 = u * RT + (int)threadIdx.x;
      if (c8 < cpr) *(uint4*)(res + row * ldr + c8 * 8) = v[u];
    }
  }
  double ss = 0.0;  // pad lanes hold zeros
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = (double)bf16_lo(wd[j]);
      const double b = (double)bf16_hi(wd[j]);
      ss += a * a;
      ss += b * b;
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < RT / 64; ++i) tot += partial[i];
  const double rstd = 1.0 / sqrt(tot / (double)hidden + eps);

#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c8 = u * RT + (int)threadIdx.x;
    const bool live = c8 < cpr;  // uniform over the four lanes of a block (cpr % 4 == 0)
    float y[8];
    uint32_t m = 0;
    if (live) {
      const uint32_t xd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const uint32_t wd[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = (float)((double)bf16_lo(xd[j]) * rstd * (1.0 + (double)bf16_lo(wd[j])));
        y[2 * j + 1] = (float)((double)bf16_hi(xd[j]) * rstd * (1.0 + (double)bf16_hi(wd[j])));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = 0.f;
    }
    m = max(m, dpp_u32<DPP_XOR1>(m));  // the four lanes of a 32-block
    m = max(m, dpp_u32<DPP_XOR2>(m));
    const uint32_t s = ue8m0_from_amax_f32_bits(m);
    const float f = inv_scale_from_ue8m0(s);
    if (live) {
      const uint32_t lo = cvt_e4m3x4(y[0] * f, y[1] * f, y[2] * f, y[3] * f);
      const uint32_t hi = cvt_e4m3x4(y[4] * f, y[5] * f, y[6] * f, y[7] * f);
      __builtin_nontemporal_store(((uint64_t)hi << 32) | lo, (uint64_t*)(q + row * hidden + c8 * 8));
      if ((threadIdx.x & 3) == 0) {
        const int b = c8 >> 2;
        if (LIN) s_lin[row * nblk + b] = (uint8_t)s;
        if (SWZ) s_swz[swizzled_offset(row, b, col_tiles)] = (uint8_t)s;
      }
    }
  }
}

template <int CPT, bool RES>
hipError_t launch_res(const uint16_t* x, const uint16_t* w, int64_t rows, int hidden, int64_t ldx, double eps,
                      uint8_t* q, uint8_t* s_lin, uint8_t* s_swz, uint16_t* res, int64_t ldr, hipStream_t stream) {
  const dim3 grid((unsigned)rows), block(RT);
  if (s_lin && s_swz)
    rmsnorm_quant_kernel<CPT, true, true, RES><<<grid, block, 0, stream>>>(x, w, hidden, ldx, eps, q, s_lin, s_swz, res, ldr);
  else if (s_lin)
    rmsnorm_quant_kernel<CPT, true, false, RES><<<grid, block, 0, stream>>>(x, w, hidden, ldx, eps, q, s_lin, s_swz, res, ldr);
  else
    rmsnorm_quant_kernel<CPT, false, true, RES><<<grid, block, 0, stream>>>(x, w, hidden, ldx, eps, q, s_lin, s_swz, res, ldr);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_cpt(const uint16_t* x, const uint16_t* w, int64_t rows, int hidden, int64_t ldx, double eps,
                      uint8_t* q, uint8_t* s_lin, uint8_t* s_swz, uint16_t* res, int64_t ldr, hipStream_t stream) {
  if (res) return launch_res<CPT, true>(x, w, rows, hidden, ldx, eps, q, s_lin, s_swz, res, ldr, stream);
  return launch_res<CPT, false>(x, w, rows, hidden, ldx, eps, q, s_lin, s_swz, nullptr, 0, stream);
}

}  // namespace

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t rows, int64_t hidden,
                                int64_t ldx, float eps, uint8_t* q, uint8_t* s_lin, uint8_t* s_swz,
                                uint16_t* res, int64_t ldr, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int cpt = (int)((hidden / 8 + RT - 1) / RT);  // 1..8 (hidden <= 16384)
  const double e = (double)eps;
  const int h = (int)hidden;
  hipError_t err;
  switch (cpt) {
    case 1: err = launch_cpt<1>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 2: err = launch_cpt<2>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 3: err = launch_cpt<3>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 4: err = launch_cpt<4>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 5: err = launch_cpt<5>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 6: err = launch_cpt<6>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    case 7: err = launch_cpt<7>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
    default: err = launch_cpt<8>(x, w, rows, h, ldx, e, q, s_lin, s_swz, res, ldr, stream); break;
  }
  if (err != hipSuccess) return err;
  if (s_swz) err = launch_swizzle_pad_zero(s_swz, rows, hidden, stream);
  return err;
}

}  // namespace mxfp8
