// kernels.h - launchers of the MXFP8 kernels (internal to the library; the C ABI is include/mxfp8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp8 {

// Arguments are validated by the C-ABI layer before any launcher runs.
hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                           uint8_t* s_lin, uint8_t* s_swz, hipStream_t stream);

// res: null, or the residual stream [rows, hidden] (row stride ldr) that x is first added to;
// it is overwritten with BF16(x + res) and the norm is taken of that sum.
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t rows, int64_t hidden,
                                int64_t ldx, float eps, uint8_t* q, uint8_t* s_lin, uint8_t* s_swz,
                                uint16_t* res, int64_t ldr, hipStream_t stream);

// Zero the pad bytes of a swizzled scale buffer for a [rows, k] operand (no-op without padding).
hipError_t launch_swizzle_pad_zero(uint8_t* s_swz, int64_t rows, int64_t k, hipStream_t stream);

// Linear scales [rows, k/32] -> 128x4 swizzled layout with zero pad bytes.
hipError_t launch_swizzle_scales(const uint8_t* lin, int64_t rows, int64_t k, uint8_t* swz, hipStream_t stream);

struct GemmShape {
  int bm, bn;  // output tile
};

// Tile shape the GEMM uses for this problem.
GemmShape gemm_pick_shape(int64_t m, int64_t n, int num_chunks, int a_layout, int b_layout);

hipError_t launch_gemm(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                       const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k, uint16_t* c,
                       int64_t ldc, int num_chunks, int first_chunk, int* chunk_done, hipStream_t stream);

// Fused dense GEMM1: gate_up GEMM (w = [gate; up], 2*inter rows), SiLU(gate) * up, MXFP8 quantisation.
hipError_t launch_gemm_silu_mul_quant(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* w,
                                      const uint8_t* ws, int w_layout, int64_t m, int64_t inter, int64_t k,
                                      uint8_t* q, uint8_t* s_lin, uint8_t* s_swz, hipStream_t stream);

}  // namespace mxfp8
