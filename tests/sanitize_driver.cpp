// sanitize_driver.cpp - exercises the CPU oracle and the library's host-only argument checks
// under the address and undefined-behaviour sanitizers (built and run by
// tests/test_sanitize_cpu.py with g++; no GPU and no HIP call). Every buffer is sized exactly,
// so an out-of-bounds access in either part is reported by the sanitizer; the checks are also
// fed adversarial sizes (negative, huge, overflowing products) that must be rejected without
// undefined arithmetic. Prints "sanitize ok" on success and exits non-zero on a wrong result.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "mxfp8.h"

extern "C" {
double oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_encode(double v);
int oracle_scale_exponent(double amax);
uint16_t oracle_bf16_from_double(double v);
int64_t oracle_scale_bytes(int64_t rows, int64_t k, int layout);
int oracle_swizzle_scales(const uint8_t* s_lin, int64_t rows, int64_t k, uint8_t* s_swz);
int oracle_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q, uint8_t* s_lin,
                          uint8_t* s_swz);
int oracle_rmsnorm_quant_mxfp8(const uint16_t* x, const uint16_t* w, int64_t rows, int64_t hidden, int64_t ldx,
                               double eps, uint8_t* q, uint8_t* s_lin, uint8_t* s_swz, float* y_out);
int oracle_add_rmsnorm_quant_mxfp8(const uint16_t* x, const uint16_t* r, const uint16_t* w, int64_t rows,
                                   int64_t hidden, int64_t ldx, int64_t ldr, double eps, uint8_t* q, uint8_t* s_lin,
                                   uint8_t* s_swz, uint16_t* h_out, float* y_out);
int oracle_mxfp8_gemm_bf16out(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                              const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k, uint16_t* c_bf16,
                              int64_t ldc, double* c_f64);
int oracle_mxfp8_gemm_sampled(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                              const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k, const int64_t* rows,
                              const int64_t* cols, int64_t count, uint16_t* out_bf16, double* out_f64);
int oracle_gemm_silu_mul_quant(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* w,
                               const uint8_t* ws, int w_layout, int64_t m, int64_t inter, int64_t k,
                               const int64_t* rows, int64_t nrows, uint8_t* q, uint8_t* s_lin, float* y_out,
                               double* gu_out);
int oracle_gemm_accum_terms(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b, const uint8_t* bs,
                            int b_layout, int64_t m, int64_t n, int64_t k, const int64_t* rows, const int64_t* cols,
                            int64_t count, int trunc_bits, double* t_out, double* s_out);
}

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static uint32_t g_state = 12345u;
static uint32_t next_u32() {  // xorshift32: deterministic inputs, no library generator
  g_state ^= g_state << 13;
  g_state ^= g_state >> 17;
  g_state ^= g_state << 5;
  return g_state;
}

// a finite BF16 value of moderate magnitude (exponent field 100..140)
static uint16_t rand_bf16() {
  uint32_t r = next_u32();
  return (uint16_t)(((r & 1u) << 15) | ((100u + (r >> 1) % 41u) << 7) | ((r >> 8) & 0x7Fu));
}

static uint8_t rand_e4m3() {
  uint8_t c = (uint8_t)(next_u32() & 0xFF);
  return (c & 0x7F) == 0x7F ? (uint8_t)(c & 0xF0) : c;  // no NaN codes
}

static void oracle_part() {
  // scalar routines at their edges
  for (int c = 0; c < 256; ++c) {
    double v = oracle_e4m3_value((uint8_t)c);
    if ((c & 0x7F) != 0x7F) EXPECT(oracle_e4m3_encode(v) == (uint8_t)c || (v == 0.0));
  }
  EXPECT(oracle_e4m3_encode(1e30) == 0x7E && oracle_e4m3_encode(-1e30) == 0xFE);
  EXPECT(oracle_scale_exponent(0.0) == -127 && oracle_scale_exponent(448.0) == 0);
  EXPECT(oracle_scale_exponent(1e300) == 127 && oracle_scale_exponent(1e-300) == -127);
  EXPECT(oracle_bf16_from_double(0.0) == 0 && oracle_bf16_from_double(-0.0) == 0x8000);
  EXPECT(oracle_bf16_from_double(1e300) == 0x7F80);

  // quantiser with a row stride, both layouts, ragged rows (37 % 128) and blocks (3 % 4)
  const int64_t rows = 37, k = 96, ldx = 128;
  std::vector<uint16_t> x(rows * ldx);
  for (auto& v : x) v = rand_bf16();
  std::vector<uint8_t> q(rows * k), s_lin(rows * (k / 32)), s_swz(oracle_scale_bytes(rows, k, 1));
  EXPECT(oracle_mxfp8_quantize(x.data(), rows, k, ldx, q.data(), s_lin.data(), s_swz.data()) == 0);
  std::vector<uint8_t> s_swz2(s_swz.size());
  EXPECT(oracle_swizzle_scales(s_lin.data(), rows, k, s_swz2.data()) == 0);
  EXPECT(memcmp(s_swz.data(), s_swz2.data(), s_swz.size()) == 0);
  EXPECT(oracle_mxfp8_quantize(x.data(), rows, k, k - 1, q.data(), s_lin.data(), nullptr) < 0);
  EXPECT(oracle_mxfp8_quantize(x.data(), -1, k, ldx, q.data(), s_lin.data(), nullptr) < 0);

  // norm quantisers
  const int64_t nr = 5, h = 256;
  std::vector<uint16_t> xn(nr * h), rn(nr * h), w(h), hout(nr * h);
  for (auto& v : xn) v = rand_bf16();
  for (auto& v : rn) v = rand_bf16();
  for (auto& v : w) v = rand_bf16();
  std::vector<uint8_t> qn(nr * h), sln(nr * (h / 32)), ssn(oracle_scale_bytes(nr, h, 1));
  std::vector<float> y(nr * h);
  EXPECT(oracle_rmsnorm_quant_mxfp8(xn.data(), w.data(), nr, h, h, 1e-6, qn.data(), sln.data(), ssn.data(),
                                    y.data()) == 0);
  EXPECT(oracle_add_rmsnorm_quant_mxfp8(xn.data(), rn.data(), w.data(), nr, h, h, h, 1e-6, qn.data(), sln.data(),
                                        ssn.data(), hout.data(), y.data()) == 0);
  EXPECT(oracle_rmsnorm_quant_mxfp8(xn.data(), w.data(), nr, 48, 48, 1e-6, qn.data(), sln.data(), nullptr,
                                    nullptr) < 0);

  // GEMM, sampled GEMM, accumulation terms, fused GEMM1: ragged M and N, both layouts
  const int64_t m = 9, n = 7, kk = 128, inter = 32;
  std::vector<uint8_t> a(m * kk), b(n * kk), wg(2 * inter * kk);
  for (auto& v : a) v = rand_e4m3();
  for (auto& v : b) v = rand_e4m3();
  for (auto& v : wg) v = rand_e4m3();
  std::vector<uint8_t> sa(m * (kk / 32)), sb(n * (kk / 32)), sw(2 * inter * (kk / 32));
  for (auto& v : sa) v = (uint8_t)(110 + next_u32() % 30);
  for (auto& v : sb) v = (uint8_t)(110 + next_u32() % 30);
  for (auto& v : sw) v = (uint8_t)(110 + next_u32() % 30);
  std::vector<uint8_t> sa_swz(oracle_scale_bytes(m, kk, 1)), sb_swz(oracle_scale_bytes(n, kk, 1));
  EXPECT(oracle_swizzle_scales(sa.data(), m, kk, sa_swz.data()) == 0);
  EXPECT(oracle_swizzle_scales(sb.data(), n, kk, sb_swz.data()) == 0);
  std::vector<uint16_t> c1(m * n), c2(m * (n + 3));
  std::vector<double> f1(m * n);
  EXPECT(oracle_mxfp8_gemm_bf16out(a.data(), sa.data(), 0, b.data(), sb.data(), 0, m, n, kk, c1.data(), n,
                                   f1.data()) == 0);
  EXPECT(oracle_mxfp8_gemm_bf16out(a.data(), sa_swz.data(), 1, b.data(), sb_swz.data(), 1, m, n, kk, c2.data(),
                                   n + 3, nullptr) == 0);
  for (int64_t i = 0; i < m; ++i) EXPECT(memcmp(&c1[i * n], &c2[i * (n + 3)], n * 2) == 0);
  std::vector<int64_t> ri = {0, 8, 3, 8}, ci = {0, 6, 2, 0};
  std::vector<uint16_t> sbits(ri.size());
  std::vector<double> sf(ri.size()), tt(ri.size()), ss(ri.size());
  EXPECT(oracle_mxfp8_gemm_sampled(a.data(), sa.data(), 0, b.data(), sb_swz.data(), 1, m, n, kk, ri.data(),
                                   ci.data(), (int64_t)ri.size(), sbits.data(), sf.data()) == 0);
  for (size_t t = 0; t < ri.size(); ++t) EXPECT(sf[t] == f1[ri[t] * n + ci[t]]);
  EXPECT(oracle_gemm_accum_terms(a.data(), sa.data(), 0, b.data(), sb.data(), 0, m, n, kk, ri.data(), ci.data(),
                                 (int64_t)ri.size(), 13, tt.data(), ss.data()) == 0);
  for (size_t t = 0; t < ri.size(); ++t) EXPECT(tt[t] >= 0.0 && ss[t] >= fabs(sf[t]) * (1.0 - 1e-12));
  std::vector<int64_t> bad_rows = {0, 9};
  EXPECT(oracle_mxfp8_gemm_sampled(a.data(), sa.data(), 0, b.data(), sb.data(), 0, m, n, kk, bad_rows.data(),
                                   ci.data(), 2, sbits.data(), sf.data()) < 0);
  std::vector<int64_t> grows = {0, 4, 8};
  std::vector<uint8_t> qg(grows.size() * inter), sg(grows.size() * (inter / 32));
  std::vector<float> yg(grows.size() * inter);
  std::vector<double> gu(grows.size() * 2 * inter);
  EXPECT(oracle_gemm_silu_mul_quant(a.data(), sa.data(), 0, wg.data(), sw.data(), 0, m, inter, kk, grows.data(),
                                    (int64_t)grows.size(), qg.data(), sg.data(), yg.data(), gu.data()) == 0);
}

static void checks_part() {
  // aligned host buffers stand in for device pointers: the checks only look at the addresses
  std::vector<uint8_t> buf(1 << 16);
  uint8_t* base = (uint8_t*)(((uintptr_t)buf.data() + 255) & ~(uintptr_t)255);
  void* p = base;
  void* p2 = base + 16384;
  void* odd = base + 2;
  const int64_t big = INT64_MAX, neg = INT64_MIN;

  EXPECT(mxfp8_scale_bytes(128, 128, 0) == 512 && mxfp8_scale_bytes(200, 96, 1) == 1024);
  EXPECT(mxfp8_scale_bytes(big, 64, 0) == -1 && mxfp8_scale_bytes(10, big - 31, 1) == -1);
  EXPECT(mxfp8_scale_bytes(neg, 64, 0) == -1 && mxfp8_scale_bytes(10, 64, 9) == -1);
  for (int s = -6; s <= 1; ++s) EXPECT(mxfp8_status_string(s) != nullptr);

  EXPECT(mxfp8_quantize_check(p, 32768, 3072, 3072, p2, p, nullptr) == MXFP8_OK);
  EXPECT(mxfp8_quantize_check(p, 0, 64, 64, nullptr, nullptr, nullptr) == MXFP8_OK);
  EXPECT(mxfp8_quantize_check(p, 4, 48, 48, p2, p, nullptr) == MXFP8_EINVAL);
  EXPECT(mxfp8_quantize_check(p, 4, 64, 64, p2, nullptr, nullptr) == MXFP8_EINVAL);
  EXPECT(mxfp8_quantize_check(odd, 4, 64, 64, p2, p, nullptr) == MXFP8_EALIGN);
  EXPECT(mxfp8_quantize_check(p, big, 64, 64, p2, p, nullptr) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_quantize_check(p, (1 << 30), 64, big - 63, p2, p, nullptr) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_quantize_check(p, neg, 64, 64, p2, p, nullptr) == MXFP8_EINVAL);

  EXPECT(rmsnorm_quant_mxfp8_check(p, p2, 1024, 6144, 6144, p, p2, nullptr) == MXFP8_OK);
  EXPECT(rmsnorm_quant_mxfp8_check(p, p2, 4, 32768, 32768, p, p2, nullptr) == MXFP8_EUNSUPPORTED);
  EXPECT(rmsnorm_quant_mxfp8_check(p, p2, (1 << 30), 6144, big - 7, p, p2, nullptr) == MXFP8_EUNSUPPORTED);
  EXPECT(add_rmsnorm_quant_mxfp8_check(p, p2, p, 4, 256, 256, 256, p, p2, nullptr) == MXFP8_OK);
  EXPECT(add_rmsnorm_quant_mxfp8_check(p, p, p2, 4, 256, 256, 256, p2, p, nullptr) == MXFP8_EINVAL);
  EXPECT(add_rmsnorm_quant_mxfp8_check(p, p2, p, 4, 256, 256, big - 7, p, p2, nullptr) == MXFP8_EUNSUPPORTED);

  EXPECT(mxfp8_swizzle_scales_check(p, 130, 96, p2) == MXFP8_OK);
  EXPECT(mxfp8_swizzle_scales_check(p, big, 96, p2) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_swizzle_scales_check(p, 130, 96, odd) == MXFP8_EALIGN);

  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, 32768, 6144, 3072, p, 6144, 4, 0) == MXFP8_OK);
  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, 32768, 6144, 96, p, 6144, 4, 0) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, 32768, 6144, 3072, p, 6144, 3, 0) == MXFP8_EINVAL);
  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, big, big, big - 127, p, big, 1, 0) == MXFP8_EINVAL);
  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, (1 << 30), (1 << 30), (int64_t)1 << 40, p, (1 << 30), 1,
                                  0) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_gemm_bf16out_check(p, p, 1, p2, p2, 1, big - 1, 8, 128, p, 8, 1, 0) == MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_gemm_bf16out_check(odd, p, 1, p2, p2, 1, 128, 128, 128, p, 128, 1, 0) == MXFP8_EALIGN);
  EXPECT(mxfp8_gemm_silu_mul_quant_check(p, p, 1, p2, p2, 1, 32768, 3072, 6144, p, nullptr, p2) == MXFP8_OK);
  EXPECT(mxfp8_gemm_silu_mul_quant_check(p, p, 1, p2, p2, 1, big, big - 31, big - 127, p, nullptr, p2) ==
         MXFP8_EUNSUPPORTED);
  EXPECT(mxfp8_gemm_silu_mul_quant_check(p, p, 1, p2, p2, 1, 64, 48, 128, p, nullptr, p2) == MXFP8_EINVAL);
}

int main() {
  oracle_part();
  checks_part();
  if (g_fail) return 1;
  printf("sanitize ok\n");
  return 0;
}
