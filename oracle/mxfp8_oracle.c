/*
 * mxfp8_oracle.c - plain CPU definition of the MXFP8 operations: the quantiser, the
 * Gemma RMSNorm quantiser (with and without a residual add), the block-scaled GEMM, the
 * fused dense GEMM1 (gate_up GEMM, SiLU(gate) * up, quantiser) and the scale swizzle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness oracle of the HIP
 * library: it is loaded by the test suite, by the smoke check and by the CPU
 * baseline leg of the benchmark, and by nothing else. The product path never
 * calls it and shares no code with it.
 *
 * Everything is written from the definitions, in fp64, element by element,
 * with no blocking, fusion or reordering:
 *
 *  - E4M3 ("FN" variant of the OCP 8-bit floating point formats): 1 sign bit,
 *    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
 *    subnormals 2^-6 * m/8; S.1111.111 is NaN; there are no infinities, so the
 *    largest finite magnitude is 1.75 * 2^8 = 448. This is the element format
 *    that vLLM PR #65496 ("Details", root-cause paragraph) names for the
 *    QuantizedActivation data.
 *  - UE8M0 (the OCP Microscaling v1.0 shared-scale format): an unsigned
 *    8-bit biased exponent, value 2^(c - 127); 0xFF is NaN and never produced.
 *    One scale covers 32 consecutive elements along K (MXFP8 as used by the
 *    GEMM-RS path of vLLM PR #64659, "Details: GEMM-RS with a quantized input").
 *  - The scale of a 32-block is the smallest power of two 2^e with
 *    amax <= 448 * 2^e, i.e. 2^ceil(log2(amax / 448)), e clamped to [-127, 127]
 *    and an all-zero block given e = -127. Elements are then encoded as
 *    E4M3(x * 2^-e), rounding to nearest with ties to even, saturating to
 *    +-448 instead of producing NaN.
 *  - The 128x4 swizzled scale layout (the "F8_128x4" layout that PR #64659's
 *    GEMM-RS kernel expects, "Details"; PR #65496 "Tradeoff" notes it cannot be
 *    concatenated by rows): scales of 128 rows x 4 K-blocks form one 512-byte
 *    tile; inside a tile row r and block c sit at (r%32)*16 + (r/32)*4 + c.
 *    Tiles are ordered row-tile major. Padding bytes are zero.
 *  - Gemma-style RMSNorm: y = x / sqrt(mean(x^2) + eps) * (1 + w) (the "Gemma
 *    norm" fused with MXFP8 quantisation in PR #64111 "Claims" and in the norm
 *    of PR #65496 "Details").
 *  - The block-scaled GEMM: C[m,n] = sum over K-blocks kb of
 *    2^(sa[m,kb]-127) * 2^(sb[n,kb]-127) * sum_{i<32} A[m,32kb+i] * B[n,32kb+i],
 *    rounded once to BF16 (round to nearest even). A is [M,K] and B is [N,K],
 *    both K-contiguous.
 *  - The fused dense GEMM1 (PR #64659 "Details", PR #64111 "Claims"): with the
 *    merged gate_up weight (gate rows, then up rows), y = SiLU(g) * u where
 *    SiLU(g) = g / (1 + e^-g), g and u exact GEMM values, y in fp64 rounded once
 *    to fp32 and quantised like the norm output.
 *  - The residual add ahead of the norm: h = BF16(x + r), one rounding of the
 *    exact sum; the norm is taken of h.
 *
 * Inexact steps: only the outer fp64 sum over K-blocks of the GEMM and the
 * fp64 RMSNorm arithmetic round. Each 32-term block product sum is exact in
 * fp64 (8-bit significand products spanning < 2^42 fit in 53 bits).
 *
 * Precision of decisions: the HIP norm and the fused GEMM1 quantise an fp32 y,
 * so this oracle rounds its fp64 y once to fp32 and takes the scale and code
 * decisions on that fp32 value, exactly (in fp64 arithmetic).
 *
 * Every function is pinned by the CPU tests (tests/test_oracle_pins.py) against
 * values fixed outside this file: golden values, torch's E4M3 and BF16 casts and
 * SiLU, closed forms, brute force on small inputs and an independent
 * reshape/transpose construction of the swizzle.
 *
 * Inputs are BF16 bit patterns (uint16). Non-finite inputs are outside the
 * contract; the quantisers report them with a negative return value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENONFINITE (-2)
#define ORACLE_ENOMEM (-3)

/* ------------------------------------------------------------------ formats */

/* Value of an E4M3 code (NaN for S.1111.111). */
double oracle_e4m3_value(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Value of a UE8M0 code: 2^(code - 127); 0xFF is NaN. */
double oracle_ue8m0_value(uint8_t code) {
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* Value of a BF16 bit pattern (its top 16 bits are an IEEE binary32). */
double oracle_bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* Magnitudes of the 127 finite non-negative codes 0x00..0x7E, ascending. */
static double g_mag[127];
static int g_mag_ready = 0;

static void init_tables(void) {
  if (g_mag_ready) return;
  for (int c = 0; c < 127; ++c) g_mag[c] = oracle_e4m3_value((uint8_t)c);
  g_mag_ready = 1;
}

/*
 * Nearest E4M3 code to v: binary search for the bracketing pair of
 * representable magnitudes, pick the closer, and on an exact tie the one with
 * an even mantissa (code LSB 0). Magnitudes >= 448 give 448 (satfinite). The
 * sign is kept, so negative values that round to zero give 0x80.
 */
uint8_t oracle_e4m3_encode(double v) {
  init_tables();
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  int code;
  if (a >= g_mag[126]) {
    code = 126;
  } else {
    int lo = 0, hi = 126; /* g_mag[lo] <= a < g_mag[hi] */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (g_mag[mid] <= a)
        lo = mid;
      else
        hi = mid;
    }
    /* both differences are exact: the bracket spans at most a factor of 2 */
    double dlo = a - g_mag[lo];
    double dhi = g_mag[hi] - a;
    if (dlo < dhi)
      code = lo;
    else if (dhi < dlo)
      code = hi;
    else
      code = (lo % 2 == 0) ? lo : hi;
  }
  return (uint8_t)(sign | code);
}

/* Smallest integer e in [-127, 127] with amax <= 448 * 2^e (127 if none). */
int oracle_scale_exponent(double amax) {
  int e = -127;
  while (e < 127 && amax > ldexp(448.0, e)) ++e;
  return e;
}

/* BF16 (round to nearest, ties to even) of an fp64 value, by one rounding. */
uint16_t oracle_bf16_from_double(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
  int lead = ex - 1;      /* a in [2^lead, 2^(lead+1)) */
  if (lead < -126) lead = -126; /* subnormal BF16: fixed spacing 2^-133 */
  double ulp = ldexp(1.0, lead - 7);
  double r = nearbyint(a / ulp) * ulp; /* default rounding mode: ties to even */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80); /* overflow */
  float rf = (float)r;    /* exact: r has at most 8 significant bits */
  uint32_t w;
  memcpy(&w, &rf, sizeof w);
  return (uint16_t)(sign | (uint16_t)(w >> 16));
}

/* ------------------------------------------------------------ scale layouts */

/* Byte offset of (row r, K-block c) in the 128x4 swizzled layout. */
int64_t oracle_swizzle_offset(int64_t r, int64_t c, int64_t nblk) {
  int64_t col_tiles = (nblk + 3) / 4;
  int64_t tile = (r / 128) * col_tiles + c / 4;
  return tile * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4);
}

/* Bytes of a scale buffer for [rows, k]: layout 0 linear, 1 swizzled. */
int64_t oracle_scale_bytes(int64_t rows, int64_t k, int layout) {
  int64_t nblk = k / 32;
  if (layout == 0) return rows * nblk;
  return ((rows + 127) / 128) * 128 * ((nblk + 3) / 4) * 4;
}

/*
 * Linear scales [rows, k/32] -> the swizzled layout, every other byte 0. The step a row-wise
 * gather of MXFP8 activations needs before the GEMM: swizzled tiles mix 128 rows, so shards
 * can only be concatenated while their scales are linear (vLLM PR #65496, "Tradeoff";
 * PR #64659, "Details"). Each byte is moved on its own by the offset definition above.
 */
int oracle_swizzle_scales(const uint8_t* s_lin, int64_t rows, int64_t k, uint8_t* s_swz) {
  if (rows < 0 || k <= 0 || k % 32 != 0) return ORACLE_EINVAL;
  if (rows == 0) return ORACLE_OK;
  if (!s_lin || !s_swz) return ORACLE_EINVAL;
  int64_t nblk = k / 32;
  memset(s_swz, 0, (size_t)oracle_scale_bytes(rows, k, 1));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < nblk; ++c) s_swz[oracle_swizzle_offset(r, c, nblk)] = s_lin[r * nblk + c];
  return ORACLE_OK;
}

static int64_t scale_index(int layout, int64_t r, int64_t c, int64_t nblk) {
  return layout == 0 ? r * nblk + c : oracle_swizzle_offset(r, c, nblk);
}

/* ---------------------------------------------------------------- quantiser */

/* Quantise one row of fp64 values; writes codes and the row's block scales. */
static void quantize_row(const double* y, int64_t k, uint8_t* q, uint8_t* scale_codes) {
  for (int64_t b = 0; b < k / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs(y[32 * b + i]);
      if (a > amax) amax = a;
    }
    int e = oracle_scale_exponent(amax);
    scale_codes[b] = (uint8_t)(e + 127);
    for (int i = 0; i < 32; ++i) q[32 * b + i] = oracle_e4m3_encode(ldexp(y[32 * b + i], -e));
  }
}

static void store_scales(const uint8_t* codes, int64_t r, int64_t nblk, uint8_t* s_lin, uint8_t* s_swz) {
  for (int64_t c = 0; c < nblk; ++c) {
    if (s_lin) s_lin[r * nblk + c] = codes[c];
    if (s_swz) s_swz[oracle_swizzle_offset(r, c, nblk)] = codes[c];
  }
}

/*
 * x: BF16 [rows, k] with row stride ldx elements. q: E4M3 [rows, k] dense.
 * s_lin: [rows, k/32] or NULL. s_swz: oracle_scale_bytes(rows,k,1) bytes or NULL.
 */
int oracle_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                          uint8_t* s_lin, uint8_t* s_swz) {
  if (rows < 0 || k <= 0 || k % 32 != 0 || ldx < k || !x || !q) return ORACLE_EINVAL;
  init_tables();
  int64_t nblk = k / 32;
  if (s_swz) memset(s_swz, 0, (size_t)oracle_scale_bytes(rows, k, 1));
  int bad = 0, nomem = 0;
#pragma omp parallel reduction(| : bad, nomem)
  {
    double* y = (double*)malloc((size_t)k * sizeof(double));
    uint8_t* codes = (uint8_t*)malloc((size_t)nblk);
    if (!y || !codes) nomem = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      if (!y || !codes) continue;
      for (int64_t i = 0; i < k; ++i) {
        y[i] = oracle_bf16_value(x[r * ldx + i]);
        if (!isfinite(y[i])) bad = 1;
      }
      quantize_row(y, k, q + r * k, codes);
      store_scales(codes, r, nblk, s_lin, s_swz);
    }
    free(y);
    free(codes);
  }
  if (nomem) return ORACLE_ENOMEM;
  return bad ? ORACLE_ENONFINITE : ORACLE_OK;
}

/* ------------------------------------------------- Gemma RMSNorm + quantiser */

/*
 * One row of the Gemma RMSNorm quantiser: y = x / sqrt(sum(x^2)/hidden + eps) * (1 + w) in
 * fp64, rounded once to fp32, then quantised as above. y (double scratch of hidden values)
 * and codes (hidden/32 bytes) are caller buffers. Returns 1 if x holds a non-finite value.
 */
static int norm_row(const uint16_t* xr, const uint16_t* w, int64_t hidden, double eps, uint8_t* q,
                    uint8_t* codes, double* y, float* y_out) {
  int bad = 0;
  double ss = 0.0;
  for (int64_t i = 0; i < hidden; ++i) {
    double xi = oracle_bf16_value(xr[i]);
    if (!isfinite(xi)) bad = 1;
    ss += xi * xi;
  }
  double rstd = 1.0 / sqrt(ss / (double)hidden + eps);
  for (int64_t i = 0; i < hidden; ++i) {
    double xi = oracle_bf16_value(xr[i]);
    double wi = oracle_bf16_value(w[i]);
    float y32 = (float)(xi * rstd * (1.0 + wi));
    if (y_out) y_out[i] = y32;
    y[i] = (double)y32;
  }
  quantize_row(y, hidden, q, codes);
  return bad;
}

/*
 * y = x / sqrt(sum(x^2)/hidden + eps) * (1 + w), in fp64, rounded once to fp32,
 * then quantised as above. x: BF16 [rows, hidden] (row stride ldx), w: BF16
 * [hidden]. y_out (optional): the fp32 y, [rows, hidden] dense.
 */
int oracle_rmsnorm_quant_mxfp8(const uint16_t* x, const uint16_t* w, int64_t rows, int64_t hidden,
                               int64_t ldx, double eps, uint8_t* q, uint8_t* s_lin, uint8_t* s_swz,
                               float* y_out) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0 || ldx < hidden || !x || !w || !q)
    return ORACLE_EINVAL;
  init_tables();
  int64_t nblk = hidden / 32;
  if (s_swz) memset(s_swz, 0, (size_t)oracle_scale_bytes(rows, hidden, 1));
  int bad = 0, nomem = 0;
#pragma omp parallel reduction(| : bad, nomem)
  {
    double* y = (double*)malloc((size_t)hidden * sizeof(double));
    uint8_t* codes = (uint8_t*)malloc((size_t)nblk);
    if (!y || !codes) nomem = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      if (!y || !codes) continue;
      bad |= norm_row(x + r * ldx, w, hidden, eps, q + r * hidden, codes, y, y_out ? y_out + r * hidden : NULL);
      store_scales(codes, r, nblk, s_lin, s_swz);
    }
    free(y);
    free(codes);
  }
  if (nomem) return ORACLE_ENOMEM;
  return bad ? ORACLE_ENONFINITE : ORACLE_OK;
}

/*
 * Residual add ahead of the norm: h = BF16(x + r) (the two BF16 values summed exactly and
 * rounded once, to nearest even) is the new residual stream, and the norm above is applied
 * to h. The pages fuse the norm and the quantisation with the all-reduce that produces x in
 * decode (vLLM PR #64111, "Claims": all-reduce + Gemma norm + MXFP8 quant); on one GPU the
 * all-reduced x is an input. x, r: BF16 [rows, hidden] with row strides ldx, ldr.
 * h_out: BF16 bits [rows, hidden] dense (required); y_out optional as above.
 */
int oracle_add_rmsnorm_quant_mxfp8(const uint16_t* x, const uint16_t* r, const uint16_t* w, int64_t rows,
                                   int64_t hidden, int64_t ldx, int64_t ldr, double eps, uint8_t* q,
                                   uint8_t* s_lin, uint8_t* s_swz, uint16_t* h_out, float* y_out) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0 || ldx < hidden || ldr < hidden || !x || !r || !w || !q ||
      !h_out)
    return ORACLE_EINVAL;
  init_tables();
  int64_t nblk = hidden / 32;
  if (s_swz) memset(s_swz, 0, (size_t)oracle_scale_bytes(rows, hidden, 1));
  int bad = 0, nomem = 0;
#pragma omp parallel reduction(| : bad, nomem)
  {
    double* y = (double*)malloc((size_t)hidden * sizeof(double));
    uint8_t* codes = (uint8_t*)malloc((size_t)nblk);
    if (!y || !codes) nomem = 1;
#pragma omp for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
      if (!y || !codes) continue;
      uint16_t* h = h_out + i * hidden;
      for (int64_t j = 0; j < hidden; ++j)
        h[j] = oracle_bf16_from_double(oracle_bf16_value(x[i * ldx + j]) + oracle_bf16_value(r[i * ldr + j]));
      bad |= norm_row(h, w, hidden, eps, q + i * hidden, codes, y, y_out ? y_out + i * hidden : NULL);
      store_scales(codes, i, nblk, s_lin, s_swz);
    }
    free(y);
    free(codes);
  }
  if (nomem) return ORACLE_ENOMEM;
  return bad ? ORACLE_ENONFINITE : ORACLE_OK;
}

/* --------------------------------------------------------------------- GEMM */

static double g_val[256];
static int g_val_ready = 0;
static void init_values(void) {
  if (g_val_ready) return;
  for (int c = 0; c < 256; ++c) g_val[c] = oracle_e4m3_value((uint8_t)c);
  g_val_ready = 1;
}

/* Exact-as-defined value of C[i,j] before BF16 rounding. */
static double gemm_element(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                           const uint8_t* bs, int b_layout, int64_t i, int64_t j, int64_t k) {
  int64_t nblk = k / 32;
  double acc = 0.0;
  for (int64_t kb = 0; kb < nblk; ++kb) {
    double blk = 0.0;
    for (int t = 0; t < 32; ++t)
      blk += g_val[a[i * k + 32 * kb + t]] * g_val[b[j * k + 32 * kb + t]];
    int sa = as[scale_index(a_layout, i, kb, nblk)];
    int sb = bs[scale_index(b_layout, j, kb, nblk)];
    acc += ldexp(blk, sa + sb - 254);
  }
  return acc;
}

/*
 * C = A * B^T with block scales. a: E4M3 [m,k]; b: E4M3 [n,k]; scales in the
 * given layouts (0 linear, 1 swizzled). c_bf16: [m, ldc] BF16 bits (may be NULL);
 * c_f64: [m, n] dense unrounded values (may be NULL).
 */
int oracle_mxfp8_gemm_bf16out(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                              const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k,
                              uint16_t* c_bf16, int64_t ldc, double* c_f64) {
  if (m < 0 || n < 0 || k <= 0 || k % 32 != 0 || !a || !b || !as || !bs) return ORACLE_EINVAL;
  if ((a_layout != 0 && a_layout != 1) || (b_layout != 0 && b_layout != 1)) return ORACLE_EINVAL;
  if (c_bf16 && ldc < n) return ORACLE_EINVAL;
  init_values();
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      double v = gemm_element(a, as, a_layout, b, bs, b_layout, i, j, k);
      if (c_f64) c_f64[i * n + j] = v;
      if (c_bf16) c_bf16[i * ldc + j] = oracle_bf16_from_double(v);
    }
  }
  return ORACLE_OK;
}

/* Same as above for `count` chosen (rows[t], cols[t]) elements only. */
int oracle_mxfp8_gemm_sampled(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* b,
                              const uint8_t* bs, int b_layout, int64_t m, int64_t n, int64_t k,
                              const int64_t* rows, const int64_t* cols, int64_t count,
                              uint16_t* out_bf16, double* out_f64) {
  if (m < 0 || n < 0 || k <= 0 || k % 32 != 0 || !a || !b || !as || !bs || !rows || !cols)
    return ORACLE_EINVAL;
  if ((a_layout != 0 && a_layout != 1) || (b_layout != 0 && b_layout != 1)) return ORACLE_EINVAL;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n) return ORACLE_EINVAL;
  init_values();
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    double v = gemm_element(a, as, a_layout, b, bs, b_layout, rows[t], cols[t], k);
    if (out_f64) out_f64[t] = v;
    if (out_bf16) out_bf16[t] = oracle_bf16_from_double(v);
  }
  return ORACLE_OK;
}

/* ------------------------------------ fused dense GEMM1: gate_up, SiLU-and-mul, quantiser */

/*
 * The dense MLP's first GEMM with its activation and quantisation fused, producing the MXFP8
 * activation down_proj consumes. vLLM PR #64659 ("Details", "GEMM-RS with a quantized input")
 * states that past its token threshold this GEMM emits MXFP8 data with scales already in the
 * swizzled layout, which the GEMM-RS path then uses without quantising again; PR #64111
 * ("Claims") lists the fused dense GEMM1 among its decode kernels. w: E4M3 [2*inter, k], rows [0, inter) the gate projection and rows
 * [inter, 2*inter) the up projection. For each listed row r of a and each j < inter:
 *   g = C[r, j], u = C[r, inter + j]          (exact values, as gemm_element above)
 *   y = g / (1 + e^-g) * u                    (SiLU(g) times up, in fp64)
 * y is rounded once to fp32 and that value is quantised per 32 along j as in the quantiser.
 * Outputs are indexed by position t in rows[]: q [nrows, inter], s_lin [nrows, inter/32],
 * y_out [nrows, inter] fp32 (optional), gu_out [nrows, 2*inter] fp64 g then u (optional).
 */
int oracle_gemm_silu_mul_quant(const uint8_t* a, const uint8_t* as, int a_layout, const uint8_t* w,
                               const uint8_t* ws, int w_layout, int64_t m, int64_t inter, int64_t k,
                               const int64_t* rows, int64_t nrows, uint8_t* q, uint8_t* s_lin,
                               float* y_out, double* gu_out) {
  if (m < 0 || inter <= 0 || inter % 32 != 0 || k <= 0 || k % 32 != 0 || nrows < 0) return ORACLE_EINVAL;
  if (!a || !as || !w || !ws || !rows || !q || !s_lin) return ORACLE_EINVAL;
  if ((a_layout != 0 && a_layout != 1) || (w_layout != 0 && w_layout != 1)) return ORACLE_EINVAL;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= m) return ORACLE_EINVAL;
  init_tables();
  init_values();
  int64_t nblk = inter / 32;
  int nomem = 0;
#pragma omp parallel reduction(| : nomem)
  {
    double* y = (double*)malloc((size_t)inter * sizeof(double));
    if (!y) nomem = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < nrows; ++t) {
      if (!y) continue;
      for (int64_t j = 0; j < inter; ++j) {
        double g = gemm_element(a, as, a_layout, w, ws, w_layout, rows[t], j, k);
        double u = gemm_element(a, as, a_layout, w, ws, w_layout, rows[t], inter + j, k);
        if (gu_out) {
          gu_out[t * 2 * inter + j] = g;
          gu_out[t * 2 * inter + inter + j] = u;
        }
        float y32 = (float)(g / (1.0 + exp(-g)) * u);
        if (y_out) y_out[t * inter + j] = y32;
        y[j] = (double)y32;
      }
      quantize_row(y, inter, q + t * inter, s_lin + t * nblk);
    }
    free(y);
  }
  return nomem ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Threads an OpenMP region of this library uses. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the threads later OpenMP regions of this library use (n >= 1); returns the previous count. */
int oracle_set_num_threads(int n) {
  int prev = oracle_num_threads();
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
  return prev;
}
