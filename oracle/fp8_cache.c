/*
 * Plain C part of the CPU oracle: the fp8 (OCP E4M3FN) KV-cache quantiser
 * and its decoder.  TEST INFRASTRUCTURE ONLY: loaded by tests/ through
 * oracle/fp8c.py; the GPU library neither links nor calls it, and it shares
 * no code with the library.
 *
 * It computes what oracle/performer.py's e4m3_encode, quantize_rows,
 * PagedCacheFP8.append and PagedCacheFP8.gather compute, written from the
 * same definitions, fast enough for the long fp8 history (2.79M tokens x 40
 * heads x 128 dims, 28.5 GB of codes), where the numpy encoder would take
 * most of an hour.  Its pins (tests/test_oracle_fp8c.py) are the numpy
 * oracle's own pins (the OCP value table, torch's float8_e4m3fn cast) and
 * bitwise equality with the numpy oracle.
 *
 * OCP 8-bit floating point, E4M3FN: sign, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is
 * NaN; no infinities; the largest finite value is 448 = 1.75 * 2^8.
 *
 * fp8 cache storage (the library's contract, not the pages'): one fp32
 * scale per (page, head) for K and for V, scale = amax / 448 over the page's
 * valid rows, code = RNE-saturate(x * (448 / amax)) with the product in
 * fp32; amax = 0 gives scale 1 and codes 0; rows past the valid ones hold
 * code 0.
 *
 * Built with gcc -std=c11 (no floating-point contraction) by oracle/fp8c.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* One E4M3FN code, round to nearest with ties to even, saturating at
 * +-448; the sign is copied from x (so -0.0 gives 0x80). */
static uint8_t e4m3_code(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double a = fabs((double)x);
  if (a > 448.0) a = 448.0;
  if (a < 0x1p-6) {
    /* subnormal range: steps of 2^-9; m = 8 is the smallest normal 2^-6,
     * whose code 0x08 follows on directly */
    const double m = nearbyint(a * 512.0);
    return sign | (uint8_t)m;
  }
  int e;
  const double f = frexp(a, &e);          /* a = f 2^e, f in [0.5, 1) */
  e -= 1;                                 /* a = (2f) 2^e, 2f in [1, 2) */
  double m = nearbyint((2.0 * f - 1.0) * 8.0);
  if (m == 8.0) {                         /* rounded up into the next binade */
    m = 0.0;
    e += 1;
  }
  return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Value of an E4M3FN code, exact in double. */
static double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = m * 0x1p-9;
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

static float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

void orc_e4m3_encode(const float* x, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(x[i]);
}

void orc_e4m3_decode(const uint8_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(c[i]);
}

/*
 * Quantise a slice of n_tok tokens that starts on a page boundary, K or V.
 *   src:    bf16 bits [n_tok][H][D]
 *   codes:  [n_pages][H][ps][D] (v_layout 0, K) or [n_pages][H][D][ps]
 *           (v_layout 1, V), n_pages = ceil(n_tok / ps); every byte written
 *   scales: [n_pages][H]
 * Page p holds tokens p*ps .. p*ps + ps - 1 of the slice (logical order).
 */
void orc_quantize_pages(const uint16_t* src, int64_t n_tok, int32_t H, int32_t D, int32_t ps,
                        int32_t v_layout, uint8_t* codes, float* scales) {
  const int64_t n_pages = (n_tok + ps - 1) / ps;
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < n_pages * H; ++blk) {
    const int64_t p = blk / H;
    const int32_t h = (int32_t)(blk % H);
    const int64_t t0 = p * ps;
    const int32_t rows = (int32_t)(n_tok - t0 < ps ? n_tok - t0 : ps);
    uint8_t* out = codes + blk * (int64_t)ps * D;
    memset(out, 0, (size_t)ps * D);
    float amax = 0.0f;
    for (int32_t r = 0; r < rows; ++r)
      for (int32_t d = 0; d < D; ++d) {
        const float a = fabsf(bf16_to_f32(src[((t0 + r) * H + h) * (int64_t)D + d]));
        if (a > amax) amax = a;
      }
    if (amax == 0.0f) {
      scales[blk] = 1.0f;
      continue;
    }
    const float scale = amax / 448.0f;
    const float inv = 448.0f / amax;
    scales[blk] = scale;
    for (int32_t r = 0; r < rows; ++r)
      for (int32_t d = 0; d < D; ++d) {
        const float y = bf16_to_f32(src[((t0 + r) * H + h) * (int64_t)D + d]) * inv;
        const uint8_t c = e4m3_code(y);
        if (v_layout) out[(int64_t)d * ps + r] = c;
        else out[(int64_t)r * D + d] = c;
      }
  }
}

/*
 * Dequantised values of one head: out[t][d] = value(code) * scale for the
 * tokens t < n_tok, in double (exact: a 4-bit significand times a 24-bit
 * one).  codes / scales as orc_quantize_pages writes them for a cache of
 * pages in logical order.
 */
void orc_decode_head(const uint8_t* codes, const float* scales, int64_t n_tok, int32_t H,
                     int32_t D, int32_t ps, int32_t head, int32_t v_layout, double* out) {
  double table[256];
  for (int c = 0; c < 256; ++c) table[c] = e4m3_value((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    const int64_t p = t / ps;
    const int32_t r = (int32_t)(t % ps);
    const int64_t blk = p * H + head;
    const uint8_t* blkc = codes + blk * (int64_t)ps * D;
    const double s = (double)scales[blk];
    for (int32_t d = 0; d < D; ++d) {
      const uint8_t c = v_layout ? blkc[(int64_t)d * ps + r] : blkc[(int64_t)r * D + d];
      out[t * D + d] = table[c] * s;
    }
  }
}
