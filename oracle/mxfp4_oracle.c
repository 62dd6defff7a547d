/*
 * MXFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU product path never calls it and
 * shares no source with it.
 *
 * MXFP4 is not the pages' format.  The "nvfp4-megamoe-kernel" pages quantize
 * to NVFP4 (16-element blocks, FP8 E4M3 block scale, fp32 tensor scale).
 * MXFP4 is the Open Compute Project "Microscaling Formats (MX)
 * Specification" v1.0 format that gfx950's scaled FP4 MFMA consumes: blocks
 * of 32 elements share one E8M0 scale (an 8-bit power-of-two exponent), each
 * element an E2M1 value, no tensor scale.  This file follows that
 * specification:
 *   - section 5.4 (E8M0): code c encodes 2^(c - 127); c = 255 is NaN (never
 *     produced here);
 *   - section 5.3.3 (E2M1): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, no
 *     infinities or NaN;
 *   - section 6.3 (conversion from scalars): the shared exponent is
 *     floor(log2(max |V_i|)) - emax, emax = 2 for E2M1, X = 2^exp, and each
 *     element is V_i / X rounded to nearest, ties to even, saturating at the
 *     largest E2M1 magnitude.
 * Readings where the specification leaves a choice (listed in the design
 * notes): an all-zero block gets scale code 0 (the smallest scale), and a
 * shared exponent below -127 is clamped to -127; the nibble sign is the sign
 * bit of V_i (so -0.0 and negative values that round to zero give nibble 8);
 * element 2i sits in the low nibble of byte i (the MFMA operand order).
 * These readings are pinned by the specification's definitions and by
 * self-consistency only (parity unpinned by the pages, which do not define
 * MXFP4).
 *
 * Precision: the scale is an exact power of two, so V_i / X is exact in
 * double; the GEMM runs in double on exactly dequantized operands.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "mxfp4_oracle.h"

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* E8M0: code c -> 2^(c - 127); 255 is NaN. */
double orc_mx_scale_value(uint32_t code) {
  if (code == 255) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* Shared-exponent code of a block whose largest magnitude is amax:
 * floor(log2(amax)) - 2 + 127, clamped to [0, 254]; 0 for amax == 0. */
uint32_t orc_mx_scale_code(double amax) {
  if (!(amax > 0.0)) return 0;
  int e;
  frexp(amax, &e); /* amax = m * 2^e, m in [0.5, 1): floor(log2(amax)) = e - 1 */
  int code = (e - 1) - 2 + 127;
  if (code < 0) code = 0;
  if (code > 254) code = 254;
  return (uint32_t)code;
}

static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_mx_e2m1_value(uint32_t nibble) {
  double v = E2M1_GRID[nibble & 7];
  return (nibble & 8) ? -v : v;
}

/* Nearest E2M1 magnitude to |v| (ties to the even code, i.e. the even
 * significand), magnitudes above 6 saturate to 6; the sign bit of v is kept. */
uint32_t orc_mx_e2m1_nibble(double v) {
  double a = fabs(v);
  uint32_t best = 7;
  if (a <= 6.0) {
    double bd = INFINITY;
    for (uint32_t c = 0; c < 8; ++c) {
      double d = fabs(a - E2M1_GRID[c]);
      if (d < bd || (d == bd && (c & 1) == 0)) {
        bd = d;
        best = c;
      }
    }
  }
  return best | (signbit(v) ? 8u : 0u);
}

/* One block of 32 bf16 values -> 16 bytes of nibbles and its scale code. */
uint32_t orc_mx_quantize_block(const uint16_t *xb, uint8_t *qb) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    double a = fabs(bf16_value(xb[i]));
    if (a > amax) amax = a;
  }
  uint32_t code = orc_mx_scale_code(amax);
  double X = orc_mx_scale_value(code);
  for (int i = 0; i < 16; ++i) {
    uint32_t lo = orc_mx_e2m1_nibble(bf16_value(xb[2 * i]) / X);
    uint32_t hi = orc_mx_e2m1_nibble(bf16_value(xb[2 * i + 1]) / X);
    qb[i] = (uint8_t)(lo | (hi << 4));
  }
  return code;
}

/* x [M][K] bf16 (K % 32 == 0) -> q [M][K/2], scale codes [M][K/32]. */
void orc_mx_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *sc) {
  for (int64_t r = 0; r < M; ++r)
    for (int64_t b = 0; b < K / 32; ++b)
      sc[r * (K / 32) + b] = (uint8_t)orc_mx_quantize_block(x + r * K + 32 * b, q + r * (K / 2) + 16 * b);
}

/* Element (r, k) of an MXFP4 matrix. */
static double mx_elem(const uint8_t *q, const uint8_t *sc, int64_t K, int64_t r, int64_t k) {
  uint8_t byte = q[r * (K / 2) + k / 2];
  uint32_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
  return orc_mx_e2m1_value(nib) * orc_mx_scale_value(sc[r * (K / 32) + k / 32]);
}

void orc_mx_dequantize(const uint8_t *q, const uint8_t *sc, int64_t M, int64_t K, double *out) {
  for (int64_t r = 0; r < M; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = mx_elem(q, sc, K, r, k);
}

/* y [M][N] = A @ W^T in double, A [M][K] and W [N][K] MXFP4. */
typedef struct {
  const uint8_t *aq, *asc, *wq, *wsc;
  int64_t M, K, N, r0, r1;
  double *y;
} linear_job;

static void *linear_worker(void *p) {
  linear_job *j = (linear_job *)p;
  double *arow = (double *)malloc(sizeof(double) * (size_t)j->K);
  for (int64_t m = j->r0; m < j->r1; ++m) {
    for (int64_t k = 0; k < j->K; ++k) arow[k] = mx_elem(j->aq, j->asc, j->K, m, k);
    for (int64_t n = 0; n < j->N; ++n) {
      double s = 0.0;
      for (int64_t k = 0; k < j->K; ++k) s += arow[k] * mx_elem(j->wq, j->wsc, j->K, n, k);
      j->y[m * j->N + n] = s;
    }
  }
  free(arow);
  return NULL;
}

void orc_mx_linear(const uint8_t *aq, const uint8_t *asc, int64_t M, int64_t K, const uint8_t *wq,
                   const uint8_t *wsc, int64_t N, double *y, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  pthread_t th[64];
  linear_job jobs[64];
  int64_t per = (M + threads - 1) / threads;
  int n = 0;
  for (int t = 0; t < threads; ++t) {
    int64_t r0 = t * per, r1 = r0 + per < M ? r0 + per : M;
    if (r0 >= r1) break;
    jobs[n] = (linear_job){aq, asc, wq, wsc, M, K, N, r0, r1, y};
    pthread_create(&th[n], NULL, linear_worker, &jobs[n]);
    ++n;
  }
  for (int t = 0; t < n; ++t) pthread_join(th[t], NULL);
}
