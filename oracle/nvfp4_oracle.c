/*
 * NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU product path never calls it and
 * shares no source with it.
 *
 * This is a plain, slow, deliberately obvious implementation of what the
 * NVFP4 MoE expert FFN computes, written from the "nvfp4-megamoe-kernel" pages:
 *   - NVFP4-1.1_APPROACH_PART_2.md: FP8 E4M3 decode/encode rules (bias 7,
 *     exponent 15 valid, 448 = 0x7e maximum, exp15/mant7 is NaN and never
 *     emitted, subnormal m * 2^-9, mantissa carry into the exponent), the
 *     two-stage E2M1 rounding (round-to-nearest-even to half steps, then a
 *     half-step -> index table), the 9-bytes-per-16-block layout.
 *   - DEBUG_LOG.md, "NVFP4 MoE Pipeline": quantize activations -> L1 GEMM
 *     with alpha = input global scale * weight global scale -> SiLU(gate)*up
 *     -> quantize -> L2 GEMM with alpha -> scatter with routing weights.
 *   - NVFP4-1.1_APPROACH.md, "Revised approach": compact SwiGLU-only output.
 *
 * Precision: the block quantization runs in IEEE fp32 with one rounding per
 * operation (the pages' kernels work in float); build with -ffp-contract=off.
 * GEMMs and SwiGLU run in fp64 on exactly dequantized operands.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   global scale g = amax / (6 * 448) is a decode multiplier, E = 1/g;
 *   block scale bsf = (bmax / 6) * E; per-block multiplier r = E / sfd;
 *   nibble sign = sign bit of x; even element in the low nibble;
 *   a zero block scale gives all-zero magnitudes; no SwiGLU clamp;
 *   the L1 output is quantized from its bf16-rounded values with a supplied
 *   global scale; one global scale per expert weight tensor.
 * Parity unpinned by the pages (fixed by these readings and self-consistency
 * only): step_to_idx entries for half steps 5, 7 and 9; the sign of nibbles
 * whose magnitude rounds to zero; nibble order within a byte; the absence of
 * a SwiGLU clamp; the operation order inside bsf and r.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

/* ---------------------------------------------------------------------- */
/* bf16 <-> float                                                          */
/* ---------------------------------------------------------------------- */

/* A bf16 value is the top half of an fp32 bit pattern, so widening is exact. */
float orc_bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double straight to the nearest bf16 (ties to even).  bf16 keeps 8
 * significant bits; below 2^-126 its spacing is fixed at 2^-133. */
uint16_t orc_double_to_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  frexp(fabs(v), &e);                   /* |v| = m * 2^e, m in [0.5, 1) */
  int qexp = e - 8;                     /* spacing of 8-significant-bit values */
  if (qexp < -133) qexp = -133;         /* bf16 subnormal spacing */
  double n = nearbyint(ldexp(v, -qexp)); /* default rounding mode: to even */
  double r = ldexp(n, qexp);
  float f = (float)r;                   /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 (NVFP4 block scale)                                           */
/* ---------------------------------------------------------------------- */

/* Decode: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent 15 holds ordinary numbers except mantissa 7, which is NaN.
 * Exponent 0 is subnormal: m * 2^-9.  (NVFP4-1.1_APPROACH_PART_2.md, the
 * subnormal correction from 1/1024 to 1/512 and the exponent-15 discussion.) */
double orc_e4m3_value(uint32_t code) {
  uint32_t s = (code >> 7) & 1u;
  uint32_t e = (code >> 3) & 15u;
  uint32_t m = code & 7u;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = (double)m * ldexp(1.0, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* Encode a non-negative value: the representable magnitude nearest to v,
 * ties to the even code, everything at or above 448 saturating to 0x7e.
 * Found by brute force over the 127 non-NaN codes.  This is the value the
 * pages' procedure (normalize, round the mantissa to nearest-even, carry an
 * overflowing mantissa into the exponent, round subnormals as v * 512, clamp
 * at 448 and never emit 0x7f) is meant to produce.  Differences of an fp32
 * value and an E4M3 value are exact in double wherever two candidates are
 * close, so the comparison below is exact where it matters. */
uint32_t orc_e4m3_encode(float v) {
  double a = (double)v;
  if (!(a >= 0.0)) a = 0.0; /* block scales are never negative; NaN -> 0 */
  if (a >= 448.0) return 0x7e;
  uint32_t best = 0;
  double bestd = INFINITY;
  for (uint32_t c = 0; c <= 0x7e; ++c) {
    double d = fabs(orc_e4m3_value(c) - a);
    if (d < bestd || (d == bestd && (c & 1u) == 0 && (best & 1u) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Element-wise encode of an array (for sweeps in tests). */
void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}

/* ---------------------------------------------------------------------- */
/* FP4 E2M1 element                                                        */
/* ---------------------------------------------------------------------- */

/* E2M1 magnitudes by 3-bit index. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Half-step -> E2M1 index table.  Entry hs is the index of the E2M1 value
 * nearest to hs/2, ties to the even index.  The pages show entries 10 -> 6
 * and 11 -> 7 (the 5.25 case); entries 5, 7 and 9 are this reading. */
static const int STEP_TO_IDX[13] = {0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7};

int orc_step_to_idx(int hs) { return (hs >= 0 && hs <= 12) ? STEP_TO_IDX[hs] : -1; }

double orc_e2m1_value(uint32_t nibble) {
  double m = E2M1_MAG[nibble & 7u];
  return (nibble & 8u) ? -m : m;
}

/* Two-stage E2M1 rounding of one scaled value s (NVFP4-1.1_APPROACH_PART_2.md:
 * clamp |s| at 6, double it, round to nearest even integer, then map the half
 * step through the table).  The sign comes from the unscaled element. */
uint32_t orc_e2m1_nibble(float s, int negative) {
  float a = fminf(fabsf(s), 6.0f);
  float twice = 2.0f * a;               /* exact */
  int hs = (int)nearbyintf(twice);      /* round half to even */
  uint32_t idx = (uint32_t)STEP_TO_IDX[hs];
  return (negative ? 8u : 0u) | idx;
}

/* ---------------------------------------------------------------------- */
/* Tensor quantize / dequantize                                            */
/* ---------------------------------------------------------------------- */

/* Dynamic per-tensor global (decode) scale: g = amax / (6 * 448), so that the
 * largest block scale lands on the E4M3 maximum; g = 1 for an all-zero
 * tensor. */
float orc_global_scale(const uint16_t *x, int64_t n) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(orc_bf16_to_float(x[i]));
    if (a > amax) amax = a;
  }
  if (amax > 0.0f) return amax / 2688.0f;
  return 1.0f;
}

/* Quantize one 16-element block.  Writes 8 packed bytes and returns the
 * scale byte.  The block-scale and multiplier formulas are this reading of
 * the pages (their values 448 and 250 -> 0x78 appear there, the formula does
 * not). */
uint32_t orc_quantize_block(const float *xb, float g, uint8_t *qb) {
  float E = 1.0f / g;
  float bmax = 0.0f;
  for (int i = 0; i < 16; ++i)
    if (fabsf(xb[i]) > bmax) bmax = fabsf(xb[i]);
  float bsf = (bmax / 6.0f) * E;
  uint32_t sf = orc_e4m3_encode(bsf);
  float sfd = (float)orc_e4m3_value(sf);
  float r = (sfd == 0.0f) ? 0.0f : E / sfd;
  uint32_t nib[16];
  for (int i = 0; i < 16; ++i) {
    float s = xb[i] * r;
    nib[i] = orc_e2m1_nibble(s, signbit(xb[i]) != 0);
  }
  for (int i = 0; i < 8; ++i)
    qb[i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
  return sf;
}

typedef struct {
  const uint16_t *x;
  int64_t K;
  float g;
  uint8_t *q, *sf;
  int64_t r0, r1;
} quant_job;

static void *quant_worker(void *p) {
  quant_job *j = (quant_job *)p;
  float xb[16];
  for (int64_t r = j->r0; r < j->r1; ++r) {
    for (int64_t b = 0; b < j->K / 16; ++b) {
      for (int i = 0; i < 16; ++i) xb[i] = orc_bf16_to_float(j->x[r * j->K + b * 16 + i]);
      j->sf[r * (j->K / 16) + b] =
          (uint8_t)orc_quantize_block(xb, j->g, j->q + r * (j->K / 2) + b * 8);
    }
  }
  return NULL;
}

/* Rows are independent given g; threads only split the row range. */
void orc_quantize(const uint16_t *x, int64_t M, int64_t K, float g, uint8_t *q, uint8_t *sf,
                  int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_t tid[256];
  quant_job jobs[256];
  for (int t = 0; t < threads; ++t) {
    jobs[t].x = x;
    jobs[t].K = K;
    jobs[t].g = g;
    jobs[t].q = q;
    jobs[t].sf = sf;
    jobs[t].r0 = M * t / threads;
    jobs[t].r1 = M * (t + 1) / threads;
    pthread_create(&tid[t], NULL, quant_worker, &jobs[t]);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* Exact (unscaled by g) value of element (row, col): +-e2m1 * block scale. */
static double deq_unscaled(const uint8_t *q, const uint8_t *sf, int64_t K, int64_t row,
                           int64_t col) {
  uint8_t byte = q[row * (K / 2) + col / 2];
  uint32_t nib = (col & 1) ? (byte >> 4) : (byte & 15u);
  double sfd = orc_e4m3_value(sf[row * (K / 16) + col / 16]);
  return orc_e2m1_value(nib) * sfd;
}

/* Dequantize: x_hat = f32(f32(+-e2m1 * sfd) * g).  The inner product is exact
 * in fp32 (at most 6 significant bits). */
void orc_dequantize(const uint8_t *q, const uint8_t *sf, float g, int64_t M, int64_t K,
                    float *out) {
  for (int64_t r = 0; r < M; ++r)
    for (int64_t c = 0; c < K; ++c) {
      float v = (float)deq_unscaled(q, sf, K, r, c);
      out[r * K + c] = v * g;
    }
}

/* bf16 output: the fp32 result above rounded to nearest-even bf16. */
void orc_dequantize_bf16(const uint8_t *q, const uint8_t *sf, float g, int64_t M, int64_t K,
                         uint16_t *out) {
  for (int64_t r = 0; r < M; ++r)
    for (int64_t c = 0; c < K; ++c) {
      float v = (float)deq_unscaled(q, sf, K, r, c);
      out[r * K + c] = orc_double_to_bf16((double)(v * g));
    }
}

/* ---------------------------------------------------------------------- */
/* Single-expert L1 GEMM + SwiGLU (+ quantize)                             */
/* ---------------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Column of gate_j / up_j in the interleaved L1 output: groups of 8 gate
 * columns alternate with groups of 8 up columns (interleave_l1_weights on
 * NVFP4-1.1_APPROACH_PART_2.md). */
static int64_t gate_col(int64_t j) { return 16 * (j / 8) + (j % 8); }
static int64_t up_col(int64_t j) { return 16 * (j / 8) + 8 + (j % 8); }

/* For one activation row: h[n] = alpha * sum_k a~[k] * w~[n][k] in fp64 over
 * the 2I interleaved weight rows, then c[j] = bf16(silu(gate_j) * up_j). */
static void l1_row(const double *arow, int64_t K, const uint8_t *wq, const uint8_t *wsf,
                   int64_t N2, double alpha, double *h, uint16_t *c) {
  for (int64_t n = 0; n < N2; ++n) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += arow[k] * deq_unscaled(wq, wsf, K, n, k);
    h[n] = acc * alpha;
  }
  for (int64_t j = 0; j < N2 / 2; ++j) c[j] = orc_double_to_bf16(silu(h[gate_col(j)]) * h[up_col(j)]);
}

typedef struct {
  const uint8_t *aq, *asf;
  int64_t K;
  const uint8_t *wq, *wsf;
  int64_t N2;
  double alpha;
  const int64_t *rows;
  int64_t nrows;
  double *h;
  uint16_t *c;
  int64_t i0, i1;
} l1_job;

static void *l1_worker(void *p) {
  l1_job *j = (l1_job *)p;
  double *arow = (double *)malloc(sizeof(double) * (size_t)j->K);
  double *h = (double *)malloc(sizeof(double) * (size_t)j->N2);
  for (int64_t i = j->i0; i < j->i1; ++i) {
    int64_t r = j->rows[i];
    for (int64_t k = 0; k < j->K; ++k) arow[k] = deq_unscaled(j->aq, j->asf, j->K, r, k);
    l1_row(arow, j->K, j->wq, j->wsf, j->N2, j->alpha, h, j->c + i * (j->N2 / 2));
    if (j->h) memcpy(j->h + i * j->N2, h, sizeof(double) * (size_t)j->N2);
  }
  free(arow);
  free(h);
  return NULL;
}

/* Dense single-expert stage for a list of activation rows:
 * alpha = f32(a_gs * w_gs); optional fp64 pre-activation h [nrows][N2];
 * compact bf16 c [nrows][N2/2]. */
void orc_l1_swiglu_rows(const uint8_t *aq, const uint8_t *asf, float a_gs, int64_t K,
                        const uint8_t *wq, const uint8_t *wsf, float w_gs, int64_t N2,
                        const int64_t *rows, int64_t nrows, double *h, uint16_t *c,
                        int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  float alpha = a_gs * w_gs;
  pthread_t tid[256];
  l1_job jobs[256];
  for (int t = 0; t < threads; ++t) {
    l1_job *j = &jobs[t];
    j->aq = aq;
    j->asf = asf;
    j->K = K;
    j->wq = wq;
    j->wsf = wsf;
    j->N2 = N2;
    j->alpha = (double)alpha;
    j->rows = rows;
    j->nrows = nrows;
    j->h = h;
    j->c = c;
    j->i0 = nrows * t / threads;
    j->i1 = nrows * (t + 1) / threads;
    pthread_create(&tid[t], NULL, l1_worker, j);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* ---------------------------------------------------------------------- */
/* Dense NVFP4 linear                                                      */
/* ---------------------------------------------------------------------- */

typedef struct {
  const uint8_t *aq, *asf, *wq, *wsf;
  int64_t K;
  double alpha;
  const int64_t *rows, *cols;
  int64_t ncols;
  float *y;
  int64_t i0, i1;
} lin_job;

static void *lin_worker(void *p) {
  lin_job *j = (lin_job *)p;
  double *arow = (double *)malloc(sizeof(double) * (size_t)j->K);
  for (int64_t i = j->i0; i < j->i1; ++i) {
    for (int64_t k = 0; k < j->K; ++k) arow[k] = deq_unscaled(j->aq, j->asf, j->K, j->rows[i], k);
    for (int64_t c = 0; c < j->ncols; ++c) {
      double acc = 0.0;
      for (int64_t k = 0; k < j->K; ++k) acc += arow[k] * deq_unscaled(j->wq, j->wsf, j->K, j->cols[c], k);
      j->y[i * j->ncols + c] = (float)(acc * j->alpha);
    }
  }
  free(arow);
  return NULL;
}

/* The pipeline's activation quantization and GEMM without routing (DEBUG_LOG.md,
 * "NVFP4 MoE Pipeline": the GEMM scales by alpha = input global scale times
 * weight global scale; "Checkpoint Layers" lists NVFP4 linear projections).
 * For the listed rows of the quantized activations aq/asf [.][K] and the
 * listed weight rows (output features) of wq/wsf [.][K]:
 *   y[i][c] = f32( f32(a_gs * w_gs) * sum_k a~[rows[i]][k] * w~[cols[c]][k] )
 * with exactly dequantized operands (e2m1 * block scale) summed in fp64. */
void orc_linear_rows(const uint8_t *aq, const uint8_t *asf, float a_gs, int64_t K, const uint8_t *wq,
                     const uint8_t *wsf, float w_gs, const int64_t *rows, int64_t nrows, const int64_t *cols,
                     int64_t ncols, float *y, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  float alpha = a_gs * w_gs;
  pthread_t tid[256];
  lin_job jobs[256];
  for (int t = 0; t < threads; ++t) {
    lin_job *j = &jobs[t];
    j->aq = aq;
    j->asf = asf;
    j->wq = wq;
    j->wsf = wsf;
    j->K = K;
    j->alpha = (double)alpha;
    j->rows = rows;
    j->cols = cols;
    j->ncols = ncols;
    j->y = y;
    j->i0 = nrows * t / threads;
    j->i1 = nrows * (t + 1) / threads;
    pthread_create(&tid[t], NULL, lin_worker, j);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* ---------------------------------------------------------------------- */
/* MoE expert FFN                                                          */
/* ---------------------------------------------------------------------- */

typedef struct {
  const orc_moe_problem *pb;
  const uint8_t *xq, *xsf;
  float x_gs;
  const int64_t *tokens;
  int64_t i0, i1;
  float *y;
  uint16_t *c_out;
  uint8_t *a2q_out, *a2sf_out;
} moe_job;

/* All k pairs of one token: L1 + SwiGLU -> compact bf16 c -> quantize with the
 * supplied global scale -> L2 with alpha -> weighted sum over the k pairs in
 * fixed order (DEBUG_LOG.md, "NVFP4 MoE Pipeline"). */
static void *moe_worker(void *p) {
  moe_job *jb = (moe_job *)p;
  const orc_moe_problem *pb = jb->pb;
  int64_t H = pb->H, I = pb->I, k = pb->topk;
  double *arow = (double *)malloc(sizeof(double) * (size_t)H);
  double *h = (double *)malloc(sizeof(double) * (size_t)(2 * I));
  double *a2row = (double *)malloc(sizeof(double) * (size_t)I);
  double *yacc = (double *)malloc(sizeof(double) * (size_t)H);
  uint16_t *c = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
  float *cf = (float *)malloc(sizeof(float) * 16);
  uint8_t *a2q = (uint8_t *)malloc((size_t)(I / 2));
  uint8_t *a2sf = (uint8_t *)malloc((size_t)(I / 16));
  for (int64_t i = jb->i0; i < jb->i1; ++i) {
    int64_t t = jb->tokens[i];
    for (int64_t kk = 0; kk < H; ++kk) arow[kk] = deq_unscaled(jb->xq, jb->xsf, H, t, kk);
    for (int64_t n = 0; n < H; ++n) yacc[n] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = pb->topk_ids[t * k + j];
      if (e < 0 || e >= pb->E) continue; /* invalid expert: pair skipped */
      const uint8_t *w1q = pb->w1_q + (int64_t)e * (2 * I) * (H / 2);
      const uint8_t *w1sf = pb->w1_sf + (int64_t)e * (2 * I) * (H / 16);
      float alpha1 = jb->x_gs * pb->w1_gs[e];
      l1_row(arow, H, w1q, w1sf, 2 * I, (double)alpha1, h, c);
      /* quantize the bf16 SwiGLU row with the supplied global scale */
      for (int64_t b = 0; b < I / 16; ++b) {
        for (int q = 0; q < 16; ++q) cf[q] = orc_bf16_to_float(c[b * 16 + q]);
        a2sf[b] = (uint8_t)orc_quantize_block(cf, pb->a2_gs, a2q + b * 8);
      }
      if (jb->c_out) memcpy(jb->c_out + i * k * I + j * I, c, sizeof(uint16_t) * (size_t)I);
      if (jb->a2q_out) memcpy(jb->a2q_out + (i * k + j) * (I / 2), a2q, (size_t)(I / 2));
      if (jb->a2sf_out) memcpy(jb->a2sf_out + (i * k + j) * (I / 16), a2sf, (size_t)(I / 16));
      for (int64_t ii = 0; ii < I; ++ii) a2row[ii] = deq_unscaled(a2q, a2sf, I, 0, ii);
      const uint8_t *w2q = pb->w2_q + (int64_t)e * H * (I / 2);
      const uint8_t *w2sf = pb->w2_sf + (int64_t)e * H * (I / 16);
      double alpha2 = (double)(pb->a2_gs * pb->w2_gs[e]);
      double wt = (double)pb->topk_w[t * k + j];
      for (int64_t n = 0; n < H; ++n) {
        double acc = 0.0;
        for (int64_t ii = 0; ii < I; ++ii) acc += a2row[ii] * deq_unscaled(w2q, w2sf, I, n, ii);
        yacc[n] += wt * (acc * alpha2);
      }
    }
    for (int64_t n = 0; n < H; ++n) jb->y[i * H + n] = (float)yacc[n];
  }
  free(arow);
  free(h);
  free(a2row);
  free(yacc);
  free(c);
  free(cf);
  free(a2q);
  free(a2sf);
  return NULL;
}

/* Compute y for a list of tokens.  Activations are quantized with the
 * supplied x_gs if non-NULL, else with the dynamic global scale of the whole
 * x.  Outputs are indexed by position in the token list:
 *   y [ntok][H] fp32; optional c [ntok][k][I] bf16, a2 q [ntok][k][I/2],
 *   a2 sf [ntok][k][I/16] (pairs of a skipped expert are left untouched).
 * Returns the global scale used for x. */
float orc_moe_tokens(const orc_moe_problem *pb, const int64_t *tokens, int64_t ntok, float *y,
                     uint16_t *c_out, uint8_t *a2q_out, uint8_t *a2sf_out, int threads) {
  int64_t T = pb->T, H = pb->H;
  float x_gs = pb->x_gs_in ? *pb->x_gs_in : orc_global_scale(pb->x, T * H);
  /* Only the listed tokens' rows are needed; quantize those rows into a
   * full-size buffer (rows are independent given the global scale). */
  uint8_t *xq = (uint8_t *)calloc((size_t)(T * (H / 2)), 1);
  uint8_t *xsf = (uint8_t *)calloc((size_t)(T * (H / 16)), 1);
  float xb[16];
  for (int64_t i = 0; i < ntok; ++i) {
    int64_t t = tokens[i];
    for (int64_t b = 0; b < H / 16; ++b) {
      for (int q = 0; q < 16; ++q) xb[q] = orc_bf16_to_float(pb->x[t * H + b * 16 + q]);
      xsf[t * (H / 16) + b] = (uint8_t)orc_quantize_block(xb, x_gs, xq + t * (H / 2) + b * 8);
    }
  }
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_t tid[256];
  moe_job jobs[256];
  for (int t = 0; t < threads; ++t) {
    moe_job *j = &jobs[t];
    j->pb = pb;
    j->xq = xq;
    j->xsf = xsf;
    j->x_gs = x_gs;
    j->tokens = tokens;
    j->i0 = ntok * t / threads;
    j->i1 = ntok * (t + 1) / threads;
    j->y = y;
    j->c_out = c_out;
    j->a2q_out = a2q_out;
    j->a2sf_out = a2sf_out;
    pthread_create(&tid[t], NULL, moe_worker, j);
  }
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
  free(xq);
  free(xsf);
  return x_gs;
}
