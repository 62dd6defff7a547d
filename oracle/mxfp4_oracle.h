/*
 * MXFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY (see mxfp4_oracle.c).
 * Host pointers throughout; nothing here touches a GPU.
 */
#ifndef MXFP4_ORACLE_H
#define MXFP4_ORACLE_H
#include <stdint.h>

double orc_mx_scale_value(uint32_t code);
uint32_t orc_mx_scale_code(double amax);
double orc_mx_e2m1_value(uint32_t nibble);
uint32_t orc_mx_e2m1_nibble(double v);
uint32_t orc_mx_quantize_block(const uint16_t *xb, uint8_t *qb);
void orc_mx_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *sc);
void orc_mx_dequantize(const uint8_t *q, const uint8_t *sc, int64_t M, int64_t K, double *out);
void orc_mx_linear(const uint8_t *aq, const uint8_t *asc, int64_t M, int64_t K, const uint8_t *wq,
                   const uint8_t *wsc, int64_t N, double *y, int threads);
#endif
