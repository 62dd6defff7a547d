/*
 * NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY (see nvfp4_oracle.c).
 * Host pointers throughout; nothing here touches a GPU.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

/* One MoE expert-FFN problem on host memory.  Shapes:
 *   x [T][H] bf16; topk_ids [T][topk] int32; topk_w [T][topk] fp32;
 *   w1 q [E][2I][H/2], sf [E][2I][H/16], gs [E]  (rows interleaved by 8: gate, up)
 *   w2 q [E][H][I/2],  sf [E][H][I/16],  gs [E]
 *   a2_gs: supplied global scale of the L1 output; x_gs_in: optional. */
typedef struct {
  int64_t T, H, I, E, topk;
  const uint16_t *x;
  const float *x_gs_in;
  const int32_t *topk_ids;
  const float *topk_w;
  const uint8_t *w1_q, *w1_sf;
  const float *w1_gs;
  const uint8_t *w2_q, *w2_sf;
  const float *w2_gs;
  float a2_gs;
} orc_moe_problem;

float orc_bf16_to_float(uint16_t h);
uint16_t orc_double_to_bf16(double v);
double orc_e4m3_value(uint32_t code);
uint32_t orc_e4m3_encode(float v);
void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out);
int orc_step_to_idx(int hs);
double orc_e2m1_value(uint32_t nibble);
uint32_t orc_e2m1_nibble(float s, int negative);
float orc_global_scale(const uint16_t *x, int64_t n);
uint32_t orc_quantize_block(const float *xb, float g, uint8_t *qb);
void orc_quantize(const uint16_t *x, int64_t M, int64_t K, float g, uint8_t *q, uint8_t *sf,
                  int threads);
void orc_dequantize(const uint8_t *q, const uint8_t *sf, float g, int64_t M, int64_t K,
                    float *out);
void orc_dequantize_bf16(const uint8_t *q, const uint8_t *sf, float g, int64_t M, int64_t K,
                         uint16_t *out);
void orc_l1_swiglu_rows(const uint8_t *aq, const uint8_t *asf, float a_gs, int64_t K,
                        const uint8_t *wq, const uint8_t *wsf, float w_gs, int64_t N2,
                        const int64_t *rows, int64_t nrows, double *h, uint16_t *c,
                        int threads);
void orc_linear_rows(const uint8_t *aq, const uint8_t *asf, float a_gs, int64_t K, const uint8_t *wq,
                     const uint8_t *wsf, float w_gs, const int64_t *rows, int64_t nrows, const int64_t *cols,
                     int64_t ncols, float *y, int threads);
float orc_moe_tokens(const orc_moe_problem *pb, const int64_t *tokens, int64_t ntok, float *y,
                     uint16_t *c_out, uint8_t *a2q_out, uint8_t *a2sf_out, int threads);
#endif
