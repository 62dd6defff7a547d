/*
 * nvfp4moe.h -- C ABI of libnvfp4moe.so, the MI355X (gfx950) NVFP4 MoE
 * expert-FFN hot path.
 *
 * Source of the operations: the "nvfp4-megamoe-kernel" pages.
 *   NVFP4-1.1_APPROACH_PART_2.md -- the NVFP4 activation quantizer: 16-element
 *     blocks, FP8 E4M3 block scale (bias 7, exponent 15 valid, 0x7e = 448 the
 *     maximum, exp15/mant7 NaN never emitted, subnormal m * 2^-9), E2M1 nibbles
 *     by two-stage round-to-nearest-even (half steps, then a table), packed two
 *     per byte; 9 bytes per block; fusing that quantizer into the SwiGLU
 *     epilogue of the L1 grouped GEMM (fp4 output, scale output, and the L2
 *     global scale as kernel inputs).
 *   NVFP4-1.1_APPROACH.md, "Revised approach: Compact SwiGLU output" -- write
 *     only the SwiGLU columns of the gate/up GEMM.
 *   DEBUG_LOG.md, "NVFP4 MoE Pipeline" -- quantize activations (fp4, scales,
 *     global scale) -> L1 GEMM with alpha = activation global scale * weight
 *     global scale -> SiLU(gate) * up -> quantize -> L2 GEMM with alpha ->
 *     scatter with routing weights.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     owned by the caller.  The library never allocates, frees, synchronizes
 *     with the host or copies to the host.  Scratch memory comes from the
 *     caller's workspace (`ws`, `ws_bytes`), sized by the matching
 *     *_workspace_size query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously on it; calls are re-entrant.
 *   - Global scales are fp32 DECODE multipliers held in device memory
 *     (a real value = e2m1 * block scale * global scale).
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - NVFP4 tensor layout for a logical [R][K] matrix (K % 16 == 0):
 *       q  uint8 [R][K/2]   element 2i in the low nibble of byte i, 2i+1 high;
 *                           nibble = sign(bit 3) | E2M1 index (bits 2..0)
 *       sf uint8 [R][K/16]  one E4M3 block scale per 16 consecutive elements
 *   - Alignment: bf16/fp32 tensors 16-byte aligned, q 4-byte aligned,
 *     workspace 256-byte aligned.
 *   - Return value: NVFP4_OK (0) or a negative nvfp4_status.  All argument
 *     checks happen before anything is enqueued, so an error return means
 *     nothing was launched.  nvfp4_last_error() gives a message (per thread).
 *   - Data-dependent conditions are not checked: non-finite inputs give
 *     unspecified bytes; out-of-range expert ids are skipped.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = -1, /* null pointer, bad size or alignment */
  NVFP4_ERR_UNSUPPORTED = -2, /* shape outside what the kernels handle */
  NVFP4_ERR_WORKSPACE = -3,   /* workspace smaller than required */
  NVFP4_ERR_HIP = -4          /* a launch failed (hipGetLastError) */
} nvfp4_status;

/*
 * nvfp4_quantize -- bf16 [M][K] -> NVFP4 (NVFP4-1.1_APPROACH_PART_2.md, the
 * quantizer whose bytes are matched 0/500 against the reference there; the
 * pages' quantize_nvfp4_gpu(x, global_scale) / stage_activation(x)).
 *   x      bf16 [M][K], M >= 0, K > 0, K % 16 == 0
 *   gs_in  nullable.  If NULL the global scale is computed from the tensor:
 *          g = max|x| / (6 * 448), or 1 for an all-zero (or empty) tensor.
 *          If non-NULL, *gs_in (device, 1 float) is used.  Supported range
 *          of g: finite and above 2^-117 (a dynamic g is below that only when
 *          0 < max|x| < ~1.6e-32); outside it the bytes are unspecified.
 *   q      uint8 [M][K/2] out;  sf uint8 [M][K/16] out
 *   gs_out device float out, the g used.  Required when gs_in is NULL;
 *          nullable otherwise (then nothing is written).
 *   ws     workspace of nvfp4_quantize_workspace_size(M, K) bytes (0 is
 *          returned when none is needed; ws may then be NULL).
 * Per block of 16: bsf = (bmax / 6) * (1/g) rounded to E4M3 (saturating at
 * 448); r = (1/g) / sfd; each element's nibble comes from x * r by the
 * two-stage E2M1 rounding.
 */
size_t nvfp4_quantize_workspace_size(int64_t M, int64_t K);
int nvfp4_quantize(const uint16_t *x, int64_t M, int64_t K, const float *gs_in, uint8_t *q,
                   uint8_t *sf, float *gs_out, void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_dequantize -- NVFP4 -> real values: x = f32(f32(e2m1 * sfd) * g),
 * rounded to nearest-even bf16 for bf16 output (FP8 E4M3 decode rules and
 * E2M1 grid of NVFP4-1.1_APPROACH_PART_2.md).
 *   q [M][K/2], sf [M][K/16], gs (device, 1 float); M >= 0, K % 16 == 0
 *   out_dtype: 0 = bf16 (uint16 [M][K]), 1 = fp32 ([M][K])
 */
int nvfp4_dequantize(const uint8_t *q, const uint8_t *sf, const float *gs, int64_t M, int64_t K,
                     int out_dtype, void *out, void *stream);

/*
 * nvfp4_gemm_swiglu_quant -- one expert's L1 stage (the fused_swiglu kernel
 * of NVFP4-1.1_APPROACH_PART_2.md in fp4 mode, with the compact output of
 * NVFP4-1.1_APPROACH.md):
 *   h[m][n] = (sum_k a[m][k] * w[n][k]) * f32(a_gs * w_gs)     n < N2 = 2I
 *   c[m][j] = bf16(silu(h[m][gate(j)]) * h[m][up(j)])          j < I
 *   (c_q, c_sf) = NVFP4 of c's rows with the supplied global scale out_gs.
 * The weight rows are interleaved by 8: rows 16t..16t+7 are gate rows
 * 8t..8t+7, rows 16t+8..16t+15 the matching up rows (interleave_l1_weights).
 *   a_q [M][K/2], a_sf [M][K/16], a_gs (device float)
 *   w_q [N2][K/2], w_sf [N2][K/16], w_gs (device float)
 *   out_gs (device float, > 0)
 *   c_bf16 bf16 [M][I] out, nullable (skips the bf16 store)
 *   c_q [M][I/2], c_sf [M][I/16] out
 *   M >= 0; K % 64 == 0; N2 % 256 == 0; M * K / 2 and N2 * K / 2 at most 4 GiB
 *   (else NVFP4_ERR_UNSUPPORTED).  a_q and w_q 16-byte, a_sf and w_sf 4-byte
 *   aligned.
 *   Workspace: with ws (nvfp4_gemm_swiglu_quant_workspace_size bytes, the
 *   exact f16 copy of the activations, 256-byte aligned; then also M * K * 2
 *   at most 4 GiB) the activations are expanded once and the GEMM reads f16;
 *   with ws == NULL the GEMM reads the NVFP4 activations itself and
 *   dequantizes each K step exactly into LDS (no workspace; measured ~6 %
 *   slower on M4096 K7168 N2 4096).  The results are identical.
 */
size_t nvfp4_gemm_swiglu_quant_workspace_size(int64_t M, int64_t K, int64_t N2);
int nvfp4_gemm_swiglu_quant(const uint8_t *a_q, const uint8_t *a_sf, const float *a_gs, int64_t M,
                            int64_t K, const uint8_t *w_q, const uint8_t *w_sf, const float *w_gs,
                            int64_t N2, const float *out_gs, uint16_t *c_bf16, uint8_t *c_q,
                            uint8_t *c_sf, void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_linear -- dense NVFP4 linear layer: the MoE's activation quantization
 * and GEMM without routing, for the checkpoint's NVFP4 projections
 * (DEBUG_LOG.md, "Checkpoint Layers": o_b_proj, q_a_proj, q_b_proj, kv_proj
 * are NVFP4; the o_a_proj BF16 -> NVFP4 question of "Next Steps").
 *   y[m][n] = f32(x_gs * w_gs) * sum_k deq(xq)[m][k] * deq(w)[n][k]
 * with xq = NVFP4(x) under x_gs (supplied, or the dynamic amax / 2688), both
 * operands exact (e2m1 * E4M3 block scale), fp32 accumulation.
 *   x bf16 [M][K] (16-byte aligned); x_gs_in nullable (device float)
 *   w_q [N][K/2], w_sf [N][K/16] (16-byte aligned), w_gs (device float)
 *   out [M][N]: bf16 (out_dtype 0) or fp32 (1), 16-byte aligned
 *   x_gs_out nullable (1 float): the activation global scale used
 *   M >= 0; K % 64 == 0; N % 256 == 0; M * K * 2 and N * K / 2 at most 4 GiB
 *   (else NVFP4_ERR_UNSUPPORTED).  Workspace: nvfp4_linear_workspace_size
 *   bytes (the NVFP4 and exact-f16 copies of x), 256-byte aligned.
 */
size_t nvfp4_linear_workspace_size(int64_t M, int64_t K, int64_t N);
int nvfp4_linear(const uint16_t *x, int64_t M, int64_t K, const float *x_gs_in, const uint8_t *w_q,
                 const uint8_t *w_sf, const float *w_gs, int64_t N, int out_dtype, void *out,
                 float *x_gs_out, void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_pair_scales -- a weight block-scale matrix sf [R][C] (C = K/16 bytes
 * per row) rewritten once, at weight preparation, in the row-paired layout
 * the 32-row MoE tiles read (nvfp4_moe_args.w1_sf_paired, w2_sf_paired):
 *   out[(r/2) * 2C + 128 * (c/64) + 64 * (r%2) + c%64] = sf[r][c]
 * so each 128-byte line holds 64 bytes of rows 2j and 2j + 1.  The MI355X
 * counterpart of the pages' remap of the scale factors into the layout
 * their hardware reads, checked there by a byte-for-byte roundtrip
 * (DEBUG_LOG.md, "Current State": the SF remap and its forward mapping).
 *   R >= 0 even, C % 64 == 0 (K % 1024 == 0); sf and out 16-byte aligned,
 *   not overlapping.  Else NVFP4_ERR_INVALID_ARG.  Asynchronous on stream.
 */
int nvfp4_pair_scales(const uint8_t *sf, int64_t R, int64_t C, uint8_t *out, void *stream);

/*
 * MoE expert FFN (DEBUG_LOG.md, "NVFP4 MoE Pipeline"), T tokens, hidden H,
 * intermediate I, E experts, top-k routing; P = T * k (token, expert) pairs,
 * pair p = t * k + j.
 */
typedef struct {
  int64_t T, H, I, E, topk;
  const uint16_t *x;        /* bf16 [T][H] */
  const float *x_gs_in;     /* nullable: supplied activation global scale */
  const int32_t *topk_ids;  /* [T][k]; ids outside [0, E) are skipped */
  const float *topk_w;      /* [T][k] routing weights */
  const uint8_t *w1_q;      /* [E][2I][H/2]  gate/up rows interleaved by 8 */
  const uint8_t *w1_sf;     /* [E][2I][H/16] */
  const float *w1_gs;       /* [E] */
  const uint8_t *w2_q;      /* [E][H][I/2] */
  const uint8_t *w2_sf;     /* [E][H][I/16] */
  const float *w2_gs;       /* [E] */
  /* device float: supplied global scale of the L1 output, which is then
     quantized in the L1 GEMM's epilogue (NVFP4-1.1_APPROACH_PART_2.md,
     fp4_mode epilogue with an l2_global_scale input).  Nullable: the
     dynamic scale amax(L1 output over the valid pairs) / 2688 is used instead
     and the L1 output is quantized in a separate pass (DEBUG_LOG.md, "NVFP4
     MoE Pipeline": stage_activation of the activated rows). */
  const float *a2_gs;
  void *out;                /* [T][H] */
  int out_dtype;            /* 0 = bf16, 1 = fp32 */
  /* nullable outputs (pair order p = t*k + j) */
  uint8_t *xq;              /* [T][H/2] */
  uint8_t *xsf;             /* [T][H/16] */
  float *x_gs_out;          /* 1 float: the activation global scale used */
  uint16_t *l1_c_bf16;      /* [P][I] compact SwiGLU output */
  uint8_t *l1_q;            /* [P][I/2] */
  uint8_t *l1_sf;           /* [P][I/16] */
  int32_t *err_count;       /* 1 int: number of skipped pairs (written, not added) */
  /* nullable, for profiling: 9 hipEvent_t created by the caller, recorded on
     `stream` before the global scale, then after the global scale, the
     activation quantization, the grouping, the L1 GEMM's main tile list
     (256-row tiles, or the 32-row tiles of tiling 32), the whole L1 stage
     (with the short tiles of the mixed tiling and any separate quantization
     pass), the L2 GEMM's main tile list, the whole L2 stage and the
     combine.  When the global scale is computed and the grouping fits one
     workgroup (at most 4096 pairs), the grouping runs in the global scale's
     launch: the first interval then holds both and the third is empty. */
  void *const *stage_events;
  /* GEMM tiling.  32: 32-row tiles that stream the weights.  256: 256-row
     MFMA tiles.  288 (mixed): 256-row tiles, except that each expert's last
     block of at most 64 rows goes on one or two 32-row tiles.  0 chooses from the
     routing shape: 32 when there are at most 16 pairs per expert on average,
     else 288; 256 when H or I is not a multiple of 256 (or equal to 128),
     which 32 and 288 need (NVFP4_ERR_UNSUPPORTED).  Other values:
     NVFP4_ERR_INVALID_ARG.  The results are the same either way up to the
     fp32 summation order inside the GEMMs. */
  int32_t tile_rows;
  /* nullable: receives the L1-output global scale used (1 float) */
  float *a2_gs_out;
  /* 0: fused.  1: with a supplied a2_gs, still write the compact bf16 L1
     output and quantize it in a separate pass (the unfused flow of
     NVFP4-1.1_APPROACH.md, "Target flow").  2: the pages' earlier flow
     (NVFP4-1.1_APPROACH_PART_2.md, the current MoE forward): the L1 GEMM
     writes an interleaved bf16 [P][2I] output, groups of 8 columns
     alternating SiLU(gate) and SiLU(gate) * up, and a separate pass
     deinterleaves and quantizes the SwiGLU groups; needs a supplied a2_gs.
     1 and 2 give the fused flow's bytes.  Any other value:
     NVFP4_ERR_INVALID_ARG. */
  int32_t l1_unfused;
  /* nullable: a second stream (hipStream_t) and two events (hipEvent_t,
     aux_events[0] and [1]), all created by the caller, on which the 32-row
     short tiles of the mixed tiling run concurrently with the 256-row
     tiles.  For each GEMM the library records aux_events[0] on `stream`,
     makes aux_stream wait for it, launches the short tiles on aux_stream,
     records aux_events[1] there and makes `stream` wait for it before the
     next stage, so the call still completes in `stream` order (and can be
     captured in a graph).  Without it, or in the other tilings, everything
     runs on `stream`; the results are the same.  aux_stream without
     aux_events: NVFP4_ERR_INVALID_ARG. */
  void *aux_stream;
  void *const *aux_events;
  /* nullable: w1_sf and w2_sf in the row-paired layout of nvfp4_pair_scales
     (prepared once with the weights), read by the 32-row tiles that stream
     the weights.  Their scale loads then use whole 128-byte lines; with the
     plain layout a line's second half is needed four 256-K steps after its
     first, when the weight stream has evicted it, and the line is fetched
     twice.  Used for w1 when H % 1024 == 0 and for w2 when I % 1024 == 0,
     ignored otherwise; the 256-row tiles read w1_sf and w2_sf.  The
     results are the same either way. */
  const uint8_t *w1_sf_paired;
  const uint8_t *w2_sf_paired;
} nvfp4_moe_args;

/*
 * moe_expert_ffn_nvfp4 -- y[t] = sum_j w[t][j] * FFN_{ids[t][j]}(x[t]) with
 *   FFN_e(x) = L2_e(NVFP4(bf16(silu(gate) * up)))  and  (gate, up) = L1_e(NVFP4(x))
 * where L1_e carries alpha1 = x_gs * w1_gs[e], L2_e carries alpha2 =
 * a2_gs * w2_gs[e], the L1 output is quantized with a2_gs (supplied, or the
 * dynamic amax / 2688 of the bf16 L1 output of all valid pairs when a2_gs is
 * NULL), and the k terms of a token are summed in fixed order j = 0..k-1 in
 * fp32.  With out_dtype 0 (bf16) the per-pair L2 rows are held in f16 with
 * one power-of-two scale per (pair, 32 columns) before that sum (relative
 * error <= 2^-11 per term, a quarter of the bf16 rounding of y); with
 * out_dtype 1 they stay fp32.
 * Requirements: T >= 0; H % 256 == 0, I % 128 == 0, E <= 512, k <= 32, and the
 * f16 GEMM operands T * H * 2, T * k * I * 2 and one expert's I * H nibble
 * bytes at most 4 GiB each (else NVFP4_ERR_UNSUPPORTED); E >= 1, k >= 1.
 * Workspace: the query's bytes, which include the per-pair rows [P][H] of
 * the L2 output (fp32, or f16 plus [P][H/32] exponent bytes for a bf16
 * output) and, for the unfused flow without l1_c_bf16, the bf16 L1 output
 * [P][I].
 */
size_t moe_expert_ffn_nvfp4_workspace_size(const nvfp4_moe_args *args);
int moe_expert_ffn_nvfp4(const nvfp4_moe_args *args, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_nvfp4_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): moe_expert_ffn_nvfp4 on the same arguments, computing
 * the same results, with its workspace taken from a static buffer of
 * NVFP4_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The caller still passes every input and output.
 * Calls whose workspace (moe_expert_ffn_nvfp4_workspace_size) exceeds that
 * size are rejected with NVFP4_ERR_WORKSPACE before anything is enqueued;
 * 64 MiB holds, e.g., the T128 H7168 I2048 k8 decode layer (29.6 MiB with a
 * bf16 output, 43.4 MiB with fp32) and T256 with a bf16 output (51.2 MiB).  The first
 * call on a device looks the buffer's device address up (no allocation);
 * make that first call outside graph capture.  Every call on one GPU uses
 * that GPU's one buffer: calls that overlap on the same GPU (two streams,
 * two threads) race and must be serialized by the caller.  Nothing is
 * allocated, freed or synchronized.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_expert_ffn_nvfp4_noalloc(const nvfp4_moe_args *args, void *stream);

/*
 * MXFP4 -- a separately labelled format, NOT the pages' NVFP4: the Open
 * Compute Project "Microscaling Formats (MX) Specification" v1.0 format
 * that gfx950's scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) consumes,
 * for measuring the FP4 matrix-core headroom next to the NVFP4 path.  Blocks
 * of 32 consecutive elements along K share one E8M0 scale code c (the value
 * 2^(c - 127), section 5.4); each element is E2M1 (section 5.3.3); there is
 * no tensor scale.  Quantization follows section 6.3: code = floor(log2(max
 * |x| of the block)) - 2 + 127, clamped to [0, 254] (0 for an all-zero
 * block), element = x / 2^(code - 127) rounded to the nearest E2M1 value,
 * ties to even, saturating at 6; the nibble sign is the sign bit of x.
 * Layout of a logical [R][K] MXFP4 matrix (K % 32 == 0):
 *   q     uint8 [R][K/2]   element 2i in the low nibble of byte i
 *   scale uint8 [R][K/32]  E8M0 codes
 *
 * mxfp4_quantize: x bf16 [M][K] (16-byte aligned) -> q (4-byte aligned),
 *   scale.  M >= 0, K % 32 == 0 (else NVFP4_ERR_INVALID_ARG).
 * mxfp4_dequantize: q, scale -> out [M][K] = e2m1 * 2^(code - 127), bf16
 *   (out_dtype 0, rounded to nearest even) or fp32 (1, exact); out 16-byte
 *   aligned.
 * mxfp4_linear: y[m][n] = sum_k deq(MXFP4(x))[m][k] * deq(w)[n][k], exact
 *   products, fp32 accumulation; x bf16 [M][K]; w_q [N][K/2] (16-byte
 *   aligned), w_scale [N][K/32] (4-byte aligned); out [M][N] bf16 (out_dtype
 *   0) or fp32 (1), 16-byte aligned.  K % 128 == 0 and N % 256 == 0, M * K / 2
 *   and N * K / 2 at most 4 GiB (else NVFP4_ERR_UNSUPPORTED).  Workspace:
 *   mxfp4_linear_workspace_size bytes (the MXFP4 copy of x), 256-byte
 *   aligned.
 */
int mxfp4_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *scale, void *stream);
int mxfp4_dequantize(const uint8_t *q, const uint8_t *scale, int64_t M, int64_t K, int out_dtype, void *out,
                     void *stream);
size_t mxfp4_linear_workspace_size(int64_t M, int64_t K, int64_t N);
int mxfp4_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *w_q, const uint8_t *w_scale, int64_t N,
                 int out_dtype, void *out, void *ws, size_t ws_bytes, void *stream);

/* Helpers. */
const char *nvfp4_status_string(int status);
const char *nvfp4_last_error(void);
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
