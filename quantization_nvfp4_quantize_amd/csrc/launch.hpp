// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// One block of up to gemm_tile_rows() rows of one expert in the
// expert-grouped (sorted) row order.
struct GemmTile {
  int expert;
  int row0;   // first sorted position
  int nrows;
  int pad;
};

// ---- quantize.hip
size_t global_scale_workspace_bytes();
// g = max|x| / 2688 (1 if all zero) over n bf16 values (n % 8 == 0) -> gs[0]
hipError_t launch_global_scale(const uint16_t* x, int64_t n, float* partial, float* gs,
                               hipStream_t s);
// The same over the rows of a [rows][cols] bf16 matrix whose row r is pair r
// of a top-k routing, skipping rows whose expert id ids[r] is outside [0, E).
hipError_t launch_global_scale_rows(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ids, int E,
                                    float* partial, float* gs, hipStream_t s);
hipError_t launch_copy_scalar(const float* src, float* dst, hipStream_t s);
// n bf16 values (n % 16 == 0) -> q [n/2], sf [n/16] with global scale gs[0];
// f16out (nullable) [n]: exact f16 of e2m1 * block scale (the GEMM operand)
hipError_t launch_quantize(const uint16_t* x, int64_t n, const float* gs, uint8_t* q, uint8_t* sf,
                           uint16_t* f16out, hipStream_t s);
// The same with the global scale formed from namax partial maxima of |x|
// (amax_part, as the second pass of launch_global_scale would) and stored to
// gs_out; f16out is required.
hipError_t launch_quantize_folded(const uint16_t* x, int64_t n, const float* amax_part, int namax, float* gs_out,
                                  uint8_t* q, uint8_t* sf, uint16_t* f16out, hipStream_t s);
// The same for the SwiGLU columns of an interleaved [rows][2I] bf16 matrix
// (groups of 8 columns alternating SiLU(gate), SiLU(gate) * up): the compact
// [rows][I] values are quantized (rows * I / 8 < 2^32).
hipError_t launch_quantize_interleaved(const uint16_t* x_il, int64_t rows, int64_t I, const float* gs,
                                       uint8_t* q, uint8_t* sf, uint16_t* f16out, hipStream_t s);
// NVFP4 (n values) -> exact f16 of e2m1 * block scale
hipError_t launch_dequantize_f16(const uint8_t* q, const uint8_t* sf, int64_t n, uint16_t* out,
                                 hipStream_t s);
// sf [R][C] -> its row-paired layout (nvfp4_pair_scales); R even, C % 64 == 0.
hipError_t launch_pair_scales(const uint8_t* sf, int64_t R, int64_t C, uint8_t* out, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* q, const uint8_t* sf, const float* gs, int64_t n,
                             bool bf16_out, void* out, hipStream_t s);

// ---- gemm.hip
int gemm_tile_rows();
// Rows per tile of the few-rows-per-expert kernels (decode shape).
int skinny_tile_rows();
// Whether those kernels take a reduction length K (a multiple of 256, or 128).
bool skinny_supports_k(int64_t K);
// L1: c = SwiGLU(alpha * A @ W^T) -> bf16 (optional) and NVFP4 (c_q, c_sf).
// tiles == nullptr: identity tiling of M rows with expert 0.  perm != nullptr:
// tile rows are sorted positions, perm gives the pair id, the activation row
// is pair / topk and the output row is the pair id.
// a_f16: exact f16 activations [rows][K]; c_f16 (nullable): exact f16 of the
// quantized SwiGLU output (the L2 operand).
hipError_t launch_l1(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                     uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                     const int* perm, int topk, hipStream_t s, uint16_t* c_il = nullptr,
                     const uint8_t* a_q = nullptr, const uint8_t* a_sf = nullptr);
// L2: o[pair] = alpha * w[pair] * (A @ W_e^T) for the routed rows (fp32), or
// without routing (tiles, perm, row_w null) over M rows of expert 0, into o
// (fp32), o_bf16 (bf16) when that is non-null, or o_f16 with o_exp (f16
// values times a power of two per row and 32-column block) when those are
// non-null.  sched (nullable): 8 work counters, zero at launch, that
// let the workgroups claim items dynamically.
hipError_t launch_l2(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w, float* o,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, const int* perm,
                     hipStream_t s, int64_t M = 0, uint16_t* o_bf16 = nullptr, int* sched = nullptr,
                     uint16_t* o_f16 = nullptr, int8_t* o_exp = nullptr);

// ---- moe.hip
size_t route_lds_bytes(int E);
// Same operations as launch_l1 / launch_l2 on tiles of at most
// skinny_tile_rows() rows (weights streamed through registers).  With
// split_ws (skinny_split_bytes(), 16-byte aligned) and split_cnt
// (skinny_split_counters() ints, zero at launch and zero again after it) the
// few items that would run alone at the end of the launch are split along K.
// Two launches that share these buffers must not overlap.  sf_paired: w_sf
// is in the row-paired layout of nvfp4_pair_scales (K % 1024 == 0, else
// hipErrorInvalidValue).
hipError_t launch_l1_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                            uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                            const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                            const int* perm, int topk, hipStream_t s, uint16_t* c_il = nullptr,
                            const uint8_t* a_q = nullptr, const uint8_t* a_sf = nullptr,
                            float* split_ws = nullptr, int* split_cnt = nullptr, bool sf_paired = false);
hipError_t launch_l2_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w,
                            float* o, const GemmTile* tiles, const int* ntiles, int max_tiles,
                            const int* perm, hipStream_t s, int64_t M = 0, uint16_t* o_bf16 = nullptr, int* sched = nullptr,
                            uint16_t* o_f16 = nullptr, int8_t* o_exp = nullptr, float* split_ws = nullptr,
                            int* split_cnt = nullptr, bool sf_paired = false);
size_t skinny_split_bytes();
constexpr int skinny_split_counters() { return 8 * 16; }
// Work counters that launch_route zeroes: [0, 16) those of the 256-row
// GEMMs, then the 32-row GEMMs' split counters.
constexpr int kSchedCounters = 16 + skinny_split_counters();
// Scratch (ints) of the many-workgroup grouping for P pairs and E experts.
size_t route_workspace_bytes(int64_t P, int E);
// Groups the pairs by expert into tiles of tile_rows rows; with small_rows
// > 0 each expert's last block of at most small_rows rows is listed in
// small / *nsmall (at most E entries) instead of tiles.  Also zeroes
// sched[0 .. kSchedCounters) (nullable): the GEMMs' work counters.
hipError_t launch_route(const int32_t* ids, int64_t P, int E, int tile_rows, int small_rows, int small_tile, int* offsets,
                        int* perm, GemmTile* tiles, int* ntiles, GemmTile* small, int* nsmall, int* err_count,
                        int* ws, int* sched, hipStream_t s);
// launch_route runs in one workgroup for these P (else in many).
bool route_single(int64_t P);
// Workgroups of the global-scale maxima that launch_amax_route uses for n8
// 8-element chunks (at most 256).
int amax_route_blocks(int64_t n8);
// launch_route (P with route_single) and, in the same launch, the first pass
// of the global scale of the n bf16 values x: namax = amax_route_blocks(n /
// 8) maxima of |x| into partial[0 .. namax), for launch_quantize_folded.
hipError_t launch_amax_route(const uint16_t* x, int64_t n, float* partial, int namax, const int32_t* ids,
                             int64_t P, int E, int tile_rows, int small_rows, int small_tile, int* offsets,
                             int* perm, GemmTile* tiles, int* ntiles, GemmTile* small, int* nsmall,
                             int* err_count, int* sched, hipStream_t s);
// y[t] = sum over the k rows of token t of o (fp32), or of the f16 form
// o_f16 * 2^o_exp when o_f16 is non-null (one exponent per 32 columns).
hipError_t launch_combine(const float* o, const int32_t* ids, int E, int64_t T, int k, int64_t H,
                          bool bf16_out, void* out, hipStream_t s, const uint16_t* o_f16 = nullptr,
                          const int8_t* o_exp = nullptr);

// ---- mxfp4.hip (OCP MX v1.0 MXFP4: E8M0 scale per 32 elements, E2M1 elements)
// n bf16 values (n % 32 == 0) -> q [n/2] (element 2i in the low nibble of
// byte i), sc [n/32] E8M0 codes
hipError_t launch_mx_quantize(const uint16_t* x, int64_t n, uint8_t* q, uint8_t* sc, hipStream_t s);
hipError_t launch_mx_dequantize(const uint8_t* q, const uint8_t* sc, int64_t n, bool bf16_out, void* out,
                                hipStream_t s);
// Tile size (rows and columns) and K step of the MXFP4 GEMM.
int mx_gemm_tile();
int mx_gemm_step_k();
// y [M][N] = A @ W^T for MXFP4 A [M][K], W [N][K] (K % mx_gemm_step_k() == 0,
// N % mx_gemm_tile() == 0) into o (fp32) or o_bf16 when that is non-null.
hipError_t launch_mx_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t M, int64_t K, const uint8_t* w_q,
                          const uint8_t* w_sc, int64_t N, float* o, uint16_t* o_bf16, hipStream_t s);

}  // namespace nvfp4
