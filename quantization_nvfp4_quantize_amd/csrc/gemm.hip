// Token-grouped NVFP4 GEMMs of the MoE expert FFN on gfx950 (the L1 gate/up
// GEMM with its fused SwiGLU -> bf16 -> NVFP4 epilogue, and the L2 down GEMM
// with the routing-weighted epilogue), after DEBUG_LOG.md "NVFP4 MoE Pipeline"
// and NVFP4-1.1_APPROACH_PART_2.md / NVFP4-1.1_APPROACH.md ("nvfp4-megamoe-
// kernel"): alpha = activation global scale * weight global scale is applied
// to the accumulator, SiLU(gate) * up is formed in the epilogue, only the
// SwiGLU columns are written (compact output), and that output is quantized
// to NVFP4 in the same pass with a supplied global scale.
//
// MI355X design (not the pages' B200 one):
//   * A workgroup of 256 threads (4 wave64s, one per SIMD) owns a 256 x 256
//     output tile; each wave owns 128 x 128 of it as 4 x 4 MFMA 32x32x16 f16
//     tiles (256 fp32 accumulators per lane, held in AGPRs).
//   * Per K step of 64, every thread loads one A row chunk and one B row chunk
//     (32 B of nibbles + 4 scale bytes each) from HBM, dequantizes them
//     exactly to f16 (E2M1 * E4M3 needs at most 6 significant bits and lies in
//     [2^-10, 2688], so f16 holds it exactly) with the gfx950 FP4 -> f16 and
//     FP8 -> f16 conversions and one packed f16 multiply, and writes them to a
//     double-buffered LDS tile.  The next step's global loads are in flight
//     while the MFMAs of the current step run.
//   * LDS rows are 64 f16 = 8 chunks of 16 B, chunk c stored at c ^ (row & 7),
//     which keeps both the row-wise writes and the MFMA operand reads free of
//     bank conflicts.
//   * The K order inside a 64-chunk is permuted identically for A and B (lane
//     half g reads physical chunk 4g + s at MFMA step s), so each lane's
//     operand bytes for the whole step are contiguous.
//   * L1: the 256 B rows of a tile are the gate/up rows of 128 compact SwiGLU
//     columns, reordered in LDS so that gate_j and up_j land in the same lane
//     and MFMA register; the epilogue writes the bf16 SwiGLU tile to LDS and
//     quantizes it with lane pairs (one 16-element block per pair).
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kStepK = 64;
constexpr int kGemmThreads = 256;
constexpr int kLdsOperand = kTileM * (kStepK / 8);  // f16x8 chunks per operand per stage

// ------------------------------------------------------------------ operands
struct RowChunk {
  uint4 q0, q1;  // 64 nibbles (K step) of one row
  uint32_t s;    // the 4 block scales of those 64 elements
};

__device__ __forceinline__ RowChunk load_row_chunk(const uint8_t* qrow, const uint8_t* sfrow,
                                                   int kb) {
  RowChunk r;
  const uint4* p = reinterpret_cast<const uint4*>(qrow + (size_t)kb * 32);
  r.q0 = p[0];
  r.q1 = p[1];
  r.s = *reinterpret_cast<const uint32_t*>(sfrow + (size_t)kb * 4);
  return r;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 sc) {
  f16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  f16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  f16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  f16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  f16x8 v = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
  return v;
}

// Dequantize one 64-element row chunk exactly into f16 and store it to the
// swizzled LDS row.
__device__ __forceinline__ void store_row_chunk(f16x8* lds, int row, const RowChunk& r) {
  f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s, 1.0f, false);
  f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s, 1.0f, true);
  f16x2 c0 = {s01[0], s01[0]}, c1 = {s01[1], s01[1]};
  f16x2 c2 = {s23[0], s23[0]}, c3 = {s23[1], s23[1]};
  lds[swz(row, 0)] = dequant8(r.q0.x, c0);
  lds[swz(row, 1)] = dequant8(r.q0.y, c0);
  lds[swz(row, 2)] = dequant8(r.q0.z, c1);
  lds[swz(row, 3)] = dequant8(r.q0.w, c1);
  lds[swz(row, 4)] = dequant8(r.q1.x, c2);
  lds[swz(row, 5)] = dequant8(r.q1.y, c2);
  lds[swz(row, 6)] = dequant8(r.q1.z, c3);
  lds[swz(row, 7)] = dequant8(r.q1.w, c3);
}

// One K step of MFMAs for this wave's 128 x 128 sub-tile.
__device__ __forceinline__ void mma_step(const f16x8* ldsA, const f16x8* ldsB, f32x16 (&acc)[4][4],
                                         int wm, int wn, int lane) {
  const int g = lane >> 5, r = lane & 31;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f16x8 a[4], b[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a[mt] = ldsA[swz(wm * 128 + mt * 32 + r, 4 * g + s)];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) b[nt] = ldsB[swz(wn * 128 + nt * 32 + r, 4 * g + s)];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
  }
}

// The whole K loop: A rows a_row[0..255], B rows b_row[0..255] (row pointers
// for this thread's A row t and B row t are passed in), nk steps of 64.
__device__ __forceinline__ void gemm_mainloop(f16x8* lds, const uint8_t* a_q_row,
                                              const uint8_t* a_sf_row, const uint8_t* b_q_row,
                                              const uint8_t* b_sf_row, int nk,
                                              f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};

  RowChunk ra = load_row_chunk(a_q_row, a_sf_row, 0);
  RowChunk rb = load_row_chunk(b_q_row, b_sf_row, 0);
  store_row_chunk(lds, tid, ra);
  store_row_chunk(lds + kLdsOperand, tid, rb);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nk;
    if (more) {
      ra = load_row_chunk(a_q_row, a_sf_row, kb + 1);
      rb = load_row_chunk(b_q_row, b_sf_row, kb + 1);
    }
    const f16x8* A = lds + cur * 2 * kLdsOperand;
    mma_step(A, A + kLdsOperand, acc, wm, wn, lane);
    if (more) {
      f16x8* N = lds + (cur ^ 1) * 2 * kLdsOperand;
      store_row_chunk(N, tid, ra);
      store_row_chunk(N + kLdsOperand, tid, rb);
    }
    __syncthreads();
  }
}

// Accumulator element i of MFMA tile (mt, nt) for this lane sits at row
// 8*(i/4) + 4*(lane/32) + i%4 and column lane%32 of that 32 x 32 tile.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// ------------------------------------------------------------------ L1
struct L1Params {
  const uint8_t* a_q;   // activations [rows][K/2]
  const uint8_t* a_sf;  // [rows][K/16]
  const float* a_gs;
  int64_t K;
  const uint8_t* w_q;   // [E][N2][K/2], rows interleaved by 8 (gate, up)
  const uint8_t* w_sf;  // [E][N2][K/16]
  const float* w_gs;    // [E]
  int64_t N2;
  const float* out_gs;  // global scale of the SwiGLU output
  uint16_t* c_bf16;     // nullable [out rows][N2/2]
  uint8_t* c_q;         // [out rows][N2/4]
  uint8_t* c_sf;        // [out rows][N2/32]
  const GemmTile* tiles;  // nullable: identity tiling of M rows, expert 0
  const int* ntiles;
  int64_t M;            // rows when tiles == nullptr
  const int* perm;      // nullable: sorted position -> pair id
  int topk;             // pair id / topk = activation row
  int n_ntiles;
};

__device__ __forceinline__ bool tile_of(const GemmTile* tiles, const int* ntiles, int64_t M, int ti,
                                        GemmTile* t) {
  if (tiles) {
    if (ti >= *ntiles) return false;
    *t = tiles[ti];
    return true;
  }
  int64_t r0 = (int64_t)ti * kTileM;
  if (r0 >= M) return false;
  t->expert = 0;
  t->row0 = (int)r0;
  t->nrows = (int)((M - r0) < kTileM ? (M - r0) : kTileM);
  t->pad = 0;
  return true;
}

// Global weight row of the l1 B tile row rb (0..255) for n tile nt: the tile
// covers compact SwiGLU columns [128 nt, 128 nt + 128); wave column half wn
// takes 64 of them: rows 32 jt + c of that half are gate (jt = 0, 1) or up
// (jt = 2, 3) of compact column 128 nt + 64 wn + 32 (jt & 1) + c.
__device__ __forceinline__ int l1_weight_row(int nt, int rb) {
  int wn = rb >> 7, jt = (rb >> 5) & 3, c = rb & 31;
  int j = 128 * nt + 64 * wn + 32 * (jt & 1) + c;
  int gate = 16 * (j >> 3) + (j & 7);
  return (jt < 2) ? gate : gate + 8;
}

__global__ __launch_bounds__(kGemmThreads) void l1_gemm_swiglu_quant_kernel(L1Params p) {
  __shared__ f16x8 lds[2 * 2 * kLdsOperand];  // 128 KiB: 2 stages x (A, B)
  __shared__ float rtab[128];
  __shared__ int out_row[kTileM];

  const int ti = blockIdx.x / p.n_ntiles;
  const int nt = blockIdx.x % p.n_ntiles;
  GemmTile t;
  if (!tile_of(p.tiles, p.ntiles, p.M, ti, &t)) return;

  const int tid = threadIdx.x;
  // A row of this thread (padding rows repeat the tile's first row; their
  // outputs are never stored)
  const int r = tid < t.nrows ? tid : 0;
  int arow, orow;
  if (p.perm) {
    int pair = p.perm[t.row0 + r];
    arow = pair / p.topk;
    orow = pair;
  } else {
    arow = t.row0 + r;
    orow = arow;
  }
  out_row[tid] = orow;
  const int64_t Kq = p.K / 2, Ks = p.K / 16;
  const uint8_t* a_q_row = p.a_q + (int64_t)arow * Kq;
  const uint8_t* a_sf_row = p.a_sf + (int64_t)arow * Ks;
  const int64_t wrow = (int64_t)t.expert * p.N2 + l1_weight_row(nt, tid);
  const uint8_t* b_q_row = p.w_q + wrow * Kq;
  const uint8_t* b_sf_row = p.w_sf + wrow * Ks;

  f32x16 acc[4][4];
  gemm_mainloop(lds, a_q_row, a_sf_row, b_q_row, b_sf_row, (int)(p.K / kStepK), acc);

  // ---- epilogue: alpha, SwiGLU, bf16 tile in LDS
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  constexpr int kCStride = 136;  // bf16 per LDS row (128 + 8 padding)
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int col = 64 * wn + 32 * jt + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float gate = acc[mt][jt][i] * alpha;
        float up = acc[mt][jt + 2][i] * alpha;
        float c = gate / (1.0f + __expf(-gate)) * up;
        __bf16 b = (__bf16)c;
        ctile[(wm * 128 + mt * 32 + acc_row(i, lane)) * kCStride + col] =
            __builtin_bit_cast(uint16_t, b);
      }
    }
  }
  const float E2 = 1.0f / p.out_gs[0];
  fill_rtab(rtab, E2, tid);
  __syncthreads();

  // ---- quantize the bf16 tile: 16 lanes per row (8 blocks, two halves each)
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
#pragma unroll 4
  for (int pass = 0; pass < kTileM / 16; ++pass) {
    const int row = pass * 16 + (tid >> 4);
    uint4 w = *reinterpret_cast<const uint4*>(ctile + row * kCStride + 8 * hb);
    uint32_t code;
    uint32_t q = quantize_half_block(w, E2, rtab, &code);
    if (row < t.nrows) {
      const int64_t o = out_row[row];
      const int64_t col0 = 128 * (int64_t)nt + 8 * hb;  // compact column of this lane's 8
      reinterpret_cast<uint32_t*>(p.c_q + o * (I / 2))[col0 / 8] = q;
      if ((hb & 1) == 0) p.c_sf[o * (I / 16) + col0 / 16] = (uint8_t)code;
      if (p.c_bf16) *reinterpret_cast<uint4*>(p.c_bf16 + o * I + col0) = w;
    }
  }
}

// ------------------------------------------------------------------ L2
struct L2Params {
  const uint8_t* a_q;   // L1 output [P][K/2] in pair order
  const uint8_t* a_sf;
  const float* a_gs;
  int64_t K;            // I
  const uint8_t* w_q;   // [E][N][K/2]
  const uint8_t* w_sf;
  const float* w_gs;
  int64_t N;            // H
  const float* row_w;   // [P] routing weight of each pair
  float* o;             // [P][N] fp32
  const GemmTile* tiles;
  const int* ntiles;
  const int* perm;
  int n_ntiles;
};

__global__ __launch_bounds__(kGemmThreads) void l2_gemm_kernel(L2Params p) {
  __shared__ f16x8 lds[2 * 2 * kLdsOperand];
  __shared__ int out_row[kTileM];
  const int ti = blockIdx.x / p.n_ntiles;
  const int nt = blockIdx.x % p.n_ntiles;
  if (ti >= *p.ntiles) return;
  const GemmTile t = p.tiles[ti];
  const int tid = threadIdx.x;
  const int r = tid < t.nrows ? tid : 0;
  const int pair = p.perm[t.row0 + r];
  out_row[tid] = pair;
  const int64_t Kq = p.K / 2, Ks = p.K / 16;
  const int64_t wrow = (int64_t)t.expert * p.N + (int64_t)nt * kTileN + tid;
  f32x16 acc[4][4];
  gemm_mainloop(lds, p.a_q + (int64_t)pair * Kq, p.a_sf + (int64_t)pair * Ks, p.w_q + wrow * Kq,
                p.w_sf + wrow * Ks, (int)(p.K / kStepK), acc);
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = wm * 128 + mt * 32 + acc_row(i, lane);
      if (row < t.nrows) {
        const int64_t pr = out_row[row];
        const float s = alpha * p.row_w[pr];
        float* orow = p.o + pr * p.N + (int64_t)nt * kTileN + wn * 128 + (lane & 31);
#pragma unroll
        for (int ntl = 0; ntl < 4; ++ntl) orow[ntl * 32] = acc[mt][ntl][i] * s;
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
int gemm_tile_rows() { return kTileM; }

hipError_t launch_l1(const uint8_t* a_q, const uint8_t* a_sf, const float* a_gs, int64_t K,
                     const uint8_t* w_q, const uint8_t* w_sf, const float* w_gs, int64_t N2,
                     const float* out_gs, uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                     const int* perm, int topk, hipStream_t s) {
  L1Params p{a_q, a_sf, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN)};
  int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l1_gemm_swiglu_quant_kernel<<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_l2(const uint8_t* a_q, const uint8_t* a_sf, const float* a_gs, int64_t K,
                     const uint8_t* w_q, const uint8_t* w_sf, const float* w_gs, int64_t N,
                     const float* row_w, float* o, const GemmTile* tiles, const int* ntiles,
                     int max_tiles, const int* perm, hipStream_t s) {
  L2Params p{a_q, a_sf, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, tiles, ntiles, perm,
             (int)(N / kTileN)};
  int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l2_gemm_kernel<<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
