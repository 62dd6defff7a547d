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
//   * Operands.  Every NVFP4 value e2m1 * E4M3-scale has at most 6
//     significant bits and lies in [2^-10, 2688], so f16 holds it exactly and
//     f16 MFMA on dequantized operands gives exact products.  The weight
//     operand (B) is dequantized inside the GEMM; the activation operand (A)
//     arrives already dequantized to exact f16 -- written once per row by its
//     producer (the activation quantizer, or the L1 epilogue for the L2 input)
//     instead of once per (row, N tile) here.  gfx950 executes a wave's VALU
//     work between that wave's MFMAs, not under them; another wave's VALU does
//     run under them, but only about 2 VALU instructions per MFMA fit.
//     Dequantizing B alone costs ~1 per MFMA; dequantizing both would cost ~2.
//   * A workgroup of 512 threads (8 wave64s, two per SIMD) owns a 256 x 256
//     output tile; wave w owns rows 128 (w & 1) .. +128 and columns
//     64 (w >> 1) .. +64 as 4 x 2 MFMA 32x32x16 f16 tiles (128 fp32
//     accumulators per lane).
//   * Per K step of 64, thread t moves half a row of each operand: 64 B of A
//     (f16) and 16 B of B nibbles plus 2 block scales, loaded two steps ahead
//     into one of two register sets.  The B half is dequantized with the
//     gfx950 FP4 -> f16 and FP8 -> f16 conversions and one packed f16
//     multiply per pair.  Both halves are written to the other stage of a
//     double-buffered LDS tile in 8 pieces placed between the wave's 32 MFMAs
//     of the step (scheduling fences keep the order); MFMA operand fragments
//     are read one sub-step ahead.
//   * LDS rows are 64 f16 = 8 chunks of 16 B, chunk c stored at
//     c ^ ((row ^ row >> 3) & 7), which keeps the row-wise writes and the MFMA
//     operand reads free of bank conflicts (16-lane groups on 64 banks).
//   * The K order inside a 64-chunk is permuted identically for A and B (lane
//     half g reads physical chunk 4g + s at MFMA step s).
//   * L1: the 256 B rows of a tile are the gate/up rows of 128 compact SwiGLU
//     columns, ordered in LDS so that gate_j and up_j land in the same lane
//     and accumulator register; the epilogue writes the bf16 SwiGLU tile to
//     LDS, quantizes it with lane pairs (one 16-element block per pair), and
//     writes the NVFP4 bytes plus the exact f16 of the quantized values (the
//     L2 operand).
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kStepK = 64;
constexpr int kGemmThreads = 512;
constexpr int kLdsOperand = kTileM * (kStepK / 8);  // f16x8 chunks per operand per stage

// ------------------------------------------------------------------ operands
// This thread's share of one K step: half an A row (32 f16) and half a B row
// (32 nibbles and their 2 block scales).
struct StepChunk {
  uint4 a[4];
  uint4 bq;
  uint32_t bs;
};

__device__ __forceinline__ StepChunk load_step(const uint16_t* a_row, const uint8_t* bq_row,
                                               const uint8_t* bsf_row, int kb, int half) {
  StepChunk c;
  const uint4* pa = reinterpret_cast<const uint4*>(a_row + (size_t)kb * 64 + half * 32);
  c.a[0] = pa[0];
  c.a[1] = pa[1];
  c.a[2] = pa[2];
  c.a[3] = pa[3];
  c.bq = *reinterpret_cast<const uint4*>(bq_row + (size_t)kb * 32 + half * 16);
  c.bs = *reinterpret_cast<const uint16_t*>(bsf_row + (size_t)kb * 4 + half * 2);
  return c;
}

// 16-byte chunk c of LDS row `row` lives at c ^ ((row ^ row >> 3) & 7): any
// 16 consecutive rows reading or writing the same logical chunk hit 16
// distinct 16-byte bank groups (64 banks), and any 8 consecutive rows hit 8.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Write piece k (0..7) of this thread's step share into LDS stage `stage`:
// pieces 0..3 are A chunks 4 half + k, pieces 4..7 the dequantized B chunks.
__device__ __forceinline__ void store_piece(f16x8* stage, int row, int half, const StepChunk& c,
                                            f16x2 s0, f16x2 s1, int k) {
  if (k < 4) {
    stage[swz(row, 4 * half + k)] = __builtin_bit_cast(f16x8, c.a[k]);
  } else {
    const int j = k - 4;
    stage[kLdsOperand + swz(row, 4 * half + j)] = dequant8(word_of(c.bq, j), (j < 2) ? s0 : s1);
  }
}

__device__ __forceinline__ void scale_pairs(uint32_t bs, f16x2* s0, f16x2* s1) {
  f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs, 1.0f, false);
  *s0 = f16x2{s[0], s[0]};
  *s1 = f16x2{s[1], s[1]};
}

__device__ __forceinline__ void store_step(f16x8* stage, int row, int half, const StepChunk& c) {
  f16x2 s0, s1;
  scale_pairs(c.bs, &s0, &s1);
#pragma unroll
  for (int k = 0; k < 8; ++k) store_piece(stage, row, half, c, s0, s1, k);
}

struct Frags {
  f16x8 a[4], b[2];
};

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One K step on LDS stage `cur` (A at cur, B at cur + kLdsOperand): the wave's
// 32 MFMAs, with this thread's next-step share `n` written into stage `nxt`
// one piece per 4 MFMAs.  Fragments of MFMA sub-step s + 1 are read while
// sub-step s runs.
__device__ __forceinline__ void mma_step_overlapped(const f16x8* cur, f16x8* nxt, int row,
                                                    int half, const StepChunk& n,
                                                    f32x16 (&acc)[4][2], int wm, int wn,
                                                    int lane) {
  const int g = lane >> 5, r = lane & 31;
  Frags f[2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) f[0].a[mt] = cur[swz(wm * 128 + mt * 32 + r, 4 * g)];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) f[0].b[nt] = cur[kLdsOperand + swz(wn * 64 + nt * 32 + r, 4 * g)];
  f16x2 s0, s1;
  scale_pairs(n.bs, &s0, &s1);
  SCHED_FENCE();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const Frags& F = f[s & 1];
    Frags& G = f[(s + 1) & 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (s < 3) {
        const int k = 4 * g + s + 1;
        if (h == 0) {
          G.a[0] = cur[swz(wm * 128 + 0 * 32 + r, k)];
          G.a[1] = cur[swz(wm * 128 + 1 * 32 + r, k)];
          G.a[2] = cur[swz(wm * 128 + 2 * 32 + r, k)];
        } else {
          G.a[3] = cur[swz(wm * 128 + 3 * 32 + r, k)];
          G.b[0] = cur[kLdsOperand + swz(wn * 64 + 0 * 32 + r, k)];
          G.b[1] = cur[kLdsOperand + swz(wn * 64 + 1 * 32 + r, k)];
        }
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int mt = 2 * h + mi;
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[mt], F.b[nt], acc[mt][nt], 0, 0, 0);
        }
      store_piece(nxt, row, half, n, s0, s1, 2 * s + h);
      SCHED_FENCE();
    }
  }
}

// The whole K loop over nk steps of 64.  a_row: this thread's A row (f16),
// bq_row / bsf_row: its B row (NVFP4); the thread moves half `half` of each.
// Global loads run two steps ahead of the MFMAs in two register sets; the
// loop body is branch-free (loads past the end re-read the last step and the
// extra pieces land in a stage nobody reads).
__device__ __forceinline__ void gemm_mainloop(f16x8* lds, const uint16_t* a_row,
                                              const uint8_t* bq_row, const uint8_t* bsf_row,
                                              int nk, f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int row = tid >> 1, half = tid & 1;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
  f16x8* S0 = lds;
  f16x8* S1 = lds + 2 * kLdsOperand;
  const int last = nk - 1;
  StepChunk c0 = load_step(a_row, bq_row, bsf_row, 0, half);
  StepChunk c1 = load_step(a_row, bq_row, bsf_row, min(1, last), half);
  store_step(S0, row, half, c0);
  __syncthreads();
  int kb = 0;
  for (; kb + 1 < nk; kb += 2) {
    // even step kb: stage S0; the next step's share is in c1; refill c0
    c0 = load_step(a_row, bq_row, bsf_row, min(kb + 2, last), half);
    mma_step_overlapped(S0, S1, row, half, c1, acc, wm, wn, lane);
    __syncthreads();
    // odd step kb + 1: stage S1; the next step's share is in c0; refill c1
    c1 = load_step(a_row, bq_row, bsf_row, min(kb + 3, last), half);
    mma_step_overlapped(S1, S0, row, half, c0, acc, wm, wn, lane);
    __syncthreads();
  }
  if (kb < nk) {
    mma_step_overlapped(S0, S1, row, half, c1, acc, wm, wn, lane);
    __syncthreads();
  }
}

// Accumulator element i of MFMA tile (mt, nt) for this lane sits at row
// 8*(i/4) + 4*(lane/32) + i%4 and column lane%32 of that 32 x 32 tile.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

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

// ------------------------------------------------------------------ L1
struct L1Params {
  const uint16_t* a_f16;  // exact f16 activations [rows][K] (e2m1 * block scale)
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
  uint16_t* c_f16;      // nullable [out rows][N2/2]: exact f16 of the quantized values
  const GemmTile* tiles;  // nullable: identity tiling of M rows, expert 0
  const int* ntiles;
  int64_t M;            // rows when tiles == nullptr
  const int* perm;      // nullable: sorted position -> pair id
  int topk;             // pair id / topk = activation row
  int n_ntiles;
};

// Global weight row of the L1 B tile row rb (0..255) for n tile nt: the tile
// covers compact SwiGLU columns [128 nt, 128 nt + 128); the 64 B rows of wave
// column wn = rb / 64 are the gate rows (rb & 32 == 0) and then the up rows of
// compact columns 128 nt + 32 wn + (rb & 31), so that MFMA n tile 0 (gate)
// and 1 (up) of a wave hold matching columns in the same lanes.
__device__ __forceinline__ int l1_weight_row(int nt, int rb) {
  int wn = rb >> 6, up = (rb >> 5) & 1, c = rb & 31;
  int j = 128 * nt + 32 * wn + c;
  int gate = 16 * (j >> 3) + (j & 7);
  return up ? gate + 8 : gate;
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
  const int row = tid >> 1;
  // A row of this thread (padding rows repeat the tile's first row; their
  // outputs are never stored)
  const int r = row < t.nrows ? row : 0;
  int arow, orow;
  if (p.perm) {
    const int pair = p.perm[t.row0 + r];
    arow = pair / p.topk;
    orow = pair;
  } else {
    arow = t.row0 + r;
    orow = arow;
  }
  if ((tid & 1) == 0) out_row[row] = orow;
  const int64_t wrow = (int64_t)t.expert * p.N2 + l1_weight_row(nt, row);

  f32x16 acc[4][2];
  gemm_mainloop(lds, p.a_f16 + (int64_t)arow * p.K, p.w_q + wrow * (p.K / 2),
                p.w_sf + wrow * (p.K / 16), (int)(p.K / kStepK), acc);

  // ---- epilogue: alpha, SwiGLU, bf16 tile in LDS
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
  constexpr int kCStride = 136;  // bf16 per LDS row (128 + 8 padding)
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds);
  const int col = 32 * wn + (lane & 31);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float gate = acc[mt][0][i] * alpha;
      float up = acc[mt][1][i] * alpha;
      float c = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up;
      __bf16 b = (__bf16)c;
      ctile[(wm * 128 + mt * 32 + acc_row(i, lane)) * kCStride + col] = __builtin_bit_cast(uint16_t, b);
    }
  }
  const float E2 = 1.0f / p.out_gs[0];
  fill_rtab(rtab, E2, tid);
  __syncthreads();

  // ---- quantize the bf16 tile: 16 lanes per row (8 blocks, two halves each)
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
#pragma unroll 2
  for (int pass = 0; pass < kTileM / (kGemmThreads / 16); ++pass) {
    const int qrow = pass * (kGemmThreads / 16) + (tid >> 4);
    uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
    uint32_t code;
    uint32_t q = quantize_half_block(w, E2, rtab, &code);
    if (qrow < t.nrows) {
      const int64_t o = out_row[qrow];
      const int64_t col0 = 128 * (int64_t)nt + 8 * hb;  // compact column of this lane's 8
      reinterpret_cast<uint32_t*>(p.c_q + o * (I / 2))[col0 / 8] = q;
      if ((hb & 1) == 0) p.c_sf[o * (I / 16) + col0 / 16] = (uint8_t)code;
      if (p.c_bf16) *reinterpret_cast<uint4*>(p.c_bf16 + o * I + col0) = w;
      if (p.c_f16) *reinterpret_cast<f16x8*>(p.c_f16 + o * I + col0) = dequant8(q, scale_pair(code));
    }
  }
}

// ------------------------------------------------------------------ L2
struct L2Params {
  const uint16_t* a_f16;  // exact f16 of the quantized L1 output [P][K], pair order
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
  const int row = tid >> 1;
  const int r = row < t.nrows ? row : 0;
  const int pair = p.perm[t.row0 + r];
  if ((tid & 1) == 0) out_row[row] = pair;
  const int64_t wrow = (int64_t)t.expert * p.N + (int64_t)nt * kTileN + row;
  f32x16 acc[4][2];
  gemm_mainloop(lds, p.a_f16 + (int64_t)pair * p.K, p.w_q + wrow * (p.K / 2),
                p.w_sf + wrow * (p.K / 16), (int)(p.K / kStepK), acc);
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int orw = wm * 128 + mt * 32 + acc_row(i, lane);
      if (orw < t.nrows) {
        const int64_t pr = out_row[orw];
        const float s = alpha * p.row_w[pr];
        float* orow = p.o + pr * p.N + (int64_t)nt * kTileN + wn * 64 + (lane & 31);
        orow[0] = acc[mt][0][i] * s;
        orow[32] = acc[mt][1][i] * s;
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
int gemm_tile_rows() { return kTileM; }

hipError_t launch_l1(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                     uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                     const int* perm, int topk, hipStream_t s) {
  L1Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf, c_f16,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN)};
  int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l1_gemm_swiglu_quant_kernel<<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_l2(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w, float* o,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, const int* perm,
                     hipStream_t s) {
  L2Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, tiles, ntiles, perm, (int)(N / kTileN)};
  int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l2_gemm_kernel<<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
