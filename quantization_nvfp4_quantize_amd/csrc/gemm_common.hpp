// Device pieces shared by the token-grouped NVFP4 GEMM kernels (the 256-row
// tile kernels for many rows per expert, the 32-row kernels for few): LDS-only
// barriers and explicit load-counter waits, direct-to-LDS loads, the XCD-aware
// work order, the operand swizzle, in-register weight dequantization, and the
// L1 (gate/up + SwiGLU + NVFP4) and L2 (down, routing-weighted) parameters.
#pragma once

#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStepK = 64;    // K per main-loop step (4 MFMA sub-steps of 16)
constexpr int kTileN = 256;   // B rows (output columns of the GEMM) per workgroup

// ------------------------------------------------------------------ sync
// Workgroup barrier over LDS only: waits for this wave's LDS traffic, not for
// its outstanding global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
  asm volatile("s_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (the counter retires loads in issue order).  The direct-to-LDS loads are
// not tracked by the compiler for later LDS reads, so their completion is
// waited for explicitly with this before the barrier that publishes them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Work item of this workgroup among W items.  Workgroup b runs on XCD b % 8;
// XCD x takes the contiguous items x q + min(x, r) .. (q = W / 8, r = W % 8,
// q + 1 items on the first r XCDs), so the workgroups running together on
// one XCD work on neighbouring items.  False for workgroups beyond W.
__device__ __forceinline__ bool work_item(int W, int* item) {
  const int b = blockIdx.x, x = b & 7, j = b >> 3;
  const int q = W >> 3, r = W & 7;
  if (j >= q + (x < r ? 1 : 0)) return false;
  *item = x * q + min(x, r) + j;
  return true;
}

// 16-byte chunk c of A row `row` lives at c ^ key(row), key(row) =
// (row ^ row >> 3) & 7: any 16 consecutive rows reading the same logical
// chunk hit 16 distinct 16-byte bank groups (64 banks).  key(32 m + r) for
// r < 32 depends only on r and on the parity of m, so the fragments of a
// wave's four A tiles are two base pointers plus compile-time offsets.
__device__ __forceinline__ int swz_key(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Direct-to-LDS loads.  They are issued from inline assembly so that the
// compiler neither orders later LDS reads of other stages behind them nor
// counts them: their completion is waited for explicitly (wait_vmcnt before
// the barrier that publishes a stage).  Waits the compiler inserts for its own
// loads can only become stricter for the loads it does not count.  M0 (the
// LDS destination) is saved and restored around each load.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// 1 KiB: lane i writes chunk i of `dst` (wave-uniform) with the 16 B at src.
__device__ __forceinline__ void dma16(f16x8* dst, const uint8_t* src) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(dst)), "v"(src)
      : "memory");
}

// The same with a wave-uniform base address (held in scalar registers) and a
// 32-bit per-lane byte offset: one VGPR per lane instead of a 64-bit
// address, and no per-lane 64-bit add.
__device__ __forceinline__ void dma16s(f16x8* dst, const uint8_t* base, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(dst)), "v"(off), "s"(base)
      : "memory");
}

__device__ __forceinline__ void dma4s(uint32_t* dst, const uint8_t* base, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(dst)), "v"(off), "s"(base)
      : "memory");
}

// 256 B: lane i writes dword i of `dst` (wave-uniform) with the 4 B at src.
__device__ __forceinline__ void dma4(uint32_t* dst, const uint8_t* src) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr(dst)), "v"(src)
      : "memory");
}

// B state of one K step in a lane: for each of its two 32-column tiles nt,
// the 16 B of nibbles of column 64 wn + 32 nt + lane % 32 at K chunks
// 4 g .. 4 g + 3 (g = lane / 32: exactly what its MFMA B fragments of the
// step need), and the column's four block-scale bytes.
struct BRaw {
  uint4 q[2];
};
struct BScale {
  uint32_t w[2];
};

// f16 pairs of the block scales 2 g and 2 g + 1 of a scale word: the
// fragments of sub-steps 0, 1 use lo, those of 2, 3 use hi.
struct ScalePairs {
  f16x2 lo[2], hi[2];
};

__device__ __forceinline__ ScalePairs scale_pairs(const BScale& sc, int g) {
  ScalePairs p;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc.w[nt] >> (16 * g), 1.0f, false);
    p.lo[nt] = f16x2{s[0], s[0]};
    p.hi[nt] = f16x2{s[1], s[1]};
  }
  return p;
}

// Exact f16 B fragment of sub-step s for column tile nt.
__device__ __forceinline__ f16x8 b_frag(const BRaw& r, const ScalePairs& p, int nt, int s) {
  return dequant8(word_of(r.q[nt], s), (s < 2) ? p.lo[nt] : p.hi[nt]);
}

// Accumulator element i of MFMA tile (mt, nt) for this lane sits at row
// 8*(i/4) + 4*(lane/32) + i%4 and column lane%32 of that 32 x 32 tile.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }


// Tile and N tile of this workgroup: tiles come from the routing (tiles,
// *ntiles), or without routing are the ceil(M / TM) row blocks of M rows
// (expert 0).  False for workgroups without work.
template <int TM>
__device__ __forceinline__ bool tile_of(const GemmTile* tiles, const int* ntiles, int64_t M,
                                        int n_ntiles, GemmTile* t, int* nt) {
  const int mtiles = tiles ? *ntiles : (int)((M + TM - 1) / TM);
  int item;
  if (!work_item(mtiles * n_ntiles, &item)) return false;
  const int ti = item / n_ntiles;
  *nt = item % n_ntiles;
  if (tiles) {
    *t = tiles[ti];
    return true;
  }
  const int64_t r0 = (int64_t)ti * TM;
  t->expert = 0;
  t->row0 = (int)r0;
  t->nrows = (int)((M - r0) < TM ? (M - r0) : TM);
  t->pad = 0;
  return true;
}

// ------------------------------------------------------------------ L1 / L2 parameters
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
  uint16_t* c_il;       // nullable [out rows][N2]: the interleaved bf16 output of the pages'
                        // earlier flow (groups of 8: SiLU(gate), then SiLU(gate) * up)
  const GemmTile* tiles;  // nullable: identity tiling of M rows, expert 0
  const int* ntiles;
  int64_t M;            // rows when tiles == nullptr
  const int* perm;      // nullable: sorted position -> pair id
  int topk;             // pair id / topk = activation row
  int n_ntiles;
  const uint8_t* a_q;   // with a_f16 null (256-row tiles): NVFP4 activations [rows][K/2],
  const uint8_t* a_sf;  // [rows][K/16], dequantized into LDS inside the GEMM
  int sf_paired;        // 32-row tiles: w_sf in the row-paired layout (K % 1024 == 0)
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

// The L2 down GEMM, and without routing (tiles == nullptr, perm == nullptr,
// row_w == nullptr) the dense NVFP4 linear y = alpha * A @ W^T.
struct L2Params {
  const uint16_t* a_f16;  // exact f16 of the quantized A rows [rows][K] (pair order for L2)
  const float* a_gs;
  int64_t K;            // I
  const uint8_t* w_q;   // [E][N][K/2]
  const uint8_t* w_sf;
  const float* w_gs;
  int64_t N;            // H
  const float* row_w;   // nullable [P]: routing weight of each pair (1 without)
  float* o;             // [rows][N] fp32 (used when o_bf16 is null)
  uint16_t* o_bf16;     // nullable [rows][N] bf16 output
  const GemmTile* tiles;  // nullable: identity tiling of M rows, expert 0
  const int* ntiles;
  int64_t M;            // rows when tiles == nullptr
  const int* perm;      // nullable: sorted position -> pair id
  int n_ntiles;
  int* sched;           // nullable: 8 zeroed work counters (one per XCD) for dynamic item claiming
  uint16_t* o_f16;      // nullable [rows][N] f16 output (used with o_exp instead of o):
  int8_t* o_exp;        // value = o_f16 * 2^o_exp, one exponent per (row, 32-column block) [rows][N/32]
  int sf_paired;        // 32-row tiles: w_sf in the row-paired layout (K % 1024 == 0)
};

// Exponent for storing the values of one (row, 32-column block) in f16:
// with m the block's largest magnitude, m * 2^-s lies in [2^14, 2^15), so no
// value overflows and values down to 2^-28 of the block maximum stay normal
// f16 numbers (full 11-bit precision).  s is clamped to [-128, 114] (int8):
// zero, subnormal, infinite or NaN maxima only need a value that keeps the
// rest finite.
__device__ __forceinline__ int f16_block_exp(float m) {
  const int ex = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;
  return max(ex - 14, -128);
}

// Epilogue writer of the L2 / linear GEMMs for one wave's 32-row x 64-column
// output block of rows r0 + 0..31, of which those below nrows are valid;
// row_of(r) gives the output row of tile row r and scale_of(r) its factor.
// Each 32 x 32 half (columns col0 + 32 half ..) goes through the wave's 4 KiB
// LDS scratch: fill(half, scratch) stores element (r, c) of the half at
// scratch[32 (r ^ ((r >> 2) & 1)) + c] (the two row groups of an MFMA
// accumulator write land in different bank halves); then lane l holds the
// 16 consecutive values 16 (l & 1) .. of row l / 2, scales them and stores
// them with 16 B writes: fp32 (o), bf16 (o_bf16), or f16 with one exponent
// per (row, 32 columns) (o_f16, o_exp).  For the f16 form the row factor sc
// is applied as sc * 2^-e: rounding is monotonic, so the largest |a * sc| of
// the block is max |a| * |sc|, and a * (sc * 2^-e) equals (a * sc) * 2^-e.
// (The accumulators are sums of exact products of NVFP4 values, so a nonzero
// max |a| is at least 2^-20 and sc * 2^-e stays finite.)  Every lane of the
// wave must take part.
__device__ __forceinline__ int l2_scratch_index(int r, int c) { return 32 * (r ^ ((r >> 2) & 1)) + c; }

template <class Fill, class RowOf, class ScaleOf>
__device__ __forceinline__ void l2_store_rows(const L2Params& p, float* scratch, int r0, int nrows, int64_t col0,
                                              int lane, Fill fill, RowOf row_of, ScaleOf scale_of) {
  const int rr = lane >> 1, h = lane & 1;
  const bool valid = r0 + rr < nrows;
  const int64_t orow = valid ? (int64_t)row_of(r0 + rr) : 0;
  const float sc = valid ? scale_of(r0 + rr) : 0.0f;
  const float* src = scratch + l2_scratch_index(rr, 16 * h);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    fill(half, scratch);
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 w = *reinterpret_cast<const float4*>(src + 4 * q);
      v[4 * q] = w.x;
      v[4 * q + 1] = w.y;
      v[4 * q + 2] = w.z;
      v[4 * q + 3] = w.w;
    }
    const int64_t col = col0 + 32 * half + 16 * h;
    if (p.o_f16) {
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(v[q]));
      m = fmaxf(m, pair_swap(m)) * fabsf(sc);
      const int e = f16_block_exp(m);
      const float s2 = m > 0.0f ? ldexpf(sc, -e) : 0.0f;
      if (valid) {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f16x2 hv{(_Float16)(v[2 * q] * s2), (_Float16)(v[2 * q + 1] * s2)};
          w[q] = __builtin_bit_cast(uint32_t, hv);
        }
        uint4* dst = reinterpret_cast<uint4*>(p.o_f16 + orow * p.N + col);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        if (h == 0) p.o_exp[orow * (p.N / 32) + col / 32] = (int8_t)e;
      }
    } else if (p.o_bf16) {
      if (valid) {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[2 * q] * sc)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(v[2 * q + 1] * sc)) << 16);
        uint4* dst = reinterpret_cast<uint4*>(p.o_bf16 + orow * p.N + col);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    } else if (valid) {
      float4* dst = reinterpret_cast<float4*>(p.o + orow * p.N + col);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q] = make_float4(v[4 * q] * sc, v[4 * q + 1] * sc, v[4 * q + 2] * sc, v[4 * q + 3] * sc);
    }
  }
}

// The same for the accumulators of two 32 x 32 MFMA tiles: a0 holds columns
// col0 + lane % 32 and a1 columns col0 + 32 + lane % 32, at rows
// acc_row(i, lane).
template <class RowOf, class ScaleOf>
__device__ __forceinline__ void l2_store_block(const L2Params& p, const f32x16& a0, const f32x16& a1,
                                               float* scratch, int r0, int nrows, int64_t col0, int lane,
                                               RowOf row_of, ScaleOf scale_of) {
  auto fill = [&](int half, float* sc) {
    const f32x16& a = half ? a1 : a0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[l2_scratch_index(acc_row(i, lane), lane & 31)] = a[i];
  };
  l2_store_rows(p, scratch, r0, nrows, col0, lane, fill, row_of, scale_of);
}

// Epilogue writer of the L2 / linear GEMMs for the transposed accumulators of
// one wave's 32-row x 64-column output block, computed as W_tile * A_tile^T
// (the MFMA operands swapped: the A and B fragments of the 32x32x16 MFMA
// have the same lane layout): lane l holds tile row r0 + (l & 31) and, in
// a[nt][i], its column col0 + 32 nt + 8 (i >> 2) + 4 (l >> 5) + (i & 3).  A
// row's 32-column block nt thus sits in lanes l and l + 32, 16 values each:
// its maximum takes one exchange between the lane halves, and the values
// written are those of l2_store_rows -- fp32 (o), bf16 (o_bf16), or f16 with
// one exponent per (row, 32 columns) (o_f16, o_exp).  fp32 rows go out as
// four 16 B runs per lane.  The 16-bit forms are packed in registers; four
// exchanges of packed pairs leave each lane with 16 consecutive columns
// (16 (l >> 5) .. of each block), which pass through the wave's 4 KiB of LDS
// (32 rows of 128 B, 16 B chunk c of row r at c ^ (r & 7)) so that every
// store instruction then writes 8 whole rows of 128 B (lane l: row l / 8 +
// 8 k, chunk l % 8); the two exponents of a row go out as one 16-bit store.
// Every lane of the wave must take part.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

template <class RowOf, class ScaleOf>
__device__ __forceinline__ void l2_store_rows_t(const L2Params& p, const f32x16 (&a)[2], uint4* scratch, int r0,
                                                int nrows, int64_t col0, int lane, RowOf row_of, ScaleOf scale_of) {
  const int g = lane >> 5, rl = lane & 31;
  const int r = r0 + rl;
  const bool valid = r < nrows;
  const float sc = valid ? scale_of(r) : 0.0f;
  if (!p.o_f16 && !p.o_bf16) {
    if (valid) {
      const int64_t orow = row_of(r);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& v = a[nt];
          *reinterpret_cast<float4*>(p.o + orow * p.N + col0 + 32 * nt + 8 * q + 4 * g) =
              make_float4(v[4 * q] * sc, v[4 * q + 1] * sc, v[4 * q + 2] * sc, v[4 * q + 3] * sc);
        }
    }
    return;
  }
  uint32_t ebits = 0;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const f32x16& v = a[nt];
    uint32_t w[8];
    if (p.o_f16) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      const auto mm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmaxf(__uint_as_float(mm[0]), __uint_as_float(mm[1])) * fabsf(sc);
      const int e = f16_block_exp(m);
      const float s2 = m > 0.0f ? ldexpf(sc, -e) : 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = pack_f16(v[2 * q] * s2, v[2 * q + 1] * s2);
      ebits |= (uint32_t)(uint8_t)e << (8 * nt);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = pack_bf16(v[2 * q] * sc, v[2 * q + 1] * sc);
    }
    // w[q] holds columns 8 (q >> 1) + 4 g + 2 (q & 1) +0, +1; after the
    // swaps lane half g holds columns 16 g .. 16 g + 15 as w0 w1 w4 w5 w2 w3 w6 w7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto s = __builtin_amdgcn_permlane32_swap(w[j], w[4 + j], false, false);
      w[j] = s[0];
      w[4 + j] = s[1];
    }
    const int c0 = 4 * nt + 2 * g;  // 16 B chunk of the row's 128 B
    scratch[8 * rl + (c0 ^ (rl & 7))] = make_uint4(w[0], w[1], w[4], w[5]);
    scratch[8 * rl + ((c0 + 1) ^ (rl & 7))] = make_uint4(w[2], w[3], w[6], w[7]);
  }
  if (p.o_f16 && valid && g == 0)
    *reinterpret_cast<uint16_t*>(p.o_exp + (int64_t)row_of(r) * (p.N / 32) + col0 / 32) = (uint16_t)ebits;
  // the wave's own scratch: its LDS writes above complete before these reads
  uint16_t* base = p.o_f16 ? p.o_f16 : p.o_bf16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = (lane >> 3) + 8 * k, c = lane & 7;
    const uint4 v = scratch[8 * rr + (c ^ (rr & 7))];
    if (r0 + rr < nrows) *reinterpret_cast<uint4*>(base + (int64_t)row_of(r0 + rr) * p.N + col0 + 8 * c) = v;
  }
}

}  // namespace nvfp4
