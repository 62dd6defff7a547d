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
//     instead of once per (row, N tile) here.
//   * A workgroup of 512 threads (8 wave64s, two per SIMD) owns a 256 x 256
//     output tile; wave w owns rows 128 (w >> 2) .. +128 and columns
//     64 (w & 3) .. +64 as 4 x 2 MFMA 32x32x16 f16 tiles (128 fp32
//     accumulators per lane).  The two waves of a SIMD (w, w + 4) hold
//     different row halves, and MFMAs of 32-row groups that lie wholly past
//     the tile's valid rows are skipped, so a partly filled tile (an expert's
//     last rows, a decode batch) costs MFMA time in proportion to its rows on
//     every SIMD.
//   * Workgroups are dealt to the 8 XCDs in turn; work items are assigned so
//     that each XCD takes one contiguous range of (M tile, N tile) items,
//     M-tile-major, and the N tiles of an M tile share one XCD's L2.
//   * K steps of 64.  A goes from global memory straight into LDS
//     (global_load_lds_dwordx4: 8 lanes fetch one 128 B row, so every request
//     uses whole cache lines and no VGPRs or LDS write instructions are
//     spent on it) through three stages, issued two steps ahead.  B moves
//     through registers: thread t loads half a row of nibbles and its two
//     block scales two steps ahead, dequantizes them with the gfx950 FP4 -> f16
//     and FP8 -> f16 conversions and one packed f16 multiply per pair, and
//     writes the next step's B stage (two stages).  The conversions and the A
//     loads are spread over the 8 MFMA groups of a step (scheduling fences
//     keep the order); MFMA operand fragments are read one sub-step ahead.
//   * LDS rows are 64 f16 = 8 chunks of 16 B, chunk c stored at
//     c ^ ((row ^ row >> 3) & 7), which keeps the B writes and the MFMA
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kStepK = 64;
constexpr int kGemmThreads = 512;
constexpr int kLdsOperand = kTileM * (kStepK / 8);  // 16 B chunks of one operand stage (32 KiB)
constexpr int kAStages = 3;
constexpr int kBStages = 2;
constexpr int kLdsB = kAStages * kLdsOperand;                    // first chunk of B stage 0
constexpr int kLdsChunks = (kAStages + kBStages) * kLdsOperand;  // 160 KiB

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

// Tile rows and columns of wave w: rows 128 wave_m .. +128, columns
// 64 wave_n .. +64 (waves w and w + 4 share a SIMD).
__device__ __forceinline__ int wave_m(int wave) { return wave >> 2; }
__device__ __forceinline__ int wave_n(int wave) { return wave & 3; }

// Active 32-row MFMA groups of a wave whose rows start at 128 wm in a tile
// of nrows valid rows (0..4).
__device__ __forceinline__ int active_groups(int nrows, int wm) {
  return min(4, max(0, (nrows - 128 * wm + 31) >> 5));
}

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

// ------------------------------------------------------------------ operands
// LDS during the main loop: A0 | A1 | A2 | B0 | B1, 32 KiB each, every stage
// 256 rows of 64 f16 = 8 chunks of 16 B.

// 16-byte chunk c of LDS row `row` lives at c ^ key(row), key(row) =
// (row ^ row >> 3) & 7: any 16 consecutive rows reading or writing the same
// logical chunk hit 16 distinct 16-byte bank groups (64 banks), and any 8
// consecutive rows hit 8.  key(32 m + r) for r < 32 depends only on r and on
// the parity of m, so the fragments of a wave's four A tiles (two B tiles)
// are two base pointers plus compile-time offsets.
__device__ __forceinline__ int swz_key(int row) { return (row ^ (row >> 3)) & 7; }

// This thread's B share of one K step: half a B row (32 nibbles) and its 2
// block scales.
struct BChunk {
  uint4 q;
  uint32_t s;
};

// bq / bsf: the workgroup's B nibbles and scales advanced to step kb (wave-
// uniform); bq_off / bsf_off: this thread's byte offsets (row and half).
__device__ __forceinline__ BChunk load_b(const uint8_t* bq, const uint8_t* bsf, uint32_t bq_off,
                                         uint32_t bsf_off) {
  BChunk c;
  c.q = *reinterpret_cast<const uint4*>(bq + bq_off);
  c.s = *reinterpret_cast<const uint16_t*>(bsf + bsf_off);
  return c;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ void scale_pairs(uint32_t bs, f16x2* s0, f16x2* s1) {
  f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs, 1.0f, false);
  *s0 = f16x2{s[0], s[0]};
  *s1 = f16x2{s[1], s[1]};
}

// Direct-to-LDS load of one 1 KiB piece of an A stage: LDS chunks
// 64 q .. 64 q + 63 (rows 8 q .. 8 q + 7), lane i writing chunk 64 q + i.
// a: the A matrix advanced to the step (wave-uniform); off: this lane's byte
// offset (row 8 q + i / 8, logical chunk (i & 7) ^ key(row)).
__device__ __forceinline__ void dma_a(f16x8* a_stage, const uint8_t* a, uint32_t off, int q) {
  __builtin_amdgcn_global_load_lds((const void*)(a + off), (lds_void*)(a_stage + q * 64), 16, 0, 0);
}

// Per-workgroup operand sources of the main loop.  Byte offsets are 32-bit:
// the A matrix and one expert's weights stay below 4 GiB.
struct Operands {
  const uint8_t* a;    // A matrix (f16 rows of K), wave-uniform
  uint32_t a_off[4];   // this lane's direct-load sources: tile rows 32 wave + 8 u + lane / 8
  const uint8_t* bq;   // B nibbles of the tile's expert, wave-uniform
  const uint8_t* bsf;  // B scales of the tile's expert, wave-uniform
  uint32_t bq_off;     // this thread's B row and half: row * K / 2 + 16 half
  uint32_t bsf_off;    // row * K / 16 + 2 half
};

struct Frags {
  f16x8 a[4], b[2];
};

// A wave's fragment pointers: the A fragment of MFMA sub-step s for rows
// wm * 128 + 32 mt + (lane & 31) of A stage st is a[s][mt & 1] + 512 (mt >> 1)
// + st * kLdsOperand; the B fragment for rows wn * 64 + 32 nt + (lane & 31) of
// B stage st is b[s][nt] + st * kLdsOperand.  Lane half g = lane >> 5 reads
// logical chunk 4 g + s (the same K permutation for A and B).
struct ReadPtrs {
  const f16x8* a[4][2];
  const f16x8* b[4][2];
};

__device__ __forceinline__ ReadPtrs read_ptrs(const f16x8* lds, int wm, int wn, int lane) {
  ReadPtrs rp;
  const int g = lane >> 5, r = lane & 31;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int ra = wm * 128 + 32 * p + r, rb = wn * 64 + 32 * p + r;
      rp.a[s][p] = lds + ra * 8 + ((4 * g + s) ^ swz_key(ra));
      rp.b[s][p] = lds + kLdsB + rb * 8 + ((4 * g + s) ^ swz_key(rb));
    }
  return rp;
}

// One K step kb on A stage KA = kb % 3 and B stage KB = kb % 2: the wave's 32
// MFMAs in 8 groups of 4 (those of row groups mt >= nmt skipped).  Between the groups the thread writes its B share of
// step kb + 1 (held in `cn`, four dequantized chunks), refills `cn` with the B
// share of step kb + 3, and issues its four direct loads of A step kb + 2
// into A stage (KA + 2) % 3.  Every step issues 6 vector-memory loads, so at
// its end at most 6 are outstanding once A of step kb + 1 (issued one step
// earlier) has landed.  Loads past the end re-read the last step; what they
// write lands in stages that are not read again.
template <int KA, int KB, bool FULL>
__device__ __forceinline__ void gemm_step(f16x8* lds, const ReadPtrs& rp, const int (&pos)[4],
                                          BChunk& cn, int kb, int last, const Operands& op,
                                          int wave, int nmt, f32x16 (&acc)[4][2]) {
  f16x8* const bw = lds + kLdsB + ((KB + 1) & 1) * kLdsOperand;
  f16x8* const aw = lds + ((KA + 2) % 3) * kLdsOperand;
  const uint8_t* const a_next = op.a + (size_t)min(kb + 2, last) * (kStepK * 2);
  const int kb3 = min(kb + 3, last);
  constexpr int aoff = KA * kLdsOperand, boff = KB * kLdsOperand;
  f16x2 s0, s1;
  scale_pairs(cn.s, &s0, &s1);
  const uint4 q = cn.q;
  // A partial wave (FULL false) reads and multiplies only its row groups
  // mt < nmt; the reads of a full wave stay unconditional, which keeps the
  // compiler's LDS wait counts exact.
  auto on = [&](int mt) { return FULL || mt < nmt; };
  Frags f[2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    if (on(mt)) f[0].a[mt] = rp.a[0][mt & 1][aoff + 512 * (mt >> 1)];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
    if (on(0)) f[0].b[nt] = rp.b[0][nt][boff];
  SCHED_FENCE();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const Frags& F = f[s & 1];
    Frags& G = f[(s + 1) & 1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (s < 3) {
        if (h == 0) {
          if (on(0)) G.a[0] = rp.a[s + 1][0][aoff];
          if (on(1)) G.a[1] = rp.a[s + 1][1][aoff];
          if (on(2)) G.a[2] = rp.a[s + 1][0][aoff + 512];
        } else {
          if (on(3)) G.a[3] = rp.a[s + 1][1][aoff + 512];
          if (on(0)) G.b[0] = rp.b[s + 1][0][boff];
          if (on(0)) G.b[1] = rp.b[s + 1][1][boff];
        }
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int mt = 2 * h + mi;
        if (on(mt)) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[mt], F.b[nt], acc[mt][nt], 0, 0, 0);
        }
      }
      const int slot = 2 * s + h;
      if (slot < 4) bw[pos[slot]] = dequant8(word_of(q, slot), (slot < 2) ? s0 : s1);
      if (slot == 3) cn = load_b(op.bq + (size_t)kb3 * 32, op.bsf + (size_t)kb3 * 4, op.bq_off, op.bsf_off);
      if (slot >= 4) dma_a(aw, a_next, op.a_off[slot - 4], 4 * wave + slot - 4);
      SCHED_FENCE();
    }
  }
  wait_vmcnt<6>();
  lds_barrier();
}

// All nk steps, A stage period 3 and B stage period 2: whole groups of 6,
// then the remaining 0..5 steps.  Both instantiations pass the same barriers.
template <bool FULL>
__device__ __forceinline__ void gemm_steps(f16x8* lds, const ReadPtrs& rp, const int (&pos)[4],
                                           BChunk& c0, BChunk& c1, int nk, const Operands& op,
                                           int wave, int nmt, f32x16 (&acc)[4][2]) {
  const int last = nk - 1;
  int kb = 0;
  for (; kb + 6 <= nk; kb += 6) {
    gemm_step<0, 0, FULL>(lds, rp, pos, c1, kb, last, op, wave, nmt, acc);
    gemm_step<1, 1, FULL>(lds, rp, pos, c0, kb + 1, last, op, wave, nmt, acc);
    gemm_step<2, 0, FULL>(lds, rp, pos, c1, kb + 2, last, op, wave, nmt, acc);
    gemm_step<0, 1, FULL>(lds, rp, pos, c0, kb + 3, last, op, wave, nmt, acc);
    gemm_step<1, 0, FULL>(lds, rp, pos, c1, kb + 4, last, op, wave, nmt, acc);
    gemm_step<2, 1, FULL>(lds, rp, pos, c0, kb + 5, last, op, wave, nmt, acc);
  }
  const int rem = nk - kb;
  if (rem > 0) gemm_step<0, 0, FULL>(lds, rp, pos, c1, kb, last, op, wave, nmt, acc);
  if (rem > 1) gemm_step<1, 1, FULL>(lds, rp, pos, c0, kb + 1, last, op, wave, nmt, acc);
  if (rem > 2) gemm_step<2, 0, FULL>(lds, rp, pos, c1, kb + 2, last, op, wave, nmt, acc);
  if (rem > 3) gemm_step<0, 1, FULL>(lds, rp, pos, c0, kb + 3, last, op, wave, nmt, acc);
  if (rem > 4) gemm_step<1, 0, FULL>(lds, rp, pos, c1, kb + 4, last, op, wave, nmt, acc);
}

// The whole K loop over nk steps of 64 (operand sources in `op`; the thread
// moves half `half` of B row tid / 2; the tile has nrows valid rows).  B register set c[j & 1] holds step j's
// share from two steps before it is written.  Ends with every load landed and
// all waves past the last LDS read, so the caller may reuse the LDS.
__device__ __forceinline__ void gemm_mainloop(f16x8* lds, const Operands& op, int nk, int nrows,
                                              f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave_m(wave), wn = wave_n(wave);
  const int nmt = __builtin_amdgcn_readfirstlane(active_groups(nrows, wm));  // tile-uniform
  const int row = tid >> 1, half = tid & 1;
  const int last = nk - 1;
  int pos[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pos[k] = row * 8 + ((4 * half + k) ^ swz_key(row));
  const int k1 = min(1, last), k2 = min(2, last);
#pragma unroll
  for (int u = 0; u < 4; ++u) dma_a(lds, op.a, op.a_off[u], 4 * wave + u);
#pragma unroll
  for (int u = 0; u < 4; ++u) dma_a(lds + kLdsOperand, op.a + (size_t)k1 * (kStepK * 2), op.a_off[u], 4 * wave + u);
  BChunk c0 = load_b(op.bq, op.bsf, op.bq_off, op.bsf_off);
  BChunk c1 = load_b(op.bq + (size_t)k1 * 32, op.bsf + (size_t)k1 * 4, op.bq_off, op.bsf_off);
  {
    f16x2 s0, s1;
    scale_pairs(c0.s, &s0, &s1);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds[kLdsB + pos[j]] = dequant8(word_of(c0.q, j), (j < 2) ? s0 : s1);
  }
  c0 = load_b(op.bq + (size_t)k2 * 32, op.bsf + (size_t)k2 * 4, op.bq_off, op.bsf_off);
  const ReadPtrs rp = read_ptrs(lds, wm, wn, lane);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
  wait_vmcnt<4>();  // A of steps 0 and 1 landed (only the two B refills may be outstanding)
  lds_barrier();
  if (nmt == 4)
    gemm_steps<true>(lds, rp, pos, c0, c1, nk, op, wave, nmt, acc);
  else
    gemm_steps<false>(lds, rp, pos, c0, c1, nk, op, wave, nmt, acc);
  wait_vmcnt<0>();
  lds_barrier();
}

// Accumulator element i of MFMA tile (mt, nt) for this lane sits at row
// 8*(i/4) + 4*(lane/32) + i%4 and column lane%32 of that 32 x 32 tile.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Tile and N tile of this workgroup: tiles come from the routing (tiles,
// *ntiles), or without routing are the ceil(M / 256) row blocks of M rows
// (expert 0).  False for workgroups without work.
__device__ __forceinline__ bool tile_of(const GemmTile* tiles, const int* ntiles, int64_t M,
                                        int n_ntiles, GemmTile* t, int* nt) {
  const int mtiles = tiles ? *ntiles : (int)((M + kTileM - 1) / kTileM);
  int item;
  if (!work_item(mtiles * n_ntiles, &item)) return false;
  const int ti = item / n_ntiles;
  *nt = item % n_ntiles;
  if (tiles) {
    *t = tiles[ti];
    return true;
  }
  const int64_t r0 = (int64_t)ti * kTileM;
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
  __shared__ f16x8 lds[kLdsChunks];

  GemmTile t;
  int nt;
  if (!tile_of(p.tiles, p.ntiles, p.M, p.n_ntiles, &t, &nt)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Output row (pair id, or activation row without routing) and activation
  // row of tile row r; padding rows repeat the tile's first row and their
  // outputs are never stored.
  auto out_row_of = [&](int r) -> int {
    const int rr = r < t.nrows ? r : 0;
    return p.perm ? p.perm[t.row0 + rr] : t.row0 + rr;
  };
  Operands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int R = 32 * wave + 8 * u + (lane >> 3);
    const int o = out_row_of(R);
    const uint32_t arow = p.perm ? (uint32_t)(o / p.topk) : (uint32_t)o;
    op.a_off[u] = arow * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
  }
  const int row = tid >> 1;
  op.bq = p.w_q + (int64_t)t.expert * p.N2 * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N2 * (p.K / 16);
  op.bq_off = (uint32_t)l1_weight_row(nt, row) * (uint32_t)(p.K / 2) + 16u * (tid & 1);
  op.bsf_off = (uint32_t)l1_weight_row(nt, row) * (uint32_t)(p.K / 16) + 2u * (tid & 1);

  f32x16 acc[4][2];
  gemm_mainloop(lds, op, (int)(p.K / kStepK), t.nrows, acc);

  // The LDS now holds the epilogue's arrays: the bf16 SwiGLU tile, the
  // reciprocal table and the output row of every tile row.
  constexpr int kCStride = 136;  // bf16 per LDS row (128 + 8 padding)
  constexpr int kCTileChunks = kTileM * kCStride * 2 / 16;
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds);
  float* rtab = reinterpret_cast<float*>(lds + kCTileChunks);
  int* out_row = reinterpret_cast<int*>(lds + kCTileChunks + 32);
  if (tid < kTileM) out_row[tid] = out_row_of(tid);
  // ---- epilogue: alpha, SwiGLU, bf16 tile in LDS
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int wm = wave_m(wave), wn = wave_n(wave);
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
  __shared__ f16x8 lds[kLdsChunks];
  GemmTile t;
  int nt;
  if (!tile_of(p.tiles, p.ntiles, 0, p.n_ntiles, &t, &nt)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // pair id of tile row r (padding rows repeat the first row, never stored)
  auto pair_of = [&](int r) -> int { return p.perm[t.row0 + (r < t.nrows ? r : 0)]; };
  Operands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int R = 32 * wave + 8 * u + (lane >> 3);
    op.a_off[u] = (uint32_t)pair_of(R) * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
  }
  const int row = tid >> 1;
  const uint32_t brow = (uint32_t)(nt * kTileN + row);
  op.bq = p.w_q + (int64_t)t.expert * p.N * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N * (p.K / 16);
  op.bq_off = brow * (uint32_t)(p.K / 2) + 16u * (tid & 1);
  op.bsf_off = brow * (uint32_t)(p.K / 16) + 2u * (tid & 1);
  f32x16 acc[4][2];
  gemm_mainloop(lds, op, (int)(p.K / kStepK), t.nrows, acc);
  int* out_row = reinterpret_cast<int*>(lds);
  if (tid < kTileM) out_row[tid] = pair_of(tid);
  __syncthreads();
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int wm = wave_m(wave), wn = wave_n(wave);
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
