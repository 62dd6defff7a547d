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
//   * K steps of 64.  A (f16), the raw B nibbles and their block scales go
//     from global memory straight into LDS (global_load_lds: no VGPRs or LDS
//     write instructions are spent on them), each load addressed as a
//     wave-uniform base plus a 32-bit lane offset: A (8 lanes per 128 B row:
//     whole cache lines) two steps ahead into three A stages, B two steps at
//     a time (4 lanes per 64 B row: half a line, where one step's 32 B
//     would use a quarter) about three steps ahead into three two-step B
//     stages, and the scales four steps at a time (4 lanes per row's 16 B,
//     where one step's 4 B took a line request of its own) into two
//     four-step scale stages.  The loads are bound by L2-to-L1 line requests
//     more than by bytes: with B and scales in single steps these two took
//     two thirds of all requests for a fifth of the bytes.  Their completion is
//     waited for with explicit load counts before the one LDS-only barrier
//     per step.  Each wave reads the raw nibbles and scales of its columns
//     from LDS and dequantizes them in registers with the gfx950 FP4 -> f16
//     and FP8 -> f16 conversions and one packed f16 multiply per pair; the
//     conversions, the A fragment reads and the direct loads are spread over
//     the 8 MFMA groups of a step (scheduling fences keep the order), and
//     operand fragments are read one sub-step ahead.
//   * LDS rows of A are 64 f16 = 8 chunks of 16 B, chunk c stored at
//     c ^ ((row ^ row >> 3) & 7); the 4 chunks of a two-step raw B row are
//     permuted with (row >> 2) & 3.  Both keep the 16-lane groups of the
//     fragment reads on distinct banks.
//   * The K order inside a 64-chunk is permuted identically for A and B (lane
//     half g reads physical chunk 4g + s at MFMA step s).
//   * L1: the 256 B rows of a tile are the gate/up rows of 128 compact SwiGLU
//     columns, ordered in LDS so that gate_j and up_j land in the same lane
//     and accumulator register; the epilogue writes the bf16 SwiGLU tile to
//     LDS, quantizes it with lane pairs (one 16-element block per pair), and
//     writes the NVFP4 bytes plus the exact f16 of the quantized values (the
//     L2 operand).
//   * L2: persistent (one workgroup per CU claiming items per XCD), with
//     the next item's first loads issued before the current item's epilogue;
//     the epilogue transposes each wave's block through LDS and writes whole
//     row segments (l2_store_block).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "gemm_common.hpp"

namespace nvfp4 {

constexpr int kTileM = 256;
constexpr int kGemmThreads = 512;
constexpr int kLdsOperand = kTileM * (kStepK / 8);  // 16 B chunks of one operand stage (32 KiB)
constexpr int kAStages = 3;     // f16 A stages
constexpr int kAStagesRaw = 4;  // A room of the NVFP4-A path (2 f16 stages + 4 raw stages)
constexpr int kBStages = 3;     // single-step B and scale stages of the NVFP4-A path
constexpr int kBRaw = kTileN * (kStepK / 2) / 16;              // 16 B chunks of raw B per stage (8 KiB)
constexpr int kBScale = kTileN * (kStepK / 16) / 16;           // 16 B chunks of B scales per stage (1 KiB)
constexpr int kBPair = 2 * kBRaw;  // 16 B chunks of a two-step B stage of the f16-A path (16 KiB)
constexpr int kBPairStages = 3;
constexpr int kSQuad = kTileN * 4;  // dwords of a four-step scale stage of the f16-A path (4 KiB)

// The main loop's LDS: three arrays (A stages, raw B stages, scale stages),
// so that the compiler can tell the A fragment reads and the raw B reads
// apart from the direct loads still in flight into the other arrays.
struct Lds {
  f16x8* a;     // kAStages (ARAW: kAStagesRaw) x kLdsOperand chunks (also the epilogue's arrays)
  f16x8* b;     // kBPairStages x kBPair chunks (ARAW: kBStages x kBRaw)
  uint32_t* s;  // 2 x kSQuad words (ARAW: kBStages x kBScale x 4)
};

// Tile rows and columns of wave w: rows 128 wave_m .. +128, columns
// 64 wave_n .. +64 (waves w and w + 4 share a SIMD).
__device__ __forceinline__ int wave_m(int wave) { return wave >> 2; }
__device__ __forceinline__ int wave_n(int wave) { return wave & 3; }

// Active 32-row MFMA groups of a wave whose rows start at 128 wm in a tile
// of nrows valid rows (0..4).
__device__ __forceinline__ int active_groups(int nrows, int wm) {
  return min(4, max(0, (nrows - 128 * wm + 31) >> 5));
}

// ------------------------------------------------------------------ operands
// LDS during the main loop (f16 A): A0 .. A2 (32 KiB each: 256 rows of 64
// f16 = 8 chunks of 16 B) | B0 .. B2 (16 KiB each, two K steps: 256 rows of
// 2 x 64 raw nibbles = 4 chunks, logical chunk 2 s + h (step s of the two,
// K half h) of row r at physical chunk (2 s + h) ^ ((r >> 2) & 3), which
// keeps the 16-lane groups of the fragment reads on distinct banks) |
// S0, S1 (4 KiB each, four K steps: row r's 4 block-scale bytes of step s
// at dword 4 r + s).  152 KiB.

// With NVFP4 activations (ARAW) the A operand arrives as nibbles and block
// scales instead of f16: A0, A1 are the f16 stages, and after them four raw
// A stages of 9 KiB (512 chunks of nibbles, row r's K half h at chunk
// 2 r + h, then the 4 scale bytes of each of the 256 rows) in the room of
// two more A stages; B and the scales then keep single-step stages (8 KiB
// each: 256 rows of 2 chunks, half h of row r at chunk 2 r + (h ^ ((r >> 3)
// & 1)); 1 KiB each: the 4 scale bytes of 256 rows).  Each
// lane loads one raw A chunk per step and, during the step before the one
// that reads it, dequantizes that chunk (32 values) into the step's f16
// stage.
constexpr int kRawChunks = kTileM * 2 + kTileM / 4;  // 576 chunks of 16 B = 9 KiB

__device__ __forceinline__ f16x8* raw_nib(const f16x8* a, int st) {
  return const_cast<f16x8*>(a) + 2 * kLdsOperand + st * kRawChunks;
}
__device__ __forceinline__ uint32_t* raw_sf(const f16x8* a, int st) {
  return reinterpret_cast<uint32_t*>(raw_nib(a, st) + 2 * kTileM);
}

// Per-workgroup operand sources of the main loop.  Byte offsets are 32-bit:
// the A matrix and one expert's weights stay below 4 GiB.
struct Operands {
  const uint8_t* a;     // A matrix (f16 rows of K), wave-uniform
  uint32_t a_off[4];    // this lane's A sources: tile rows 32 wave + 8 u + lane / 8
  const uint8_t* aq;    // ARAW: A nibbles (rows of K / 2 bytes), wave-uniform
  uint32_t aq_off;      // its source: tile row 32 wave + lane / 2, K half lane & 1
  const uint8_t* asf;   // ARAW: A block scales (rows of K / 16 bytes), wave-uniform
  uint32_t asf_off;     // its scale source: tile row 64 (wave % 4) + lane
  const uint8_t* bq;    // B nibbles of the tile's expert, wave-uniform
  uint32_t bq_off;      // ARAW: this lane's B source: tile row 32 wave + lane / 2, half (lane ^ lane >> 4) & 1
  const uint8_t* bsf;   // B scales of the tile's expert, wave-uniform
  uint32_t bsf_off;     // ARAW: this lane's scale source: tile row 64 (wave % 4) + lane
  uint32_t bq_row[2];   // f16-A path: byte offsets of the B rows 32 wave + 16 u + lane / 4
  uint32_t bq_lc;       // 16 x the logical chunk this lane loads: (lane & 3) ^ ((lane >> 4) & 3)
  uint32_t bq_lim;      // K / 2 - 16: last 16 B of a row
  uint32_t sf_lim;      // K / 16 - 4: last 4 B of a scale row
};

struct Frags {
  f16x8 a[4], b[2];
};

// A wave's A fragment pointers: the fragment of MFMA sub-step s for rows
// wm * 128 + 32 mt + (lane & 31) of A stage st is a[s][mt & 1] + 512 (mt >> 1)
// + st * kLdsOperand.  Lane half g = lane >> 5 reads logical chunk 4 g + s
// (B uses the same K permutation).
struct ReadPtrs {
  const f16x8* a[4][2];
  const f16x8* b;     // ARAW: this lane's raw B chunk of column tile 0 in B stage 0 (tile 1: + 64,
                      // rows 32 apart keep the same swizzle bit)
  const uint32_t* s;  // ARAW: its scale word of column tile 0 in scale stage 0 (tile 1: + 32)
  const f16x8* bp[2];  // f16-A path: the raw B chunk of step parity s' in two-step stage 0 (tile 1: + 128)
  const uint32_t* sq;  // f16-A path: its scale words of four-step scale stage 0 (step j: + j % 4; tile 1: + 128)
};

__device__ __forceinline__ ReadPtrs read_ptrs(const Lds& L, int wm, int wn, int lane) {
  ReadPtrs rp;
  const int g = lane >> 5, r = lane & 31;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int ra = wm * 128 + 32 * p + r;
      rp.a[s][p] = L.a + ra * 8 + ((4 * g + s) ^ swz_key(ra));
    }
  rp.b = L.b + 2 * (wn * 64 + r) + (g ^ ((r >> 3) & 1));
  rp.s = L.s + wn * 64 + r;
  const int key4 = (r >> 2) & 3;
  rp.bp[0] = L.b + 4 * (wn * 64 + r) + (g ^ key4);
  rp.bp[1] = L.b + 4 * (wn * 64 + r) + ((2 + g) ^ key4);
  rp.sq = L.s + 4 * (wn * 64 + r);
  return rp;
}

// One K step kb on A stage KA (f16 A: kb % 3; ARAW: kb % 4); bs = kb % 3 is
// the single-step B / scale stage holding step kb (ARAW only), and the
// register sets R, S alternate with KB = kb % 2.
// The wave's 32 MFMAs run in 8 groups of 4 (those of row groups mt >= nmt
// skipped); ahead of each group it reads the next A fragments from LDS and
// dequantizes the next B fragments in registers, the last group preparing the
// B fragments of sub-step 0 of step kb + 1 (bf).  Between the groups it reads
// the raw B and the scales of step kb + 1 into R[KB ^ 1], S[KB ^ 1], then
// issues, in this order, the direct loads of B, of scales and of A step
// kb + 2 into A stage (KA + 2) % 3.  f16 A: B goes two steps at a time,
// each step one half of the rows of a two-step stage (16 rows per load): in
// step kb the rows 16 (KB ^ 1) .. of each wave's 32 for the steps 2P,
// 2P + 1, P = (kb + 5) / 2, into two-step stage P % 3 (the one of steps
// kb - 1, kb or kb, kb - 1, read by step kb - 1 at the latest).  The scales
// go four steps at a time, half of the rows per load, in the steps
// kb % 4 == 3 and 0 (see there).  A wave issues 5 or 6 loads per step, and
// everything that step kb + 1 reads (A of step kb + 1, B and scales of step
// kb + 2) was issued before step kb, so waiting at the end of step kb until
// at most 5 are outstanding (the loads retire in order) is enough.  Loads
// past the end re-read the last step (the last pair or group), and a lane's
// bytes past the end of a row (a step count that is not a multiple of 2 or
// 4) re-read the row's last ones; what they write is never read.  ARAW: B
// and the scales of step kb + 3 (waves 4 KB .. 4 KB + 3, a quarter of the
// rows each) one step at a time into stage bs, A step kb + 3 as raw nibbles
// and scales, 3 loads per step (see the end of the step).
// ARAW: dequantize word j (0..3: 8 values) of this lane's raw A chunk in raw
// stage st (row tid / 2, K half tid & 1; block scale 2 (tid & 1) + j / 2)
// into its 16 B chunk of f16 stage fst.  The word and the scale byte are
// read here, so nothing stays live between the calls.
// Byte offsets (from L.a) are formed from the lane index each time: the
// caller passes a copy the compiler cannot treat as loop-invariant, so no
// per-lane addresses stay live across the K loop.
__device__ __forceinline__ void expand_a_word(const Lds& L, int st, int fst, int wave, int lane, int j) {
  const uint32_t tid = (uint32_t)(wave * 64 + lane);
  const uint32_t r = tid >> 1, h = tid & 1;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(L.a) + 2 * kLdsOperand * 16 + st * kRawChunks * 16;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(base + 16 * tid + 4 * j);
  const uint32_t code = base[2 * kTileM * 16 + 2 * tid + (j >> 1)];  // row r's scale 2 h + j / 2
  const uint32_t dst = (r * 128 + 16 * ((4 * h) ^ (uint32_t)swz_key((int)r))) ^ (16u * j);
  *reinterpret_cast<f16x8*>(reinterpret_cast<uint8_t*>(L.a) + fst * kLdsOperand * 16 + dst) =
      dequant8(w, scale_pair(code));
}

template <int KA, int KB, bool FULL, bool SWAP, bool ARAW>
__device__ __forceinline__ void gemm_step(const Lds& L, const ReadPtrs& rp, BRaw (&R)[2],
                                          BScale (&S)[2], f16x8 (&bf)[2], int kb, int bs, int last,
                                          const Operands& op, int wave, int lane, int nmt,
                                          f32x16 (&acc)[4][2]) {
  const int g = lane >> 5;
  const bool scales = (wave >> 2) == KB;  // this wave loads a quarter of the scales
  f16x8* const a_dst = L.a + (ARAW ? 0 : ((KA + 2) % 3)) * kLdsOperand + (4 * wave) * 64;
  f16x8* const b_dst = L.b + bs * kBRaw + wave * 64;
  uint32_t* const s_dst = L.s + bs * kBScale * 4 + (wave & 3) * 64;
  const int bn = (bs == 2) ? 0 : bs + 1;  // B / scale stage of step kb + 1
  // f16 A: kb % 6 from the stage periods; step kb + 1 sits in two-step
  // stage ((kb + 1) % 6) / 2 at parity (kb + 1) & 1
  constexpr int kb6 = (3 * KB + 4 * KA) % 6, n6 = (kb6 + 1) % 6;
  const f16x8* const b_next = ARAW ? rp.b + bn * kBRaw : rp.bp[n6 & 1] + (n6 >> 1) * kBPair;
  const uint32_t* const s_next =
      ARAW ? rp.s + bn * kBScale * 4 : rp.sq + (((kb + 1) >> 2) & 1) * kSQuad + ((kb + 1) & 3);
  const uint8_t* const a_src = op.a + (size_t)min(kb + 2, last) * (kStepK * 2);
  const uint8_t* const b_src = op.bq + (size_t)min(kb + 3, last) * (kStepK / 2);
  const uint8_t* const s_src = op.bsf + (size_t)min(kb + 3, last) * (kStepK / 16);
  constexpr int aoff = (ARAW ? (KA & 1) : KA) * kLdsOperand;
  // A partial wave (FULL false) reads and multiplies only its row groups
  // mt < nmt; the reads of a full wave stay unconditional, which keeps the
  // compiler's LDS wait counts exact.
  auto on = [&](int mt) { return FULL || mt < nmt; };
  ScalePairs pc;
  if (on(0)) pc = scale_pairs(S[KB], g);
  Frags f[2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    if (on(mt)) f[0].a[mt] = rp.a[0][mt & 1][aoff + 512 * (mt >> 1)];
  f[0].b[0] = bf[0];
  f[0].b[1] = bf[1];
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
        }
        if (on(0)) G.b[h] = b_frag(R[KB], pc, h, s + 1);
      } else if (on(0)) {
        const ScalePairs pn = scale_pairs(S[KB ^ 1], g);
        bf[h] = b_frag(R[KB ^ 1], pn, h, 0);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int mt = 2 * h + mi;
        if (on(mt)) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_f16(F.b[nt], F.a[mt], acc[mt][nt], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[mt], F.b[nt], acc[mt][nt], 0, 0, 0);
        }
      }
      const int slot = 2 * s + h;
      if (slot == 0) {
        if (on(0)) {  // a wave without valid rows needs no B
          R[KB ^ 1].q[0] = __builtin_bit_cast(uint4, b_next[0]);
          R[KB ^ 1].q[1] = __builtin_bit_cast(uint4, b_next[ARAW ? 64 : 128]);
          S[KB ^ 1].w[0] = s_next[0];
          S[KB ^ 1].w[1] = s_next[ARAW ? 32 : 128];
        }
        if (ARAW) {
          dma16s(b_dst, b_src, op.bq_off);
        } else {
          // half lu of the rows of the two-step stage of steps 2P, 2P + 1,
          // P = (kb + 5) / 2 (64 B of each row: half of a line)
          constexpr int lst = ((kb6 + 5) % 6) >> 1, lu = KB ^ 1;
          const int P = min((kb + 5) >> 1, last >> 1);
          const uint32_t off = op.bq_row[lu] + min((uint32_t)(64 * P) + op.bq_lc, op.bq_lim);
          dma16s(L.b + lst * kBPair + (32 * wave + 16 * lu) * 4, op.bq, off);
        }
        if (!ARAW) {
          // scales four steps at a time: group Q (steps 4Q .. 4Q + 3) into
          // four-step stage Q & 1, rows 16 u .. of each wave's 32 in step
          // 4Q - 5 + u, 16 B per row in 4 lanes (the stage of steps
          // 4Q - 8 .. 4Q - 5, read by step 4Q - 6 at the latest)
          const int k4 = kb & 3;
          if (k4 == 3 || k4 == 0) {
            const int u = k4 == 0 ? 1 : 0, Q = (kb + 5) >> 2;
            // the scale row of B row bq_row / (K / 2) starts at bq_row / 8
            const uint32_t row = u ? op.bq_row[1] : op.bq_row[0];  // a select: no indexed private array
            const uint32_t off = (row >> 3) +
                                 min((uint32_t)(16 * min(Q, last >> 2)) + 4u * (uint32_t)(lane & 3), op.sf_lim);
            dma4s(L.s + (Q & 1) * kSQuad + 4 * (32 * wave + 16 * u), op.bsf, off);
          }
        } else if (scales) {
          dma4s(s_dst, s_src, op.bsf_off);
        } else {  // the other half of the waves loads the A scales
          const int j = min(kb + 3, last);
          dma4s(raw_sf(L.a, (KA + 3) % 4) + (wave & 3) * 64, op.asf + (size_t)j * (kStepK / 16), op.asf_off);
        }
      }
      if (ARAW) {
        if (slot == 1) {
          const int j = min(kb + 3, last);
          dma16s(raw_nib(L.a, (KA + 3) % 4) + wave * 64, op.aq + (size_t)j * (kStepK / 2), op.aq_off);
        }
        if (slot >= 2 && slot < 6) {
          int lane_o = lane;
          asm volatile("" : "+v"(lane_o));
          expand_a_word(L, (KA + 1) % 4, (KA + 1) & 1, wave, lane_o, slot - 2);
        }
      } else if (slot >= 1 && slot < 5) {
        dma16s(a_dst + (slot - 1) * 64, a_src, op.a_off[slot - 1]);
      }
      SCHED_FENCE();
    }
  }
  // ARAW: 3 loads per step (B, a quarter of the B or A scales, A), so <= 3
  // outstanding means everything issued during step kb - 1 (all operands
  // of step kb + 2, needed during step kb + 1) has landed
  if (ARAW)
    wait_vmcnt<3>();
  else
    wait_vmcnt<5>();
  lds_barrier();
}

// All nk steps.  f16 A: A stage period 3 and register-set period 2, whole
// groups of 6, then the remaining 0..5 steps (the two-step B and four-step
// scale stages follow from kb itself).  ARAW: A stage period 4, groups of 4;
// bs runs through the single-step B / scale stages 0, 1, 2.
// Both instantiations (FULL) pass the same barriers.
template <bool FULL, bool SWAP, bool ARAW>
__device__ __forceinline__ void gemm_steps(const Lds& L, const ReadPtrs& rp, BRaw (&R)[2],
                                           BScale (&S)[2], f16x8 (&bf)[2], int nk,
                                           const Operands& op, int wave, int lane, int nmt,
                                           f32x16 (&acc)[4][2]) {
  const int last = nk - 1;
  int kb = 0, bs = 0;
  auto next = [](int b) { return b == 2 ? 0 : b + 1; };
  if (ARAW) {
    for (; kb + 4 <= nk; kb += 4) {
      gemm_step<0, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb, bs, last, op, wave, lane, nmt, acc);
      bs = next(bs);
      gemm_step<1, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 1, bs, last, op, wave, lane, nmt, acc);
      bs = next(bs);
      gemm_step<2, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 2, bs, last, op, wave, lane, nmt, acc);
      bs = next(bs);
      gemm_step<3, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 3, bs, last, op, wave, lane, nmt, acc);
      bs = next(bs);
    }
    const int rem = nk - kb;
    if (rem > 0) gemm_step<0, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb, bs, last, op, wave, lane, nmt, acc);
    if (rem > 1) gemm_step<1, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 1, next(bs), last, op, wave, lane, nmt, acc);
    if (rem > 2) gemm_step<2, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 2, next(next(bs)), last, op, wave, lane, nmt, acc);
    return;
  }
  // f16 A: stage period 3 (KA = kb % 3 = bs), register sets period 2
  for (; kb + 6 <= nk; kb += 6) {
    gemm_step<0, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb, 0, last, op, wave, lane, nmt, acc);
    gemm_step<1, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 1, 1, last, op, wave, lane, nmt, acc);
    gemm_step<2, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 2, 2, last, op, wave, lane, nmt, acc);
    gemm_step<0, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 3, 0, last, op, wave, lane, nmt, acc);
    gemm_step<1, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 4, 1, last, op, wave, lane, nmt, acc);
    gemm_step<2, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 5, 2, last, op, wave, lane, nmt, acc);
  }
  const int rem = nk - kb;
  if (rem > 0) gemm_step<0, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb, 0, last, op, wave, lane, nmt, acc);
  if (rem > 1) gemm_step<1, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 1, 1, last, op, wave, lane, nmt, acc);
  if (rem > 2) gemm_step<2, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 2, 2, last, op, wave, lane, nmt, acc);
  if (rem > 3) gemm_step<0, 1, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 3, 0, last, op, wave, lane, nmt, acc);
  if (rem > 4) gemm_step<1, 0, FULL, SWAP, ARAW>(L, rp, R, S, bf, kb + 4, 1, last, op, wave, lane, nmt, acc);
}

// The prologue of a tile's K loop.  f16 A: the direct loads of A steps 0, 1,
// of B steps 0..3 and the first half of the rows of steps 4, 5 (two-step
// stages 0, 1 and half of 2), and of the scales of steps 0..3 and the first
// half of the rows of steps 4..7.  ARAW: B, A and the scales of steps 0..2.  The LDS stages must be
// free (every wave past its last read of them).
template <bool ARAW = false>
__device__ __forceinline__ void gemm_prologue(const Lds& L, const Operands& op, int nk, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int last = nk - 1;
  if (!ARAW) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* a_src = op.a + (size_t)min(j, last) * (kStepK * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dma16s(L.a + j * kLdsOperand + (4 * wave + u) * 64, a_src, op.a_off[u]);
    }
  }
  if (!ARAW) {  // two-step B stages 0, 1 and the first half of stage 2
#pragma unroll
    for (int P = 0; P < 3; ++P)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (P == 2 && u == 1) break;
        const uint32_t off =
            op.bq_row[u] + min((uint32_t)(64 * min(P, last >> 1)) + op.bq_lc, op.bq_lim);
        dma16s(L.b + P * kBPair + (32 * wave + 16 * u) * 4, op.bq, off);
      }
  }
  if (!ARAW) {  // scales: four-step group 0 and the first half of group 1
#pragma unroll
    for (int Q = 0; Q < 2; ++Q)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (Q == 1 && u == 1) break;
        const uint32_t off = (op.bq_row[u] >> 3) +
                             min((uint32_t)(16 * min(Q, last >> 2)) + 4u * (uint32_t)(tid & 3), op.sf_lim);
        dma4s(L.s + Q * kSQuad + 4 * (32 * wave + 16 * u), op.bsf, off);
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int jj = min(j, last);
    if (ARAW) dma16s(L.b + j * kBRaw + wave * 64, op.bq + (size_t)jj * (kStepK / 2), op.bq_off);
    if ((wave >> 2) == (j & 1))
      dma4s(L.s + j * kBScale * 4 + (wave & 3) * 64, op.bsf + (size_t)jj * (kStepK / 16), op.bsf_off);
    else if (ARAW)
      dma4s(raw_sf(L.a, j) + (wave & 3) * 64, op.asf + (size_t)jj * (kStepK / 16), op.asf_off);
    if (ARAW) dma16s(raw_nib(L.a, j) + wave * 64, op.aq + (size_t)jj * (kStepK / 2), op.aq_off);
  }
}

// The rest of the K loop over nk steps of 64 (operand sources in `op`; the
// tile has nrows valid rows), after gemm_prologue: waits for the prologue's
// loads (and any earlier memory operation of the wave), reads the raw B and
// scales of step 0 and dequantizes its sub-step 0 fragments, then runs the
// steps.  Ends with every load landed and all waves past the last LDS read,
// so the caller may reuse the LDS.
template <bool SWAP, bool ARAW = false>
__device__ __forceinline__ void gemm_body(const Lds& L, const Operands& op, int nk, int nrows,
                                          f32x16 (&acc)[4][2], int tid) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave_m(wave), wn = wave_n(wave), g = lane >> 5;
  const int nmt = __builtin_amdgcn_readfirstlane(active_groups(nrows, wm));  // tile-uniform
  const ReadPtrs rp = read_ptrs(L, wm, wn, lane);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
  wait_vmcnt<0>();
  lds_barrier();
  if (ARAW) {  // step 0's A into f16 stage 0 (published by the barrier below)
#pragma unroll
    for (int j = 0; j < 4; ++j) expand_a_word(L, 0, 0, wave, lane, j);
  }
  BRaw R[2];
  BScale S[2];
  const f16x8* const b0 = ARAW ? rp.b : rp.bp[0];  // step 0: stage 0 (parity 0 of two-step stage 0)
  R[0].q[0] = __builtin_bit_cast(uint4, b0[0]);
  R[0].q[1] = __builtin_bit_cast(uint4, b0[ARAW ? 64 : 128]);
  const uint32_t* const s0 = ARAW ? rp.s : rp.sq;  // step 0: scale stage 0
  S[0].w[0] = s0[0];
  S[0].w[1] = s0[ARAW ? 32 : 128];
  f16x8 bf[2];
  {
    const ScalePairs p0 = scale_pairs(S[0], g);
    bf[0] = b_frag(R[0], p0, 0, 0);
    bf[1] = b_frag(R[0], p0, 1, 0);
  }
  lds_barrier();  // B and scale stage 0 are refilled during step 0
  if (nmt == 4)
    gemm_steps<true, SWAP, ARAW>(L, rp, R, S, bf, nk, op, wave, lane, nmt, acc);
  else
    gemm_steps<false, SWAP, ARAW>(L, rp, R, S, bf, nk, op, wave, lane, nmt, acc);
  wait_vmcnt<0>();
  lds_barrier();
}

// The whole K loop of one tile.
template <bool ARAW>
__device__ __forceinline__ void gemm_mainloop(const Lds& L, const Operands& op, int nk, int nrows,
                                              f32x16 (&acc)[4][2]) {
  gemm_prologue<ARAW>(L, op, nk, threadIdx.x);
  gemm_body<true, ARAW>(L, op, nk, nrows, acc, threadIdx.x);
}

// ------------------------------------------------------------------ persistent grid
// The L2 GEMM runs one workgroup per CU (a multiple of 8) over W (row tile,
// column tile) items, row-tile-major.  The XCD x = b % 8 of workgroup b owns
// the contiguous range start .. end - 1 of items that work_item would deal
// it, so the workgroups running together on one XCD work on neighbouring
// items.  With work counters (sched), the workgroups of an XCD claim its
// items one at a time in order (item = start + the counter's old value), so
// a workgroup that drew short items (an expert's last few rows) takes more
// of them; without, they take them in turn.  The next item's operand offsets
// and prologue loads are issued before the current item's epilogue, so its
// load latency, the epilogue and the absent workgroup launch overlap.
struct XcdRange {
  int start, end;
};

__device__ __forceinline__ XcdRange xcd_range(int W) {
  const int x = blockIdx.x & 7, q = W >> 3, r = W & 7;
  const int start = x * q + min(x, r);
  return {start, start + q + (x < r ? 1 : 0)};
}

// ------------------------------------------------------------------ L1
template <bool ARAW>
__global__ __launch_bounds__(kGemmThreads) void l1_gemm_swiglu_quant_kernel(L1Params p) {
  __shared__ f16x8 lds_a[(ARAW ? kAStagesRaw : kAStages) * kLdsOperand];
  __shared__ f16x8 lds_b[ARAW ? kBStages * kBRaw : kBPairStages * kBPair];
  __shared__ uint32_t lds_s[ARAW ? kBStages * kBScale * 4 : 2 * kSQuad];
  const Lds L{lds_a, lds_b, lds_s};

  GemmTile t;
  int nt;
  if (!tile_of<kTileM>(p.tiles, p.ntiles, p.M, p.n_ntiles, &t, &nt)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Output row (pair id, or activation row without routing) and activation
  // row of tile row r; padding rows repeat the tile's first row and their
  // outputs are never stored.
  auto out_row_of = [&](int r) -> int {
    const int rr = r < t.nrows ? r : 0;
    return p.perm ? p.perm[t.row0 + rr] : t.row0 + rr;
  };
  auto act_row = [&](int r) -> uint32_t {
    const int o = out_row_of(r);
    return p.perm ? (uint32_t)(o / p.topk) : (uint32_t)o;
  };
  Operands op;
  if (ARAW) {
    op.aq = p.a_q;
    op.aq_off = act_row(32 * wave + (lane >> 1)) * (uint32_t)(p.K / 2) + 16u * (lane & 1);
    op.asf = p.a_sf;
    op.asf_off = act_row(64 * (wave & 3) + lane) * (uint32_t)(p.K / 16);
  } else {
    op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int R = 32 * wave + 8 * u + (lane >> 3);
      op.a_off[u] = act_row(R) * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
    }
  }
  op.bq = p.w_q + (int64_t)t.expert * p.N2 * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N2 * (p.K / 16);
  op.bq_off = (uint32_t)l1_weight_row(nt, 32 * wave + (lane >> 1)) * (uint32_t)(p.K / 2) +
              16u * ((lane ^ (lane >> 4)) & 1);
  op.bsf_off = (uint32_t)l1_weight_row(nt, 64 * (wave & 3) + lane) * (uint32_t)(p.K / 16);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    op.bq_row[u] = (uint32_t)l1_weight_row(nt, 32 * wave + 16 * u + (lane >> 2)) * (uint32_t)(p.K / 2);
  op.bq_lc = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  op.bq_lim = (uint32_t)(p.K / 2) - 16u;
  op.sf_lim = (uint32_t)(p.K / 16) - 4u;

  f32x16 acc[4][2];
  gemm_mainloop<ARAW>(L, op, (int)(p.K / kStepK), t.nrows, acc);

  // The LDS now holds the epilogue's arrays: the bf16 SwiGLU tile, the
  // reciprocal table and the output row of every tile row.
  constexpr int kCStride = 136;  // bf16 per LDS row (128 + 8 padding)
  constexpr int kCTileChunks = kTileM * kCStride * 2 / 16;
  static_assert(kCTileChunks + 32 + kTileM / 4 <= kAStages * kLdsOperand, "epilogue LDS");
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds_a);
  float* rtab = reinterpret_cast<float*>(lds_a + kCTileChunks);
  int* out_row = reinterpret_cast<int*>(lds_a + kCTileChunks + 32);
  if (tid < kTileM) out_row[tid] = out_row_of(tid);
  // ---- epilogue: alpha, SwiGLU, bf16 tile in LDS
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int wm = wave_m(wave), wn = wave_n(wave);
  // only the row groups holding valid rows (rows past nrows are never stored)
  const int nmt = __builtin_amdgcn_readfirstlane(active_groups(t.nrows, wm));
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
  const int npass = (t.nrows + kGemmThreads / 16 - 1) / (kGemmThreads / 16);
  // bf16 tile of SiLU(gate) (gate_only) or SiLU(gate) * up in LDS.  The
  // accumulators are transposed (the MFMA computed W_tile * A_tile^T): lane l
  // holds tile row 128 wm + 32 mt + (l & 31) and, in register i of n tile 0
  // (gate) and 1 (up), compact column 32 wn + 8 (i >> 2) + 4 (l >> 5) +
  // (i & 3).  The 16 values are packed in pairs, four exchanges between the
  // lane halves make them columns 32 wn + 16 (l >> 5) .. + 15 in order, and
  // two 16 B writes store them.
  auto fill_ctile = [&](bool gate_only) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nmt) {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float c2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float gate = acc[mt][0][2 * q + h] * alpha;
            const float sg = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate));
            c2[h] = gate_only ? sg : sg * (acc[mt][1][2 * q + h] * alpha);
          }
          w[q] = pack_bf16(c2[0], c2[1]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const auto sw = __builtin_amdgcn_permlane32_swap(w[j], w[4 + j], false, false);
          w[j] = sw[0];
          w[4 + j] = sw[1];
        }
        uint4* dst = reinterpret_cast<uint4*>(ctile + (wm * 128 + mt * 32 + (lane & 31)) * kCStride +
                                              32 * wn + 16 * (lane >> 5));
        dst[0] = make_uint4(w[0], w[1], w[4], w[5]);
        dst[1] = make_uint4(w[2], w[3], w[6], w[7]);
      }
    }
  };
  if (p.c_il) {
    // interleaved output: the SiLU(gate) groups first (16 lanes per row, 8
    // columns each, 32 rows per pass)
    fill_ctile(true);
    __syncthreads();
    for (int pass = 0; pass < npass; ++pass) {
      const int qrow = pass * (kGemmThreads / 16) + (tid >> 4);
      if (qrow < t.nrows) {
        const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
        const int64_t g8 = 16 * (int64_t)nt + hb;  // group of 8 compact columns
        *reinterpret_cast<uint4*>(p.c_il + (int64_t)out_row[qrow] * p.N2 + 16 * g8) = w;
      }
    }
    __syncthreads();
  }
  fill_ctile(false);
  const float E2 = p.c_q ? 1.0f / p.out_gs[0] : 1.0f;  // no quantization without c_q
  fill_rtab(rtab, E2, tid);
  __syncthreads();

  // ---- quantize the bf16 tile: 16 lanes per row (8 blocks, two halves
  // each), 32 rows per pass, passes up to the last valid row
  for (int pass = 0; pass < npass; ++pass) {
    const int qrow = pass * (kGemmThreads / 16) + (tid >> 4);
    uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
    uint32_t code = 0, q = 0;
    if (p.c_q) q = quantize_half_block(w, E2, rtab, &code);  // tile-uniform branch
    if (qrow < t.nrows) {
      const int64_t o = out_row[qrow];
      const int64_t col0 = 128 * (int64_t)nt + 8 * hb;  // compact column of this lane's 8
      if (p.c_q) {
        reinterpret_cast<uint32_t*>(p.c_q + o * (I / 2))[col0 / 8] = q;
        if ((hb & 1) == 0) p.c_sf[o * (I / 16) + col0 / 16] = (uint8_t)code;
        if (p.c_f16) *reinterpret_cast<f16x8*>(p.c_f16 + o * I + col0) = dequant8(q, scale_pair(code));
      }
      if (p.c_bf16) *reinterpret_cast<uint4*>(p.c_bf16 + o * I + col0) = w;
      if (p.c_il) *reinterpret_cast<uint4*>(p.c_il + o * p.N2 + 2 * col0 + 8) = w;
    }
  }
}

// ------------------------------------------------------------------ L2
// Persistent (its K loop is short, so the per-item prologue, epilogue and
// workgroup launch were a large share of its time); the epilogue needs only
// the output rows and scales, which live outside the operand stages.  The
// L1 GEMM (K = H) stays one workgroup per item: in a persistent loop its
// larger epilogue state pushed the K loop into register spills.
__global__ __launch_bounds__(kGemmThreads) void l2_gemm_kernel(L2Params p) {
  __shared__ f16x8 lds_a[kAStages * kLdsOperand];
  __shared__ f16x8 lds_b[kBPairStages * kBPair];
  __shared__ uint32_t lds_s[2 * kSQuad];
  __shared__ int out_row[kTileM];
  __shared__ float out_scale[kTileM];
  const Lds L{lds_a, lds_b, lds_s};
  __shared__ int s_claim[2];
  const int tid = threadIdx.x;
  const int mtiles = p.tiles ? *p.ntiles : (int)((p.M + kTileM - 1) / kTileM);
  const XcdRange xr = xcd_range(mtiles * p.n_ntiles);
  int* const counter = p.sched ? p.sched + (blockIdx.x & 7) : nullptr;
  // the first two items of this workgroup (claimed, or in turn)
  int item, next;
  if (counter) {
    if (tid == 0) {
      s_claim[0] = xr.start + atomicAdd(counter, 1);
      s_claim[1] = xr.start + atomicAdd(counter, 1);
    }
    __syncthreads();
    item = s_claim[0];
    next = s_claim[1];
  } else {
    item = xr.start + (int)(blockIdx.x >> 3);
    next = item + (int)(gridDim.x >> 3);
  }
  if (item >= xr.end) return;
  const int nk = (int)(p.K / kStepK);

  // tile, column tile and this lane's operand sources of an item
  auto setup = [&](int it, GemmTile& t, int& nt, Operands& op, int tid_s) {
    const int lane = tid_s & 63, wave = tid_s >> 6;
    // Dense (unrouted) rows: items in groups of 4 row tiles, row tile
    // fastest inside a group, so the workgroups running together on an XCD
    // share 4 A tiles and 8 weight tiles in its L2 instead of 1 A tile and
    // 32 weight tiles (-2 % on M4096 K4096 N16384).  Routed tiles keep the
    // row-tile-major order: an expert's 2-3 row tiles already run together,
    // and grouping them measured slower.
    const int gr = p.tiles ? 1 : 4;
    const int group = it / (gr * p.n_ntiles);
    const int t0 = group * gr, gm = min(gr, mtiles - t0);
    const int within = it - group * gr * p.n_ntiles;
    const int ti = t0 + within % gm;
    nt = within / gm;
    if (p.tiles) {
      t = p.tiles[ti];
    } else {
      const int64_t r0 = (int64_t)ti * kTileM;
      t.expert = 0;
      t.row0 = (int)r0;
      t.nrows = (int)((p.M - r0) < kTileM ? (p.M - r0) : kTileM);
      t.pad = 0;
    }
    op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int R = 32 * wave + 8 * u + (lane >> 3);
      const int rr = t.row0 + (R < t.nrows ? R : 0);  // padding rows repeat the first row
      const int pr = p.perm ? p.perm[rr] : rr;
      op.a_off[u] = (uint32_t)pr * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
    }
    op.bq = p.w_q + (int64_t)t.expert * p.N * (p.K / 2);
    op.bsf = p.w_sf + (int64_t)t.expert * p.N * (p.K / 16);
    op.bq_off = (uint32_t)(nt * kTileN + 32 * wave + (lane >> 1)) * (uint32_t)(p.K / 2) +
                16u * ((lane ^ (lane >> 4)) & 1);
    op.bsf_off = (uint32_t)(nt * kTileN + 64 * (wave & 3) + lane) * (uint32_t)(p.K / 16);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      op.bq_row[u] = (uint32_t)(nt * kTileN + 32 * wave + 16 * u + (lane >> 2)) * (uint32_t)(p.K / 2);
    op.bq_lc = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    op.bq_lim = (uint32_t)(p.K / 2) - 16u;
    op.sf_lim = (uint32_t)(p.K / 16) - 4u;
  };

  GemmTile t;
  int nt;
  Operands op;
  setup(item, t, nt, op, tid);
  gemm_prologue(L, op, nk, tid);
  int tid_i = tid;
  for (;;) {
    // threadIdx.x behind an empty asm statement: the per-lane addresses
    // derived from it are recomputed per item instead of being hoisted out of
    // the loop (which would hold dozens of them across the K loop)
    asm volatile("" : "+v"(tid_i));
    const int lane_i = tid_i & 63;
    // claim the item after `next` now; its index is needed only after this
    // item's epilogue, when the loads before it have landed anyway
    int claimed = 0;
    if (counter && tid_i == 0) claimed = atomicAdd(counter, 1);
    f32x16 acc[4][2];
    gemm_body<true>(L, op, nk, t.nrows, acc, tid_i);
    if (counter && tid_i == 0) s_claim[0] = xr.start + claimed;  // published by the epilogue's barrier
    // output row (pair id) and scale alpha * routing weight of every tile row
    if (tid_i < t.nrows) {
      const int pr = p.perm ? p.perm[t.row0 + tid_i] : t.row0 + tid_i;
      const float alpha = p.a_gs[0] * p.w_gs[t.expert];
      out_row[tid_i] = pr;
      out_scale[tid_i] = p.row_w ? alpha * p.row_w[pr] : alpha;
    }
    const bool more = next < xr.end;  // workgroup-uniform
    GemmTile tn = t;
    int ntn = nt;
    if (more) {
      setup(next, tn, ntn, op, tid_i);  // op now describes the next item
      gemm_prologue(L, op, nk, tid_i);  // the stages are free: gemm_body ended with a barrier
    }
    __syncthreads();
    const int after = counter ? s_claim[0] : next + (int)(gridDim.x >> 3);
    const int wm = wave_m(tid_i >> 6), wn = wave_n(tid_i >> 6);
    const int64_t col0 = (int64_t)nt * kTileN + wn * 64;
    // A stage 3 is free here (the next item's prologue fills stages 0..2 and
    // its first step refills stage 3 only after the barrier that ends every
    // wave's epilogue): 4 KiB of it per wave for the epilogue's transposition
    uint4* const scratch = reinterpret_cast<uint4*>(lds_a + 2 * kLdsOperand) + (tid_i >> 6) * 256;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (wm * 128 + mt * 32 >= t.nrows) break;  // wave-uniform
      l2_store_rows_t(p, acc[mt], scratch, wm * 128 + mt * 32, t.nrows, col0, lane_i,
                      [&](int r) { return out_row[r]; }, [&](int r) { return out_scale[r]; });
    }
    if (!more) break;
    item = next;
    next = after;
    t = tn;
    nt = ntn;
  }
}

// ------------------------------------------------------------------ launchers
int gemm_tile_rows() { return kTileM; }

// Persistent grid for up to `items` items: one workgroup per CU of the
// current device, a multiple of 8 (the XCDs), no more than the items need.
// The CU count is queried once per device.
static unsigned persistent_grid(int64_t items) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cu_count[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  int cus = dev >= 0 ? cu_count[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    if (dev >= 0) cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  return (unsigned)std::min<int64_t>((items + 7) / 8 * 8, (int64_t)(cus / 8 * 8));
}

hipError_t launch_l1(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                     uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                     const int* perm, int topk, hipStream_t s, uint16_t* c_il, const uint8_t* a_q,
                     const uint8_t* a_sf) {
  L1Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf, c_f16, c_il,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN), a_q, a_sf};
  int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  if (a_f16)
    l1_gemm_swiglu_quant_kernel<false><<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  else if (a_q && a_sf)
    l1_gemm_swiglu_quant_kernel<true><<<(unsigned)grid, kGemmThreads, 0, s>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_l2(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                     const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w, float* o,
                     const GemmTile* tiles, const int* ntiles, int max_tiles, const int* perm,
                     hipStream_t s, int64_t M, uint16_t* o_bf16, int* sched, uint16_t* o_f16,
                     int8_t* o_exp) {
  L2Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, o_bf16, tiles, ntiles, M, perm, (int)(N / kTileN),
             sched, o_f16, o_exp};
  const int64_t items = (int64_t)max_tiles * p.n_ntiles;
  if (items == 0) return hipSuccess;
  l2_gemm_kernel<<<persistent_grid(items), kGemmThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
