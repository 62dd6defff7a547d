// Token-grouped NVFP4 GEMMs for tiles of at most 32 rows: the decode shape of
// the MoE expert FFN, where each touched expert gets a handful of tokens and
// the GEMMs stream the experts' weights ("NVFP4 MoE Pipeline" in
// DEBUG_LOG.md; the L1 gate/up GEMM with the fused SwiGLU -> bf16 -> NVFP4
// epilogue and the L2 down GEMM with the routing-weighted epilogue are the
// same operations as in the 256-row tile kernels).
//
// MI355X design.  A 256-row tile leaves one workgroup per CU, and the weight
// bytes one CU keeps in flight are far below what HBM latency needs; with few
// rows the MFMAs are idle anyway.  Here:
//   * A workgroup of 4 waves owns 32 rows x 256 B rows (output columns); wave
//     w owns B rows 64 w .. +64 as four 16-column tiles of the 16x16x32 f16
//     MFMA (for L1: gate columns 0..15, 16..31, then the up columns 0..15,
//     16..31 of the same 32 SwiGLU columns, so SwiGLU stays within a lane),
//     and both 16-row halves of the tile: 32 fp32 accumulators per lane.
//   * Weights never touch LDS: each lane loads its 16 B pieces of nibbles
//     straight into registers one super-step (256 K) ahead, two register
//     sets, and dequantizes them to exact f16 in registers (each weight
//     once).  The 16x16x32 operand layout (lane = column l % 16, four lanes
//     per column) lets each load instruction cover 16 weight rows x 64
//     contiguous bytes: loads that touch 32 rows each (the 32x32x16 operand
//     layout) stream at ~5.2 TB/s on this part, 16-row loads at ~6.3 TB/s.
//   * K order: in a super-step, lane group g = lane / 16 holds the nibbles
//     of K [128 h + 32 g, +32) (h = 0, 1: its two loads), and MFMA step
//     (h, s) takes K [128 h + 32 g + 8 s, +8) from it.  The activations use
//     the same order.
//   * The 32 activation rows (exact f16) of a super-step go to one of two LDS
//     buffers with direct-to-LDS loads issued one super-step ahead (region j
//     of a buffer holds K [64 j, 64 j + 64)); one LDS-only barrier per
//     super-step.
//   * 32 KiB of LDS for the activations plus 18 KiB of scales, and at most
//     168 VGPRs, so three workgroups (12 waves) share a CU.
//   * Tail split.  Each XCD runs its contiguous range of items `slots` at a
//     time (resident workgroups per XCD).  When that range is a few items
//     past a whole number of rounds, those last items would run nearly
//     alone at the end of the launch; instead each of them is split along K
//     into a few pieces run by as many workgroups.  A piece writes its fp32
//     accumulators to a partial slot; the last piece of an item to arrive
//     (an atomic count) adds the item's partials in piece order and runs
//     the epilogue.  No workgroup waits for another.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "gemm_common.hpp"

namespace nvfp4 {

constexpr int kSkTileM = 32;
constexpr int kSkThreads = 256;
constexpr int kSkSteps = 4;                          // K steps of 64 per super-step
constexpr int kSkAStage = kSkTileM * (kStepK / 8);  // 16 B chunks of one A step (4 KiB)
constexpr int kSkABuf = kSkSteps * kSkAStage;       // one super-step of A (16 KiB)

// Per-workgroup operand sources (32-bit byte offsets, as in the 256-row
// kernels).  Within a super-step (256 K, or a K tail of 128), MFMA step
// (h, s) of lane group g = lane / 16 takes K [128 h + 32 g + 8 s, +8), for A
// and for B alike.
struct SkOperands {
  const uint8_t* a;     // A matrix (f16 rows of K), wave-uniform
  uint32_t a_base;      // this lane's A row (tile row 8 wave + lane / 8) + 16 c, c = (lane & 7) ^ key(row)
  const uint8_t* bq;    // B nibbles of the tile's expert, wave-uniform
  const uint8_t* bsf;   // B scales of the tile's expert, wave-uniform
  uint32_t bq_row;      // byte offset of this lane's nibbles in column tile 0: tile row 64 wave + lane % 16, + 16 (lane / 16)
  uint32_t bq_step[4];  // wave-uniform: from it to column tile ct (tile rows 64 wave + 16 ct + lane % 16)
  uint32_t sf_dma;      // scale-row offset of the tile row 64 wave + lane / 4 (row-paired: of its pair's
                        // line half)
  uint32_t sf_step[4];  // wave-uniform: from it to the scale rows of the tile rows 64 wave + 16 i + lane / 4
  uint32_t sf_ss0;      // wave-uniform: the first super-step of the piece (its scales' column offset)
  bool sf_pair;         // wave-uniform: the scales are in the row-paired layout
  bool a_rows;          // wave-uniform: this wave's 8 A rows include a valid one
};

// The nibbles of one super-step in a lane: for each column tile ct, the
// 16 B of K [128 h + 32 g, +32) (h = 0, 1; a K tail of 128 has h = 0 only).
struct SkB {
  uint4 q[4][2];
};

// Scales in LDS.  Every 256 K (one super-step) a weight row has 16 scale
// bytes.  The scales of four whole super-steps (a macro-step: 64 B per row,
// 16 KiB per tile) are brought in with one direct load per lane and wave for
// each quarter of the rows, 4 lanes per row, so each scale line is fetched by
// loads issued together.  Row tr keeps its 16 B chunk c (super-step c of the
// macro-step) at position c ^ ((tr >> 2) & 3), which spreads the 32 rows one
// read instruction touches over distinct banks.  The 8 scale bytes of a K
// tail of 128 go to a separate 2 KiB area (row tr at bytes 8 tr).
constexpr int kSkSfMacro = kTileN * 64;  // bytes
constexpr int kSkSfTail = kTileN * 8;
__device__ __forceinline__ int sk_sf_swz(int tr) { return (tr >> 2) & 3; }

// Steps of super-step ss (nfull whole super-steps, then a tail of 2 steps if
// the K steps are not a multiple of 4).
__device__ __forceinline__ int sk_steps(int ss, int nfull) { return ss < nfull ? kSkSteps : 2; }

// Direct loads of A for super-step ss into buf: region j holds K [64 j,
// 64 j + 64) of the 32 rows (128 B each, 16 B chunk c at c ^ key(row)); wave
// w fetches rows 8 w .. 8 w + 7 (1 KiB per region).  A tail super-step (m =
// 2 steps) loads its two regions twice (the second copy is not read).  A wave
// whose rows are all past the tile's valid rows loads nothing: those rows of
// the buffer keep stale values, which reach only accumulator rows that are
// never stored (an MFMA output row depends on its own A row alone).
__device__ __forceinline__ void sk_load_a(f16x8* buf, const SkOperands& op, int ss, int m, int wave) {
  if (!op.a_rows) return;
  const uint8_t* base = op.a + (size_t)ss * (kSkSteps * kStepK * 2);
#pragma unroll
  for (int j = 0; j < kSkSteps; ++j)
    dma16s(buf + j * kSkAStage + wave * 64, base, op.a_base + 128u * (uint32_t)(j & (m - 1)));
}

// Nibbles of super-step ss: per column tile, the 16 B of K [128 h + 32 g,
// +32) for h = 0, 1 (h = 0 only in a tail super-step): each load covers 16
// weight rows x 64 contiguous bytes.
__device__ __forceinline__ SkB sk_load_b(const SkOperands& op, int ss, int m) {
  SkB b;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    // a wave-uniform base plus a 32-bit lane offset: the scalar-base form of
    // the load, no 64-bit address per lane
    const uint8_t* base = op.bq + (size_t)ss * (kSkSteps * kStepK / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b.q[ct][h] = *reinterpret_cast<const uint4*>(base + (op.bq_row + op.bq_step[ct] + 64u * (uint32_t)(h & (m >> 2))));
  }
  return b;
}

// Direct loads of the scales of macro-step mac (super-steps 4 mac .. 4 mac
// + 3 of the piece; chunks past the last whole super-step re-read it and are
// not used).  Super-step j's 16 B of a row sit at 16 j in the plain layout,
// and at 128 (j / 4) + 16 (j % 4) past the row's half of its pair's lines in
// the row-paired one (then every line a load touches is used whole).
__device__ __forceinline__ void sk_load_sf_macro(uint8_t* sfbuf, const SkOperands& op, int mac, int nfull,
                                                 int wave, int lane) {
  // the lane writes position lane & 3 of its rows tr = 64 wave + 16 i +
  // lane / 4, which holds chunk (lane & 3) ^ sk_sf_swz(tr) = (lane & 3) ^
  // ((lane >> 4) & 3); recomputed here rather than held across the K loop
  int l = lane;
  asm volatile("" : "+v"(l));
  const int sf_c = (l & 3) ^ ((l >> 4) & 3);
  const uint32_t j = op.sf_ss0 + (uint32_t)min(4 * mac + sf_c, nfull - 1);
  const uint32_t off = op.sf_dma + (op.sf_pair ? 128u * (j >> 2) + 16u * (j & 3) : 16u * j);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dma16s(reinterpret_cast<f16x8*>(sfbuf + 1024 * (4 * wave + i)), op.bsf + op.sf_step[i], off);
}

// Direct loads of the 8 tail scale bytes of every tile row (dword d of the
// area holds half d & 1 of row d >> 1); row_of maps a tile row to its scale
// row offset (plain layout: a K with a tail is never row-paired).
template <class RowOf>
__device__ __forceinline__ void sk_load_sf_tail(uint8_t* sftail, const SkOperands& op, int nfull, int wave,
                                                int lane, RowOf row_of) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = 256 * i + 64 * wave + lane;
    dma4(reinterpret_cast<uint32_t*>(sftail + 1024 * i + 256 * wave),
         op.bsf + row_of(d >> 1) + 16 * (op.sf_ss0 + nfull) + 4 * (d & 1));
  }
}

// This lane's block-scale pairs of super-step ss for its four column tiles:
// s[ct][h] holds, in its low 16 bits, the scales of the 16-K blocks 8 h + 2 g
// and 8 h + 2 g + 1 (those of MFMA steps (h, 0..1) and (h, 2..3)).  The
// rows tr = 64 wave + 16 ct + lane % 16 of the four column tiles share
// sk_sf_swz(tr) = (lane % 16) / 4 & 3, so one lane address and immediate
// offsets (1024 B, resp. 128 B of the tail area, per column tile) reach all
// four.
__device__ __forceinline__ void sk_read_sf(const uint8_t* sfbuf, const uint8_t* sftail, int ss, int nfull,
                                           int wave, int lane, uint32_t (&s)[4][2]) {
  const int g = lane >> 4, sh = 16 * (g & 1), r = lane & 15;
  if (ss < nfull) {
    const uint8_t* const p = sfbuf + 64 * (64 * wave + r) + 16 * ((ss & 3) ^ ((r >> 2) & 3));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 1024 * ct);
      s[ct][0] = word_of(v, g >> 1) >> sh;
      s[ct][1] = word_of(v, 2 + (g >> 1)) >> sh;
    }
  } else {
    const uint8_t* const p = sftail + 8 * (64 * wave + r) + 4 * (g >> 1);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      s[ct][0] = *reinterpret_cast<const uint32_t*>(p + 128 * ct) >> sh;
      s[ct][1] = 0;
    }
  }
}

// The MFMAs of K half h of a super-step (4 steps of 32) from A buffer buf,
// nibbles W and scale pairs sw; ra[s] is this lane's A chunk of step (h = 0,
// s) in row group 0 (row group 1: ra[s ^ 2] + 128, since key(r + 16) =
// key(r) ^ 2 for r < 16).
__device__ __forceinline__ void sk_half(const f16x8* buf, const int (&ra)[4], const SkB& W,
                                        const uint32_t (&sw)[4][2], int h, f32x4 (&acc)[2][4]) {
  f16x2 lo[4], hi[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[ct][h], 1.0f, false);
    lo[ct] = f16x2{sc[0], sc[0]};
    hi[ct] = f16x2{sc[1], sc[1]};
  }
  const int off = 2 * h * kSkAStage;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x8 a0 = buf[ra[s] + off];
    const f16x8 a1 = buf[ra[s ^ 2] + off + 128];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f16x8 b = dequant8(word_of(W.q[ct][h], s), s < 2 ? lo[ct] : hi[ct]);
      acc[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b, acc[0][ct], 0, 0, 0);
      acc[1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b, acc[1][ct], 0, 0, 0);
    }
  }
  SCHED_FENCE();  // keeps each half's fragments from being hoisted into the previous one
}

struct SkLds {
  f16x8* a;        // two A buffers of one super-step
  uint8_t* sf;     // scales of one macro-step
  uint8_t* sftail; // scales of the K tail
};

// Super-step ss on A buffer BUF and register set W[BUF]: wait for its loads
// (issued one super-step earlier) and publish them with a barrier (which
// also tells every wave that A buffer BUF ^ 1 is no longer read), read its
// scale words; at the end of a macro-step, once every wave has read them,
// fetch the next macro-step's scales; issue the loads of super-step ss + 1
// (A first, then B, and the tail's scales with the tail; the last super-step
// issues none: a wasted super-step of loads per item, which the epilogue
// would also wait for, cost the 8-super-step L2 items 3 %), then run its
// MFMAs.
template <int BUF, class RowOf>
__device__ __forceinline__ void sk_super(const SkLds& L, const int (&ra)[4], SkB (&W)[2], const SkOperands& op,
                                         int ss, int nss, int nfull, int wave, int lane, f32x4 (&acc)[2][4],
                                         RowOf row_of) {
  wait_vmcnt<0>();
  lds_barrier();
  uint32_t sw[4][2];
  sk_read_sf(L.sf, L.sftail, ss, nfull, wave, lane, sw);
  if ((ss & 3) == 3 && ss + 1 < nfull) {
    lds_barrier();
    sk_load_sf_macro(L.sf, op, (ss + 1) >> 2, nfull, wave, lane);
  }
  if (ss + 1 < nss) {
    const int nx = ss + 1;
    const int mx = sk_steps(nx, nfull);
    sk_load_a(L.a + (BUF ^ 1) * kSkABuf, op, nx, mx, wave);
    W[BUF ^ 1] = sk_load_b(op, nx, mx);
    if (nx == nfull && nss > nfull) sk_load_sf_tail(L.sftail, op, nfull, wave, lane, row_of);
  }
  SCHED_FENCE();
  const f16x8* buf = L.a + BUF * kSkABuf;
  sk_half(buf, ra, W[BUF], sw, 0, acc);
  if (ss < nfull) sk_half(buf, ra, W[BUF], sw, 1, acc);
}

// The K loop over nk steps of 64 (nk even); ends with all loads landed and
// every wave past its last LDS read.  row_of(tr) is the byte offset of the
// scale row of tile row tr within the expert's scales.  a_base_of() gives
// this lane's A source (op.a_base), asked for once the first weight and scale
// loads are out; after_first() runs once the first loads are issued (loads
// it issues then land with them).
template <class RowOf, class ABase, class AfterFirst>
__device__ __forceinline__ void sk_mainloop(const SkLds& L, SkOperands& op, int nk, f32x4 (&acc)[2][4],
                                            RowOf row_of, ABase a_base_of, AfterFirst after_first) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int nfull = nk / kSkSteps;
  const int nss = nfull + (nk % kSkSteps ? 1 : 0);
  SkB W[2];
  // the weights first: their addresses need only the tile; the activation
  // rows' (a_base_of) also the routing permutation, whose load then
  // overlaps these
  W[0] = sk_load_b(op, 0, sk_steps(0, nfull));
  if (nfull > 0)
    sk_load_sf_macro(L.sf, op, 0, nfull, wave, lane);
  else
    sk_load_sf_tail(L.sftail, op, nfull, wave, lane, row_of);
  op.a_base = a_base_of();
  sk_load_a(L.a, op, 0, sk_steps(0, nfull), wave);
  after_first();
  // A fragment of step (0, s) for row r (group 0): K [32 g + 8 s, +8) is
  // chunk 4 (g & 1) + s of region g >> 1
  int ra[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ra[s] = (g >> 1) * kSkAStage + r * 8 + ((4 * (g & 1) + s) ^ swz_key(r));
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = f32x4{};
  for (int ss = 0; ss < nss; ss += 2) {
    sk_super<0>(L, ra, W, op, ss, nss, nfull, wave, lane, acc, row_of);
    if (ss + 1 < nss) sk_super<1>(L, ra, W, op, ss + 1, nss, nfull, wave, lane, acc, row_of);
  }
  wait_vmcnt<0>();
  lds_barrier();
}

// This lane's A source (a_base) for A row `arow` at tile row R = 8 wave +
// lane / 8.
__device__ __forceinline__ uint32_t sk_a_base(uint32_t arow, int64_t K, int lane, int R) {
  return arow * (uint32_t)(K * 2) + 16u * (uint32_t)((lane & 7) ^ swz_key(R));
}

// Weight and scale sources of this lane for a tile (a_base is set by the
// main loop); wrow(tr) gives the global weight row of tile row tr.
template <class WRow>
__device__ __forceinline__ void sk_operands(SkOperands& op, int64_t K, int wave, int lane, int nrows, bool sf_pair,
                                            WRow wrow) {
  const int b0 = wrow(64 * wave + (lane & 15));
  op.bq_row = (uint32_t)b0 * (uint32_t)(K / 2) + 16u * (uint32_t)(lane >> 4);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
    op.bq_step[ct] =
        (uint32_t)__builtin_amdgcn_readfirstlane((wrow(64 * wave + 16 * ct + (lane & 15)) - b0) * (int)(K / 2));
  // the weight rows of tile rows 64 wave + 16 i + r (r < 16) lie the same
  // number of rows after that of 64 wave + r for every r (plain order: 16 i;
  // the L1 gate/up order: 32 (i & 1) + 8 (i >> 1)), so the steps are scalars
  // row-paired scales: pair w0 / 2 starts at (w0 & ~1) K / 16 and row w0's
  // half of each line at + 64 (w0 & 1); the rows 16 i after w0 have its
  // parity, so the steps below are the same in both layouts
  const int w0 = wrow(64 * wave + (lane >> 2));
  op.sf_dma = sf_pair ? (uint32_t)(w0 & ~1) * (uint32_t)(K / 16) + 64u * (uint32_t)(w0 & 1)
                      : (uint32_t)w0 * (uint32_t)(K / 16);
  op.sf_pair = sf_pair;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    op.sf_step[i] = (uint32_t)__builtin_amdgcn_readfirstlane((wrow(64 * wave + 16 * i + (lane >> 2)) - w0) * (int)(K / 16));
  op.a_rows = __builtin_amdgcn_readfirstlane(8 * wave < nrows ? 1 : 0) != 0;
}

// ------------------------------------------------------------------ work items
constexpr int kSplitItems = skinny_split_counters() / 8;  // at most this many items per XCD are split
constexpr int kSplitPieces = 32;  // pieces (partial slots) per XCD
constexpr int kSplitMax = 4;      // pieces per item
constexpr int kSplitMinSteps = 6; // super-steps per piece, at least (shorter pieces cost more than they save)

// The split's buffers (partial null: no split).
struct SkSplit {
  f32x4* partial;  // 8 x kSplitPieces slots of 8 x kSkThreads f32x4 (32 KiB each)
  int* count;      // 8 x kSplitItems arrival counters, zero at launch
  int slots;       // workgroups resident per XCD
};

// A workgroup's work: super-steps [ss0, ss0 + nss) of item (t, nt), piece
// `piece` of `npieces` (1: the whole item, nk steps of 64 from step 0).
struct SkWork {
  GemmTile t;
  int nt;
  int nk;       // K steps of 64 of this piece
  int ss0;      // its first super-step
  int piece, npieces;
  int slot;     // partial slot of piece 0 of the item (piece p: slot + p)
  int counter;  // the item's arrival counter
};

// Items are numbered M-tile-major (item = tile * n_ntiles + nt) and dealt to
// the XCDs in contiguous ranges as in work_item: block b runs on XCD b % 8
// as its (b / 8)-th workgroup.  XCD x's n items, with R = n % slots: the
// first n - R are whole; with a split, each of the last R (R <= kSplitItems)
// becomes s = min(kSplitMax, kSplitPieces / R, nss / kSplitMinSteps) >= 2
// pieces, numbered item-major after the whole items.  False for workgroups
// without work.
__device__ __forceinline__ bool sk_work_of(const GemmTile* tiles, const int* ntiles, int64_t M, int n_ntiles,
                                           int nk, const SkSplit& sp, SkWork* w) {
  const int mtiles = tiles ? *ntiles : (int)((M + kSkTileM - 1) / kSkTileM);
  const int W = mtiles * n_ntiles;
  const int b = blockIdx.x, x = b & 7, j = b >> 3;
  const int q = W >> 3, r = W & 7;
  const int n = q + (x < r ? 1 : 0), base = x * q + min(x, r);
  const int nss = nk / kSkSteps;
  int R = 0, s = 1;
  if (sp.partial && sp.slots > 0 && nk % kSkSteps == 0) {
    R = __builtin_amdgcn_readfirstlane(n % sp.slots);
    s = (R > 0 && R <= kSplitItems) ? __builtin_amdgcn_readfirstlane(min(min(kSplitMax, kSplitPieces / R), nss / kSplitMinSteps)) : 1;
    if (s < 2) {
      R = 0;
      s = 1;
    }
  }
  const int whole = n - R;
  int item;
  w->nk = nk;
  w->ss0 = 0;
  w->piece = 0;
  w->npieces = 1;
  w->slot = 0;
  w->counter = 0;
  if (j < whole) {
    item = base + j;
  } else {
    const int k = j - whole;  // piece k % s of split item k / s
    if (k >= R * s) return false;
    // (the divisions run on the vector ALU: readfirstlane keeps these
    // workgroup-uniform values in scalar registers across the K loop)
    const int ks = __builtin_amdgcn_readfirstlane(k / s);
    item = base + whole + ks;
    w->piece = k - ks * s;
    w->npieces = s;
    w->ss0 = __builtin_amdgcn_readfirstlane(w->piece * nss / s);
    w->nk = (__builtin_amdgcn_readfirstlane((w->piece + 1) * nss / s) - w->ss0) * kSkSteps;
    w->slot = x * kSplitPieces + ks * s;
    w->counter = x * kSplitItems + ks;
  }
  const int ti = item / n_ntiles;
  w->nt = item % n_ntiles;
  if (tiles) {
    w->t = tiles[ti];
  } else {
    const int64_t r0 = (int64_t)ti * kSkTileM;
    w->t = GemmTile{0, (int)r0, (int)((M - r0) < kSkTileM ? (M - r0) : kSkTileM), 0};
  }
  return true;
}

// A piece of a split item: store its accumulators to its partial slot and
// count its arrival.  The last piece of the item to arrive (true) gets the
// sum of all pieces' partials, added in piece order (the same result
// whichever arrives last), and resets the item's counter for the next
// launch; the others (false) are done.
__device__ __forceinline__ bool sk_split_sum(const SkSplit& sp, const SkWork& w, f32x4 (&acc)[2][4], int tid,
                                             int* flag) {
  f32x4* const part = sp.partial + (size_t)w.slot * (8 * kSkThreads);
#pragma unroll
  for (int i = 0; i < 8; ++i) part[(w.piece * 8 + i) * kSkThreads + tid] = acc[i >> 2][i & 3];
  // Release: every thread's partial before the count.  The workgroup's
  // stores are ordered before thread 0's agent-scope release RMW by the
  // workgroup-scope fence and barrier (one agent-scope fence per workgroup,
  // not per thread: each costs an L2 write-back).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    int* const c = sp.count + w.counter;
    const int old = __hip_atomic_fetch_add(c, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == w.npieces - 1;
    if (last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  if (!*flag) return false;
  // acquire: thread 0's RMW, then the barrier, orders every piece's partial
  // before these loads
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x4 v = part[i * kSkThreads + tid];
    for (int pc = 1; pc < w.npieces; ++pc) v += part[(pc * 8 + i) * kSkThreads + tid];
    acc[i >> 2][i & 3] = v;
  }
  return true;
}

#define SK_LDS_DECL                                              \
  __shared__ f16x8 lds_a[2 * kSkABuf];                           \
  __shared__ __attribute__((aligned(16))) uint8_t lds_sf[kSkSfMacro]; \
  __shared__ __attribute__((aligned(16))) uint8_t lds_sft[kSkSfTail]; \
  const SkLds L{lds_a, lds_sf, lds_sft}

// ------------------------------------------------------------------ L1
__global__ __launch_bounds__(kSkThreads, 3) void l1_skinny_kernel(L1Params p, SkSplit sp) {
  SK_LDS_DECL;
  __shared__ int last_piece;
  SkWork wk;
  if (!sk_work_of(p.tiles, p.ntiles, p.M, p.n_ntiles, (int)(p.K / kStepK), sp, &wk)) return;
  const GemmTile t = wk.t;
  const int nt = wk.nt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto out_row_of = [&](int r) -> int {
    const int rr = r < t.nrows ? r : 0;
    return p.perm ? p.perm[t.row0 + rr] : t.row0 + rr;
  };
  auto wrow = [&](int tr) { return l1_weight_row(nt, tr); };
  auto sf_row = [&](int tr) { return (uint32_t)l1_weight_row(nt, tr) * (uint32_t)(p.K / 16); };
  SkOperands op;
  // a piece starts at super-step ss0: the row offsets stay, the bases move
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16) + (size_t)wk.ss0 * (kSkSteps * kStepK * 2);
  op.bq = p.w_q + (int64_t)t.expert * p.N2 * (p.K / 2) + (size_t)wk.ss0 * (kSkSteps * kStepK / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N2 * (p.K / 16);  // the piece's scales: sf_ss0
  op.sf_ss0 = (uint32_t)wk.ss0;
  // what the epilogue reads from memory, loaded as raw values beside the A
  // rows (used only there, so nothing waits for them before): the pair of
  // tile row tid, alpha's factors, the output scale -- each would otherwise
  // cost the epilogue a round trip
  int my_perm = 0;
  if (tid < kSkTileM && p.perm) my_perm = p.perm[t.row0 + (tid < t.nrows ? tid : 0)];
  const float a_gs = p.a_gs[0], w_gs = p.w_gs[t.expert];
  const float out_gs = p.c_q ? p.out_gs[0] : 1.0f;
  const int R = 8 * wave + (lane >> 3);
  const int o = out_row_of(R);  // the A row's pair, used once the weights' first loads are out
  sk_operands(op, p.K, wave, lane, t.nrows, p.sf_paired != 0, wrow);
  f32x4 acc[2][4];
  sk_mainloop(L, op, wk.nk, acc, sf_row,
              [&] { return sk_a_base(p.perm ? (uint32_t)(o / p.topk) : (uint32_t)o, p.K, lane, R); }, [] {});
  // a piece that is not its item's last runs the epilogue with no rows (an
  // early return here made the compiler spill in the K loop)
  const int nrows = (wk.npieces > 1 && !sk_split_sum(sp, wk, acc, tid, &last_piece)) ? 0 : t.nrows;

  // epilogue: SwiGLU -> bf16 tile (32 x 128) in LDS, then NVFP4 of its rows
  constexpr int kCStride = 136;
  constexpr int kCTileChunks = kSkTileM * kCStride * 2 / 16;
  static_assert(kCTileChunks + 32 + kSkTileM / 4 <= 2 * kSkABuf, "epilogue LDS");
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds_a);
  float* rtab = reinterpret_cast<float*>(lds_a + kCTileChunks);
  int* out_row = reinterpret_cast<int*>(lds_a + kCTileChunks + 32);
  if (tid < kSkTileM) out_row[tid] = p.perm ? my_perm : t.row0 + (tid < t.nrows ? tid : 0);
  const float alpha = a_gs * w_gs;
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
  const int npass = (nrows + kSkThreads / 16 - 1) / (kSkThreads / 16);
  // bf16 tile of SiLU(gate) (gate_only) or SiLU(gate) * up in LDS: column
  // tiles ct and ct + 2 (ct < 2) hold the gate and up values of SwiGLU
  // columns 32 wave + 16 ct + lane % 16, at rows 16 mt + 4 (lane / 16) + i
  auto fill_ctile = [&](bool gate_only) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gate = acc[mt][ct][i] * alpha;
          const float sg = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate));
          const float c = gate_only ? sg : sg * (acc[mt][ct + 2][i] * alpha);
          const int row = 16 * mt + 4 * (lane >> 4) + i, col = 32 * wave + 16 * ct + (lane & 15);
          ctile[row * kCStride + col] = __builtin_bit_cast(uint16_t, (__bf16)c);
        }
  };
  if (p.c_il) {
    // interleaved output: the SiLU(gate) groups first
    fill_ctile(true);
    __syncthreads();
    for (int pass = 0; pass < npass; ++pass) {
      const int qrow = pass * (kSkThreads / 16) + (tid >> 4);
      if (qrow < nrows) {
        const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
        const int64_t g8 = 16 * (int64_t)nt + hb;
        *reinterpret_cast<uint4*>(p.c_il + (int64_t)out_row[qrow] * p.N2 + 16 * g8) = w;
      }
    }
    __syncthreads();
  }
  fill_ctile(false);
  const float E2 = p.c_q ? 1.0f / out_gs : 1.0f;  // no quantization without c_q
  fill_rtab(rtab, E2, tid);
  __syncthreads();
  for (int pass = 0; pass < npass; ++pass) {
    const int qrow = pass * (kSkThreads / 16) + (tid >> 4);
    const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
    uint32_t code = 0, q = 0;
    if (p.c_q) q = quantize_half_block(w, E2, rtab, &code);  // tile-uniform branch
    if (qrow < nrows) {
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
__global__ __launch_bounds__(kSkThreads, 3) void l2_skinny_kernel(L2Params p, SkSplit sp) {
  SK_LDS_DECL;
  __shared__ int last_piece;
  SkWork wk;
  if (!sk_work_of(p.tiles, p.ntiles, p.M, p.n_ntiles, (int)(p.K / kStepK), sp, &wk)) return;
  const GemmTile t = wk.t;
  const int nt = wk.nt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto pair_of = [&](int r) -> int {
    const int rr = t.row0 + (r < t.nrows ? r : 0);
    return p.perm ? p.perm[rr] : rr;
  };
  auto wrow = [&](int tr) { return nt * kTileN + tr; };
  auto sf_row = [&](int tr) { return (uint32_t)(nt * kTileN + tr) * (uint32_t)(p.K / 16); };
  SkOperands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16) + (size_t)wk.ss0 * (kSkSteps * kStepK * 2);
  op.bq = p.w_q + (int64_t)t.expert * p.N * (p.K / 2) + (size_t)wk.ss0 * (kSkSteps * kStepK / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N * (p.K / 16);  // the piece's scales: sf_ss0
  op.sf_ss0 = (uint32_t)wk.ss0;
  const int R = 8 * wave + (lane >> 3);
  const int a_pair = pair_of(R);  // used once the weights' first loads are out
  sk_operands(op, p.K, wave, lane, t.nrows, p.sf_paired != 0, wrow);
  // what the epilogue reads from memory, loaded as raw values with the first
  // operands (used only there): the pair of tile row tid (read beside the A
  // rows), alpha's factors, and, once the first operands are on their way,
  // the pair's routing weight -- each would otherwise cost the epilogue a
  // round trip
  const int my_pair = tid < kSkTileM ? pair_of(tid) : 0;
  const float a_gs = p.a_gs[0], w_gs = p.w_gs[t.expert];
  float my_w = 1.0f;
  f32x4 acc[2][4];
  sk_mainloop(
      L, op, wk.nk, acc, sf_row, [&] { return sk_a_base((uint32_t)a_pair, p.K, lane, R); },
      [&] {
        if (tid < kSkTileM && p.row_w) my_w = p.row_w[my_pair];
      });
  // a piece that is not its item's last runs the epilogue with no rows (an
  // early return here made the compiler spill in the K loop)
  const int nrows = (wk.npieces > 1 && !sk_split_sum(sp, wk, acc, tid, &last_piece)) ? 0 : t.nrows;
  // the scales' LDS holds the output rows and their scales, the A buffers
  // each wave's 4 KiB transposition scratch
  int* out_row = reinterpret_cast<int*>(lds_sf);
  float* row_scale = reinterpret_cast<float*>(lds_sf) + kSkTileM;
  if (tid < kSkTileM) {
    const float alpha = a_gs * w_gs;
    out_row[tid] = my_pair;
    row_scale[tid] = p.row_w ? alpha * my_w : alpha;
  }
  __syncthreads();
  float* const scratch = reinterpret_cast<float*>(lds_a) + wave * 1024;
  // half h of the wave's 64 columns is column tiles 2 h, 2 h + 1
  auto fill = [&](int half, float* sc) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[l2_scratch_index(16 * mt + 4 * (lane >> 4) + i, 16 * c2 + (lane & 15))] = acc[mt][2 * half + c2][i];
  };
  l2_store_rows(p, scratch, 0, nrows, (int64_t)nt * kTileN + wave * 64, lane, fill,
                [&](int r) { return out_row[r]; },
                [&](int r) { return row_scale[r]; });
}

// ------------------------------------------------------------------ launchers
int skinny_tile_rows() { return kSkTileM; }

size_t skinny_split_bytes() { return (size_t)8 * kSplitPieces * 8 * kSkThreads * sizeof(f32x4); }

namespace {

// Workgroups of `kernel` resident per XCD on the current device (CUs / 8 x
// workgroups per CU), looked up once per device and kernel; 0 if unknown.
template <class Kernel>
int resident_per_xcd(Kernel kernel, std::atomic<int> (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kSkThreads, 0) != hipSuccess)
    return 0;
  v = std::max(0, cus / 8 * per_cu);
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

std::atomic<int> g_l1_slots[64], g_l2_slots[64];

// Blocks for W items at most: each XCD's range, plus its pieces beyond the
// items they split.
int64_t skinny_grid(int64_t W, bool split) { return 8 * ((W + 7) / 8 + (split ? kSplitPieces : 0)); }

}  // namespace

// K of whole super-steps (the scale rows then stay 16-byte aligned for the
// direct loads), or a single tail super-step of 128.
bool skinny_supports_k(int64_t K) { return K > 0 && (K % (kSkSteps * kStepK) == 0 || K == 2 * kStepK); }

hipError_t launch_l1_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                            uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                            const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                            const int* perm, int topk, hipStream_t s, uint16_t* c_il, const uint8_t* a_q,
                            const uint8_t* a_sf, float* split_ws, int* split_cnt, bool sf_paired) {
  (void)a_q;
  (void)a_sf;
  if (!a_f16) return hipErrorInvalidValue;  // the 32-row tiles take f16 activations only
  if (sf_paired && K % 1024 != 0) return hipErrorInvalidValue;
  L1Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf, c_f16, c_il,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN)};
  p.sf_paired = sf_paired ? 1 : 0;
  const int64_t W = (int64_t)max_tiles * p.n_ntiles;
  if (W == 0) return hipSuccess;
  if (!skinny_supports_k(K)) return hipErrorInvalidValue;
  SkSplit sp{nullptr, nullptr, 0};
  if (split_ws && split_cnt) sp = SkSplit{reinterpret_cast<f32x4*>(split_ws), split_cnt, resident_per_xcd(l1_skinny_kernel, g_l1_slots)};
  l1_skinny_kernel<<<(unsigned)skinny_grid(W, sp.slots > 0), kSkThreads, 0, s>>>(p, sp);
  return hipGetLastError();
}

hipError_t launch_l2_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w,
                            float* o, const GemmTile* tiles, const int* ntiles, int max_tiles,
                            const int* perm, hipStream_t s, int64_t M, uint16_t* o_bf16, int* sched,
                            uint16_t* o_f16, int8_t* o_exp, float* split_ws, int* split_cnt, bool sf_paired) {
  (void)sched;  // one workgroup per item (or piece) here
  if (sf_paired && K % 1024 != 0) return hipErrorInvalidValue;
  L2Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, o_bf16, tiles, ntiles, M, perm, (int)(N / kTileN),
             nullptr, o_f16, o_exp};
  p.sf_paired = sf_paired ? 1 : 0;
  const int64_t W = (int64_t)max_tiles * p.n_ntiles;
  if (W == 0) return hipSuccess;
  if (!skinny_supports_k(K)) return hipErrorInvalidValue;
  SkSplit sp{nullptr, nullptr, 0};
  if (split_ws && split_cnt) sp = SkSplit{reinterpret_cast<f32x4*>(split_ws), split_cnt, resident_per_xcd(l2_skinny_kernel, g_l2_slots)};
  l2_skinny_kernel<<<(unsigned)skinny_grid(W, sp.slots > 0), kSkThreads, 0, s>>>(p, sp);
  return hipGetLastError();
}

}  // namespace nvfp4
