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
//     w owns B rows 64 w .. +64 as two 32-column MFMA tiles (for L1: the gate
//     and the up rows of the same 32 SwiGLU columns, so SwiGLU stays within a
//     lane), 32 fp32 accumulators per lane.
//   * K advances in super-steps of 256 (four MFMA steps of 64).  The K order
//     inside a super-step is permuted identically for A and B so that lane
//     half g of a column holds the contiguous K range [128 g, 128 g + 128):
//     the two lanes of a column read one whole 128 B line of nibbles with
//     four back-to-back 16 B loads (plus 8 scale bytes), so every line of the
//     weight stream is used by loads issued together instead of by loads one
//     K step apart, which the L2 would have to keep the line for.
//   * Weights never touch LDS: each lane loads its super-step of nibbles and
//     scales straight into registers one super-step ahead (two register sets)
//     and dequantizes them to exact f16 in registers (each weight once).
//   * The 32 activation rows (exact f16) of a super-step go to one of two LDS
//     buffers with direct-to-LDS loads issued one super-step ahead; one
//     LDS-only barrier per super-step.
//   * 32 KiB of LDS and at most 168 VGPRs, so three workgroups (12 waves)
//     share a CU.
#include <hip/hip_runtime.h>

#include "gemm_common.hpp"

namespace nvfp4 {

constexpr int kSkTileM = 32;
constexpr int kSkThreads = 256;
constexpr int kSkSteps = 4;                          // K steps of 64 per super-step
constexpr int kSkAStage = kSkTileM * (kStepK / 8);  // 16 B chunks of one A step (4 KiB)
constexpr int kSkABuf = kSkSteps * kSkAStage;       // one super-step of A (16 KiB)

// Per-workgroup operand sources (32-bit byte offsets, as in the 256-row
// kernels).  A super-step of m K steps (m = 4, or m = 2 for a K tail of 128)
// starting at K step kb0 holds K chunks of 8 (physical index q within the
// super-step) as follows: MFMA step j, sub-step s, lane half g uses
// q = 4 m g + 4 j + s, for A and for B alike.
struct SkOperands {
  const uint8_t* a;     // A matrix (f16 rows of K), wave-uniform
  uint32_t a_base;      // this lane's A row (tile row 8 wave + lane / 8) + 16 (c & 3)
  uint32_t a_hi;        // 64 (c >> 2); c = (lane & 7) ^ key(row) is the logical chunk it fetches
  const uint8_t* bq;    // B nibbles of the tile's expert, wave-uniform
  const uint8_t* bsf;   // B scales of the tile's expert, wave-uniform
  uint32_t bq_row[2];   // byte offsets of this lane's column rows (tile rows 64 wave + 32 nt + lane % 32)
  uint32_t sf_dma[4];   // scale-row offsets of the tile rows 64 wave + 16 i + lane / 4 (i < 4)
  int sf_tr[4];         // those tile rows
  int g;                // lane half
};

// The nibbles of one super-step in a lane: for each column tile nt, the 16 B
// of each MFMA step j.
struct SkB {
  uint4 q[2][kSkSteps];
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

// Direct loads of A for super-step ss into buf: step j's 32 rows x 128 B;
// wave w fetches rows 8 w .. 8 w + 7 (1 KiB per step).  A tail super-step
// loads its two steps twice (the second copy is not read).
__device__ __forceinline__ void sk_load_a(f16x8* buf, const SkOperands& op, int ss, int m, int wave) {
  const uint8_t* base = op.a + (size_t)ss * (kSkSteps * kStepK * 2);
  const uint32_t off = op.a_hi * (uint32_t)m + op.a_base;
#pragma unroll
  for (int j = 0; j < kSkSteps; ++j) dma16s(buf + j * kSkAStage + wave * 64, base, off + 64u * (j & (m - 1)));
}

// Nibbles of super-step ss: four 16 B loads of consecutive addresses per
// column tile (one 128 B line for the two lanes of a column); a tail
// super-step repeats its two steps.
__device__ __forceinline__ SkB sk_load_b(const SkOperands& op, int ss, int m) {
  SkB b;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint8_t* q = op.bq + (size_t)ss * (kSkSteps * kStepK / 2) + op.bq_row[nt] + 16 * m * op.g;
#pragma unroll
    for (int j = 0; j < kSkSteps; ++j) b.q[nt][j] = *reinterpret_cast<const uint4*>(q + 16 * (j & (m - 1)));
  }
  return b;
}

// Direct loads of the scales of macro-step mac (super-steps 4 mac .. 4 mac
// + 3; chunks past the last whole super-step re-read it and are not used).
__device__ __forceinline__ void sk_load_sf_macro(uint8_t* sfbuf, const SkOperands& op, int mac, int nfull,
                                                 int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (lane & 3) ^ sk_sf_swz(op.sf_tr[i]);
    const int ssrc = min(4 * mac + c, nfull - 1);
    dma16s(reinterpret_cast<f16x8*>(sfbuf + 1024 * (4 * wave + i)), op.bsf, op.sf_dma[i] + 16u * ssrc);
  }
}

// Direct loads of the 8 tail scale bytes of every tile row (dword d of the
// area holds half d & 1 of row d >> 1); row_of maps a tile row to its scale
// row offset.
template <class RowOf>
__device__ __forceinline__ void sk_load_sf_tail(uint8_t* sftail, const SkOperands& op, int nfull, int wave,
                                                int lane, RowOf row_of) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = 256 * i + 64 * wave + lane;
    dma4(reinterpret_cast<uint32_t*>(sftail + 1024 * i + 256 * wave),
         op.bsf + row_of(d >> 1) + 16 * nfull + 4 * (d & 1));
  }
}

// This lane's scale words of super-step ss for its two column tiles: step j's
// pair of block scales is bits 16 (j & 1) of s[nt][j >> 1].
__device__ __forceinline__ void sk_read_sf(const uint8_t* sfbuf, const uint8_t* sftail, int ss, int nfull,
                                           int wave, int lane, uint32_t (&s)[2][2]) {
  const int g = lane >> 5;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int tr = 64 * wave + 32 * nt + (lane & 31);
    if (ss < nfull) {
      const uint2 v = *reinterpret_cast<const uint2*>(sfbuf + 64 * tr + 16 * ((ss & 3) ^ sk_sf_swz(tr)) + 8 * g);
      s[nt][0] = v.x;
      s[nt][1] = v.y;
    } else {
      s[nt][0] = *reinterpret_cast<const uint32_t*>(sftail + 8 * tr + 4 * g);
      s[nt][1] = 0;
    }
  }
}

// The MFMAs of step j from A buffer buf, nibbles W and scale words sw.
__device__ __forceinline__ void sk_step(const f16x8* buf, const int (&ra)[4], const SkB& W,
                                        const uint32_t (&sw)[2][2], int j, f32x16 (&acc)[2]) {
  f16x2 lo[2], hi[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[nt][j >> 1] >> (16 * (j & 1)), 1.0f, false);
    lo[nt] = f16x2{sc[0], sc[0]};
    hi[nt] = f16x2{sc[1], sc[1]};
  }
  const int off = j * kSkAStage;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f16x8 fa = buf[ra[s] + off];
    const f16x8 b0 = dequant8(word_of(W.q[0][j], s), s < 2 ? lo[0] : hi[0]);
    const f16x8 b1 = dequant8(word_of(W.q[1][j], s), s < 2 ? lo[1] : hi[1]);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, b1, acc[1], 0, 0, 0);
  }
  SCHED_FENCE();  // keeps each step's fragments from being hoisted into the previous one
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
// (A first, then B; past the end they repeat the last super-step and are not
// used, and the tail's scales with the tail), then run its MFMAs.
template <int BUF, class RowOf>
__device__ __forceinline__ void sk_super(const SkLds& L, const int (&ra)[4], SkB (&W)[2], const SkOperands& op,
                                         int ss, int nss, int nfull, int wave, int lane, f32x16 (&acc)[2],
                                         RowOf row_of) {
  wait_vmcnt<0>();
  lds_barrier();
  uint32_t sw[2][2];
  sk_read_sf(L.sf, L.sftail, ss, nfull, wave, lane, sw);
  if ((ss & 3) == 3 && ss + 1 < nfull) {
    lds_barrier();
    sk_load_sf_macro(L.sf, op, (ss + 1) >> 2, nfull, wave, lane);
  }
  const int nx = min(ss + 1, nss - 1);
  const int mx = sk_steps(nx, nfull);
  sk_load_a(L.a + (BUF ^ 1) * kSkABuf, op, nx, mx, wave);
  W[BUF ^ 1] = sk_load_b(op, nx, mx);
  if (ss + 1 == nfull && nss > nfull) sk_load_sf_tail(L.sftail, op, nfull, wave, lane, row_of);
  SCHED_FENCE();
  const f16x8* buf = L.a + BUF * kSkABuf;
  sk_step(buf, ra, W[BUF], sw, 0, acc);
  sk_step(buf, ra, W[BUF], sw, 1, acc);
  if (ss < nfull) {
    sk_step(buf, ra, W[BUF], sw, 2, acc);
    sk_step(buf, ra, W[BUF], sw, 3, acc);
  }
}

// The K loop over nk steps of 64 (nk even); ends with all loads landed and
// every wave past its last LDS read.  row_of(tr) is the byte offset of the
// scale row of tile row tr within the expert's scales.
template <class RowOf>
__device__ __forceinline__ void sk_mainloop(const SkLds& L, const SkOperands& op, int nk, f32x16 (&acc)[2],
                                            RowOf row_of) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  const int nfull = nk / kSkSteps;
  const int nss = nfull + (nk % kSkSteps ? 1 : 0);
  SkB W[2];
  sk_load_a(L.a, op, 0, sk_steps(0, nfull), wave);
  if (nfull > 0)
    sk_load_sf_macro(L.sf, op, 0, nfull, wave, lane);
  else
    sk_load_sf_tail(L.sftail, op, nfull, wave, lane, row_of);
  W[0] = sk_load_b(op, 0, sk_steps(0, nfull));
  // A fragment chunk of sub-step s: row r, logical chunk 4 g + s
  int ra[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ra[s] = r * 8 + ((4 * g + s) ^ swz_key(r));
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  for (int ss = 0; ss < nss; ss += 2) {
    sk_super<0>(L, ra, W, op, ss, nss, nfull, wave, lane, acc, row_of);
    if (ss + 1 < nss) sk_super<1>(L, ra, W, op, ss + 1, nss, nfull, wave, lane, acc, row_of);
  }
  wait_vmcnt<0>();
  lds_barrier();
}

// Operand sources of this lane for a tile: A row `arow` (lane's tile row is
// 8 wave + lane / 8); row_of(tr) gives the global weight row of tile row tr.
template <class WRow>
__device__ __forceinline__ void sk_operands(SkOperands& op, uint32_t arow, int64_t K, int wave, int lane, int R,
                                            WRow wrow) {
  const int c = (lane & 7) ^ swz_key(R);
  op.a_base = arow * (uint32_t)(K * 2) + 16u * (uint32_t)(c & 3);
  op.a_hi = 64u * (uint32_t)(c >> 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) op.bq_row[j] = (uint32_t)wrow(64 * wave + 32 * j + (lane & 31)) * (uint32_t)(K / 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    op.sf_tr[i] = 64 * wave + 16 * i + (lane >> 2);
    op.sf_dma[i] = (uint32_t)wrow(op.sf_tr[i]) * (uint32_t)(K / 16);
  }
  op.g = lane >> 5;
}

#define SK_LDS_DECL                                              \
  __shared__ f16x8 lds_a[2 * kSkABuf];                           \
  __shared__ __attribute__((aligned(16))) uint8_t lds_sf[kSkSfMacro]; \
  __shared__ __attribute__((aligned(16))) uint8_t lds_sft[kSkSfTail]; \
  const SkLds L{lds_a, lds_sf, lds_sft}

// ------------------------------------------------------------------ L1
__global__ __launch_bounds__(kSkThreads, 3) void l1_skinny_kernel(L1Params p) {
  SK_LDS_DECL;
  GemmTile t;
  int nt;
  if (!tile_of<kSkTileM>(p.tiles, p.ntiles, p.M, p.n_ntiles, &t, &nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto out_row_of = [&](int r) -> int {
    const int rr = r < t.nrows ? r : 0;
    return p.perm ? p.perm[t.row0 + rr] : t.row0 + rr;
  };
  auto wrow = [&](int tr) { return l1_weight_row(nt, tr); };
  auto sf_row = [&](int tr) { return (uint32_t)l1_weight_row(nt, tr) * (uint32_t)(p.K / 16); };
  SkOperands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
  op.bq = p.w_q + (int64_t)t.expert * p.N2 * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N2 * (p.K / 16);
  {
    const int R = 8 * wave + (lane >> 3);
    const int o = out_row_of(R);
    const uint32_t arow = p.perm ? (uint32_t)(o / p.topk) : (uint32_t)o;
    sk_operands(op, arow, p.K, wave, lane, R, wrow);
  }
  f32x16 acc[2];
  sk_mainloop(L, op, (int)(p.K / kStepK), acc, sf_row);

  // epilogue: SwiGLU -> bf16 tile (32 x 128) in LDS, then NVFP4 of its rows
  constexpr int kCStride = 136;
  constexpr int kCTileChunks = kSkTileM * kCStride * 2 / 16;
  static_assert(kCTileChunks + 32 + kSkTileM / 4 <= 2 * kSkABuf, "epilogue LDS");
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds_a);
  float* rtab = reinterpret_cast<float*>(lds_a + kCTileChunks);
  int* out_row = reinterpret_cast<int*>(lds_a + kCTileChunks + 32);
  if (tid < kSkTileM) out_row[tid] = out_row_of(tid);
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int col = 32 * wave + (lane & 31);
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
  const int npass = (t.nrows + kSkThreads / 16 - 1) / (kSkThreads / 16);
  // bf16 tile of SiLU(gate) (gate_only) or SiLU(gate) * up in LDS
  auto fill_ctile = [&](bool gate_only) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float gate = acc[0][i] * alpha;
      const float sg = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate));
      const float c = gate_only ? sg : sg * (acc[1][i] * alpha);
      ctile[acc_row(i, lane) * kCStride + col] = __builtin_bit_cast(uint16_t, (__bf16)c);
    }
  };
  if (p.c_il) {
    // interleaved output: the SiLU(gate) groups first
    fill_ctile(true);
    __syncthreads();
    for (int pass = 0; pass < npass; ++pass) {
      const int qrow = pass * (kSkThreads / 16) + (tid >> 4);
      if (qrow < t.nrows) {
        const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
        const int64_t g8 = 16 * (int64_t)nt + hb;
        *reinterpret_cast<uint4*>(p.c_il + (int64_t)out_row[qrow] * p.N2 + 16 * g8) = w;
      }
    }
    __syncthreads();
  }
  fill_ctile(false);
  const float E2 = p.c_q ? 1.0f / p.out_gs[0] : 1.0f;  // no quantization without c_q
  fill_rtab(rtab, E2, tid);
  __syncthreads();
  for (int pass = 0; pass < npass; ++pass) {
    const int qrow = pass * (kSkThreads / 16) + (tid >> 4);
    const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
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
__global__ __launch_bounds__(kSkThreads, 3) void l2_skinny_kernel(L2Params p) {
  SK_LDS_DECL;
  GemmTile t;
  int nt;
  if (!tile_of<kSkTileM>(p.tiles, p.ntiles, p.M, p.n_ntiles, &t, &nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto pair_of = [&](int r) -> int {
    const int rr = t.row0 + (r < t.nrows ? r : 0);
    return p.perm ? p.perm[rr] : rr;
  };
  auto wrow = [&](int tr) { return nt * kTileN + tr; };
  auto sf_row = [&](int tr) { return (uint32_t)(nt * kTileN + tr) * (uint32_t)(p.K / 16); };
  SkOperands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
  op.bq = p.w_q + (int64_t)t.expert * p.N * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N * (p.K / 16);
  sk_operands(op, (uint32_t)pair_of(8 * wave + (lane >> 3)), p.K, wave, lane, 8 * wave + (lane >> 3), wrow);
  f32x16 acc[2];
  sk_mainloop(L, op, (int)(p.K / kStepK), acc, sf_row);
  // the scales' LDS holds the output rows, the A buffers each wave's
  // 4 KiB transposition scratch
  int* out_row = reinterpret_cast<int*>(lds_sf);
  if (tid < kSkTileM) out_row[tid] = pair_of(tid);
  __syncthreads();
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  float* const scratch = reinterpret_cast<float*>(lds_a) + wave * 1024;
  l2_store_block(p, acc[0], acc[1], scratch, 0, t.nrows, (int64_t)nt * kTileN + wave * 64, lane,
                 [&](int r) { return out_row[r]; },
                 [&](int r) { return p.row_w ? alpha * p.row_w[out_row[r]] : alpha; });
}

// ------------------------------------------------------------------ launchers
int skinny_tile_rows() { return kSkTileM; }

// K of whole super-steps (the scale rows then stay 16-byte aligned for the
// direct loads), or a single tail super-step of 128.
bool skinny_supports_k(int64_t K) { return K > 0 && (K % (kSkSteps * kStepK) == 0 || K == 2 * kStepK); }

hipError_t launch_l1_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                            uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                            const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                            const int* perm, int topk, hipStream_t s, uint16_t* c_il) {
  L1Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf, c_f16, c_il,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN)};
  const int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  if (!skinny_supports_k(K)) return hipErrorInvalidValue;
  l1_skinny_kernel<<<(unsigned)grid, kSkThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_l2_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w,
                            float* o, const GemmTile* tiles, const int* ntiles, int max_tiles,
                            const int* perm, hipStream_t s, int64_t M, uint16_t* o_bf16, int* sched,
                            uint16_t* o_f16, int8_t* o_exp) {
  (void)sched;  // one workgroup per item here
  L2Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, o_bf16, tiles, ntiles, M, perm, (int)(N / kTileN),
             nullptr, o_f16, o_exp};
  const int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  if (!skinny_supports_k(K)) return hipErrorInvalidValue;
  l2_skinny_kernel<<<(unsigned)grid, kSkThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
