// Token-grouped NVFP4 GEMMs for tiles of at most 32 rows: the decode shape of
// the MoE expert FFN, where each touched expert gets a handful of tokens and
// the GEMMs stream the experts' weights ("NVFP4 MoE Pipeline" in
// DEBUG_LOG.md; the L1 gate/up GEMM with the fused SwiGLU -> bf16 -> NVFP4
// epilogue and the L2 down GEMM with the routing-weighted epilogue are the
// same operations as in the 256-row tile kernels).
//
// MI355X design.  A 256-row tile leaves one workgroup per CU, and the weight
// bytes one CU keeps in flight (two steps of 9 KiB) are far below what HBM
// latency needs; with few rows the MFMAs are idle anyway.  Here:
//   * A workgroup of 4 waves owns 32 rows x 256 B rows (output columns); wave
//     w owns B rows 64 w .. +64 as two 32-column MFMA tiles (for L1: the gate
//     and the up rows of the same 32 SwiGLU columns, so SwiGLU stays within a
//     lane), 32 fp32 accumulators per lane.
//   * Weights never touch LDS: each lane loads, per K step of 64, the 16 B of
//     nibbles its MFMA B fragments need from each of its two column tiles
//     plus their scale words straight into registers, four steps ahead, and
//     dequantizes them to exact f16 in registers (each weight once).
//   * The 32 activation rows (exact f16) go through a 4-stage LDS ring with
//     direct-to-LDS loads, one 1 KiB load per wave and step, issued three
//     steps ahead; one LDS-only barrier per step.
//   * At most 128 VGPRs and 16 KiB of LDS, so four workgroups (16 waves) share
//     a CU and about 128 KiB of weights are in flight per CU.
#include <hip/hip_runtime.h>

#include "gemm_common.hpp"

namespace nvfp4 {

constexpr int kSkTileM = 32;
constexpr int kSkThreads = 256;
constexpr int kSkAStage = kSkTileM * (kStepK / 8);  // 16 B chunks of one A stage (4 KiB)
constexpr int kSkAStages = 4;
constexpr int kSkDepth = 4;  // weight register sets: step kb's are loaded during step kb - 4

// Per-workgroup operand sources (32-bit byte offsets, as in the 256-row
// kernels).
struct SkOperands {
  const uint8_t* a;      // A matrix (f16 rows of K), wave-uniform
  uint32_t a_off;        // this lane's A source: tile row 8 wave + lane / 8, chunk (lane & 7) ^ key
  const uint8_t* bq;     // B nibbles of the tile's expert, wave-uniform
  const uint8_t* bsf;    // B scales of the tile's expert, wave-uniform
  uint32_t bq_off[2];    // this lane's nibbles: tile rows 64 wave + 32 nt + lane % 32, K half lane / 32
  uint32_t bsf_off[2];   // and their scale words
};

// Weights of one K step in a lane (both column tiles): nibbles and scales.
struct SkB {
  BRaw r;
  BScale s;
};

__device__ __forceinline__ SkB sk_load_b(const SkOperands& op, int kb) {
  SkB b;
  const uint8_t* q = op.bq + (size_t)kb * (kStepK / 2);
  const uint8_t* sf = op.bsf + (size_t)kb * (kStepK / 16);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    b.r.q[nt] = *reinterpret_cast<const uint4*>(q + op.bq_off[nt]);
    b.s.w[nt] = *reinterpret_cast<const uint32_t*>(sf + op.bsf_off[nt]);
  }
  return b;
}

// One K step kb on A stage KA = kb % 4 with weight set W[KA]: 8 MFMAs (4
// sub-steps x 2 column tiles), each sub-step's B fragments dequantized just
// before its MFMAs.  Then W[KA] is refilled with step kb + 4 (4 loads) and the
// wave's direct load of A step kb + 3 goes to A stage (KA + 3) % 4 (last read
// in step kb - 1), in that order: 5 loads per step, so waiting at the end of
// step kb until at most 10 are outstanding means A of step kb + 1 (the last
// load of step kb - 2) has landed.  Loads past the end re-read the last step.
template <int KA>
__device__ __forceinline__ void sk_step(f16x8* lds_a, const f16x8* const (&ra)[4], SkB (&W)[kSkDepth],
                                        int kb, int last, const SkOperands& op, int wave, int lane,
                                        f32x16 (&acc)[2]) {
  const int g = lane >> 5;
  const ScalePairs pc = scale_pairs(W[KA].s, g);
  constexpr int aoff = KA * kSkAStage;
  f16x8 fa[2];
  fa[0] = ra[0][aoff];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) fa[(s + 1) & 1] = ra[s + 1][aoff];
    const f16x8 b0 = b_frag(W[KA].r, pc, 0, s);
    const f16x8 b1 = b_frag(W[KA].r, pc, 1, s);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s & 1], b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s & 1], b1, acc[1], 0, 0, 0);
  }
  SCHED_FENCE();
  W[KA] = sk_load_b(op, min(kb + kSkDepth, last));
  dma16(lds_a + ((KA + 3) % 4) * kSkAStage + wave * 64,
        op.a + (size_t)min(kb + 3, last) * (kStepK * 2) + op.a_off);
  SCHED_FENCE();
  wait_vmcnt<10>();
  lds_barrier();
}

// The K loop over nk steps; ends with all loads landed and every wave past
// its last LDS read.
__device__ __forceinline__ void sk_mainloop(f16x8* lds_a, const SkOperands& op, int nk,
                                            f32x16 (&acc)[2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  const int last = nk - 1;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    dma16(lds_a + j * kSkAStage + wave * 64, op.a + (size_t)min(j, last) * (kStepK * 2) + op.a_off);
  SkB W[kSkDepth];
#pragma unroll
  for (int j = 0; j < kSkDepth; ++j) W[j] = sk_load_b(op, min(j, last));
  // A fragment pointers of sub-step s: row r, logical chunk 4 g + s
  const f16x8* ra[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ra[s] = lds_a + r * 8 + ((4 * g + s) ^ swz_key(r));
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  wait_vmcnt<0>();
  lds_barrier();
  int kb = 0;
  for (; kb + 4 <= nk; kb += 4) {
    sk_step<0>(lds_a, ra, W, kb, last, op, wave, lane, acc);
    sk_step<1>(lds_a, ra, W, kb + 1, last, op, wave, lane, acc);
    sk_step<2>(lds_a, ra, W, kb + 2, last, op, wave, lane, acc);
    sk_step<3>(lds_a, ra, W, kb + 3, last, op, wave, lane, acc);
  }
  const int rem = nk - kb;
  if (rem > 0) sk_step<0>(lds_a, ra, W, kb, last, op, wave, lane, acc);
  if (rem > 1) sk_step<1>(lds_a, ra, W, kb + 1, last, op, wave, lane, acc);
  if (rem > 2) sk_step<2>(lds_a, ra, W, kb + 2, last, op, wave, lane, acc);
  wait_vmcnt<0>();
  lds_barrier();
}

// ------------------------------------------------------------------ L1
__global__ __launch_bounds__(kSkThreads, 4) void l1_skinny_kernel(L1Params p) {
  __shared__ f16x8 lds_a[kSkAStages * kSkAStage];
  GemmTile t;
  int nt;
  if (!tile_of<kSkTileM>(p.tiles, p.ntiles, p.M, p.n_ntiles, &t, &nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto out_row_of = [&](int r) -> int {
    const int rr = r < t.nrows ? r : 0;
    return p.perm ? p.perm[t.row0 + rr] : t.row0 + rr;
  };
  SkOperands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
  {
    const int R = 8 * wave + (lane >> 3);
    const int o = out_row_of(R);
    const uint32_t arow = p.perm ? (uint32_t)(o / p.topk) : (uint32_t)o;
    op.a_off = arow * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
  }
  op.bq = p.w_q + (int64_t)t.expert * p.N2 * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N2 * (p.K / 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t row = (uint32_t)l1_weight_row(nt, 64 * wave + 32 * j + (lane & 31));
    op.bq_off[j] = row * (uint32_t)(p.K / 2) + 16u * (lane >> 5);
    op.bsf_off[j] = row * (uint32_t)(p.K / 16);
  }
  f32x16 acc[2];
  sk_mainloop(lds_a, op, (int)(p.K / kStepK), acc);

  // epilogue: SwiGLU -> bf16 tile (32 x 128) in LDS, then NVFP4 of its rows
  constexpr int kCStride = 136;
  constexpr int kCTileChunks = kSkTileM * kCStride * 2 / 16;
  static_assert(kCTileChunks + 32 + kSkTileM / 4 <= kSkAStages * kSkAStage, "epilogue LDS");
  uint16_t* ctile = reinterpret_cast<uint16_t*>(lds_a);
  float* rtab = reinterpret_cast<float*>(lds_a + kCTileChunks);
  int* out_row = reinterpret_cast<int*>(lds_a + kCTileChunks + 32);
  if (tid < kSkTileM) out_row[tid] = out_row_of(tid);
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
  const int col = 32 * wave + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float gate = acc[0][i] * alpha;
    const float up = acc[1][i] * alpha;
    const float c = gate * __builtin_amdgcn_rcpf(1.0f + __expf(-gate)) * up;
    ctile[acc_row(i, lane) * kCStride + col] = __builtin_bit_cast(uint16_t, (__bf16)c);
  }
  const float E2 = 1.0f / p.out_gs[0];
  fill_rtab(rtab, E2, tid);
  __syncthreads();
  const int64_t I = p.N2 / 2;
  const int hb = tid & 15;
  const int npass = (t.nrows + kSkThreads / 16 - 1) / (kSkThreads / 16);
  for (int pass = 0; pass < npass; ++pass) {
    const int qrow = pass * (kSkThreads / 16) + (tid >> 4);
    const uint4 w = *reinterpret_cast<const uint4*>(ctile + qrow * kCStride + 8 * hb);
    uint32_t code;
    const uint32_t q = quantize_half_block(w, E2, rtab, &code);
    if (qrow < t.nrows) {
      const int64_t o = out_row[qrow];
      const int64_t col0 = 128 * (int64_t)nt + 8 * hb;
      reinterpret_cast<uint32_t*>(p.c_q + o * (I / 2))[col0 / 8] = q;
      if ((hb & 1) == 0) p.c_sf[o * (I / 16) + col0 / 16] = (uint8_t)code;
      if (p.c_bf16) *reinterpret_cast<uint4*>(p.c_bf16 + o * I + col0) = w;
      if (p.c_f16) *reinterpret_cast<f16x8*>(p.c_f16 + o * I + col0) = dequant8(q, scale_pair(code));
    }
  }
}

// ------------------------------------------------------------------ L2
__global__ __launch_bounds__(kSkThreads, 4) void l2_skinny_kernel(L2Params p) {
  __shared__ f16x8 lds_a[kSkAStages * kSkAStage];
  GemmTile t;
  int nt;
  if (!tile_of<kSkTileM>(p.tiles, p.ntiles, 0, p.n_ntiles, &t, &nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto pair_of = [&](int r) -> int { return p.perm[t.row0 + (r < t.nrows ? r : 0)]; };
  SkOperands op;
  op.a = reinterpret_cast<const uint8_t*>(p.a_f16);
  {
    const int R = 8 * wave + (lane >> 3);
    op.a_off = (uint32_t)pair_of(R) * (uint32_t)(p.K * 2) + 16u * ((lane & 7) ^ swz_key(R));
  }
  op.bq = p.w_q + (int64_t)t.expert * p.N * (p.K / 2);
  op.bsf = p.w_sf + (int64_t)t.expert * p.N * (p.K / 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t row = (uint32_t)(nt * kTileN + 64 * wave + 32 * j + (lane & 31));
    op.bq_off[j] = row * (uint32_t)(p.K / 2) + 16u * (lane >> 5);
    op.bsf_off[j] = row * (uint32_t)(p.K / 16);
  }
  f32x16 acc[2];
  sk_mainloop(lds_a, op, (int)(p.K / kStepK), acc);
  int* out_row = reinterpret_cast<int*>(lds_a);
  if (tid < kSkTileM) out_row[tid] = pair_of(tid);
  __syncthreads();
  const float alpha = p.a_gs[0] * p.w_gs[t.expert];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int orw = acc_row(i, lane);
    if (orw < t.nrows) {
      const int64_t pr = out_row[orw];
      const float s = alpha * p.row_w[pr];
      float* orow = p.o + pr * p.N + (int64_t)nt * kTileN + wave * 64 + (lane & 31);
      orow[0] = acc[0][i] * s;
      orow[32] = acc[1][i] * s;
    }
  }
}

// ------------------------------------------------------------------ launchers
int skinny_tile_rows() { return kSkTileM; }

hipError_t launch_l1_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N2, const float* out_gs,
                            uint16_t* c_bf16, uint8_t* c_q, uint8_t* c_sf, uint16_t* c_f16,
                            const GemmTile* tiles, const int* ntiles, int max_tiles, int64_t M,
                            const int* perm, int topk, hipStream_t s) {
  L1Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf, c_f16,
             tiles, ntiles, M, perm, topk, (int)(N2 / kTileN)};
  const int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l1_skinny_kernel<<<(unsigned)grid, kSkThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_l2_skinny(const uint16_t* a_f16, const float* a_gs, int64_t K, const uint8_t* w_q,
                            const uint8_t* w_sf, const float* w_gs, int64_t N, const float* row_w,
                            float* o, const GemmTile* tiles, const int* ntiles, int max_tiles,
                            const int* perm, hipStream_t s) {
  L2Params p{a_f16, a_gs, K, w_q, w_sf, w_gs, N, row_w, o, tiles, ntiles, perm, (int)(N / kTileN)};
  const int64_t grid = (int64_t)max_tiles * p.n_ntiles;
  if (grid == 0) return hipSuccess;
  l2_skinny_kernel<<<(unsigned)grid, kSkThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
