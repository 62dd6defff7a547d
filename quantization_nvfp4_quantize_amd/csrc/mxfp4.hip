// MXFP4 quantize, dequantize and GEMM on gfx950: the separately labelled
// scaled-MFMA variant next to the pages' NVFP4.  MXFP4 is the format of the
// Open Compute Project "Microscaling Formats (MX) Specification" v1.0: 32
// consecutive elements share one E8M0 scale (code c = 2^(c - 127), section
// 5.4), each element is E2M1 (section 5.3.3), there is no tensor scale.  The
// conversion of section 6.3 sets the shared exponent to floor(log2(max |V|))
// - 2 and rounds V / 2^exp to nearest E2M1, ties to even, saturating at 6.
// It is not NVFP4 (E4M3 scale per 16 elements, fp32 tensor scale, the pages'
// two-stage E2M1 rounding): an NVFP4 block scale is not a power of two, so
// NVFP4 operands cannot be fed to the scaled MFMA exactly, which is why the
// NVFP4 GEMMs dequantize to f16.
//
// MI355X design:
//   * Quantize: one lane per 8 elements (a 16 B load), the 4 lanes of a block
//     take its maximum with two DPP steps; the shared exponent comes straight
//     from the maximum's exponent bits (code = max(biased exponent - 2, 0):
//     every subnormal or zero maximum clamps to code 0); the elements are
//     scaled by the exact power of two 2^(127 - code) and converted with the
//     gfx950 FP4 conversion, which rounds to nearest even on the E2M1 grid,
//     saturates at 6 and keeps the sign of zero.
//   * GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 and one
//     E8M0 scale per lane (row, 32-element K block): the operands go from
//     HBM straight into LDS and from LDS straight into the MFMA -- no
//     dequantization at all.  A workgroup of 8 wave64s owns a 256 x 256
//     output tile, wave w rows 128 (w >> 2) .. +128 and columns 64 (w & 3)
//     .. +64 as 4 x 2 MFMA tiles; K steps of 128 (two MFMA sub-steps of 64),
//     operands loaded four steps ahead into four LDS stages, and each step's
//     fragments read from LDS one step ahead into registers, so that the
//     MFMAs never wait for LDS.  The loads are bound by L2-to-L1 line
//     requests (128 B lines): a step's 64 B of a row takes a line request,
//     and so does its 4 B of scale codes.  For K % 512 == 0 (mx_gemm_kernel)
//     the scale codes come 16 B per row for 4 steps at a time, which takes
//     3/8 of the requests away (about 15% of the GEMM's time on the
//     4096 x 4096 x 16384 linear); other K (mx_gemm_kernel_k128) load them
//     per step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "gemm_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ quantize
constexpr int kMxQThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
constexpr int kMxQUnroll = 4;
constexpr int kMxQChunksPerWG = kMxQThreads * kMxQUnroll;

// Maximum over the 4 lanes of a quad (quad_perm [1,0,3,2], then [2,3,0,1]).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
}

// E8M0 code of a block whose largest magnitude is m >= 0 (finite):
// floor(log2(m)) - 2 + 127 = biased exponent - 2 for a normal m, clamped at
// 0, which also covers subnormal and zero maxima (their exponent is below
// -126, so the code would be negative).
__device__ __forceinline__ uint32_t mx_scale_code(float m) {
  const int ef = (int)(__float_as_uint(m) >> 23);
  return (uint32_t)max(ef - 2, 0);
}

// n8 chunks of 8 bf16 (4 chunks per block, n8 % 4 == 0) -> q (one dword of
// 8 nibbles per chunk, element 2i in the low nibble of byte i), sc (one code
// per block).
__global__ __launch_bounds__(kMxQThreads) void mx_quantize_kernel(const uint4* __restrict__ x, int64_t n8,
                                                                  uint32_t* __restrict__ q,
                                                                  uint8_t* __restrict__ sc) {
  const int64_t base = (int64_t)blockIdx.x * kMxQChunksPerWG + threadIdx.x;
  uint4 w[kMxQUnroll];
#pragma unroll
  for (int u = 0; u < kMxQUnroll; ++u) {
    const int64_t i = base + u * kMxQThreads;
    w[u] = (i < n8) ? load_stream(x + i) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kMxQUnroll; ++u) {
    const int64_t i = base + u * kMxQThreads;  // chunks 4b .. 4b + 3 of block b sit in one quad
    const uint32_t code = mx_scale_code(quad_max(abs_max8(w[u])));
    const float r = __uint_as_float((254u - code) << 23);  // 2^(127 - code), exact
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16_lo(w[u].x) * r, bf16_hi(w[u].x) * r, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16_lo(w[u].y) * r, bf16_hi(w[u].y) * r, 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16_lo(w[u].z) * r, bf16_hi(w[u].z) * r, 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16_lo(w[u].w) * r, bf16_hi(w[u].w) * r, 1.0f, 3);
    if (i < n8) {  // not read back by this pass: streaming stores
      __builtin_nontemporal_store(p, q + i);
      if ((i & 3) == 0) __builtin_nontemporal_store((uint8_t)code, sc + (i >> 2));
    }
  }
}

// ------------------------------------------------------------------ dequantize
// x = e2m1 * 2^(code - 127), exact (ldexp keeps subnormal results).
template <bool BF16_OUT>
__global__ __launch_bounds__(kMxQThreads) void mx_dequantize_kernel(const uint32_t* __restrict__ q,
                                                                    const uint8_t* __restrict__ sc, int64_t n8,
                                                                    void* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kMxQThreads + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * kMxQThreads) {
    const uint32_t p = q[i];
    const int e = (int)sc[i >> 2] - 127;
    const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
    const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
    const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
    const float v[8] = {ldexpf(f0[0], e), ldexpf(f0[1], e), ldexpf(f1[0], e), ldexpf(f1[1], e),
                        ldexpf(f2[0], e), ldexpf(f2[1], e), ldexpf(f3[0], e), ldexpf(f3[1], e)};
    if (BF16_OUT) {
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * j]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * j + 1]) << 16);
      reinterpret_cast<uint4*>(out)[i] = make_uint4(h[0], h[1], h[2], h[3]);
    } else {
      float4* o = reinterpret_cast<float4*>(out) + 2 * i;
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// ------------------------------------------------------------------ GEMM, any K % 128 == 0
constexpr int kMxTile = 256;          // rows and columns of a workgroup tile
constexpr int kMxThreads = 512;
constexpr int kMxStepK = 128;         // K per main-loop step
constexpr int kMxStages = 4;
constexpr int kMxOperand = kMxTile * (kMxStepK / 2) / 16;  // 16 B chunks of one operand stage (16 KiB)
constexpr int kMxScales = kMxTile;                         // dwords of one scale stage (1 KiB)
constexpr int kMxGroupRows = 4;                            // row tiles per group of the work order

// LDS: A and B stages (256 rows of 64 B = 4 chunks of 32 E2M1 values, logical
// chunk c of row r stored at c ^ ((r >> 2) & 3), so that the 16 rows a
// fragment read covers per 16 lanes land on 16 distinct 16 B bank groups),
// and per stage one dword of 4 scale codes per row.  136 KiB in all.
struct MxLds {
  uint4* a;      // kMxStages x kMxOperand
  uint4* b;      // kMxStages x kMxOperand
  uint32_t* sa;  // kMxStages x kMxScales
  uint32_t* sb;
};

struct MxOperands {
  const uint8_t* a;    // A nibbles [M][K/2], wave-uniform
  uint32_t a_off[2];   // this lane's sources: tile rows 32 wave + 16 u + lane / 4
  const uint8_t* b;    // W nibbles [N][K/2]
  uint32_t b_off[2];
  const uint8_t* s;    // scale source of this wave (A scales for waves 0..3, W scales for 4..7)
  uint32_t s_off;      // this lane's scale row: 64 (wave & 3) + lane of the tile
};

// Direct loads of step j into stage st: A and B (2 x 1 KiB each per wave),
// then the wave's 256 B of scales.
__device__ __forceinline__ void mx_load_step(const MxLds& L, const MxOperands& op, int j, int st, int wave) {
  const uint8_t* a_src = op.a + (size_t)j * (kMxStepK / 2);
  const uint8_t* b_src = op.b + (size_t)j * (kMxStepK / 2);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    dma16s(reinterpret_cast<f16x8*>(L.a + st * kMxOperand + (32 * wave + 16 * u) * 4), a_src, op.a_off[u]);
    dma16s(reinterpret_cast<f16x8*>(L.b + st * kMxOperand + (32 * wave + 16 * u) * 4), b_src, op.b_off[u]);
  }
  uint32_t* s_dst = ((wave >> 2) ? L.sb : L.sa) + st * kMxScales + 64 * (wave & 3);
  dma4s(s_dst, op.s + (size_t)j * (kMxStepK / 32), op.s_off);
}

__device__ __forceinline__ i32x8 widen(const uint4& v) {
  i32x4 w = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}

struct MxParams {
  const uint8_t* a_q;   // [M][K/2]
  const uint8_t* a_sc;  // [M][K/32]
  const uint8_t* w_q;   // [N][K/2]
  const uint8_t* w_sc;  // [N][K/32]
  int64_t M, K, N;
  float* o;             // [M][N] fp32 (when o_bf16 is null)
  uint16_t* o_bf16;     // nullable [M][N] bf16
};

__global__ __launch_bounds__(kMxThreads) void mx_gemm_kernel_k128(MxParams p) {
  __shared__ uint4 lds_a[kMxStages * kMxOperand];
  __shared__ uint4 lds_b[kMxStages * kMxOperand];
  __shared__ uint32_t lds_sa[kMxStages * kMxScales];
  __shared__ uint32_t lds_sb[kMxStages * kMxScales];
  const MxLds L{lds_a, lds_b, lds_sa, lds_sb};

  const int ntn = (int)(p.N / kMxTile);
  const int mtiles = (int)((p.M + kMxTile - 1) / kMxTile);
  int item;
  if (!work_item(mtiles * ntn, &item)) return;
  // Items in groups of kMxGroupRows row tiles, row tile fastest inside a
  // group: the 32 workgroups that run together on one XCD (contiguous items)
  // then cover 4 row tiles x 8 column tiles, 12 operand tiles instead of the
  // 33 of a row-major order, which keeps most of their loads in the XCD's L2.
  const int group = item / (kMxGroupRows * ntn);
  const int tm0 = group * kMxGroupRows, gm = min(kMxGroupRows, mtiles - tm0);
  const int within = item - group * kMxGroupRows * ntn;
  const int tm = tm0 + within % gm, tn = within / gm;
  const int64_t m0 = (int64_t)tm * kMxTile, n0 = (int64_t)tn * kMxTile;
  const int nrows = (int)min((int64_t)kMxTile, p.M - m0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t K2 = (uint32_t)(p.K / 2), K32 = (uint32_t)(p.K / 32);
  MxOperands op;
  op.a = p.a_q + m0 * K2;
  op.b = p.w_q + n0 * K2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int R = 32 * wave + 16 * u + (lane >> 2);  // tile row; its key (R >> 2) & 3 is (lane >> 4) & 3
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    op.a_off[u] = (uint32_t)min(R, nrows - 1) * K2 + chunk;  // rows past M repeat the last one (never stored)
    op.b_off[u] = (uint32_t)R * K2 + chunk;
  }
  const int srow = 64 * (wave & 3) + lane;
  if (wave >> 2) {
    op.s = p.w_sc + n0 * K32;
    op.s_off = (uint32_t)srow * K32;
  } else {
    op.s = p.a_sc + m0 * K32;
    op.s_off = (uint32_t)min(srow, nrows - 1) * K32;
  }

  const int nk = (int)(p.K / kMxStepK), last = nk - 1;
#pragma unroll
  for (int j = 0; j < kMxStages; ++j) mx_load_step(L, op, min(j, last), j, wave);

  // fragment addresses: row r of the wave's row group mt (A) or column group
  // nt (B) reads logical chunk 2 s + g at sub-step s; the XOR key of its row
  // is (lane >> 2) & 3 (row groups start at multiples of 32)
  const int wm = wave >> 2, wn = wave & 3, g = lane >> 5, r = lane & 31;
  const int key = (lane >> 2) & 3;
  const uint4* a_frag[2];
  const uint4* b_frag[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    a_frag[s] = L.a + (128 * wm + r) * 4 + ((2 * s + g) ^ key);
    b_frag[s] = L.b + (64 * wn + r) * 4 + ((2 * s + g) ^ key);
  }
  const uint32_t* a_scale = L.sa + 128 * wm + r;
  const uint32_t* b_scale = L.sb + 64 * wn + r;

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};

  // The sub-step s fragments of stage st, and the stage's scale dwords (as
  // read; shifted right by 8 g where they are used, so that byte 0 is the K
  // block of sub-step 0 and byte 2 that of sub-step 1 for this lane's half g).
  auto read_frags = [&](int st, int s, uint4 (&fa)[4], uint4 (&fb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fa[mt] = a_frag[s][st * kMxOperand + 128 * mt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) fb[nt] = b_frag[s][st * kMxOperand + 128 * nt];
  };
  auto read_scales = [&](int st, uint32_t (&sa)[4], uint32_t (&sb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sa[mt] = a_scale[st * kMxScales + 32 * mt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) sb[nt] = b_scale[st * kMxScales + 32 * nt];
  };
  // the 8 MFMAs of one sub-step (OPSEL 0: sub-step 0, scale byte 0; 2:
  // sub-step 1, scale byte 2)
  auto mfmas0 = [&](const uint4 (&fa)[4], const uint4 (&fb)[2], const uint32_t (&sa)[4], const uint32_t (&sb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fa[mt]), widen(fb[nt]), acc[mt][nt],
                                                                     4, 4, 0, (int)sa[mt], 0, (int)sb[nt]);
  };
  auto mfmas1 = [&](const uint4 (&fa)[4], const uint4 (&fb)[2], const uint32_t (&sa)[4], const uint32_t (&sb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fa[mt]), widen(fb[nt]), acc[mt][nt],
                                                                     4, 4, 2, (int)sa[mt], 2, (int)sb[nt]);
  };

  // Software pipeline, one step kb per iteration: c0 holds the step's
  // sub-step 0 fragments (and sa, sb its scale dwords), read during the
  // previous iteration.  Read the sub-step 1 fragments c1, shift the scale
  // dwords into sa1, sb1 (the shift waits for those reads: done here, a
  // sub-step after them, rather than right after the barrier, where it held
  // back the fragment reads and loads that follow, -1.5 %), and run the
  // sub-step 0 MFMAs; then the barrier, which ends every wave's reads of stage kb and
  // publishes stage kb + 1; then read the sub-step 0 fragments and scales of
  // step kb + 1 (a stale but valid stage in the last iteration), load step
  // kb + 4 into the stage of step kb, and run the sub-step 1 MFMAs while
  // those reads land.  The iteration is one basic block with scheduling
  // fences between its phases, so the barrier stays between the two MFMA
  // groups.  5 loads per step: at most 10 outstanding at the barrier means
  // every load of step kb - 3 and earlier has landed, including step kb + 1.
  uint4 c0a[4], c0b[2], c1a[4], c1b[2];
  uint32_t sa[4], sb[2], sa1[4], sb1[2];
  wait_vmcnt<0>();
  lds_barrier();
  read_scales(0, sa, sb);
  read_frags(0, 0, c0a, c0b);
  for (int kb = 0; kb < nk; ++kb) {
    const int st = kb & 3;
    read_frags(st, 1, c1a, c1b);
    SCHED_FENCE();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sa1[mt] = sa[mt] >> (8 * g);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) sb1[nt] = sb[nt] >> (8 * g);
    mfmas0(c0a, c0b, sa1, sb1);
    SCHED_FENCE();
    wait_vmcnt<10>();
    lds_barrier();
    SCHED_FENCE();
    read_scales((kb + 1) & 3, sa, sb);
    read_frags((kb + 1) & 3, 0, c0a, c0b);
    mx_load_step(L, op, min(kb + kMxStages, last), st, wave);
    SCHED_FENCE();
    mfmas1(c1a, c1b, sa1, sb1);
    SCHED_FENCE();
  }
  wait_vmcnt<0>();
  lds_barrier();

  // epilogue: each wave's 32 x 64 blocks through 4 KiB of LDS, rows of 16 B stores
  L2Params ep{};
  ep.N = p.N;
  ep.o = p.o;
  ep.o_bf16 = p.o_bf16;
  float* const scratch = reinterpret_cast<float*>(lds_a) + wave * 1024;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (128 * wm + 32 * mt >= nrows) break;  // wave-uniform
    l2_store_block(ep, acc[mt][0], acc[mt][1], scratch, 128 * wm + 32 * mt, nrows, n0 + 64 * wn, lane,
                   [&](int rr) { return m0 + rr; }, [&](int) { return 1.0f; });
  }
}

// ------------------------------------------------------------------ GEMM, K % 512 == 0
// The same tiles, waves and A/B stages as mx_gemm_kernel_k128; the scale
// codes instead come 16 B per row (4 steps) at a time into two 4-step scale
// stages of 256 rows x 16 B per operand.  A row's scale codes are one
// contiguous run of K/32 bytes, so each step's 4 B per row of the general
// kernel costs a whole cache-line request per row (512 requests per step
// for 2 KiB); this way one request per row brings 4 steps.
constexpr int kMxQuad = kMxTile * 4;  // dwords of one 4-step scale stage of one operand (4 KiB)

__global__ __launch_bounds__(kMxThreads) void mx_gemm_kernel(MxParams p) {
  __shared__ uint4 lds_a[kMxStages * kMxOperand];
  __shared__ uint4 lds_b[kMxStages * kMxOperand];
  __shared__ uint32_t lds_sa[2 * kMxQuad];
  __shared__ uint32_t lds_sb[2 * kMxQuad];

  const int ntn = (int)(p.N / kMxTile);
  const int mtiles = (int)((p.M + kMxTile - 1) / kMxTile);
  int item;
  if (!work_item(mtiles * ntn, &item)) return;
  const int group = item / (kMxGroupRows * ntn);
  const int tm0 = group * kMxGroupRows, gm = min(kMxGroupRows, mtiles - tm0);
  const int within = item - group * kMxGroupRows * ntn;
  const int tm = tm0 + within % gm, tn = within / gm;
  const int64_t m0 = (int64_t)tm * kMxTile, n0 = (int64_t)tn * kMxTile;
  const int nrows = (int)min((int64_t)kMxTile, p.M - m0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t K2 = (uint32_t)(p.K / 2), K32 = (uint32_t)(p.K / 32);
  const uint8_t* const a_src0 = p.a_q + m0 * K2;
  const uint8_t* const b_src0 = p.w_q + n0 * K2;
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int R = 32 * wave + 16 * u + (lane >> 2);  // tile row; its key (R >> 2) & 3 is (lane >> 4) & 3
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    a_off[u] = (uint32_t)min(R, nrows - 1) * K2 + chunk;  // rows past M repeat the last one (never stored)
    b_off[u] = (uint32_t)R * K2 + chunk;
  }
  // scale rows: waves 0..3 the A rows 64 wave + lane, waves 4..7 the W rows 64 (wave - 4) + lane
  const int srow = 64 * (wave & 3) + lane;
  const uint8_t* const s_src0 = (wave >> 2) ? p.w_sc + n0 * K32 : p.a_sc + m0 * K32;
  const uint32_t s_off = (uint32_t)((wave >> 2) ? srow : min(srow, nrows - 1)) * K32;
  uint32_t* const s_dst0 = ((wave >> 2) ? lds_sb : lds_sa) + 4 * 64 * (wave & 3);

  const int nk = (int)(p.K / kMxStepK), last = nk - 1, lastq = nk / 4 - 1;
  auto load_ab = [&](int j, int st) {
    const uint8_t* a_src = a_src0 + (size_t)j * (kMxStepK / 2);
    const uint8_t* b_src = b_src0 + (size_t)j * (kMxStepK / 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      dma16s(reinterpret_cast<f16x8*>(lds_a + st * kMxOperand + (32 * wave + 16 * u) * 4), a_src, a_off[u]);
      dma16s(reinterpret_cast<f16x8*>(lds_b + st * kMxOperand + (32 * wave + 16 * u) * 4), b_src, b_off[u]);
    }
  };
  auto load_quad = [&](int q) {
    dma16s(reinterpret_cast<f16x8*>(s_dst0 + (q & 1) * kMxQuad), s_src0 + (size_t)min(q, lastq) * 16, s_off);
  };
  // 4 loads per step and one per 4 steps, in the order quad 0, steps 0..3,
  // quad 1 here and, in the main loop, step kb + 4 in every iteration and
  // after it quad kb / 4 + 2 in iterations kb % 4 == 3
  load_quad(0);
#pragma unroll
  for (int j = 0; j < kMxStages; ++j) load_ab(min(j, last), j);
  load_quad(1);

  const int wm = wave >> 2, wn = wave & 3, g = lane >> 5, r = lane & 31;
  const int key = (lane >> 2) & 3;
  const uint4* a_frag[2];
  const uint4* b_frag[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    a_frag[s] = lds_a + (128 * wm + r) * 4 + ((2 * s + g) ^ key);
    b_frag[s] = lds_b + (64 * wn + r) * 4 + ((2 * s + g) ^ key);
  }
  const uint32_t* a_scale = lds_sa + (128 * wm + r) * 4;
  const uint32_t* b_scale = lds_sb + (64 * wn + r) * 4;

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};

  auto read_frags = [&](int st, int s, uint4 (&fa)[4], uint4 (&fb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fa[mt] = a_frag[s][st * kMxOperand + 128 * mt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) fb[nt] = b_frag[s][st * kMxOperand + 128 * nt];
  };
  // scale dwords of step j: quad stage (j / 4) & 1, dword j % 4 of each row
  auto read_scales = [&](int j, uint32_t (&sa)[4], uint32_t (&sb)[2]) {
    const int o = ((j >> 2) & 1) * kMxQuad + (j & 3);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sa[mt] = a_scale[o + 4 * 32 * mt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) sb[nt] = b_scale[o + 4 * 32 * nt];
  };
  auto mfmas0 = [&](const uint4 (&fa)[4], const uint4 (&fb)[2], const uint32_t (&sa)[4], const uint32_t (&sb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fa[mt]), widen(fb[nt]), acc[mt][nt],
                                                                     4, 4, 0, (int)sa[mt], 0, (int)sb[nt]);
  };
  auto mfmas1 = [&](const uint4 (&fa)[4], const uint4 (&fb)[2], const uint32_t (&sa)[4], const uint32_t (&sb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fa[mt]), widen(fb[nt]), acc[mt][nt],
                                                                     4, 4, 2, (int)sa[mt], 2, (int)sb[nt]);
  };

  uint4 c0a[4], c0b[2], c1a[4], c1b[2];
  uint32_t sa[4], sb[2], sa1[4], sb1[2];
  // step 0 and quad 0 landed: at most the 12 loads of steps 1..3 and quad 1 outstanding
  wait_vmcnt<13>();
  lds_barrier();
  read_scales(0, sa, sb);
  read_frags(0, 0, c0a, c0b);
  // Iteration kb as in mx_gemm_kernel_k128.  At its barrier step kb + 1
  // must have landed (and, for kb % 4 == 3, quad kb / 4 + 1, issued before
  // it): after step kb + 1's loads come those of steps kb + 2 and kb + 3
  // and, unless kb % 4 == 3, one quad.
  auto iter = [&](int kb, auto km) {
    constexpr int KM = decltype(km)::value;
    const int st = kb & 3;
    read_frags(st, 1, c1a, c1b);
    SCHED_FENCE();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sa1[mt] = sa[mt] >> (8 * g);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) sb1[nt] = sb[nt] >> (8 * g);
    mfmas0(c0a, c0b, sa1, sb1);
    SCHED_FENCE();
    wait_vmcnt<KM == 3 ? 8 : 9>();
    lds_barrier();
    SCHED_FENCE();
    read_scales(kb + 1, sa, sb);
    read_frags((kb + 1) & 3, 0, c0a, c0b);
    load_ab(min(kb + kMxStages, last), st);
    if (KM == 3) load_quad((kb >> 2) + 2);
    SCHED_FENCE();
    mfmas1(c1a, c1b, sa1, sb1);
    SCHED_FENCE();
  };
  for (int kb = 0; kb < nk; kb += 4) {
    iter(kb, std::integral_constant<int, 0>{});
    iter(kb + 1, std::integral_constant<int, 1>{});
    iter(kb + 2, std::integral_constant<int, 2>{});
    iter(kb + 3, std::integral_constant<int, 3>{});
  }
  wait_vmcnt<0>();
  lds_barrier();

  L2Params ep{};
  ep.N = p.N;
  ep.o = p.o;
  ep.o_bf16 = p.o_bf16;
  float* const scratch = reinterpret_cast<float*>(lds_a) + wave * 1024;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (128 * wm + 32 * mt >= nrows) break;  // wave-uniform
    l2_store_block(ep, acc[mt][0], acc[mt][1], scratch, 128 * wm + 32 * mt, nrows, n0 + 64 * wn, lane,
                   [&](int rr) { return m0 + rr; }, [&](int) { return 1.0f; });
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_mx_quantize(const uint16_t* x, int64_t n, uint8_t* q, uint8_t* sc, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t wg = (n8 + kMxQChunksPerWG - 1) / kMxQChunksPerWG;
  mx_quantize_kernel<<<(unsigned)wg, kMxQThreads, 0, s>>>(reinterpret_cast<const uint4*>(x), n8,
                                                          reinterpret_cast<uint32_t*>(q), sc);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* q, const uint8_t* sc, int64_t n, bool bf16_out, void* out,
                                hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t wg = std::min<int64_t>((n8 + kMxQThreads - 1) / kMxQThreads, 65536);
  if (bf16_out)
    mx_dequantize_kernel<true><<<(unsigned)wg, kMxQThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(q), sc,
                                                                    n8, out);
  else
    mx_dequantize_kernel<false><<<(unsigned)wg, kMxQThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(q), sc,
                                                                     n8, out);
  return hipGetLastError();
}

int mx_gemm_tile() { return kMxTile; }
int mx_gemm_step_k() { return kMxStepK; }

hipError_t launch_mx_gemm(const uint8_t* a_q, const uint8_t* a_sc, int64_t M, int64_t K, const uint8_t* w_q,
                          const uint8_t* w_sc, int64_t N, float* o, uint16_t* o_bf16, hipStream_t s) {
  if (M == 0) return hipSuccess;
  MxParams p{a_q, a_sc, w_q, w_sc, M, K, N, o, o_bf16};
  const int64_t items = ((M + kMxTile - 1) / kMxTile) * (N / kMxTile);
  const unsigned grid = (unsigned)((items + 7) / 8 * 8);
  if (K % 512 == 0 && ((uintptr_t)a_sc & 15) == 0 && ((uintptr_t)w_sc & 15) == 0)
    mx_gemm_kernel<<<grid, kMxThreads, 0, s>>>(p);
  else
    mx_gemm_kernel_k128<<<grid, kMxThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace nvfp4
