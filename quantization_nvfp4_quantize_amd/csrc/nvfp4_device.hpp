// Device primitives of the NVFP4 path on gfx950.
//
// Format (NVFP4-1.1_APPROACH_PART_2.md, "nvfp4-megamoe-kernel"): blocks of 16
// elements share one FP8 E4M3 scale (bias 7, exponent 15 holds numbers except
// mantissa 7 = NaN, largest value 0x7e = 448, subnormal m * 2^-9); each element
// is an E2M1 nibble (sign bit 3, index bits 2..0 into {0,.5,1,1.5,2,3,4,6})
// chosen by rounding 2*min(|s|,6) to the nearest even integer and mapping that
// half step through a table; two nibbles per byte, element 2i in the low nibble.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------------ E4M3
// Decode a non-negative E4M3 code (0..0x7e) exactly.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;                 // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));     // 2^(e-7) * (1 + m/8)
}

// Decode any E4M3 byte (sign, exponent 15 valid, 0x7f/0xff NaN) with the
// gfx950 FP8 conversion, which is exact on all 256 codes.
__device__ __forceinline__ float e4m3_decode_signed(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// Encode a non-negative fp32 value: nearest E4M3 magnitude, ties to the even
// code, values at or above 448 saturate to 0x7e (never the NaN code 0x7f).
// The gfx950 FP8 conversion rounds to nearest even exactly like that on
// [0, 448] (checked against the integer rounding on every third fp32 pattern
// of that range); it would emit NaN from 464-ish up, hence the clamp first.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(v, 448.0f), 0.0f, 0, false) & 0xffu;
}

// f32(b / 6) for every bf16 value b >= 0: one reciprocal product plus one
// fused correction step (the remainder b - 6*q0 is exact).  Equal to the
// correctly rounded division for all 2^15 non-negative finite bf16 inputs
// (checked exhaustively on the host); 3 instructions instead of ~10.
__device__ __forceinline__ float div6_bf16(float b) {
  const float c = 0.16666667163372039794921875f;  // RN(1/6)
  float q0 = b * c;
  float r = __builtin_fmaf(-q0, 6.0f, b);
  return __builtin_fmaf(r, c, q0);
}

// ------------------------------------------------------------------ E2M1
// Two scaled values -> two nibbles written into byte SEL of `packed` (first
// value in the low nibble).  Stage 1 rounds 2*clamp(s, -6, 6) to the nearest
// even integer (v_rndne keeps the sign of a zero result, so the nibble sign
// is the element's sign); stage 2 is the gfx950 FP4 conversion of that half
// step count divided by its scale operand 2: a round-to-nearest-even onto the
// E2M1 grid, which maps the half steps exactly as the table does
// (2.5 -> 2, 3.5 -> 4, 4.5 -> 4, 5 -> 4, 5.5 -> 6; the rest are exact).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t packed, float s0, float s1) {
  float h0 = __builtin_rintf(__builtin_amdgcn_fmed3f(s0 + s0, -12.0f, 12.0f));
  float h1 = __builtin_rintf(__builtin_amdgcn_fmed3f(s1 + s1, -12.0f, 12.0f));
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, h0, h1, 2.0f, SEL);
}

// ------------------------------------------------------------------ lanes
// Value of the neighbouring lane in a pair (lanes 2i <-> 2i+1), via DPP.
__device__ __forceinline__ float pair_swap(float v) {
  // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float abs_max8(uint4 w) {
  float m = fmaxf(fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x))), fabsf(bf16_lo(w.y)));
  m = fmaxf(fmaxf(m, fabsf(bf16_hi(w.y))), fabsf(bf16_lo(w.z)));
  m = fmaxf(fmaxf(m, fabsf(bf16_hi(w.z))), fabsf(bf16_lo(w.w)));
  return fmaxf(m, fabsf(bf16_hi(w.w)));
}

// Quantize the 8 bf16 values held by this lane, half of a 16-element block
// whose other half sits in the paired lane.  E = 1/g; rtab[c] = E / decode(c)
// for every code c (0 for c = 0).  Returns the 8 nibbles as one dword and the
// block's scale byte in *sf.  Both lanes of the pair must call this.
__device__ __forceinline__ uint32_t quantize_half_block(uint4 w, float E, const float* rtab,
                                                        uint32_t* sf) {
  float m = abs_max8(w);
  float bmax = fmaxf(m, pair_swap(m));
  float bsf = div6_bf16(bmax) * E;  // f32(f32(bmax / 6) * E)
  uint32_t code = e4m3_encode(bsf);
  *sf = code;
  float r = rtab[code];
  uint32_t p = 0;
  p = e2m1_pack2<0>(p, bf16_lo(w.x) * r, bf16_hi(w.x) * r);
  p = e2m1_pack2<1>(p, bf16_lo(w.y) * r, bf16_hi(w.y) * r);
  p = e2m1_pack2<2>(p, bf16_lo(w.z) * r, bf16_hi(w.z) * r);
  p = e2m1_pack2<3>(p, bf16_lo(w.w) * r, bf16_hi(w.w) * r);
  return p;
}

// 8 E2M1 nibbles (one dword) times one block scale (as an f16 pair) -> the 8
// exact products as f16 (at most 6 significant bits, within f16's normal
// range for every E4M3 scale): gfx950 FP4 -> f16 conversion, then one packed
// f16 multiply per pair.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 sc) {
  f16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  f16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  f16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  f16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  f16x8 v = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
  return v;
}

// An E4M3 scale byte as an f16 pair {s, s} (exact).
__device__ __forceinline__ f16x2 scale_pair(uint32_t code) {
  f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false);
  return f16x2{s[0], s[0]};
}

// Fill the per-tensor multiplier table rtab[c] = f32(E / decode(c)) (c < 127),
// rtab[0] = 0.  Call with at least 128 threads, then barrier.
__device__ __forceinline__ void fill_rtab(float* rtab, float E, int tid) {
  if (tid < 128) {
    float d = (tid < 127) ? e4m3_decode((uint32_t)tid) : 0.0f;
    rtab[tid] = (d == 0.0f) ? 0.0f : E / d;
  }
}

}  // namespace nvfp4
