// NVFP4 quantize / dequantize / global-scale kernels for gfx950.
//
// The tensor is handled as a flat sequence of 16-element blocks (rows are
// contiguous and K % 16 == 0, so no block straddles a row and the scale index
// of block b is simply b).  Each lane loads 16 bytes (8 bf16 = half a block)
// with one dwordx4 load, so a wavefront reads 1 KiB of consecutive memory per
// load instruction; the two lanes of a block exchange their partial maxima
// with one DPP swap.  Each lane stores one dword of nibbles (a wavefront
// stores 256 consecutive bytes), the even lane of a pair stores the scale.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;  // threads per workgroup
constexpr int kQUnroll = 4;     // 8-element chunks per thread (loads in flight)
constexpr int kQChunksPerWG = kQThreads * kQUnroll;
constexpr int kAmaxMaxWG = 2048;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ amax
// Pass 1: per-workgroup max |x| over a grid-stride range of 8-element chunks.
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(const uint4* __restrict__ x,
                                                                 int64_t n8,
                                                                 float* __restrict__ partial) {
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * kQThreads)
    m = fmaxf(m, abs_max8(load_nt(x + i)));
  // wavefront reduction then across the 4 wavefronts
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kQThreads / 64; ++w) r = fmaxf(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// Pass 1 over the rows of a [rows][cols] matrix that belong to valid (token,
// expert) pairs: row r counts when 0 <= ids[r] < E.  rc8 = cols / 8 chunks per
// row; the chunk index stays below 2^32.
__global__ __launch_bounds__(kQThreads) void amax_rows_partial_kernel(const uint4* __restrict__ x,
                                                                      int64_t n8, uint32_t rc8,
                                                                      const int32_t* __restrict__ ids,
                                                                      int E, float* __restrict__ partial) {
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * kQThreads) {
    const int32_t e = ids[(uint32_t)i / rc8];
    if (e >= 0 && e < E) m = fmaxf(m, abs_max8(load_nt(x + i)));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kQThreads / 64; ++w) r = fmaxf(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// Pass 2: one workgroup reduces the partials; g = amax / (6 * 448), or 1 when
// the tensor is all zero (or empty).
__global__ __launch_bounds__(1024) void amax_finalize_kernel(const float* __restrict__ partial,
                                                             int npartial, float* __restrict__ gs) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += 1024) m = fmaxf(m, partial[i]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[16];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < 16; ++w) r = fmaxf(r, red[w]);
    gs[0] = (r > 0.0f) ? r / 2688.0f : 1.0f;
  }
}

__global__ void copy_scalar_kernel(const float* __restrict__ src, float* __restrict__ dst) {
  if (threadIdx.x == 0) dst[0] = src[0];
}

// ------------------------------------------------------------------ quantize
// F16OUT: also write the exact f16 of each quantized value (e2m1 * block
// scale, without the global scale) -- the GEMM operand form of the tensor.
// IL: the input is an interleaved [rows][2 * 8 il8] matrix whose 8-column
// groups alternate SiLU(gate) and SwiGLU values; chunk i of the compact
// [rows][8 il8] tensor is its row's group 2 (i % il8) + 1.
// With amax_part (namax per-workgroup maxima of |x|) instead of gs, every
// workgroup reduces the maxima itself and forms g = amax / (6 * 448) (1 for
// an all-zero tensor) exactly as amax_finalize_kernel does, and workgroup 0
// stores it to gs_out: the reduction pass without a launch of its own.
template <bool F16OUT, bool IL = false>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t n8,
                                                             const float* __restrict__ gs,
                                                             uint32_t* __restrict__ q,
                                                             uint8_t* __restrict__ sf,
                                                             f16x8* __restrict__ f16out,
                                                             uint32_t il8 = 0,
                                                             const float* __restrict__ amax_part = nullptr,
                                                             int namax = 0, float* __restrict__ gs_out = nullptr) {
  __shared__ float rtab[128];
  __shared__ float red[kQThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kQChunksPerWG + threadIdx.x;
  uint4 w[kQUnroll];
#pragma unroll
  for (int u = 0; u < kQUnroll; ++u) {
    int64_t i = base + u * kQThreads;
    int64_t src = i;
    if (IL) {
      const uint32_t r = (uint32_t)i / il8, c = (uint32_t)i - r * il8;
      src = 2 * (int64_t)r * il8 + 2 * c + 1;
    }
    w[u] = (i < n8) ? load_nt(x + src) : make_uint4(0, 0, 0, 0);
  }
  float g;
  if (amax_part) {  // kernel-uniform
    float m = 0.0f;
    for (int i = threadIdx.x; i < namax; i += kQThreads) m = fmaxf(m, amax_part[i]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float r = red[0];
    for (int k = 1; k < kQThreads / 64; ++k) r = fmaxf(r, red[k]);
    g = (r > 0.0f) ? r / 2688.0f : 1.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) gs_out[0] = g;
  } else {
    g = gs[0];
  }
  const float E = 1.0f / g;
  fill_rtab(rtab, E, threadIdx.x);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kQUnroll; ++u) {
    int64_t i = base + u * kQThreads;  // i and i^1 hold the two halves of block i/2
    uint32_t code;
    uint32_t p = quantize_half_block(w[u], E, rtab, &code);
    if (i < n8) {  // the NVFP4 bytes are not read back by this pass: streaming stores
      __builtin_nontemporal_store(p, q + i);
      if ((i & 1) == 0) __builtin_nontemporal_store((uint8_t)code, sf + (i >> 1));
      if (F16OUT) f16out[i] = dequant8(p, scale_pair(code));
    }
  }
}

// ------------------------------------------------------------------ dequantize
// Each lane handles kQUnroll chunks of 8 elements (one dword of nibbles and
// its block scale each, loaded together before any is converted); the bf16
// output is written with streaming stores.
// x = f32(f32(e2m1 * sfd) * g); the gfx950 FP4 -> f32 conversion gives the
// exact E2M1 values, the product with the E4M3 scale is exact in fp32.
template <bool BF16_OUT>
__global__ __launch_bounds__(kQThreads) void dequantize_kernel(const uint32_t* __restrict__ q,
                                                               const uint8_t* __restrict__ sf,
                                                               const float* __restrict__ gs,
                                                               int64_t n8, void* __restrict__ out) {
  const float g = gs[0];
  const int64_t base = (int64_t)blockIdx.x * kQChunksPerWG + threadIdx.x;
  uint32_t pq[kQUnroll];
  uint32_t cs[kQUnroll];
#pragma unroll
  for (int u = 0; u < kQUnroll; ++u) {
    const int64_t i = base + u * kQThreads;
    pq[u] = (i < n8) ? __builtin_nontemporal_load(q + i) : 0u;
    cs[u] = (i < n8) ? sf[i >> 1] : 0u;
  }
#pragma unroll
  for (int u = 0; u < kQUnroll; ++u) {
    const int64_t i = base + u * kQThreads;
    if (i >= n8) break;
    const uint32_t p = pq[u];
    const float sfd = e4m3_decode_signed(cs[u]);
    float v[8];
    auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
    auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
    auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
    v[0] = (f0[0] * sfd) * g;
    v[1] = (f0[1] * sfd) * g;
    v[2] = (f1[0] * sfd) * g;
    v[3] = (f1[1] * sfd) * g;
    v[4] = (f2[0] * sfd) * g;
    v[5] = (f2[1] * sfd) * g;
    v[6] = (f3[0] * sfd) * g;
    v[7] = (f3[1] * sfd) * g;
    if (BF16_OUT) {
      __bf16 h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) h[k] = (__bf16)v[k];
      u32x4 o;
      __builtin_memcpy(&o, h, 16);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + i);
    } else {
      float4* o = reinterpret_cast<float4*>(out) + 2 * i;
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// NVFP4 -> exact f16 of e2m1 * block scale (no global scale): the GEMM
// operand form of an already-quantized tensor.
__global__ __launch_bounds__(kQThreads) void dequantize_f16_kernel(const uint32_t* __restrict__ q,
                                                                   const uint8_t* __restrict__ sf,
                                                                   int64_t n8,
                                                                   f16x8* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * kQThreads)
    out[i] = dequant8(q[i], scale_pair(sf[i >> 1]));
}

// ------------------------------------------------------------------ launchers
int amax_workgroups(int64_t n8) {
  int64_t wg = (n8 + kQChunksPerWG - 1) / kQChunksPerWG;
  if (wg < 1) wg = 1;
  if (wg > kAmaxMaxWG) wg = kAmaxMaxWG;
  return (int)wg;
}

size_t global_scale_workspace_bytes() { return kAmaxMaxWG * sizeof(float); }

hipError_t launch_global_scale(const uint16_t* x, int64_t n, float* partial, float* gs,
                               hipStream_t s) {
  int64_t n8 = n / 8;
  int wg = amax_workgroups(n8);
  amax_partial_kernel<<<wg, kQThreads, 0, s>>>(reinterpret_cast<const uint4*>(x), n8, partial);
  amax_finalize_kernel<<<1, 1024, 0, s>>>(partial, wg, gs);
  return hipGetLastError();
}

hipError_t launch_global_scale_rows(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ids, int E,
                                    float* partial, float* gs, hipStream_t s) {
  const int64_t n8 = rows * cols / 8;
  if (cols % 8 != 0 || n8 >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  const int wg = amax_workgroups(n8);
  amax_rows_partial_kernel<<<wg, kQThreads, 0, s>>>(reinterpret_cast<const uint4*>(x), n8,
                                                    (uint32_t)(cols / 8), ids, E, partial);
  amax_finalize_kernel<<<1, 1024, 0, s>>>(partial, wg, gs);
  return hipGetLastError();
}

hipError_t launch_copy_scalar(const float* src, float* dst, hipStream_t s) {
  copy_scalar_kernel<<<1, 64, 0, s>>>(src, dst);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t n, const float* gs, uint8_t* q, uint8_t* sf,
                           uint16_t* f16out, hipStream_t s) {
  int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  int64_t wg = (n8 + kQChunksPerWG - 1) / kQChunksPerWG;
  if (f16out)
    quantize_kernel<true><<<(unsigned)wg, kQThreads, 0, s>>>(
        reinterpret_cast<const uint4*>(x), n8, gs, reinterpret_cast<uint32_t*>(q), sf,
        reinterpret_cast<f16x8*>(f16out));
  else
    quantize_kernel<false><<<(unsigned)wg, kQThreads, 0, s>>>(
        reinterpret_cast<const uint4*>(x), n8, gs, reinterpret_cast<uint32_t*>(q), sf, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_folded(const uint16_t* x, int64_t n, const float* amax_part, int namax, float* gs_out,
                                  uint8_t* q, uint8_t* sf, uint16_t* f16out, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  if (!amax_part || namax < 1 || !gs_out || !f16out) return hipErrorInvalidValue;
  const int64_t wg = (n8 + kQChunksPerWG - 1) / kQChunksPerWG;
  quantize_kernel<true><<<(unsigned)wg, kQThreads, 0, s>>>(
      reinterpret_cast<const uint4*>(x), n8, nullptr, reinterpret_cast<uint32_t*>(q), sf,
      reinterpret_cast<f16x8*>(f16out), 0u, amax_part, namax, gs_out);
  return hipGetLastError();
}

hipError_t launch_quantize_interleaved(const uint16_t* x_il, int64_t rows, int64_t I, const float* gs,
                                       uint8_t* q, uint8_t* sf, uint16_t* f16out, hipStream_t s) {
  const int64_t n8 = rows * I / 8;
  if (n8 == 0) return hipSuccess;
  if (I % 16 != 0 || n8 >= ((int64_t)1 << 32) || !f16out) return hipErrorInvalidValue;
  const int64_t wg = (n8 + kQChunksPerWG - 1) / kQChunksPerWG;
  quantize_kernel<true, true><<<(unsigned)wg, kQThreads, 0, s>>>(
      reinterpret_cast<const uint4*>(x_il), n8, gs, reinterpret_cast<uint32_t*>(q), sf,
      reinterpret_cast<f16x8*>(f16out), (uint32_t)(I / 8));
  return hipGetLastError();
}

hipError_t launch_dequantize_f16(const uint8_t* q, const uint8_t* sf, int64_t n, uint16_t* out,
                                 hipStream_t s) {
  int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  int64_t wg = (n8 + kQThreads - 1) / kQThreads;
  if (wg > 65536) wg = 65536;
  dequantize_f16_kernel<<<(unsigned)wg, kQThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(q), sf,
                                                            n8, reinterpret_cast<f16x8*>(out));
  return hipGetLastError();
}

// ------------------------------------------------------------------ paired scale rows
// The row-paired layout of a block-scale matrix [R][C] (R even, C % 64 == 0):
// byte c of row r goes to (r / 2) 2C + 128 (c / 64) + 64 (r % 2) + c % 64, so
// each 128-byte line holds 64 bytes of rows 2j and 2j + 1, the form in which
// the 32-row GEMMs load a tile's scales in whole lines.  One 16-byte chunk
// per thread (all offsets below in chunks).
__global__ __launch_bounds__(256) void pair_scales_kernel(const uint4* __restrict__ sf, int64_t R, int64_t c16,
                                                          uint4* __restrict__ out) {
  const int64_t n = R * c16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / c16, cc = i - r * c16;
    out[(r >> 1) * (2 * c16) + 8 * (cc >> 2) + 4 * (r & 1) + (cc & 3)] = sf[i];
  }
}

hipError_t launch_pair_scales(const uint8_t* sf, int64_t R, int64_t C, uint8_t* out, hipStream_t s) {
  const int64_t n = R * (C / 16);
  if (n == 0) return hipSuccess;
  if ((R & 1) || C % 64 != 0) return hipErrorInvalidValue;
  const int64_t wg = std::min<int64_t>((n + 255) / 256, 65536);
  pair_scales_kernel<<<(unsigned)wg, 256, 0, s>>>(reinterpret_cast<const uint4*>(sf), R, C / 16,
                                                   reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* q, const uint8_t* sf, const float* gs, int64_t n,
                             bool bf16_out, void* out, hipStream_t s) {
  int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  int64_t wg = (n8 + kQChunksPerWG - 1) / kQChunksPerWG;
  if (bf16_out)
    dequantize_kernel<true><<<(unsigned)wg, kQThreads, 0, s>>>(
        reinterpret_cast<const uint32_t*>(q), sf, gs, n8, out);
  else
    dequantize_kernel<false><<<(unsigned)wg, kQThreads, 0, s>>>(
        reinterpret_cast<const uint32_t*>(q), sf, gs, n8, out);
  return hipGetLastError();
}

}  // namespace nvfp4
