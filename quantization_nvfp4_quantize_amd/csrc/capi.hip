// extern "C" boundary of libnvfp4moe.so: argument validation, workspace
// carving and the launch sequence on the caller's stream.  Every check runs
// before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/nvfp4moe.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

constexpr int64_t kMaxOperandBytes = (int64_t)1 << 32;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

int nvfp4_version(void) { return 1; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported shape";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_last_error; }

// ------------------------------------------------------------------ quantize
size_t nvfp4_quantize_workspace_size(int64_t M, int64_t K) {
  (void)M;
  (void)K;
  return nvfp4::global_scale_workspace_bytes();
}

int nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K, const float* gs_in, uint8_t* q,
                   uint8_t* sf, float* gs_out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || K % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_quantize: need M >= 0, K > 0, K %% 16 == 0 (M=%lld K=%lld)",
                (long long)M, (long long)K);
  if (M > 0 && (!x || !q || !sf))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_quantize: x, q and sf must be non-null");
  if (!gs_in && !gs_out)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_quantize: gs_out is required when gs_in is null");
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(gs_in, 4) || !aligned(gs_out, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_quantize: x must be 16-byte and q 4-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n = M * K;
  const float* gs = gs_in;
  if (!gs_in) {
    size_t need = nvfp4_quantize_workspace_size(M, K);
    if (ws_bytes < need || !ws)
      return fail(NVFP4_ERR_WORKSPACE, "nvfp4_quantize: workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_quantize: ws must be 256-byte aligned");
    int st = hip_status(nvfp4::launch_global_scale(x, n, static_cast<float*>(ws), gs_out, s),
                        "nvfp4_quantize (global scale)");
    if (st) return st;
    gs = gs_out;
  } else if (gs_out) {
    int st = hip_status(nvfp4::launch_copy_scalar(gs_in, gs_out, s), "nvfp4_quantize (copy scale)");
    if (st) return st;
  }
  return hip_status(nvfp4::launch_quantize(x, n, gs, q, sf, nullptr, s), "nvfp4_quantize");
}

// ------------------------------------------------------------------ dequantize
int nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, const float* gs, int64_t M, int64_t K,
                     int out_dtype, void* out, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || K % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_dequantize: need M >= 0, K > 0, K %% 16 == 0");
  if (out_dtype != 0 && out_dtype != 1)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_dequantize: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (M > 0 && (!q || !sf || !gs || !out))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_dequantize: null pointer");
  if (!aligned(q, 4) || !aligned(out, 16) || !aligned(gs, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_dequantize: q must be 4-byte and out 16-byte aligned");
  return hip_status(nvfp4::launch_dequantize(q, sf, gs, M * K, out_dtype == 0, out,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "nvfp4_dequantize");
}

// ------------------------------------------------------------------ paired scale rows
int nvfp4_pair_scales(const uint8_t* sf, int64_t R, int64_t C, uint8_t* out, void* stream) {
  g_last_error[0] = 0;
  if (R < 0 || C < 0 || (R & 1) || C % 64 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_pair_scales: need R >= 0 even and C %% 64 == 0 (R=%lld C=%lld)",
                (long long)R, (long long)C);
  const size_t n = (size_t)(R * C);
  if (n == 0) return NVFP4_OK;
  if (!sf || !out) return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_pair_scales: null pointer");
  if (!aligned(sf, 16) || !aligned(out, 16))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_pair_scales: sf and out must be 16-byte aligned");
  if (sf < out + n && out < sf + n) return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_pair_scales: sf and out overlap");
  return hip_status(nvfp4::launch_pair_scales(sf, R, C, out, reinterpret_cast<hipStream_t>(stream)),
                    "nvfp4_pair_scales");
}

// ------------------------------------------------------------------ GEMM stage
size_t nvfp4_gemm_swiglu_quant_workspace_size(int64_t M, int64_t K, int64_t N2) {
  (void)N2;
  if (M <= 0 || K <= 0) return 0;
  return round_up((size_t)(M * K) * sizeof(uint16_t), 256);  // exact f16 copy of the activations
}

int nvfp4_gemm_swiglu_quant(const uint8_t* a_q, const uint8_t* a_sf, const float* a_gs, int64_t M,
                            int64_t K, const uint8_t* w_q, const uint8_t* w_sf, const float* w_gs,
                            int64_t N2, const float* out_gs, uint16_t* c_bf16, uint8_t* c_q,
                            uint8_t* c_sf, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || N2 <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_gemm_swiglu_quant: need M >= 0, K > 0, N2 > 0");
  if (K % 64 != 0 || N2 % 256 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "nvfp4_gemm_swiglu_quant: need K %% 64 == 0 and N2 %% 256 == 0 (K=%lld N2=%lld)",
                (long long)K, (long long)N2);
  if (M > (int64_t)1 << 30) return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_gemm_swiglu_quant: M too large");
  // the GEMM addresses its operands with 32-bit byte offsets
  if ((__int128)M * (K / 2) > kMaxOperandBytes || (__int128)N2 * (K / 2) > kMaxOperandBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_gemm_swiglu_quant: an operand exceeds 4 GiB");
  if (M == 0) return NVFP4_OK;
  if (!a_q || !a_sf || !a_gs || !w_q || !w_sf || !w_gs || !out_gs || !c_q || !c_sf)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_gemm_swiglu_quant: null pointer");
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(a_sf, 4) || !aligned(w_sf, 4) ||
      !aligned(c_q, 4) || !aligned(c_bf16, 16))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_gemm_swiglu_quant: misaligned pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int tiles = (int)((M + nvfp4::gemm_tile_rows() - 1) / nvfp4::gemm_tile_rows());
  if (!ws) {  // no workspace: the GEMM dequantizes the NVFP4 activations into LDS itself
    return hip_status(nvfp4::launch_l1(nullptr, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf,
                                       nullptr, nullptr, nullptr, tiles, M, nullptr, 1, s, nullptr, a_q, a_sf),
                      "nvfp4_gemm_swiglu_quant");
  }
  // with a workspace: expand the activations to exact f16 once, then the GEMM
  // (measured faster: the expansion inside the MFMA loop costs it more time
  // than this pass takes)
  if ((__int128)M * K * 2 > kMaxOperandBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_gemm_swiglu_quant: the f16 activations exceed 4 GiB (pass ws = NULL)");
  const size_t need = nvfp4_gemm_swiglu_quant_workspace_size(M, K, N2);
  if (ws_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "nvfp4_gemm_swiglu_quant: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_gemm_swiglu_quant: ws must be 256-byte aligned");
  uint16_t* a_f16 = static_cast<uint16_t*>(ws);
  int st = hip_status(nvfp4::launch_dequantize_f16(a_q, a_sf, M * K, a_f16, s),
                      "nvfp4_gemm_swiglu_quant (operand)");
  if (st) return st;
  return hip_status(nvfp4::launch_l1(a_f16, a_gs, K, w_q, w_sf, w_gs, N2, out_gs, c_bf16, c_q, c_sf,
                                     nullptr, nullptr, nullptr, tiles, M, nullptr, 1, s),
                    "nvfp4_gemm_swiglu_quant");
}

// ------------------------------------------------------------------ dense linear
namespace {

struct LinearLayout {
  size_t partial, gs, xq, xsf, x_f16, total;
};

LinearLayout linear_layout(int64_t M, int64_t K) {
  LinearLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t r = off;
    off = round_up(off + bytes, 256);
    return r;
  };
  L.partial = take(nvfp4::global_scale_workspace_bytes());
  L.gs = take(sizeof(float));
  L.xq = take((size_t)(M * K / 2));
  L.xsf = take((size_t)(M * K / 16));
  L.x_f16 = take(sizeof(uint16_t) * (size_t)(M * K));
  L.total = off;
  return L;
}

// Rows up to which the 32-row kernels (weights streamed) take the linear.
constexpr int64_t kLinearSkinnyRows = 64;

}  // namespace

size_t nvfp4_linear_workspace_size(int64_t M, int64_t K, int64_t N) {
  (void)N;
  if (M < 0 || K <= 0) return 0;
  return linear_layout(M, K).total;
}

int nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, const float* x_gs_in, const uint8_t* w_q,
                 const uint8_t* w_sf, const float* w_gs, int64_t N, int out_dtype, void* out,
                 float* x_gs_out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || N <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_linear: need M >= 0, K > 0, N > 0");
  if (out_dtype != 0 && out_dtype != 1)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_linear: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (K % 64 != 0 || N % 256 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_linear: need K %% 64 == 0 and N %% 256 == 0 (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (M > (int64_t)1 << 30) return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_linear: M too large");
  if ((__int128)M * K * 2 > kMaxOperandBytes || (__int128)N * (K / 2) > kMaxOperandBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_linear: an operand exceeds 4 GiB");
  if (M == 0) return NVFP4_OK;
  if (!x || !w_q || !w_sf || !w_gs || !out)
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_linear: null pointer");
  // the GEMM epilogues write out with 16-byte vector stores
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_sf, 16) || !aligned(out, 16) ||
      !aligned(x_gs_in, 4) || !aligned(x_gs_out, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_linear: misaligned pointer (x, w_q, w_sf and out need 16 bytes)");
  const LinearLayout L = linear_layout(M, K);
  if (!ws || ws_bytes < L.total)
    return fail(NVFP4_ERR_WORKSPACE, "nvfp4_linear: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_INVALID_ARG, "nvfp4_linear: ws must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int st;
  const float* gs = x_gs_in;
  if (!gs) {
    float* g = x_gs_out ? x_gs_out : reinterpret_cast<float*>(w + L.gs);
    if ((st = hip_status(nvfp4::launch_global_scale(x, M * K, reinterpret_cast<float*>(w + L.partial), g, s),
                         "nvfp4_linear (global scale)")))
      return st;
    gs = g;
  } else if (x_gs_out &&
             (st = hip_status(nvfp4::launch_copy_scalar(x_gs_in, x_gs_out, s), "nvfp4_linear (copy scale)"))) {
    return st;
  }
  uint16_t* x_f16 = reinterpret_cast<uint16_t*>(w + L.x_f16);
  if ((st = hip_status(nvfp4::launch_quantize(x, M * K, gs, reinterpret_cast<uint8_t*>(w + L.xq),
                                              reinterpret_cast<uint8_t*>(w + L.xsf), x_f16, s),
                       "nvfp4_linear (quantize x)")))
    return st;
  const bool skinny = M <= kLinearSkinnyRows && nvfp4::skinny_supports_k(K);
  const int64_t tm = skinny ? nvfp4::skinny_tile_rows() : nvfp4::gemm_tile_rows();
  const int tiles = (int)((M + tm - 1) / tm);
  float* o32 = out_dtype == 1 ? static_cast<float*>(out) : nullptr;
  uint16_t* o16 = out_dtype == 0 ? static_cast<uint16_t*>(out) : nullptr;
  return hip_status(skinny ? nvfp4::launch_l2_skinny(x_f16, gs, K, w_q, w_sf, w_gs, N, nullptr, o32, nullptr,
                                                     nullptr, tiles, nullptr, s, M, o16)
                           : nvfp4::launch_l2(x_f16, gs, K, w_q, w_sf, w_gs, N, nullptr, o32, nullptr, nullptr,
                                              tiles, nullptr, s, M, o16),
                    "nvfp4_linear");
}

// ------------------------------------------------------------------ MXFP4
// The separately labelled OCP MX v1.0 format (E8M0 scale per 32 elements)
// on gfx950's scaled FP4 MFMA.
int mxfp4_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* scale, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || K % 32 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_quantize: need M >= 0, K > 0, K %% 32 == 0 (M=%lld K=%lld)",
                (long long)M, (long long)K);
  if (M == 0) return NVFP4_OK;
  if (!x || !q || !scale) return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_quantize: x, q and scale must be non-null");
  if (!aligned(x, 16) || !aligned(q, 4))
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_quantize: x must be 16-byte and q 4-byte aligned");
  return hip_status(nvfp4::launch_mx_quantize(x, M * K, q, scale, reinterpret_cast<hipStream_t>(stream)),
                    "mxfp4_quantize");
}

int mxfp4_dequantize(const uint8_t* q, const uint8_t* scale, int64_t M, int64_t K, int out_dtype, void* out,
                     void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || K % 32 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_dequantize: need M >= 0, K > 0, K %% 32 == 0");
  if (out_dtype != 0 && out_dtype != 1)
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_dequantize: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (M == 0) return NVFP4_OK;
  if (!q || !scale || !out) return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_dequantize: null pointer");
  if (!aligned(q, 4) || !aligned(out, 16))
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_dequantize: q must be 4-byte and out 16-byte aligned");
  return hip_status(nvfp4::launch_mx_dequantize(q, scale, M * K, out_dtype == 0, out,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "mxfp4_dequantize");
}

namespace {
struct MxLayout {
  size_t xq, xsc, total;
};
MxLayout mx_layout(int64_t M, int64_t K) {
  MxLayout L;
  L.xq = 0;
  L.xsc = round_up((size_t)(M * K / 2), 256);
  L.total = round_up(L.xsc + (size_t)(M * K / 32), 256);
  return L;
}
}  // namespace

size_t mxfp4_linear_workspace_size(int64_t M, int64_t K, int64_t N) {
  (void)N;
  if (M < 0 || K <= 0) return 0;
  return mx_layout(M, K).total;
}

int mxfp4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w_q, const uint8_t* w_scale, int64_t N,
                 int out_dtype, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K <= 0 || N <= 0) return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_linear: need M >= 0, K > 0, N > 0");
  if (out_dtype != 0 && out_dtype != 1)
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_linear: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (K % nvfp4::mx_gemm_step_k() != 0 || N % nvfp4::mx_gemm_tile() != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "mxfp4_linear: need K %% %d == 0 and N %% %d == 0 (K=%lld N=%lld)",
                nvfp4::mx_gemm_step_k(), nvfp4::mx_gemm_tile(), (long long)K, (long long)N);
  if (M > (int64_t)1 << 30) return fail(NVFP4_ERR_UNSUPPORTED, "mxfp4_linear: M too large");
  if ((__int128)M * (K / 2) > kMaxOperandBytes || (__int128)N * (K / 2) > kMaxOperandBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "mxfp4_linear: an operand exceeds 4 GiB");
  if (M == 0) return NVFP4_OK;
  if (!x || !w_q || !w_scale || !out) return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_linear: null pointer");
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4) || !aligned(out, 16))
    return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_linear: misaligned pointer");
  const MxLayout L = mx_layout(M, K);
  if (!ws || ws_bytes < L.total)
    return fail(NVFP4_ERR_WORKSPACE, "mxfp4_linear: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_INVALID_ARG, "mxfp4_linear: ws must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  uint8_t* xq = reinterpret_cast<uint8_t*>(w + L.xq);
  uint8_t* xsc = reinterpret_cast<uint8_t*>(w + L.xsc);
  int st;
  if ((st = hip_status(nvfp4::launch_mx_quantize(x, M * K, xq, xsc, s), "mxfp4_linear (quantize x)"))) return st;
  return hip_status(nvfp4::launch_mx_gemm(xq, xsc, M, K, w_q, w_scale, N,
                                          out_dtype == 1 ? static_cast<float*>(out) : nullptr,
                                          out_dtype == 0 ? static_cast<uint16_t*>(out) : nullptr, s),
                    "mxfp4_linear");
}

// ------------------------------------------------------------------ MoE
namespace {

struct MoeLayout {
  size_t partial, x_gs, xq, xsf, x_f16, offsets, perm, tiles, ntiles, small, nsmall, err, route, sched, split,
      a2_gs, c, a2q, a2sf, a2_f16, o, oexp, total;
  int max_tiles;
};

// The L1 output is quantized in a separate pass (from its bf16 rows) when its
// global scale is dynamic or the caller asks for the unfused flow; flow 2 is
// the pages' earlier one (interleaved bf16 output, deinterleave + quantize).
bool moe_unfused(const nvfp4_moe_args* a) { return a->a2_gs == nullptr || a->l1_unfused == 1; }
bool moe_interleaved(const nvfp4_moe_args* a) { return a->l1_unfused == 2; }

// With a bf16 output the L2 GEMM writes its per-pair rows in f16 with one
// power-of-two exponent per (pair, 32 columns) (relative error <= 2^-11 per
// value, 4x below the bf16 rounding of y), which halves the bytes written and
// read back by the combine; an fp32 output keeps fp32 rows.
bool moe_f16_rows(const nvfp4_moe_args* a) { return a->out_dtype == 0; }

// GEMM tiling: 32-row tiles (weights streamed through registers) when the
// experts get few rows each; else 256-row tiles (MFMA-bound), each expert's
// last block of at most 64 rows on one or two 32-row tiles of its own when
// the 32-row kernels take H and I (mixed, tile_rows 256 + 32: such a short
// block would cost a 256-row tile most of a full tile's time, two 32-row
// tiles about 60 % of it).
int kMixedTileRows() { return nvfp4::gemm_tile_rows() + nvfp4::skinny_tile_rows(); }
constexpr int kMaxShortTiles = 2;  // 32-row tiles per expert's short last block

bool moe_skinny_fits(const nvfp4_moe_args* a) {
  return nvfp4::skinny_supports_k(a->H) && nvfp4::skinny_supports_k(a->I);
}

int64_t moe_tile_rows(const nvfp4_moe_args* a) {
  if (a->tile_rows) return a->tile_rows;
  const int64_t P = a->T * a->topk;
  if (!moe_skinny_fits(a)) return nvfp4::gemm_tile_rows();
  return P <= 16 * a->E ? nvfp4::skinny_tile_rows() : kMixedTileRows();
}

MoeLayout moe_layout(const nvfp4_moe_args* a) {
  MoeLayout L;
  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, P = a->T * a->topk;
  const int64_t bm = moe_tile_rows(a) == nvfp4::skinny_tile_rows() ? nvfp4::skinny_tile_rows()
                                                                    : nvfp4::gemm_tile_rows();
  L.max_tiles = (int)((P + bm - 1) / bm + E);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t r = off;
    off = round_up(off + bytes, 256);
    return r;
  };
  L.partial = take(nvfp4::global_scale_workspace_bytes());
  L.x_gs = take(sizeof(float));
  L.xq = take((size_t)(T * H / 2));
  L.xsf = take((size_t)(T * H / 16));
  L.x_f16 = take(sizeof(uint16_t) * (size_t)(T * H));
  L.offsets = take(sizeof(int) * (size_t)(E + 1));
  L.perm = take(sizeof(int) * (size_t)(P > 0 ? P : 1));
  L.tiles = take(sizeof(nvfp4::GemmTile) * (size_t)L.max_tiles);
  L.ntiles = take(sizeof(int));
  L.small = take(sizeof(nvfp4::GemmTile) * (size_t)kMaxShortTiles * (size_t)E);
  L.nsmall = take(sizeof(int));
  L.err = take(sizeof(int));
  L.route = take(nvfp4::route_workspace_bytes(P, (int)E));
  L.sched = take(nvfp4::kSchedCounters * sizeof(int));
  // the 32-row GEMMs' partial sums of the items they split along K
  L.split = take(moe_tile_rows(a) == nvfp4::skinny_tile_rows() ? nvfp4::skinny_split_bytes() : 0);
  L.a2_gs = take(sizeof(float));
  L.c = take(moe_interleaved(a) ? sizeof(uint16_t) * (size_t)(2 * P * I)
             : moe_unfused(a) && !a->l1_c_bf16 ? sizeof(uint16_t) * (size_t)(P * I) : 0);
  L.a2q = take((size_t)(P * I / 2));
  L.a2sf = take((size_t)(P * I / 16));
  L.a2_f16 = take(sizeof(uint16_t) * (size_t)(P * I));
  L.o = take((moe_f16_rows(a) ? sizeof(uint16_t) : sizeof(float)) * (size_t)(P * H));
  L.oexp = take(moe_f16_rows(a) ? (size_t)(P * H / 32) : 0);
  L.total = off;
  return L;
}

int moe_validate(const nvfp4_moe_args* a) {
  if (!a) return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: args is null");
  if (a->T < 0 || a->H <= 0 || a->I <= 0 || a->E < 1 || a->topk < 1)
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: need T >= 0, H, I > 0, E >= 1, topk >= 1");
  if (a->H % 256 != 0 || a->I % 128 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4: need H %% 256 == 0 and I %% 128 == 0 (H=%lld I=%lld)",
                (long long)a->H, (long long)a->I);
  if (a->E > 512 || a->topk > 32)
    return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4: need E <= 512 and topk <= 32");
  if (a->T * a->topk > ((int64_t)1 << 30))
    return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4: too many (token, expert) pairs");
  // the GEMMs address the f16 activations and one expert's weights with
  // 32-bit byte offsets
  if ((__int128)a->T * a->H * 2 > kMaxOperandBytes ||
      (__int128)a->T * a->topk * a->I * 2 > kMaxOperandBytes ||
      (__int128)a->I * a->H > kMaxOperandBytes)
    return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4: a GEMM operand exceeds 4 GiB");
  if (a->out_dtype != 0 && a->out_dtype != 1)
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (a->tile_rows != 0 && a->tile_rows != nvfp4::skinny_tile_rows() &&
      a->tile_rows != nvfp4::gemm_tile_rows() && a->tile_rows != kMixedTileRows())
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: tile_rows must be 0, %d, %d or %d",
                nvfp4::skinny_tile_rows(), nvfp4::gemm_tile_rows(), kMixedTileRows());
  if (a->l1_unfused < 0 || a->l1_unfused > 2)
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: l1_unfused must be 0, 1 or 2");
  if (a->l1_unfused == 2 && !a->a2_gs)
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: the interleaved flow needs a supplied a2_gs");
  if (a->aux_stream && (!a->aux_events || !a->aux_events[0] || !a->aux_events[1]))
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: aux_stream needs two aux_events");
  if ((a->tile_rows == nvfp4::skinny_tile_rows() || a->tile_rows == kMixedTileRows()) && !moe_skinny_fits(a))
    return fail(NVFP4_ERR_UNSUPPORTED,
                "moe_expert_ffn_nvfp4: tile_rows %d needs H and I multiples of 256 (or 128)", a->tile_rows);
  if (a->T > 0 && (!a->x || !a->topk_ids || !a->topk_w || !a->w1_q || !a->w1_sf || !a->w1_gs ||
                   !a->w2_q || !a->w2_sf || !a->w2_gs || !a->out))
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: null required pointer");
  if (!aligned(a->x, 16) || !aligned(a->w1_q, 16) || !aligned(a->w2_q, 16) || !aligned(a->out, 16) ||
      !aligned(a->xq, 16) || !aligned(a->l1_q, 16) || !aligned(a->l1_c_bf16, 16) ||
      !aligned(a->w1_sf, 4) || !aligned(a->w2_sf, 4) || !aligned(a->xsf, 4) || !aligned(a->l1_sf, 4) ||
      !aligned(a->w1_sf_paired, 16) || !aligned(a->w2_sf_paired, 16))
    return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: misaligned pointer");
  return NVFP4_OK;
}

}  // namespace

size_t moe_expert_ffn_nvfp4_workspace_size(const nvfp4_moe_args* args) {
  if (!args || args->T < 0 || args->topk < 1 || args->E < 1 || args->tile_rows < 0) return 0;
  return moe_layout(args).total;
}

int moe_expert_ffn_nvfp4(const nvfp4_moe_args* a, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  int st = moe_validate(a);
  if (st) return st;
  const MoeLayout L = moe_layout(a);
  if (!ws || ws_bytes < L.total)
    return fail(NVFP4_ERR_WORKSPACE, "moe_expert_ffn_nvfp4: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (!aligned(ws, 256)) return fail(NVFP4_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4: ws must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, k = a->topk, P = T * k;
  auto mark = [&](int i) {
    if (a->stage_events) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a->stage_events[i]), s);
  };
  mark(0);

  // a1: activation global scale.  With a computed scale and a grouping that
  // runs in one workgroup, the grouping (a3) shares the launch of the first
  // pass of the scale, and the second pass runs inside the quantization.
  const int64_t mode = moe_tile_rows(a);
  const bool skinny = mode == nvfp4::skinny_tile_rows(), mixed = mode == kMixedTileRows();
  const int route_tile = skinny ? nvfp4::skinny_tile_rows() : nvfp4::gemm_tile_rows();
  const int route_small = mixed ? kMaxShortTiles * nvfp4::skinny_tile_rows() : 0;
  int* offsets = reinterpret_cast<int*>(w + L.offsets);
  int* perm = reinterpret_cast<int*>(w + L.perm);
  nvfp4::GemmTile* tiles = reinterpret_cast<nvfp4::GemmTile*>(w + L.tiles);
  int* ntiles = reinterpret_cast<int*>(w + L.ntiles);
  int* err = a->err_count ? a->err_count : reinterpret_cast<int*>(w + L.err);
  nvfp4::GemmTile* small = reinterpret_cast<nvfp4::GemmTile*>(w + L.small);
  int* nsmall = reinterpret_cast<int*>(w + L.nsmall);
  int* sched = reinterpret_cast<int*>(w + L.sched);
  const int namax = nvfp4::amax_route_blocks(T * H / 8);
  const bool fold = !a->x_gs_in && T > 0 && nvfp4::route_single(P) && namax < 256;
  float* partial = reinterpret_cast<float*>(w + L.partial);
  const float* x_gs;
  if (fold) {
    if ((st = hip_status(nvfp4::launch_amax_route(a->x, T * H, partial, namax, a->topk_ids, P, (int)E, route_tile,
                                                  route_small, nvfp4::skinny_tile_rows(), offsets, perm, tiles,
                                                  ntiles, small, nsmall, err, sched, s),
                         "global scale + route")))
      return st;
    x_gs = a->x_gs_out ? a->x_gs_out : reinterpret_cast<float*>(w + L.x_gs);
  } else if (a->x_gs_in) {
    x_gs = a->x_gs_in;
    if (a->x_gs_out && (st = hip_status(nvfp4::launch_copy_scalar(a->x_gs_in, a->x_gs_out, s), "copy x_gs")))
      return st;
  } else {
    float* g = a->x_gs_out ? a->x_gs_out : reinterpret_cast<float*>(w + L.x_gs);
    if ((st = hip_status(nvfp4::launch_global_scale(a->x, T * H, partial, g, s), "global scale"))) return st;
    x_gs = g;
  }
  mark(1);
  if (T == 0) {
    for (int i = 2; i < 9; ++i) mark(i);
    return NVFP4_OK;
  }
  // a2: quantize the activations
  uint8_t* xq = a->xq ? a->xq : reinterpret_cast<uint8_t*>(w + L.xq);
  uint8_t* xsf = a->xsf ? a->xsf : reinterpret_cast<uint8_t*>(w + L.xsf);
  uint16_t* x_f16 = reinterpret_cast<uint16_t*>(w + L.x_f16);
  if ((st = hip_status(fold ? nvfp4::launch_quantize_folded(a->x, T * H, partial, namax,
                                                            const_cast<float*>(x_gs), xq, xsf, x_f16, s)
                            : nvfp4::launch_quantize(a->x, T * H, x_gs, xq, xsf, x_f16, s),
                       "quantize x")))
    return st;
  mark(2);
  // a3: group pairs by expert (done above when folded)
  // the short tiles of the mixed tiling run on the caller's second stream
  // when it gave one: fork after the work they depend on, join before the
  // work that depends on them
  const bool concurrent = mixed && a->aux_stream;
  hipStream_t aux = concurrent ? reinterpret_cast<hipStream_t>(a->aux_stream) : s;
  auto fork = [&]() -> hipError_t {
    if (!concurrent) return hipSuccess;
    hipEvent_t ev = reinterpret_cast<hipEvent_t>(a->aux_events[0]);
    hipError_t e = hipEventRecord(ev, s);
    return e == hipSuccess ? hipStreamWaitEvent(aux, ev, 0) : e;
  };
  auto join = [&]() -> hipError_t {
    if (!concurrent) return hipSuccess;
    hipEvent_t ev = reinterpret_cast<hipEvent_t>(a->aux_events[1]);
    hipError_t e = hipEventRecord(ev, aux);
    return e == hipSuccess ? hipStreamWaitEvent(s, ev, 0) : e;
  };
  if (!fold && (st = hip_status(nvfp4::launch_route(a->topk_ids, P, (int)E, route_tile, route_small,
                                                    nvfp4::skinny_tile_rows(), offsets, perm, tiles, ntiles,
                                                    small, nsmall, err, reinterpret_cast<int*>(w + L.route),
                                                    sched, s),
                                "route")))
    return st;
  mark(3);
  // a4-a6: L1 GEMM + SwiGLU + compact bf16 + NVFP4 (fused: in the GEMM's
  // epilogue with the supplied scale; unfused: the GEMM writes the bf16 rows,
  // then the scale (supplied, or the dynamic amax of the valid pairs' rows)
  // and a separate quantization pass)
  uint8_t* a2q = a->l1_q ? a->l1_q : reinterpret_cast<uint8_t*>(w + L.a2q);
  uint8_t* a2sf = a->l1_sf ? a->l1_sf : reinterpret_cast<uint8_t*>(w + L.a2sf);
  uint16_t* a2_f16 = reinterpret_cast<uint16_t*>(w + L.a2_f16);
  // the L1 GEMM over the tile list (and the short tiles of the mixed tiling)
  // 32-row tiles only: the buffers of the tail split (its counters follow
  // the 256-row GEMMs' in the zeroed sched area)
  float* split_ws = skinny ? reinterpret_cast<float*>(w + L.split) : nullptr;
  int* split_cnt = skinny ? reinterpret_cast<int*>(w + L.sched) + 16 : nullptr;
  // the 32-row tiles' weight scales: the row-paired copies when given and
  // K (H for L1, I for L2) is a multiple of 1024
  const bool pair1 = a->w1_sf_paired && H % 1024 == 0, pair2 = a->w2_sf_paired && I % 1024 == 0;
  const uint8_t* w1_sf_sk = pair1 ? a->w1_sf_paired : a->w1_sf;
  const uint8_t* w2_sf_sk = pair2 ? a->w2_sf_paired : a->w2_sf;
  auto l1 = [&](const float* out_gs, uint16_t* c_bf16, uint8_t* cq, uint8_t* csf, uint16_t* cf16,
                uint16_t* c_il) {
    hipError_t e = fork();
    if (e == hipSuccess)
      e = skinny ? nvfp4::launch_l1_skinny(x_f16, x_gs, H, a->w1_q, w1_sf_sk, a->w1_gs, 2 * I, out_gs, c_bf16, cq,
                                           csf, cf16, tiles, ntiles, L.max_tiles, 0, perm, (int)k, s, c_il,
                                           nullptr, nullptr, split_ws, split_cnt, pair1)
                 : nvfp4::launch_l1(x_f16, x_gs, H, a->w1_q, a->w1_sf, a->w1_gs, 2 * I, out_gs, c_bf16, cq, csf,
                                    cf16, tiles, ntiles, L.max_tiles, 0, perm, (int)k, s, c_il);
    mark(4);
    if (e == hipSuccess && mixed)
      e = nvfp4::launch_l1_skinny(x_f16, x_gs, H, a->w1_q, w1_sf_sk, a->w1_gs, 2 * I, out_gs, c_bf16, cq, csf,
                                  cf16, small, nsmall, kMaxShortTiles * (int)E, 0, perm, (int)k, aux, c_il,
                                  nullptr, nullptr, nullptr, nullptr, pair1);
    if (e == hipSuccess) e = join();
    return hip_status(e, "L1 GEMM");
  };
  const float* a2_gs = a->a2_gs;
  if (moe_interleaved(a)) {
    uint16_t* c_il = reinterpret_cast<uint16_t*>(w + L.c);
    if ((st = l1(nullptr, a->l1_c_bf16, nullptr, nullptr, nullptr, c_il))) return st;
    if (a->a2_gs_out && (st = hip_status(nvfp4::launch_copy_scalar(a2_gs, a->a2_gs_out, s), "copy a2_gs")))
      return st;
    if ((st = hip_status(nvfp4::launch_quantize_interleaved(c_il, P, I, a2_gs, a2q, a2sf, a2_f16, s),
                         "deinterleave + quantize L1 output")))
      return st;
  } else if (!moe_unfused(a)) {
    if ((st = l1(a->a2_gs, a->l1_c_bf16, a2q, a2sf, a2_f16, nullptr))) return st;
    if (a->a2_gs_out && (st = hip_status(nvfp4::launch_copy_scalar(a->a2_gs, a->a2_gs_out, s), "copy a2_gs")))
      return st;
  } else {
    uint16_t* c = a->l1_c_bf16 ? a->l1_c_bf16 : reinterpret_cast<uint16_t*>(w + L.c);
    if ((st = l1(nullptr, c, nullptr, nullptr, nullptr, nullptr))) return st;
    if (!a2_gs) {
      float* g2 = a->a2_gs_out ? a->a2_gs_out : reinterpret_cast<float*>(w + L.a2_gs);
      if ((st = hip_status(nvfp4::launch_global_scale_rows(c, P, I, a->topk_ids, (int)E,
                                                           reinterpret_cast<float*>(w + L.partial), g2, s),
                           "L1-output global scale")))
        return st;
      a2_gs = g2;
    } else if (a->a2_gs_out &&
               (st = hip_status(nvfp4::launch_copy_scalar(a2_gs, a->a2_gs_out, s), "copy a2_gs"))) {
      return st;
    }
    if ((st = hip_status(nvfp4::launch_quantize(c, P * I, a2_gs, a2q, a2sf, a2_f16, s), "quantize L1 output")))
      return st;
  }
  mark(5);
  // a7: L2 GEMM, weighted by the routing weights
  const bool f16_rows = moe_f16_rows(a);
  float* o = f16_rows ? nullptr : reinterpret_cast<float*>(w + L.o);
  uint16_t* o16 = f16_rows ? reinterpret_cast<uint16_t*>(w + L.o) : nullptr;
  int8_t* oexp = f16_rows ? reinterpret_cast<int8_t*>(w + L.oexp) : nullptr;
  {
    hipError_t e = fork();
    if (e == hipSuccess)
      e = skinny ? nvfp4::launch_l2_skinny(a2_f16, a2_gs, I, a->w2_q, w2_sf_sk, a->w2_gs, H, a->topk_w, o, tiles,
                                           ntiles, L.max_tiles, perm, s, 0, nullptr, nullptr, o16, oexp, split_ws,
                                           split_cnt, pair2)
                 : nvfp4::launch_l2(a2_f16, a2_gs, I, a->w2_q, a->w2_sf, a->w2_gs, H, a->topk_w, o, tiles, ntiles,
                                    L.max_tiles, perm, s, 0, nullptr, reinterpret_cast<int*>(w + L.sched) + 8, o16,
                                    oexp);
    mark(6);
    if (e == hipSuccess && mixed)
      e = nvfp4::launch_l2_skinny(a2_f16, a2_gs, I, a->w2_q, w2_sf_sk, a->w2_gs, H, a->topk_w, o, small, nsmall,
                                  kMaxShortTiles * (int)E, perm, aux, 0, nullptr, nullptr, o16, oexp, nullptr,
                                  nullptr, pair2);
    if (e == hipSuccess) e = join();
    if ((st = hip_status(e, "L2 GEMM"))) return st;
  }
  mark(7);
  // a8: combine the k rows of every token
  if ((st = hip_status(nvfp4::launch_combine(o, a->topk_ids, (int)E, T, (int)k, H, a->out_dtype == 0, a->out, s,
                                             o16, oexp),
                       "combine")))
    return st;
  mark(8);
  return NVFP4_OK;
}

// ------------------------------------------------------------------ no-allocation MoE
// The workspace of moe_expert_ffn_nvfp4_noalloc: a static device array, one
// copy per GPU (each holds it until the process ends).  In host code the
// name `scratch` is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_expert_ffn_nvfp4_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_expert_ffn_nvfp4_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(NVFP4_ERR_HIP, "moe_expert_ffn_nvfp4_noalloc: no device address for the scratch buffer");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

}  // namespace

int moe_expert_ffn_nvfp4_noalloc(const nvfp4_moe_args* a, void* stream) {
  g_last_error[0] = 0;
  int st = moe_validate(a);
  if (st) return st;
  const size_t need = moe_layout(a).total;
  if (need > NVFP4_NOALLOC_SCRATCH_BYTES)
    return fail(NVFP4_ERR_WORKSPACE,
                "moe_expert_ffn_nvfp4_noalloc: this call needs %zu bytes of workspace, more than the %zu-byte "
                "static buffer (use moe_expert_ffn_nvfp4 with a caller workspace)",
                need, (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  // the launch sequence writes every workspace byte it reads (the grouping
  // kernels zero their own counters), so the previous call's contents do
  // not matter
  return moe_expert_ffn_nvfp4(a, ws, NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
