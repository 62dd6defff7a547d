// extern "C" boundary of libnvfp4moe.so: argument validation, workspace
// carving and the launch sequence on the caller's stream.  Every check runs
// before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/nvfp4moe.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

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
  return hip_status(nvfp4::launch_quantize(x, n, gs, q, sf, s), "nvfp4_quantize");
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

// ------------------------------------------------------------------ GEMM stage
size_t nvfp4_gemm_swiglu_quant_workspace_size(int64_t M, int64_t K, int64_t N2) {
  (void)M;
  (void)K;
  (void)N2;
  return 0;
}

int nvfp4_gemm_swiglu_quant(const uint8_t* a_q, const uint8_t* a_sf, const float* a_gs, int64_t M,
                            int64_t K, const uint8_t* w_q, const uint8_t* w_sf, const float* w_gs,
                            int64_t N2, const float* out_gs, uint16_t* c_bf16, uint8_t* c_q,
                            uint8_t* c_sf, void* ws, size_t ws_bytes, void* stream) {
  (void)a_q; (void)a_sf; (void)a_gs; (void)M; (void)K; (void)w_q; (void)w_sf; (void)w_gs;
  (void)N2; (void)out_gs; (void)c_bf16; (void)c_q; (void)c_sf; (void)ws; (void)ws_bytes;
  (void)stream;
  return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_gemm_swiglu_quant: not available in this build");
}

// ------------------------------------------------------------------ MoE
size_t moe_expert_ffn_nvfp4_workspace_size(const nvfp4_moe_args* args) {
  (void)args;
  return 0;
}

int moe_expert_ffn_nvfp4(const nvfp4_moe_args* args, void* ws, size_t ws_bytes, void* stream) {
  (void)args; (void)ws; (void)ws_bytes; (void)stream;
  return fail(NVFP4_ERR_UNSUPPORTED, "moe_expert_ffn_nvfp4: not available in this build");
}

}  // extern "C"
