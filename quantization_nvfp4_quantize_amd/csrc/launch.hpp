// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// ---- quantize.hip
size_t global_scale_workspace_bytes();
// g = max|x| / 2688 (1 if all zero) over n bf16 values (n % 8 == 0) -> gs[0]
hipError_t launch_global_scale(const uint16_t* x, int64_t n, float* partial, float* gs,
                               hipStream_t s);
hipError_t launch_copy_scalar(const float* src, float* dst, hipStream_t s);
// n bf16 values (n % 16 == 0) -> q [n/2], sf [n/16] with global scale gs[0]
hipError_t launch_quantize(const uint16_t* x, int64_t n, const float* gs, uint8_t* q, uint8_t* sf,
                           hipStream_t s);
hipError_t launch_dequantize(const uint8_t* q, const uint8_t* sf, const float* gs, int64_t n,
                             bool bf16_out, void* out, hipStream_t s);

}  // namespace nvfp4
