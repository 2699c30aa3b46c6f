// Internal launcher interface between the C ABI (api.cpp) and the kernel files.
// Arguments are validated by the caller; every launcher enqueues on `stream` and returns
// the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4impl {

enum { FMT_NV = 0, FMT_MX = 1 };
enum { DT_F32 = 0, DT_BF16 = 1 };

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int fmt, int hadamard,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale, bool compute_scale,
                           float* dbg, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             int64_t M, int64_t K, int fmt, int hadamard, void* y, int dtype,
                             hipStream_t stream);

hipError_t launch_residual_quantize(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                                    float eps, const int32_t* perm, int64_t S, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, bool compute_scale,
                                    float* dbg, hipStream_t stream);

hipError_t launch_residual_quantize_mx(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                                       float eps, const int32_t* perm, int64_t S, uint8_t* codes,
                                       uint8_t* scales, float* dbg, hipStream_t stream);

struct PackLayout {
  size_t off_micro, off_group, total;
};
PackLayout pack_layout(int64_t M, int64_t K);

hipError_t launch_pack(const uint16_t* x, int64_t M, int64_t K, uint8_t* packed, float* dbg,
                       hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, int64_t M, int64_t K, uint16_t* y, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, void* c, int ctype, hipStream_t stream);

}  // namespace fp4impl
