// C ABI entry points: argument validation, status mapping and dispatch to the launchers.
// Validation happens before any HIP call; no entry point allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/fp4.h"
#include "fp4_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

fp4_status fail(fp4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fp4_status ok() {
  g_last_error[0] = '\0';
  return FP4_OK;
}

fp4_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(FP4_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host-side fault injection for testing the error path without a GPU: with the
// environment variable FP4_FAULT_INJECT=launch, every entry point that passes its
// argument validation reports a launch failure through the same status mapping as a
// real one, and enqueues nothing.  Read on every call, so a test can switch it.
bool launch_failure_injected() {
  const char* v = std::getenv("FP4_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "launch") == 0;
}

#define INJECT_POINT(where)                                                                   \
  do {                                                                                        \
    if (launch_failure_injected()) return hip_status(hipErrorLaunchFailure, where " (injected)"); \
  } while (0)

#define REQUIRE(cond, status, ...) \
  do {                              \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* fp4_status_str(fp4_status s) {
  switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_E_NULL: return "FP4_E_NULL";
    case FP4_E_SHAPE: return "FP4_E_SHAPE";
    case FP4_E_ALIGN: return "FP4_E_ALIGN";
    case FP4_E_UNSUPPORTED: return "FP4_E_UNSUPPORTED";
    case FP4_E_HIP: return "FP4_E_HIP";
  }
  return "FP4_E_UNKNOWN";
}

const char* fp4_last_error(void) { return g_last_error; }

fp4_status fp4_quantize(const void* x, fp4_dtype xt, int64_t M, int64_t K, fp4_format fmt, int hadamard,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale, fp4_scale_mode mode,
                        float* dbg_rotated, void* stream) {
  REQUIRE(fmt == FP4_NVFP4 || fmt == FP4_MXFP4, FP4_E_UNSUPPORTED, "fp4_quantize: unknown format %d", (int)fmt);
  REQUIRE(xt == FP4_F32 || xt == FP4_BF16, FP4_E_UNSUPPORTED, "fp4_quantize: unknown input dtype %d", (int)xt);
  REQUIRE(hadamard == 0 || hadamard == 16 || hadamard == 32 || hadamard == 128, FP4_E_UNSUPPORTED,
          "fp4_quantize: hadamard must be 0, 16, 32 or 128 (got %d)", hadamard);
  REQUIRE(mode == FP4_SCALE_COMPUTE || mode == FP4_SCALE_GIVEN, FP4_E_UNSUPPORTED, "fp4_quantize: bad scale mode");
  REQUIRE(M >= 0 && K >= 0, FP4_E_SHAPE, "fp4_quantize: negative size M=%lld K=%lld", (long long)M, (long long)K);
  REQUIRE(K % 32 == 0, FP4_E_SHAPE, "fp4_quantize: K=%lld is not a multiple of 32", (long long)K);
  REQUIRE(hadamard != 128 || K % 128 == 0, FP4_E_SHAPE,
          "fp4_quantize: the two-level 128 rotation needs K %% 128 == 0 (K=%lld)", (long long)K);
  const bool empty = (M == 0 || K == 0);
  if (fmt == FP4_NVFP4) {
    REQUIRE(tensor_scale != nullptr, FP4_E_NULL, "fp4_quantize: NVFP4 needs tensor_scale");
    REQUIRE(aligned(tensor_scale, 4), FP4_E_ALIGN, "fp4_quantize: tensor_scale not 4-byte aligned");
  } else {
    REQUIRE(tensor_scale == nullptr, FP4_E_UNSUPPORTED, "fp4_quantize: MXFP4 takes no tensor_scale");
  }
  if (!empty) {
    REQUIRE(x && codes && scales, FP4_E_NULL, "fp4_quantize: x, codes and scales are required");
    REQUIRE(aligned(x, 16) && aligned(codes, 16), FP4_E_ALIGN, "fp4_quantize: x and codes must be 16-byte aligned");
    REQUIRE(aligned(scales, 4), FP4_E_ALIGN, "fp4_quantize: scales must be 4-byte aligned");
    REQUIRE(!dbg_rotated || aligned(dbg_rotated, 16), FP4_E_ALIGN, "fp4_quantize: dbg_rotated not 16-byte aligned");
  }
  // an empty tensor only has a tensor scale (0) to produce, and only when computing it
  if (empty && !(fmt == FP4_NVFP4 && mode == FP4_SCALE_COMPUTE)) return ok();
  INJECT_POINT("fp4_quantize");
  hipError_t e = fp4impl::launch_quantize(x, xt == FP4_BF16 ? fp4impl::DT_BF16 : fp4impl::DT_F32, M, K,
                                          fmt == FP4_MXFP4 ? fp4impl::FMT_MX : fp4impl::FMT_NV, hadamard,
                                          codes, scales, tensor_scale,
                                          fmt == FP4_NVFP4 && mode == FP4_SCALE_COMPUTE, dbg_rotated,
                                          reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_quantize");
}

fp4_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t M,
                          int64_t K, fp4_format fmt, int inverse_hadamard, void* y, fp4_dtype yt, void* stream) {
  REQUIRE(fmt == FP4_NVFP4 || fmt == FP4_MXFP4, FP4_E_UNSUPPORTED, "fp4_dequantize: unknown format %d", (int)fmt);
  REQUIRE(yt == FP4_F32 || yt == FP4_BF16, FP4_E_UNSUPPORTED, "fp4_dequantize: unknown output dtype");
  REQUIRE(inverse_hadamard == 0 || inverse_hadamard == 16 || inverse_hadamard == 32 || inverse_hadamard == 128,
          FP4_E_UNSUPPORTED, "fp4_dequantize: inverse_hadamard must be 0, 16, 32 or 128");
  REQUIRE(M >= 0 && K >= 0, FP4_E_SHAPE, "fp4_dequantize: negative size");
  REQUIRE(K % 32 == 0, FP4_E_SHAPE, "fp4_dequantize: K=%lld is not a multiple of 32", (long long)K);
  REQUIRE(inverse_hadamard != 128 || K % 128 == 0, FP4_E_SHAPE,
          "fp4_dequantize: the two-level 128 rotation needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (M == 0 || K == 0) return ok();
  REQUIRE(codes && scales && y, FP4_E_NULL, "fp4_dequantize: codes, scales and y are required");
  REQUIRE(fmt == FP4_MXFP4 || tensor_scale, FP4_E_NULL, "fp4_dequantize: NVFP4 needs tensor_scale");
  REQUIRE(aligned(codes, 16) && aligned(y, 16), FP4_E_ALIGN, "fp4_dequantize: codes and y must be 16-byte aligned");
  REQUIRE(aligned(scales, 4), FP4_E_ALIGN, "fp4_dequantize: scales must be 4-byte aligned");
  INJECT_POINT("fp4_dequantize");
  hipError_t e = fp4impl::launch_dequantize(codes, scales, tensor_scale, M, K,
                                            fmt == FP4_MXFP4 ? fp4impl::FMT_MX : fp4impl::FMT_NV, inverse_hadamard,
                                            y, yt == FP4_BF16 ? fp4impl::DT_BF16 : fp4impl::DT_F32,
                                            reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_dequantize");
}

fp4_status fp4_residual_quantize(const void* x, int64_t M, int64_t K, const float* gamma, float eps,
                                 const int32_t* perm, int64_t S, uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, fp4_scale_mode mode, float* dbg_normed, void* stream) {
  REQUIRE(mode == FP4_SCALE_COMPUTE || mode == FP4_SCALE_GIVEN, FP4_E_UNSUPPORTED, "fp4_residual_quantize: bad scale mode");
  REQUIRE(M >= 0, FP4_E_SHAPE, "fp4_residual_quantize: negative M");
  REQUIRE(K >= 16 && K <= 16384 && K % 16 == 0, FP4_E_SHAPE,
          "fp4_residual_quantize: K=%lld must be a multiple of 16 in [16, 16384]", (long long)K);
  REQUIRE(S >= 0 && S <= K && S % 16 == 0, FP4_E_SHAPE,
          "fp4_residual_quantize: S=%lld must be a multiple of 16 in [0, K]", (long long)S);
  REQUIRE(eps >= 0.0f, FP4_E_SHAPE, "fp4_residual_quantize: eps must be >= 0");
  REQUIRE(tensor_scale != nullptr, FP4_E_NULL, "fp4_residual_quantize: tensor_scale is required");
  REQUIRE(aligned(tensor_scale, 4), FP4_E_ALIGN, "fp4_residual_quantize: tensor_scale not 4-byte aligned");
  REQUIRE(perm != nullptr, FP4_E_NULL, "fp4_residual_quantize: perm is required");
  REQUIRE(aligned(perm, 4) && (!gamma || aligned(gamma, 4)), FP4_E_ALIGN, "fp4_residual_quantize: perm/gamma misaligned");
  if (M > 0) {
    REQUIRE(x && codes && scales, FP4_E_NULL, "fp4_residual_quantize: x, codes and scales are required");
    REQUIRE(aligned(x, 16) && aligned(codes, 16), FP4_E_ALIGN, "fp4_residual_quantize: x and codes must be 16-byte aligned");
    REQUIRE(!dbg_normed || aligned(dbg_normed, 16), FP4_E_ALIGN, "fp4_residual_quantize: dbg_normed misaligned");
  }
  INJECT_POINT("fp4_residual_quantize");
  hipError_t e = fp4impl::launch_residual_quantize(reinterpret_cast<const uint16_t*>(x), M, K, gamma, eps, perm, S,
                                                   codes, scales, tensor_scale, mode == FP4_SCALE_COMPUTE,
                                                   dbg_normed, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_residual_quantize");
}

fp4_status fp4_residual_quantize_mx(const void* x, int64_t M, int64_t K, const float* gamma, float eps,
                                    const int32_t* perm, int64_t S, uint8_t* codes, uint8_t* scales,
                                    float* dbg_normed, void* stream) {
  REQUIRE(M >= 0, FP4_E_SHAPE, "fp4_residual_quantize_mx: negative M");
  REQUIRE(K >= 32 && K <= 16384 && K % 32 == 0, FP4_E_SHAPE,
          "fp4_residual_quantize_mx: K=%lld must be a multiple of 32 in [32, 16384]", (long long)K);
  REQUIRE(S >= 0 && S <= K && S % 32 == 0, FP4_E_SHAPE,
          "fp4_residual_quantize_mx: S=%lld must be a multiple of 32 in [0, K]", (long long)S);
  REQUIRE(eps >= 0.0f, FP4_E_SHAPE, "fp4_residual_quantize_mx: eps must be >= 0");
  REQUIRE(perm != nullptr, FP4_E_NULL, "fp4_residual_quantize_mx: perm is required");
  REQUIRE(aligned(perm, 4) && (!gamma || aligned(gamma, 4)), FP4_E_ALIGN,
          "fp4_residual_quantize_mx: perm/gamma misaligned");
  if (M > 0) {
    REQUIRE(x && codes && scales, FP4_E_NULL, "fp4_residual_quantize_mx: x, codes and scales are required");
    REQUIRE(aligned(x, 16) && aligned(codes, 16), FP4_E_ALIGN,
            "fp4_residual_quantize_mx: x and codes must be 16-byte aligned");
    REQUIRE(!dbg_normed || aligned(dbg_normed, 16), FP4_E_ALIGN, "fp4_residual_quantize_mx: dbg_normed misaligned");
  }
  INJECT_POINT("fp4_residual_quantize_mx");
  hipError_t e = fp4impl::launch_residual_quantize_mx(reinterpret_cast<const uint16_t*>(x), M, K, gamma, eps, perm,
                                                      S, codes, scales, dbg_normed,
                                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_residual_quantize_mx");
}

size_t fp4_pack_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K % 128 != 0) return 0;
  return fp4impl::pack_layout(M, K).total;
}

fp4_status fp4_pack(const void* x, int64_t M, int64_t K, void* packed, float* dbg_rotated, void* stream) {
  REQUIRE(M >= 0 && K >= 0, FP4_E_SHAPE, "fp4_pack: negative size");
  REQUIRE(K % 128 == 0, FP4_E_SHAPE, "fp4_pack: K=%lld is not a multiple of 128", (long long)K);
  if (M == 0 || K == 0) return ok();
  REQUIRE(x && packed, FP4_E_NULL, "fp4_pack: x and packed are required");
  REQUIRE(aligned(x, 16) && aligned(packed, 256), FP4_E_ALIGN, "fp4_pack: x must be 16-byte, packed 256-byte aligned");
  REQUIRE(!dbg_rotated || aligned(dbg_rotated, 16), FP4_E_ALIGN, "fp4_pack: dbg_rotated misaligned");
  INJECT_POINT("fp4_pack");
  hipError_t e = fp4impl::launch_pack(reinterpret_cast<const uint16_t*>(x), M, K, reinterpret_cast<uint8_t*>(packed),
                                      dbg_rotated, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_pack");
}

fp4_status fp4_unpack(const void* packed, int64_t M, int64_t K, void* y, void* stream) {
  REQUIRE(M >= 0 && K >= 0, FP4_E_SHAPE, "fp4_unpack: negative size");
  REQUIRE(K % 128 == 0, FP4_E_SHAPE, "fp4_unpack: K=%lld is not a multiple of 128", (long long)K);
  if (M == 0 || K == 0) return ok();
  REQUIRE(packed && y, FP4_E_NULL, "fp4_unpack: packed and y are required");
  REQUIRE(aligned(y, 16) && aligned(packed, 256), FP4_E_ALIGN, "fp4_unpack: y must be 16-byte, packed 256-byte aligned");
  INJECT_POINT("fp4_unpack");
  hipError_t e = fp4impl::launch_unpack(reinterpret_cast<const uint8_t*>(packed), M, K, reinterpret_cast<uint16_t*>(y),
                                        reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_unpack");
}

fp4_status fp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                    int64_t M, int64_t N, int64_t K, void* c, fp4_dtype ct, void* stream) {
  REQUIRE(ct == FP4_F32 || ct == FP4_BF16, FP4_E_UNSUPPORTED, "fp4_gemm: unknown output dtype");
  REQUIRE(M >= 0 && N >= 0 && K >= 0, FP4_E_SHAPE, "fp4_gemm: negative size");
  REQUIRE(K % 128 == 0 && K > 0, FP4_E_SHAPE, "fp4_gemm: K=%lld must be a positive multiple of 128", (long long)K);
  REQUIRE(M * (K / 2) < (1ll << 31) && N * (K / 2) < (1ll << 31), FP4_E_SHAPE,
          "fp4_gemm: each operand's codes must stay below 2 GiB");
  if (M == 0 || N == 0) return ok();
  REQUIRE(a_codes && a_scales && b_codes && b_scales && c, FP4_E_NULL, "fp4_gemm: every operand is required");
  REQUIRE(aligned(a_codes, 16) && aligned(b_codes, 16) && aligned(c, 16), FP4_E_ALIGN,
          "fp4_gemm: codes and c must be 16-byte aligned");
  REQUIRE(aligned(a_scales, 4) && aligned(b_scales, 4), FP4_E_ALIGN, "fp4_gemm: scales must be 4-byte aligned");
  INJECT_POINT("fp4_gemm");
  hipError_t e = fp4impl::launch_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, c,
                                      ct == FP4_BF16 ? fp4impl::DT_BF16 : fp4impl::DT_F32,
                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "fp4_gemm");
}

}  // extern "C"
