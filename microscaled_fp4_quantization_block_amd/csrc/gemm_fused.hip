// Fused-quantization experiment: the W4A4 GEMM with the activation quantization inside it.
// Each workgroup rotates (H_32) and quantizes (MXFP4) the bf16 rows of A its tile needs,
// buffer by buffer, straight into LDS, instead of reading the codes that a separate
// fp4_quantize launch wrote.  Same tiling, pipeline, arithmetic and MFMA order as the
// library's GEMM (gemm_core.hpp with FA = true), so its output equals fp4_gemm's on
// fp4_quantize(A, MXFP4, 32).  Measured against that two-launch step; every tile of a
// tile row repeats its A panel's quantization (N / 256 times over).
//
// Source: MR-GPTQ abstract (hyper.ai, Résumé): activations rotated and quantized on the
// fly ahead of FP4 GEMM kernels.
#include "gemm_core.hpp"

#include "../../include/fp4_probe.h"

extern "C" int fp4probe_gemm_fused_a(const void* a_bf16, const uint8_t* b_codes, const uint8_t* b_scales,
                                     int64_t M, int64_t N, int64_t K, void* c, int bf16_out, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 256 != 0) return 1;
  if (M * K >= (1ll << 31) || N * (K / 2) >= (1ll << 31)) return 1;
  if (M == 0 || N == 0) return 0;
  if (!a_bf16 || !b_codes || !b_scales || !c) return 1;
  if ((reinterpret_cast<uintptr_t>(a_bf16) | reinterpret_cast<uintptr_t>(b_codes) |
       reinterpret_cast<uintptr_t>(c)) % 16 != 0 || reinterpret_cast<uintptr_t>(b_scales) % 4 != 0)
    return 1;
  constexpr int kWaves = 8;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm<kWaves, true><<<dim3((unsigned)tiles), dim3(64 * kWaves), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint8_t*>(a_bf16), nullptr, b_codes, b_scales, (int)M, (int)N, (int)K, c,
      bf16_out ? fp4impl::DT_BF16 : fp4impl::DT_F32);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
