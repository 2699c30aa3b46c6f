// W4A4 MXFP4 GEMM of the library (fp4_gemm): the launcher.  The kernel (k_gemm, its tiling,
// LDS pipeline and epilogue) is in gemm_core.hpp.
//
// Sources: MR-GPTQ abstract (hyper.ai, Résumé): FP4 GEMM kernels with the rotation folded
// into the weights and activations quantized on the fly; ARCQuant summary (gist.science,
// Méthodologie item 4): a single GEMM over the reduction axis whose high-precision
// accumulator sums every product.
#include "gemm_core.hpp"

namespace fp4impl {

constexpr int kWaves = 8;

hipError_t launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, void* c, int ctype, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm<kWaves><<<dim3((unsigned)tiles), dim3(64 * kWaves), 0, st>>>(a, sa, b, sb, (int)M, (int)N, (int)K, c, ctype);
  return hipGetLastError();
}

}  // namespace fp4impl
