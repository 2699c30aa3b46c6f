/*
 * fp4.h -- C ABI of the micro-scaled FP4 quantization library for AMD Instinct MI355X
 * (gfx950).  Every entry point takes plain pointers and sizes; no C++ or PyTorch type
 * crosses this boundary.
 *
 * Common rules
 * ------------
 * - Pointers are DEVICE memory unless a comment says otherwise; the caller allocates
 *   and owns every buffer.  The library never allocates, frees or synchronises.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *   enqueued on it in call order; results are visible after the caller synchronises.
 * - Tensors are row-major [M][K] with K (the channel / reduction axis) contiguous.
 * - E2M1 codes: two per byte, element 2j in bits 0-3, element 2j+1 in bits 4-7; a code
 *   is sign(bit 3) | magnitude index (0..7 for 0, .5, 1, 1.5, 2, 3, 4, 6).
 * - Scales: one byte per block, row-major [M][K / block]: E4M3 bit patterns (NVFP4,
 *   block 16) or E8M0 biased exponents (MXFP4, block 32, value 2^(code-127)).
 * - Every call validates its arguments before any HIP call and returns a status; it
 *   never throws, aborts or prints.  Launch failures map to FP4_E_HIP.  Device faults
 *   surface at the caller's next synchronisation.  Inputs must be finite.
 * - Data pointers must be 16-byte aligned (scale and permutation pointers: 4-byte).
 * - The library is stateless and thread-safe.
 */
#ifndef FP4_MI355X_H
#define FP4_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_E_NULL = 1,        /* a required pointer is NULL                                  */
  FP4_E_SHAPE = 2,       /* negative size, or a size not a multiple of the block/group  */
  FP4_E_ALIGN = 3,       /* a pointer misses its alignment                               */
  FP4_E_UNSUPPORTED = 4, /* format / rotation / dtype combination not provided           */
  FP4_E_HIP = 5          /* the HIP runtime reported an error                            */
} fp4_status;

typedef enum { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;
typedef enum { FP4_F32 = 0, FP4_BF16 = 1 } fp4_dtype;
typedef enum { FP4_SCALE_COMPUTE = 0, FP4_SCALE_GIVEN = 1 } fp4_scale_mode;

/*
 * fp4_quantize -- block Hadamard rotation (optional) + micro-scaled FP4 quantization.
 *
 * Defined by: the MR-GPTQ abstract (hyper.ai, Résumé: block Hadamard transforms before
 * MXFP4 / NVFP4 quantization, activations rotated on the fly) and the ARCQuant summary
 * (gist.science, Énoncé du Problème: NVFP4 blocks of 16; Méthodologie item 2: standard
 * block NVFP4).
 *
 *   x            [M][K] input, dtype xt (FP4_F32 or FP4_BF16)
 *   fmt          FP4_NVFP4: E4M3 scale per 16 + one fp32 tensor scale
 *                FP4_MXFP4: E8M0 scale per 32
 *   hadamard     0 (none), 16 or 32: orthonormal Sylvester H_n applied to every
 *                contiguous n-block of a row before quantization; 128: the two-level
 *                transform of every contiguous 128-group (H_16 inside each 16-element
 *                micro-group, then H_8 across the group's 8 micro-groups; equal to the
 *                Sylvester H_128), after the FP4Quant abstract (paperdot.bitmofang.com:
 *                hybrid two-level FWHT)
 *   codes        [M][K/2] output bytes
 *   scales       [M][K/16] (NVFP4) or [M][K/32] (MXFP4) output bytes
 *   tensor_scale NVFP4 only, one fp32: written (FP4_SCALE_COMPUTE: fl32(amax/2688) of the
 *                rotated tensor) or read (FP4_SCALE_GIVEN).  Must be NULL for MXFP4.
 *   dbg_rotated  optional [M][K] fp32 output of the rotated values (NULL = not written)
 * Shapes: M >= 0, K >= 0, K % 32 == 0 (K % 128 == 0 with hadamard 128).  M*K == 0 is a
 * no-op (NVFP4 COMPUTE writes 0).
 * Unrotated codes and scales are the exact round-to-nearest-even decisions of x/scale.
 * Rotated input is quantized from its binary32 rotated values with binary32 scale and
 * element arithmetic: a decision can differ from the exact one only where the real
 * quotient lies within a few binary32 ulps of a rounding boundary.
 */
fp4_status fp4_quantize(const void* x, fp4_dtype xt, int64_t M, int64_t K, fp4_format fmt,
                        int hadamard, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                        fp4_scale_mode mode, float* dbg_rotated, void* stream);

/*
 * fp4_dequantize -- values of quantized codes, with the optional inverse rotation.
 *
 * Mirror of fp4_quantize (same sources).  y[m][k] = fl32(V(code) * s_b * s_t) for
 * NVFP4 or V(code) * 2^(e-127) for MXFP4, then H_n applied per n-block when
 * inverse_hadamard is 16 or 32, or the two-level 128 transform per 128-group when it is
 * 128 (each is its own inverse), then rounded to yt (bf16: nearest-even from the fp32
 * value).  tensor_scale: NVFP4 only (1 fp32, read).  Shapes as fp4_quantize.
 */
fp4_status fp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                          int64_t M, int64_t K, fp4_format fmt, int inverse_hadamard,
                          void* y, fp4_dtype yt, void* stream);

/*
 * fp4_residual_quantize -- ARCQuant fused activation kernel: RMSNorm, channel reorder,
 * primary NVFP4 and residual NVFP4 of the first S reordered channels.
 *
 * Defined by the ARCQuant summary (gist.science/fr/paper/2601.07475), Méthodologie
 * items 1-3 and 5: channels reordered by absolute maximum (the order is a calibration
 * product and arrives as `perm`), primary block NVFP4, residual (original minus primary
 * quantized value) of the outlier channels quantized into extra NVFP4 channels,
 * concatenated along K; one fused kernel produces the GEMM-ready layout.
 *
 *   x            [M][K] bf16 activations
 *   gamma        [K] fp32 RMSNorm weight, or NULL for unit weight
 *   eps          RMSNorm epsilon: y = x / sqrt(mean(x^2) + eps) * gamma
 *   perm         [K] int32 permutation: reordered channel c takes y[:, perm[c]]
 *   S            residual channels (the first S reordered ones), S % 16 == 0, S <= K
 *   codes        [M][(K+S)/2] output: per row K/2 primary bytes then S/2 residual bytes
 *   scales       [M][(K+S)/16] output E4M3: K/16 primary then S/16 residual
 *   tensor_scale one fp32 shared by both parts: written (COMPUTE: fl32(max|z|/2688)) or
 *                read (GIVEN)
 *   dbg_normed   optional [M][K] fp32 output of the normalized, reordered values z
 * Shapes: K % 16 == 0, 16 <= K <= 16384.  perm must be a permutation (not checked).
 */
fp4_status fp4_residual_quantize(const void* x, int64_t M, int64_t K, const float* gamma, float eps,
                                 const int32_t* perm, int64_t S, uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, fp4_scale_mode mode, float* dbg_normed,
                                 void* stream);

/*
 * fp4_residual_quantize_mx -- MXFP4 flavour of fp4_residual_quantize: RMSNorm, channel
 * reorder, primary MXFP4 and residual MXFP4 of the first S reordered channels.
 *
 * Defined by the ARCQuant summary (gist.science/fr/paper/2601.07475): Méthodologie
 * items 1-3 for the steps, Résultats Expérimentaux (Généralisabilité) for the extension
 * of the augmented-residual scheme to MXFP4.  Per 32-channel block of z: E8M0 scale
 * 2^(floor(log2 amax) - 2), codes E2M1_RNE(z / scale); residual r = z - (primary value)
 * on the first S channels, quantized the same way with its own scales.  No tensor scale.
 * The output feeds fp4_gemm directly with K' = K + S against weights whose columns are
 * reordered by `perm` and whose first S reordered columns are repeated after them.
 *
 *   x, gamma, eps, perm   as for fp4_residual_quantize
 *   S            residual channels, S % 32 == 0, S <= K
 *   codes        [M][(K+S)/2] output: K/2 primary bytes then S/2 residual bytes per row
 *   scales       [M][(K+S)/32] output E8M0: K/32 primary then S/32 residual
 *   dbg_normed   optional [M][K] fp32 output of the normalized, reordered values z
 * Shapes: K % 32 == 0, 32 <= K <= 16384.  perm must be a permutation (not checked).
 */
fp4_status fp4_residual_quantize_mx(const void* x, int64_t M, int64_t K, const float* gamma, float eps,
                                    const int32_t* perm, int64_t S, uint8_t* codes, uint8_t* scales,
                                    float* dbg_normed, void* stream);

/*
 * fp4_pack_bytes -- HOST function, no device work: size in bytes of the packed
 * dual-scale message of an [M][K] tensor (K % 128 == 0), or 0 for invalid sizes.
 *
 * Layout (FP4Quant abstract, paperdot.bitmofang.com: micro-grouped dual-scale FP4 with
 * sub-byte packing; the layout itself is this library's): three planar sections, each
 * starting at a multiple of 256 bytes:
 *   [0]            E2M1 codes, [M][K/2] bytes
 *   [off_micro]    E4M3 micro-group scales, one per 16 elements, [M][K/16] bytes
 *   [off_group]    fp32 group scales, one per 128 elements, [M][K/128], little-endian
 * off_micro = align256(M*K/2), off_group = align256(off_micro + M*K/16),
 * total = align256(off_group + 4*M*K/128).
 */
size_t fp4_pack_bytes(int64_t M, int64_t K);

/*
 * fp4_pack -- FP4Quant micro-grouped dual-scale FP4 compression of a bf16 tensor.
 *
 * Defined by the FP4Quant abstract (paperdot.bitmofang.com): a hybrid two-level FWHT
 * lowers quantization error, a micro-grouped dual-scale quantization keeps local
 * distribution characteristics, and packing gives a compact sub-byte message.  Per
 * 128-group: y = H_8 across the 8 micro-groups of (H_16 within each micro-group of x);
 * s_g = fl32(amax(y)/2688); per micro-group s_m = E4M3(amax/(6 s_g)); codes
 * E2M1(y/(s_m s_g)).  packed must hold fp4_pack_bytes(M, K) bytes; K % 128 == 0.
 * dbg_rotated: optional [M][K] fp32 output of y.
 */
fp4_status fp4_pack(const void* x, int64_t M, int64_t K, void* packed, float* dbg_rotated,
                    void* stream);

/*
 * fp4_unpack -- inverse of fp4_pack: y_hat = fl32(V * s_m * s_g), the same two-level
 * FWHT (its own inverse), bf16 nearest-even output y [M][K].
 */
fp4_status fp4_unpack(const void* packed, int64_t M, int64_t K, void* y, void* stream);

/*
 * fp4_gemm -- W4A4 MXFP4 GEMM: C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulation.
 *
 * Defined by the MR-GPTQ abstract (hyper.ai, Résumé: FP4 GEMM kernels with the rotation
 * fused into the weights offline, activations rotated and quantized on the fly) and
 * the ARCQuant summary (Méthodologie item 4: one GEMM over the reduction axis, the
 * high-precision accumulator summing every product).  A and B are MXFP4 (E2M1 codes,
 * E8M0 scale per 32 along K), both K-contiguous ("TN"):
 *   a_codes [M][K/2], a_scales [M][K/32], b_codes [N][K/2], b_scales [N][K/32],
 *   c [M][N] in ct (FP4_BF16: nearest-even from the fp32 sum; FP4_F32).
 * Shapes: M, N >= 0, K > 0, K % 128 == 0, M*K/2 and N*K/2 below 2^31 bytes.
 * Reads nothing outside the four operands, for every admitted shape: where a load's
 * 16 bytes would reach past an operand's last row (ragged M/N tiles, a half last
 * 256-element step of K, a half last scale group), the hardware range check returns zeros.
 * Deterministic: the fp32 summation order of C[m][n] depends only on K and on the parity
 * of n / 256, so a product over the rows of B from a multiple of 512 onward (a column
 * shard) gives the same bits as those columns of the wider product.
 */
fp4_status fp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c, fp4_dtype ct,
                    void* stream);

/* Human-readable name of a status (static string; host function). */
const char* fp4_status_str(fp4_status s);

/* Detail of the last failing call on this host thread (static per-thread buffer). */
const char* fp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_H */
