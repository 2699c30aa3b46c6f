/*
 * fp4_probe.h -- roofline probes of MI355X (gfx950) and a fused-quantization experiment,
 * built as libfp4probe.so next to the quantization library.  The probes measure the
 * practical ceilings that the quantization kernels (HBM bandwidth) and the W4A4 GEMM
 * (scaled FP4 MFMA throughput) are compared with, beside the published peaks.  Not part
 * of the quantization ABI (fp4.h); the benchmark's calibration and experiment workloads
 * call them.
 *
 * Pointers are device memory owned by the caller; `stream` is a hipStream_t as void*
 * (NULL = default stream).  Return 0 on success, 1 for invalid arguments (nothing is
 * launched), 2 when the launch reports an error.  Nothing is allocated or synchronised.
 */
#ifndef FP4_MI355X_PROBE_H
#define FP4_MI355X_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fp4probe_hbm_read -- read `bytes` (a multiple of 16) of `buf` once with coalesced
 * 16-byte loads over `blocks` workgroups of 256 lanes: each workgroup walks contiguous
 * 32 KiB chunks (grid-stride), eight loads in flight per lane.  sink: [blocks * 256]
 * uint32 output, one folded word per lane.
 */
int fp4probe_hbm_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, void* stream);

/*
 * fp4probe_mfma_loop -- `iters` iterations of eight v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1
 * operands, E8M0 scales) per wave in registers, `blocks` workgroups of eight waves (two
 * per SIMD).  FLOP per launch = blocks * 8 * iters * 8 * 131072.
 *   mode 0: constant operand bytes; 1: fixed random bytes; 2: bytes changed every iteration.
 * sink: [blocks * 512] fp32 output (the accumulator sums, so the loop is not removed).
 */
int fp4probe_mfma_loop(int iters, int mode, int blocks, float* sink, void* stream);

/*
 * fp4probe_gemm_fused_a -- the W4A4 MXFP4 GEMM with the activation quantization fused into
 * it: C [M][N] = A B^T where A is bf16 [M][K], rotated by H_32 and quantized to MXFP4 inside
 * every tile (MR-GPTQ abstract, hyper.ai, Résumé: activations rotated and quantized on the
 * fly), and B is MXFP4 as for fp4_gemm (b_codes [N][K/2], b_scales [N][K/32] E8M0).  The
 * result equals fp4_gemm on fp4_quantize(A, MXFP4, 32)'s output.  An experiment measured
 * against that two-launch step, not a library entry point.  K % 256 == 0, M K < 2^31;
 * pointers 16-byte aligned (scales 4).  c: bf16 (bf16_out != 0) or fp32.
 */
int fp4probe_gemm_fused_a(const void* a_bf16, const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                          int64_t N, int64_t K, void* c, int bf16_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_PROBE_H */
