// Roofline probes: the practical ceilings that the quantization kernels and the GEMM are
// measured against, next to the published peaks.
//
// - fp4probe_hbm_read: workgroups stream contiguous 32 KiB chunks with 16-byte loads,
//   eight in flight per lane, and fold them into one word, so the only traffic is the
//   read itself.  Achieved bytes / time is the read ceiling for a working set of that
//   size.
// - fp4probe_mfma_loop: a register-only loop of v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1
//   operands, shaped like the GEMM's waves (eight waves per workgroup, two per SIMD, a
//   2 x 4 block of 32 x 32 accumulators per wave) and no memory traffic inside the loop.
//   Operand bytes are constant, fixed random, or changed every iteration: the FP4 MFMA
//   power, and under the board's power limit the clock, depends on how the operand bits
//   toggle.
//
// Built as its own library (libfp4probe.so); the quantization library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4_probe.h"

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadDepth = 8;                               // 16-byte loads in flight per lane
constexpr uint64_t kReadChunk = 16ull * kReadThreads * kReadDepth;   // 32 KiB per workgroup step

// Workgroups walk contiguous 32 KiB chunks (grid-stride); in a chunk, load j of lane l
// reads bytes 16 (l + 256 j) .. +15, so every load instruction covers 4 KiB contiguous.
__global__ void __launch_bounds__(kReadThreads) k_hbm_read(const uint4* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t per = kReadChunk / 16;
  uint32_t acc = 0;
  uint64_t c = blockIdx.x;
  for (; (c + 1) * per <= n16; c += gridDim.x) {
    const uint4* q = p + c * per + threadIdx.x;
    uint4 v[kReadDepth];
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) v[j] = q[j * kReadThreads];
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (uint64_t i = c * per + threadIdx.x; i < n16; i += kReadThreads) {    // partial last chunk
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(uint64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

constexpr int kMfmaThreads = 512;   // eight waves, two per SIMD

__global__ void __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_mfma_loop(int iters, int mode, float* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t gid = blockIdx.x * kMfmaThreads + threadIdx.x;
  v8i a[2], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i][r] = mode == 0 ? 0x35353535 : (int)mix(gid * 64u + 8u * i + r);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j][r] = mode == 0 ? 0x53535353 : (int)mix(gid * 64u + 32u + 8u * j + r);
  }
#pragma unroll
  for (int r = 4; r < 8; ++r) {
    a[0][r] = a[1][r] = 0;
    b[0][r] = b[1][r] = b[2][r] = b[3][r] = 0;
  }
  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  const int sa = 127, sb = 120;     // 2^0 and 2^-7: sums stay finite for any iteration count
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 4, 4, 0, sb, 0, sa);
    if (mode == 2) {              // new operand bits every iteration
      const int h = (int)mix((uint32_t)it * 0x9E3779B9u + gid);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[0][r] ^= h; a[1][r] ^= h << 1;
        b[0][r] ^= h >> 1; b[1][r] ^= h << 2; b[2][r] ^= h >> 2; b[3][r] ^= h << 3;
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[gid] = s;
#endif
}

}  // namespace

extern "C" {

int fp4probe_hbm_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks <= 0 || bytes % 16 != 0) return 1;
  k_hbm_read<<<dim3((unsigned)blocks), dim3(kReadThreads), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int fp4probe_mfma_loop(int iters, int mode, int blocks, float* sink, void* stream) {
  if (!sink || blocks <= 0 || iters < 0 || mode < 0 || mode > 2) return 1;
  k_mfma_loop<<<dim3((unsigned)blocks), dim3(kMfmaThreads), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      iters, mode, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
