// ARCQuant fused activation kernel: RMSNorm + channel reorder + primary NVFP4 + residual
// NVFP4 of the first S reordered channels, written as one [K | S] row.
//
// Source: ARCQuant summary (gist.science/fr/paper/2601.07475), Méthodologie: channels
// reordered by absolute maximum (item 1); primary block NVFP4 and residual = original
// minus primary quantized value for the outlier channels, quantized into a second set of
// NVFP4 channels (item 2); residual channels concatenated along K (item 3); one fused
// kernel for reorder, RMSNorm, primary and residual quantization emitting the GEMM-ready
// layout (item 5).
//
// One workgroup walks rows (persistent, stride gridDim.x).  Per row: coalesced 16-element
// loads accumulate sum(x^2) and park x as fp32 in LDS; a workgroup reduction gives
// 1/rms; each lane then gathers its 16 reordered channels z[c] = x[perm[c]] / rms * gamma
// from LDS (perm is staged in LDS once per workgroup) and encodes them; lanes whose block
// lies in the first S channels also encode the residual z - V s_b s_t (one fma, a single
// rounding of the exact difference).  The dynamic tensor scale needs max|z| first: the
// same kernel runs once in statistics mode (identical arithmetic up to z) before the
// quantizing launch.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ void k_zero_scalar(float* p) { *p = 0.0f; }
__global__ void k_finalize_tensor_scale(float* p) { *p = *p / 2688.0f; }

template <bool STATS>
__global__ void __launch_bounds__(kThreads)
k_arcquant(const uint16_t* __restrict__ x, int64_t M, int K, const float* __restrict__ gamma, float eps,
           const int32_t* __restrict__ perm, int S, uint8_t* __restrict__ codes,
           uint8_t* __restrict__ scales, float* tensor_scale, float* __restrict__ dbg) {
  extern __shared__ float smem[];
  float* xs = smem;                                        // [K] row values
  int32_t* ps = reinterpret_cast<int32_t*>(smem + K);      // [K] permutation
  __shared__ float red[kWaves];

  const int t = threadIdx.x;
  const int nblk = K / 16;
  // an index outside [0, K) (not a permutation: caller error) is clamped, never dereferenced
  for (int c = t; c < K; c += kThreads) ps[c] = (int32_t)min((uint32_t)perm[c], (uint32_t)(K - 1));
  const float s_t = STATS ? 0.0f : *tensor_scale;
  const int64_t row_codes = (K + S) / 2, row_scales = (K + S) / 16;
  float tmax = 0.0f;

  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const uint16_t* xr = x + r * K;
    float ss = 0.0f;
    for (int b = t; b < nblk; b += kThreads) {
      float v[16];
      load_bf16<16>(xr + 16 * b, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(v[i], v[i], ss);
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<float4*>(xs + 16 * b + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();                                       // xs, ps and red complete
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += red[w];
    const float inv_rms = 1.0f / sqrtf(tot / (float)K + eps);

    for (int b = t; b < nblk; b += kThreads) {
      float z[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int p = ps[16 * b + i];
        float y = xs[p] * inv_rms;
        z[i] = gamma ? y * gamma[p] : y;
      }
      if (dbg) store_f32<16>(dbg + r * K + 16 * b, z);
      if constexpr (STATS) {
        tmax = fmaxf(tmax, absmax<16>(z));
      } else {
        uint32_t sb = nvfp4_block_scale(absmax<16>(z), s_t);
        float sbv = e4m3_value(sb);
        float S32 = sbv * s_t;
        float E = S32 > 0.0f ? 1.0f / S32 : 0.0f;
        uint2 w = nvfp4_encode16_fast(z, E);
        *reinterpret_cast<uint2*>(codes + r * row_codes + 8 * b) = w;
        scales[r * row_scales + b] = (uint8_t)sb;
        if (16 * b < S) {
          float q[16];
          e2m1_decode8(w.x, 1.0f, q);
          e2m1_decode8(w.y, 1.0f, q + 8);
#pragma unroll
          for (int i = 0; i < 16; ++i) q[i] = fmaf(-(q[i] * sbv), s_t, z[i]);   // z - V s_b s_t
          uint32_t sr = nvfp4_block_scale(absmax<16>(q), s_t);
          float R32 = e4m3_value(sr) * s_t;
          float Er = R32 > 0.0f ? 1.0f / R32 : 0.0f;
          *reinterpret_cast<uint2*>(codes + r * row_codes + K / 2 + 8 * b) = nvfp4_encode16_fast(q, Er);
          scales[r * row_scales + nblk + b] = (uint8_t)sr;
        }
      }
    }
    __syncthreads();                                       // xs reused by the next row
  }
  if constexpr (STATS) {
    tmax = wave_max(tmax);
    if ((t & 63) == 0 && tmax > 0.0f) atomic_max_nonneg(tensor_scale, tmax);
  }
}

}  // namespace

namespace fp4impl {

hipError_t launch_residual_quantize(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                                    float eps, const int32_t* perm, int64_t S, uint8_t* codes,
                                    uint8_t* scales, float* ts, bool compute, float* dbg,
                                    hipStream_t st) {
  size_t lds = (size_t)K * 8;
  if (lds > 65536) {   // rows beyond 8192 channels need more than the default 64 KiB of LDS
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_arcquant<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_arcquant<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  unsigned grid = (unsigned)(M < 2048 ? (M > 0 ? M : 1) : 2048);
  if (compute) {
    k_zero_scalar<<<1, 1, 0, st>>>(ts);
    if (M) k_arcquant<true><<<grid, kThreads, lds, st>>>(x, M, (int)K, gamma, eps, perm, (int)S, codes,
                                                        scales, ts, nullptr);
    k_finalize_tensor_scale<<<1, 1, 0, st>>>(ts);
  }
  if (M) k_arcquant<false><<<grid, kThreads, lds, st>>>(x, M, (int)K, gamma, eps, perm, (int)S, codes,
                                                       scales, ts, dbg);
  return hipGetLastError();
}

}  // namespace fp4impl
