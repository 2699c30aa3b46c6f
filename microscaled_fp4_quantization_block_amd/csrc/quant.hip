// Block-Hadamard + micro-scaled FP4 quantization and dequantization (NVFP4 and MXFP4).
//
// Work decomposition: one lane owns one 32-element chunk of a row (K % 32 == 0, so a
// chunk never straddles rows and its codes are one 16-byte store).  A chunk holds whole
// Hadamard blocks (16 or 32), one MXFP4 block or two NVFP4 blocks, so rotation, block
// maxima, scale choice and encoding all stay in the lane's registers; the only
// cross-lane step is the per-tensor maximum of NVFP4 (a grid-stride pass before the
// quantization launch, reduced over each workgroup before its one atomic), and for the
// two-level 128 rotation the DPP butterflies across a quad of chunks.
//
// Sources: MR-GPTQ abstract (hyper.ai, Résumé) for block Hadamard before MXFP4 / NVFP4
// quantization and online activation rotation; ARCQuant summary (gist.science, Énoncé du
// Problème) for NVFP4 blocks of 16.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr float kTensorDivisor = 2688.0f;   // largest E4M3 scale (448) x largest E2M1 value (6)

template <int DT>
__device__ __forceinline__ void load_chunk(const void* x, int64_t chunk, float* v) {
  if constexpr (DT == fp4impl::DT_BF16)
    load_bf16<32>(reinterpret_cast<const uint16_t*>(x) + chunk * 32, v);
  else
    load_f32<32>(reinterpret_cast<const float*>(x) + chunk * 32, v);
}

__global__ void k_zero_scalar(float* p) { *p = 0.0f; }

// Tensor scale s_t = fl32(max|H x| / 2688) by a running atomic max into *ts (which starts
// at 0).  A grid-stride walk over the chunks, reduced over the workgroup before its one
// atomic: atomics on a single address serialise, so the grid is capped at kAmaxGroups.
// Each workgroup contributes fl32(m / 2688) of its own maximum m: correctly rounded
// division by a positive constant is monotone, so the maximum of the rounded quotients is
// the rounded quotient of the maximum, and no finishing step is needed.
constexpr int kAmaxThreads = 1024, kAmaxGroups = 256;
template <int DT, int H>
__global__ void __launch_bounds__(kAmaxThreads) k_amax(const void* x, int64_t nchunks, float* ts) {
  __shared__ float wm[kAmaxThreads / 64];
  float m = 0.0f;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * blockDim.x) {
    float v[32];
    load_chunk<DT>(x, c, v);
    chunk_rotate<H>(v, c);
    m = fmaxf(m, absmax<32>(v));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, wm[w]);
    if (m > 0.0f) atomic_max_nonneg(ts, m / kTensorDivisor);
  }
}

template <int DT, int H>
__global__ void __launch_bounds__(kThreads)
k_quant_mx(const void* x, int64_t nchunks, uint8_t* codes, uint8_t* scales, float* dbg) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  float v[32];
  load_chunk<DT>(x, c, v);
  chunk_rotate<H>(v, c);
  if (dbg) store_f32<32>(dbg + c * 32, v);
  uint32_t e = e8m0_from_amax(absmax<32>(v));
  store_out(reinterpret_cast<uint4*>(codes) + c, e2m1_encode32(v, e8m0_value(e)));
  store_out(scales + c, (uint8_t)e);
}

// NVFP4: two 16-blocks per chunk.  Unrotated input takes the exact scale and element
// decisions (binary32 with a certified margin, float64 quotients where the margin is too
// thin); rotated input (already fp32-rounded) the fast ones.
template <int DT, int H>
__global__ void __launch_bounds__(kThreads)
k_quant_nv(const void* x, int64_t nchunks, uint8_t* codes, uint8_t* scales,
           const float* tensor_scale, float* dbg) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  const float s_t = *tensor_scale;
  float v[32];
  load_chunk<DT>(x, c, v);
  chunk_rotate<H>(v, c);
  if (dbg) store_f32<32>(dbg + c * 32, v);
  uint2 w[2];
  uint32_t sb[2];
  const float inv6s = recip_fast(6.0f * s_t);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if constexpr (H == 0) {
      // Exact decisions: binary32 with a certified margin, float64 where it is too thin.
      const float amax = absmax<16>(v + 16 * b);
      bool ok = checked_divisor(6.0f * s_t) && nvfp4_block_scale_checked(amax, inv6s, sb[b]);
      if (!ok) sb[b] = nvfp4_block_scale(amax, s_t);
      const float S32 = e4m3_value(sb[b]) * s_t;
      ok = checked_divisor(S32) && nvfp4_encode16_checked(v + 16 * b, recip_fast(S32), w[b]);
      if (!ok) {
        w[b] = nvfp4_encode16_exact(v + 16 * b, (double)e4m3_value(sb[b]) * (double)s_t);   // S exact
      }
    } else {
      sb[b] = nvfp4_block_scale_fast(absmax<16>(v + 16 * b), inv6s);
      w[b] = nvfp4_encode16_fast(v + 16 * b, recip_fast(e4m3_value(sb[b]) * s_t));
    }
  }
  store_out(reinterpret_cast<uint4*>(codes) + c, make_uint4(w[0].x, w[0].y, w[1].x, w[1].y));
  store_out(reinterpret_cast<uint16_t*>(scales) + c, (uint16_t)(sb[0] | (sb[1] << 8)));
}

// Dequantization: fl32(V s_b s_t) (NVFP4) or V 2^(e-127) (MXFP4), optional H, store.
// Written by quads: lane p of a quad owns elements 8 p .. 8 p + 7 of a 32-element chunk
// (one 4-byte code word), so the stores of a wave are 1 KiB contiguous for bf16 output;
// rotation finishes with DPP butterflies across the quad.  kDeqUnits units per lane,
// all loads issued before any conversion.
constexpr int kDeqUnits = 4;

template <int FMT, int H, int OUT>
__global__ void __launch_bounds__(kThreads)
k_dequant(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t n8, void* y) {
  const int64_t base = (int64_t)blockIdx.x * (kDeqUnits * blockDim.x) + threadIdx.x;
  uint32_t cw[kDeqUnits], sc[kDeqUnits];
#pragma unroll
  for (int u = 0; u < kDeqUnits; ++u) {
    const int64_t i = base + (int64_t)u * blockDim.x;
    const bool ok = i < n8;
    cw[u] = ok ? reinterpret_cast<const uint32_t*>(codes)[i] : 0u;
    sc[u] = ok ? (uint32_t)scales[FMT == fp4impl::FMT_MX ? (i >> 2) : (i >> 1)] : 0u;
  }
  const float s_t = FMT == fp4impl::FMT_MX ? 0.0f : *tensor_scale;
#pragma unroll
  for (int u = 0; u < kDeqUnits; ++u) {
    const int64_t i = base + (int64_t)u * blockDim.x;
    float v[8];
    if constexpr (FMT == fp4impl::FMT_MX) {
      e2m1_decode8(cw[u], e8m0_value(sc[u]), v);
    } else {
      e2m1_decode8(cw[u], 1.0f, v);
      const float sb = e4m3_value(sc[u]);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (v[j] * sb) * s_t;     // V s_b exact
    }
    unit_rotate8<H>(v, threadIdx.x);                            // every lane takes part
    if (i < n8) {
      if constexpr (OUT == fp4impl::DT_F32)
        store_f32_out<8>(reinterpret_cast<float*>(y) + i * 8, v);
      else
        store_bf16_out<8>(reinterpret_cast<uint16_t*>(y) + i * 8, v);
    }
  }
}

// Small tensors get 64-thread workgroups, so that their few thousand lanes still spread
// over many CUs (256-thread groups would leave most of the chip idle below ~4M elements).
inline int threads_for(int64_t nchunks) { return nchunks < 16384 ? 64 : kThreads; }
inline dim3 grid_for(int64_t nchunks) {
  const int t = threads_for(nchunks);
  return dim3((unsigned)((nchunks + t - 1) / t));
}

template <int DT, int H>
hipError_t quantize_t(const void* x, int64_t nchunks, int fmt, uint8_t* codes, uint8_t* scales,
                      float* ts, bool compute, float* dbg, hipStream_t st) {
  dim3 g = grid_for(nchunks), b(threads_for(nchunks));
  if (fmt == fp4impl::FMT_MX) {
    if (nchunks) k_quant_mx<DT, H><<<g, b, 0, st>>>(x, nchunks, codes, scales, dbg);
    return hipGetLastError();
  }
  if (compute) {
    k_zero_scalar<<<1, 1, 0, st>>>(ts);
    if (nchunks) {
      const int64_t t = nchunks >= 65536 ? kAmaxThreads : kThreads;
      const int64_t wg = (nchunks + t - 1) / t;
      k_amax<DT, H><<<dim3((unsigned)(wg < kAmaxGroups ? wg : kAmaxGroups)), dim3((unsigned)t), 0, st>>>(x, nchunks, ts);
    }
  }
  if (nchunks) k_quant_nv<DT, H><<<g, b, 0, st>>>(x, nchunks, codes, scales, ts, dbg);
  return hipGetLastError();
}

template <int FMT, int H>
hipError_t dequant_t(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t nchunks,
                     void* y, int dt, hipStream_t st) {
  if (!nchunks) return hipSuccess;
  const int t = threads_for(nchunks);
  const int64_t n8 = nchunks * 4, per_block = (int64_t)kDeqUnits * t;
  dim3 g((unsigned)((n8 + per_block - 1) / per_block)), b(t);
  if (dt == fp4impl::DT_F32)
    k_dequant<FMT, H, fp4impl::DT_F32><<<g, b, 0, st>>>(codes, scales, ts, n8, y);
  else
    k_dequant<FMT, H, fp4impl::DT_BF16><<<g, b, 0, st>>>(codes, scales, ts, n8, y);
  return hipGetLastError();
}

}  // namespace

namespace fp4impl {

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int fmt, int hadamard,
                           uint8_t* codes, uint8_t* scales, float* ts, bool compute, float* dbg,
                           hipStream_t st) {
  int64_t n = M * K / 32;
  if (dtype == DT_BF16) {
    if (hadamard == 0) return quantize_t<DT_BF16, 0>(x, n, fmt, codes, scales, ts, compute, dbg, st);
    if (hadamard == 16) return quantize_t<DT_BF16, 16>(x, n, fmt, codes, scales, ts, compute, dbg, st);
    if (hadamard == 128) return quantize_t<DT_BF16, 128>(x, n, fmt, codes, scales, ts, compute, dbg, st);
    return quantize_t<DT_BF16, 32>(x, n, fmt, codes, scales, ts, compute, dbg, st);
  }
  if (hadamard == 0) return quantize_t<DT_F32, 0>(x, n, fmt, codes, scales, ts, compute, dbg, st);
  if (hadamard == 16) return quantize_t<DT_F32, 16>(x, n, fmt, codes, scales, ts, compute, dbg, st);
  if (hadamard == 128) return quantize_t<DT_F32, 128>(x, n, fmt, codes, scales, ts, compute, dbg, st);
  return quantize_t<DT_F32, 32>(x, n, fmt, codes, scales, ts, compute, dbg, st);
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t M,
                             int64_t K, int fmt, int hadamard, void* y, int dt, hipStream_t st) {
  int64_t n = M * K / 32;
  if (fmt == FMT_MX) {
    if (hadamard == 0) return dequant_t<FMT_MX, 0>(codes, scales, ts, n, y, dt, st);
    if (hadamard == 16) return dequant_t<FMT_MX, 16>(codes, scales, ts, n, y, dt, st);
    if (hadamard == 128) return dequant_t<FMT_MX, 128>(codes, scales, ts, n, y, dt, st);
    return dequant_t<FMT_MX, 32>(codes, scales, ts, n, y, dt, st);
  }
  if (hadamard == 0) return dequant_t<FMT_NV, 0>(codes, scales, ts, n, y, dt, st);
  if (hadamard == 16) return dequant_t<FMT_NV, 16>(codes, scales, ts, n, y, dt, st);
  if (hadamard == 128) return dequant_t<FMT_NV, 128>(codes, scales, ts, n, y, dt, st);
  return dequant_t<FMT_NV, 32>(codes, scales, ts, n, y, dt, st);
}

}  // namespace fp4impl
