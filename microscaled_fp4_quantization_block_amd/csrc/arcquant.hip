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
// Work decomposition (gfx950): one wave owns one row at a time, so the row reduction is a
// wave reduction and no workgroup barrier sits on the per-row path.
//   1. The row streams in with coalesced 16-byte loads (eight per lane in flight), its
//      sum of squares accumulates in registers, and the raw bf16 row is parked in the
//      wave's own LDS slice.
//   2. A DPP reduction gives every lane the same sum, hence the same 1/rms.
//   3. Lane l then encodes blocks l, l + 64, ...: the 16 channel indices of a block come
//      from the permutation, staged once per workgroup in LDS as 16-bit byte offsets into the
//      row (2 c, below 2^15 for K <= 16384; one SDWA add forms each address), and the
//      16 values are gathered from the LDS row.  Codes leave as 8-byte stores (512
//      contiguous bytes per wave instruction), block scales as bytes (64 contiguous).
//      Lanes whose block lies in the first S channels also encode the residual
//      z - V s_b s_t (one fma: a single rounding of the exact difference).
// Rows of up to 4096 channels are one load per wave.  A workgroup requests its rows in
// groups of two waves (four with a gain vector), each group released once the previous
// one has half its rows in, so rows land in a steady stream and the early ones are
// encoded under the later ones' traffic (see k_arcquant).  With a gain vector, gamma is
// staged in LDS once per workgroup, already permuted to output order (see gain_slot).
// The dynamic tensor scale needs max|z| over the tensor first.  The maximum does not
// depend on channel order, so the statistics pass streams rows without the gather, with
// the same per-element arithmetic as the quantizing pass.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int kMaxWaves = 8;
constexpr int kLdsLimit = 144 * 1024;       // dynamic LDS per workgroup used here
constexpr int kUnroll = 8;          // 16-byte loads in flight per lane
// Rows of at most 64 kUnroll 16-byte units (K <= kPipeK) are software-pipelined: at most
// kPipeTotal waves in all (16 per CU), each walking several rows with the next row's
// loads in flight.  Without a gain vector, 8 waves per workgroup (two workgroups per
// CU); with one, 16 (one per CU), so that gamma (K floats) sits in LDS once per CU.
constexpr int kPipeK = 8 * 64 * kUnroll;
constexpr int kPipeTotal = 4096;
template <bool kGamma>
constexpr int pipe_waves() { return kGamma ? 16 : 8; }
constexpr int kMaxGroups = 8;       // load groups per workgroup, at most
// Waves per load group: two in a workgroup of 8 waves, four in one of 16 (gain vector), so
// that both chains release four groups one after another.
template <bool kGamma>
constexpr int group_waves() { return kGamma ? 4 : 2; }
// Statistics passes end in one atomic maximum per workgroup; atomics on one address
// serialise, so their grids are capped at kStatsGroups workgroups.
constexpr int kStatsGroups = 256;

__global__ void k_zero_scalar(float* p) { *p = 0.0f; }

// Make this wave's LDS writes visible to its own later LDS reads (and the reverse).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// One chunk of a row: kUnroll 16-byte units per lane (unit u0 + 64 i + lane), zero past
// the end.
__device__ __forceinline__ void load_units(const uint16_t* __restrict__ xr, int u0, int units, int lane,
                                           uint4 (&raw)[kUnroll]) {
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int u = u0 + 64 * i + lane;
    raw[i] = u < units ? reinterpret_cast<const uint4*>(xr)[u] : make_uint4(0, 0, 0, 0);
  }
}

// The same chunk of a row of at most 64 kUnroll units, through a buffer resource over its
// `units` 16-byte units: units past the end read as zero without a branch, so the loads
// are straight-line code and a later wait can count them exactly.
__device__ __forceinline__ void load_units_rsrc(const uint16_t* xr, int units, int lane, uint4 (&raw)[kUnroll]) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xr), (short)0, units * 16, 0x00020000);
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (64 * i + lane) * 16, 0, 0);
    raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// Lane-local sum of squares of one chunk (fixed order) and its copy into the LDS row.
__device__ __forceinline__ float park_units(const uint4 (&raw)[kUnroll], int u0, int units, int lane,
                                            uint16_t* xs, float ss) {
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf16_lo(w[k]), b = bf16_hi(w[k]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
    const int u = u0 + 64 * i + lane;
    if (u < units) reinterpret_cast<uint4*>(xs)[u] = raw[i];
  }
  return ss;
}

// Stream one row: sum of squares in a fixed order (lane-local over its units, then a
// wave reduction), raw bf16 parked at xs.  Identical arithmetic in every pass.
__device__ __forceinline__ float load_row(const uint16_t* __restrict__ xr, int units, int lane, uint16_t* xs) {
  float ss = 0.0f;
  for (int u0 = 0; u0 < units; u0 += 64 * kUnroll) {
    uint4 raw[kUnroll];
    load_units(xr, u0, units, lane, raw);
    ss = park_units(raw, u0, units, lane, xs, ss);
  }
  return wave_sum(ss);
}

// 1 / sqrt(ss / K + eps): one fused multiply-add and the hardware reciprocal square root
// (v_rsq_f32, within 1 ulp), well inside the tolerance the normalised values are held to.
__device__ __forceinline__ float inv_rms_of(float ss, int K, float eps) {
  return __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / (float)K, eps));
}

// z = fl(x / rms), times the channel's gamma value g when the norm has a gain (kGamma):
// the normalised value of one channel.  Whether a gain is present is a template
// parameter, so the per-element path has no branch and the gains of a block are loaded
// together before use.
template <bool kGamma>
__device__ __forceinline__ float norm_value(uint16_t xb, float inv_rms, float g) {
  const float y = __uint_as_float((uint32_t)xb << 16) * inv_rms;
  return kGamma ? y * g : y;
}

// Maximum m of max|z| over the workgroup, then one atomic max of fl32(m / 2688) into the
// tensor scale *ts (which starts at 0).  Correctly rounded division by a positive constant
// is monotone, so the largest rounded quotient is fl32(max|z| / 2688) of the whole tensor.
// Every thread of the workgroup calls it (it holds a barrier).
__device__ __forceinline__ void workgroup_tensor_scale(float m, float* ts) {
  __shared__ float wmax[kMaxWaves];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, wmax[w]);
    if (m > 0.0f) atomic_max_nonneg(ts, m / 2688.0f);
  }
}

// Statistics pass for rows of any length: each wave streams its rows through its LDS
// slice in chunks, keeping a running max|z|.
template <bool kGamma>
__global__ void __launch_bounds__(64 * kMaxWaves)
k_arc_stats(const uint16_t* __restrict__ x, int64_t M, int K, const float* __restrict__ gamma, float eps,
            float* tensor_scale) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint16_t* xs = smem + (size_t)wave * K;
  const int units = K / 8;
  float tmax = 0.0f;
  for (int64_t r = (int64_t)blockIdx.x * W + wave; r < M; r += (int64_t)gridDim.x * W) {
    const float ss = load_row(x + r * K, units, lane, xs);
    const float inv_rms = inv_rms_of(ss, K, eps);
    wave_lds_sync();
    for (int u = lane; u < units; u += 64) {
      const uint4 w = reinterpret_cast<const uint4*>(xs)[u];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      float g[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) g[k] = kGamma ? gamma[8 * u + k] : 1.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        tmax = fmaxf(tmax, fabsf(norm_value<kGamma>((uint16_t)ws[k], inv_rms, g[2 * k])));
        tmax = fmaxf(tmax, fabsf(norm_value<kGamma>((uint16_t)(ws[k] >> 16), inv_rms, g[2 * k + 1])));
      }
    }
    wave_lds_sync();
  }
  workgroup_tensor_scale(tmax, tensor_scale);
}

// Statistics pass for rows of at most 64 kUnroll units: rows stay in registers (no LDS
// copy), two per wave per step with both rows' loads in flight.  The sum of squares takes
// the same per-lane order as park_units and the same wave reduction, so 1/rms is the
// quantizing pass's to the bit.  Without a gain vector the row's max|z| is max|x| times
// 1/rms, which by monotone rounding equals the maximum of the rounded products; with one,
// every element's fl(fl(x / rms) g) is formed as norm_value does.

template <bool kGamma>
__device__ __forceinline__ float row_absmax(const uint4 (&raw)[kUnroll], int units, int lane, int K, float eps,
                                            const float* __restrict__ gamma) {
  float ss = 0.0f, am = 0.0f;
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf16_lo(w[k]), b = bf16_hi(w[k]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
      am = fmaxf(am, fmaxf(fabsf(a), fabsf(b)));
    }
  }
  const float inv_rms = inv_rms_of(wave_sum(ss), K, eps);
  if constexpr (!kGamma) return am * inv_rms;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int u = 64 * i + lane;
    if (u < units) {
      float g[8];                                          // gamma is only 4-byte aligned
#pragma unroll
      for (int k = 0; k < 8; ++k) g[k] = gamma[8 * u + k];
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = fmaxf(m, fabsf(norm_value<true>((uint16_t)w[k], inv_rms, g[2 * k])));
        m = fmaxf(m, fabsf(norm_value<true>((uint16_t)(w[k] >> 16), inv_rms, g[2 * k + 1])));
      }
    }
  }
  return m;
}

template <bool kGamma>
__global__ void __launch_bounds__(64 * kMaxWaves)
k_arc_stats_rows(const uint16_t* __restrict__ x, int64_t M, int K, const float* __restrict__ gamma, float eps,
                 float* tensor_scale) {
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int units = K / 8;
  const int64_t stride = (int64_t)gridDim.x * W;
  float tmax = 0.0f;
  for (int64_t r = (int64_t)blockIdx.x * W + wave; r < M; r += 2 * stride) {
    const int64_t r2 = r + stride < M ? r + stride : r;   // a missing second row repeats the first
    uint4 a[kUnroll], b[kUnroll];
    load_units_rsrc(x + r * K, units, lane, a);
    load_units_rsrc(x + r2 * K, units, lane, b);
    tmax = fmaxf(tmax, row_absmax<kGamma>(a, units, lane, K, eps, gamma));
    tmax = fmaxf(tmax, row_absmax<kGamma>(b, units, lane, K, eps, gamma));
  }
  workgroup_tensor_scale(tmax, tensor_scale);
}

// Encode one 16-channel block: primary NVFP4 codes and scale, and for blocks inside the
// first S channels the residual z - V s_b s_t and its codes and scale.
__device__ __forceinline__ void encode_block(const float (&z)[16], int b, int K, int nblk, int sblk, float s_t,
                                             uint8_t* __restrict__ crow, uint8_t* __restrict__ srow) {
  const float inv6s = recip_fast(6.0f * s_t);
  const uint32_t sb = nvfp4_block_scale_fast(absmax<16>(z), inv6s);
  const float sbv = e4m3_value(sb);
  const uint2 w = nvfp4_encode16_fast(z, recip_fast(sbv * s_t));
  store_out(reinterpret_cast<uint2*>(crow + 8 * b), w);
  store_out(srow + b, (uint8_t)sb);
  if (b < sblk) {
    float q[16];
    e2m1_decode8(w.x, 1.0f, q);
    e2m1_decode8(w.y, 1.0f, q + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = fmaf(-(q[i] * sbv), s_t, z[i]);   // z - V s_b s_t
    const uint32_t sr = nvfp4_block_scale_fast(absmax<16>(q), inv6s);
    store_out(reinterpret_cast<uint2*>(crow + K / 2 + 8 * b), nvfp4_encode16_fast(q, recip_fast(e4m3_value(sr) * s_t)));
    store_out(srow + nblk + b, (uint8_t)sr);
  }
}

// encode_block for z = fl(x inv_rms) without forming z on the primary path (no gain
// vector).  The block maximum is max|x| times inv_rms, which equals the maximum of the
// rounded products since rounding is monotone, so the block scale is the same as
// encode_block's.  The elements are encoded as x fl(inv_rms / (s_b s_t)) instead of
// fl(x inv_rms) / (s_b s_t): the product rounds once less, which moves an element's code
// only when its quotient lies within a few ulp of a rounding boundary.  The residual
// lanes form z as encode_block does.
__device__ __forceinline__ void encode_block_unnormed(const float (&x)[16], float inv_rms, int b, int K, int nblk,
                                                      int sblk, float s_t, uint8_t* __restrict__ crow,
                                                      uint8_t* __restrict__ srow) {
  const float inv6s = recip_fast(6.0f * s_t);
  const uint32_t sb = nvfp4_block_scale_fast(absmax<16>(x) * inv_rms, inv6s);
  const float sbv = e4m3_value(sb);
  const uint2 w = nvfp4_encode16_fast(x, inv_rms * recip_fast(sbv * s_t));
  store_out(reinterpret_cast<uint2*>(crow + 8 * b), w);
  store_out(srow + b, (uint8_t)sb);
  if (b < sblk) {
    // z = fl(x inv_rms) is formed here, not shared with the debug copy: shared, the
    // compiler hoists its 16 products above both branches into every block.
    float ir = inv_rms;
    asm volatile("" : "+v"(ir));
    float q[16];
    e2m1_decode8(w.x, 1.0f, q);
    e2m1_decode8(w.y, 1.0f, q + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = fmaf(-(q[i] * sbv), s_t, x[i] * ir);   // z - V s_b s_t
    const uint32_t sr = nvfp4_block_scale_fast(absmax<16>(q), inv6s);
    store_out(reinterpret_cast<uint2*>(crow + K / 2 + 8 * b), nvfp4_encode16_fast(q, recip_fast(e4m3_value(sr) * s_t)));
    store_out(srow + nblk + b, (uint8_t)sr);
  }
}

// Gather, normalise and encode row r from its LDS copy: lane l takes blocks l + 64 j.
// kBlocks blocks per lane are gathered together (all their LDS reads in flight at once)
// before any of them is encoded.
constexpr int kBlocks = 1;
// Gamma staged in LDS for a workgroup (rows of at most kPipeK channels): already
// permuted to output order, gl holds gamma[perm[c]] for output channel c = BS b + 4 q + e
// (BS channels per scale block) at float 4 (q (K / BS) + b) + e.  Lane l's gains for
// block b are then BS / 4 16-byte reads at 16-byte steps across the lanes, with no
// address arithmetic and no bank conflicts, where a gain looked up by input channel
// would be one random 4-byte read per element.
template <int BS>
__device__ __forceinline__ int gain_slot(int c, int K) {
  return 4 * (((c % BS) >> 2) * (K / BS) + c / BS) + (c & 3);
}

template <int BS>
__device__ __forceinline__ void gains_of_block(const float* gl, int b, int nblk, float (&g)[BS]) {
  const float4* g4 = reinterpret_cast<const float4*>(gl) + b;
#pragma unroll
  for (int q = 0; q < BS / 4; ++q) {
    const float4 t = g4[q * nblk];
    g[4 * q] = t.x;
    g[4 * q + 1] = t.y;
    g[4 * q + 2] = t.z;
    g[4 * q + 3] = t.w;
  }
}

// Gain of the channel at byte offset `off` of the bf16 row, from global memory (longer rows).
__device__ __forceinline__ float gain_global(const float* __restrict__ gamma, uint32_t off) {
  return gamma[off >> 1];
}

template <bool kGamma, bool kLdsGamma>
__device__ __forceinline__ void encode_row(const uint16_t* xs, const uint16_t* ps, int64_t r, int K, int S,
                                           int lane, float inv_rms, const float* __restrict__ gamma,
                                           const float* gl, float s_t, uint8_t* __restrict__ codes,
                                           uint8_t* __restrict__ scales, float* __restrict__ dbg) {
  const int nblk = K / 16, sblk = S / 16;
  const int64_t row_codes = (K + S) / 2, row_scales = (K + S) / 16;
  uint8_t* crow = codes + r * row_codes;
  uint8_t* srow = scales + r * row_scales;
  for (int b0 = lane; b0 < nblk; b0 += 64 * kBlocks) {
    uint4 pw[kBlocks][2];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      const int b = min(b0 + 64 * j, nblk - 1);            // past the end: a valid dummy block
      pw[j][0] = reinterpret_cast<const uint4*>(ps)[2 * b];
      pw[j][1] = reinterpret_cast<const uint4*>(ps)[2 * b + 1];
    }
    uint16_t xv[kBlocks][16];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      const uint32_t w[8] = {pw[j][0].x, pw[j][0].y, pw[j][0].z, pw[j][0].w,
                             pw[j][1].x, pw[j][1].y, pw[j][1].z, pw[j][1].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xv[j][2 * k] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(xs) + (w[k] & 0xFFFFu));
        xv[j][2 * k + 1] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(xs) + (w[k] >> 16));
      }
    }
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      const int b = b0 + 64 * j;
      if (b >= nblk) break;
      const uint32_t w[8] = {pw[j][0].x, pw[j][0].y, pw[j][0].z, pw[j][0].w,
                             pw[j][1].x, pw[j][1].y, pw[j][1].z, pw[j][1].w};
      if constexpr (kGamma) {
        float g[16];
        if constexpr (kLdsGamma) {
          gains_of_block<16>(gl, b, nblk, g);
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            g[2 * k] = gain_global(gamma, w[k] & 0xFFFFu);
            g[2 * k + 1] = gain_global(gamma, w[k] >> 16);
          }
        }
        float z[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) z[k] = norm_value<true>(xv[j][k], inv_rms, g[k]);
        if (dbg) store_f32<16>(dbg + r * K + 16 * b, z);
        encode_block(z, b, K, nblk, sblk, s_t, crow, srow);
      } else {
        float xf[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) xf[k] = __uint_as_float((uint32_t)xv[j][k] << 16);
        if (dbg) {
          float z[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) z[k] = xf[k] * inv_rms;
          store_f32<16>(dbg + r * K + 16 * b, z);
        }
        encode_block_unnormed(xf, inv_rms, b, K, nblk, sblk, s_t, crow, srow);
      }
    }
  }
}

// MXFP4 flavour: 32-channel blocks, one E8M0 scale per block (floor(log2 amax) - 2), codes
// by the hardware convert (exact: power-of-two scale).  The residual z - V 2^(e-127) is
// exact in binary32: z lies within a factor of two of its nearest grid point, or the
// grid point is 0.  Lane l takes blocks l, l + 64, ...
template <bool kGamma, bool kLdsGamma>
__device__ __forceinline__ void encode_row_mx(const uint16_t* xs, const uint16_t* ps, int64_t r, int K, int S,
                                              int lane, float inv_rms, const float* __restrict__ gamma,
                                              const float* gl,
                                              uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                              float* __restrict__ dbg) {
  const int nblk = K / 32, sblk = S / 32;
  const int64_t row_codes = (K + S) / 2, row_scales = (K + S) / 32;
  uint8_t* crow = codes + r * row_codes;
  uint8_t* srow = scales + r * row_scales;
  for (int b = lane; b < nblk; b += 64) {
    uint4 pw4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pw4[q] = reinterpret_cast<const uint4*>(ps)[4 * b + q];
    int c[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {pw4[q].x, pw4[q].y, pw4[q].z, pw4[q].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[8 * q + 2 * k] = (int)(w[k] & 0xFFFFu);         // byte offsets
        c[8 * q + 2 * k + 1] = (int)(w[k] >> 16);
      }
    }
    float g[32];
    if constexpr (kGamma && kLdsGamma) {
      gains_of_block<32>(gl, b, nblk, g);
    } else {
#pragma unroll
      for (int k = 0; k < 32; ++k) g[k] = kGamma ? gain_global(gamma, (uint32_t)c[k]) : 1.0f;
    }
    float z[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
      z[k] = norm_value<kGamma>(*reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(xs) + c[k]), inv_rms, g[k]);
    if (dbg) store_f32<32>(dbg + r * K + 32 * b, z);
    const uint32_t e = e8m0_from_amax(absmax<32>(z));
    const float sc = e8m0_value(e);
    const uint4 w = e2m1_encode32(z, sc);
    store_out(reinterpret_cast<uint4*>(crow + 16 * b), w);
    store_out(srow + b, (uint8_t)e);
    if (b < sblk) {
      float q[32];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) e2m1_decode8(ws[i], sc, q + 8 * i);
#pragma unroll
      for (int i = 0; i < 32; ++i) q[i] = z[i] - q[i];
      const uint32_t er = e8m0_from_amax(absmax<32>(q));
      store_out(reinterpret_cast<uint4*>(crow + K / 2 + 16 * b), e2m1_encode32(q, e8m0_value(er)));
      store_out(srow + nblk + b, (uint8_t)er);
    }
  }
}

template <int FMT, bool kGamma>
__global__ void __launch_bounds__(64 * pipe_waves<kGamma>())
k_arcquant(const uint16_t* __restrict__ x, int64_t M, int K, const float* __restrict__ gamma, float eps,
           const int32_t* __restrict__ perm, int S, uint8_t* __restrict__ codes,
           uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, float* __restrict__ dbg) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int units = K / 8;
  const bool pipelined = units <= 64 * kUnroll;
  // LDS: [K] permutation as byte offsets 2 perm[c]; with a gain vector and short rows,
  // [K] fp32 gamma permuted to output order (gain_slot); then one [K] bf16 row per wave.
  constexpr int BS = FMT == fp4impl::FMT_NV ? 16 : 32;
  const bool lds_gamma = kGamma && pipelined;
  uint16_t* ps = smem;
  float* gl = reinterpret_cast<float*>(smem + K);   // used only when lds_gamma
  uint16_t* xs = smem + (size_t)(lds_gamma ? 3 : 1) * K + (size_t)wave * K;

  const int64_t stride = (int64_t)gridDim.x * W;
  int64_t r = (int64_t)blockIdx.x * W + wave;
  // An index outside [0, K) (not a permutation: caller error) is clamped, never dereferenced.
  // With a gain vector the table and gamma are staged by the waves past group 0 only:
  // gamma[perm[c]] is a load that depends on perm[c], and group 0's row loads, issued
  // first, must not wait behind it.
  constexpr int kGW = group_waves<kGamma>();
  constexpr int kLead = kGamma ? kGW : 0;
  constexpr int kStW = 64 * (pipe_waves<kGamma>() - kLead);
  constexpr int kSt = (kPipeK + kStW - 1) / kStW;              // staging batch per thread
  const int nst = (int)blockDim.x - 64 * kLead, st = (int)threadIdx.x - 64 * kLead;
  uint4 raw[kUnroll];
  static_assert(pipe_waves<kGamma>() % kGW == 0 && pipe_waves<kGamma>() / kGW <= kMaxGroups, "load groups");
  if (pipelined && (int)blockDim.x == 64 * pipe_waves<kGamma>() && K <= kSt * nst) {
    // The permutation's loads (L2-resident after the first workgroups) go out first.  The
    // rows are then requested in groups of kGW waves: group 0 at once, group g once every
    // wave of group g - 1 has the first half of its row in (an LDS counter per group).
    // Rows thus land in a steady stream, and each group is encoded while the next ones
    // arrive: with every row requested at once, all of them would land together at the
    // end and the encode would start only then.  Group 0 waits for nothing, every wave
    // counts itself unconditionally, and the workgroup's waves (8 or 16) are a multiple of
    // kGW, so every group has kGW waves and every wait ends.  A row past M reloads row
    // M - 1, which is then never used, so every wave takes part.
    uint32_t pv[kSt];
    float gv[kGamma ? kSt : 1];
    if (st >= 0) {
#pragma unroll
      for (int i = 0; i < kSt; ++i) pv[i] = (uint32_t)perm[min(st + i * nst, K - 1)];
      if constexpr (kGamma) {
#pragma unroll
        for (int i = 0; i < kSt; ++i) gv[i] = gamma[min(pv[i], (uint32_t)(K - 1))];
      }
    }
    __shared__ uint32_t landed[kMaxGroups];
    const int64_t r0 = r < M ? r : M - 1;
    const int grp = wave / kGW;
    if (threadIdx.x < kMaxGroups) landed[threadIdx.x] = 0u;
    if (grp == 0) load_units_rsrc(x + r0 * K, units, lane, raw);   // pipelined: one chunk
    if (st >= 0) {
#pragma unroll
      for (int i = 0; i < kSt; ++i) {
        const int c = st + i * nst;
        if (c < K) {
          ps[c] = (uint16_t)(2 * min(pv[i], (uint32_t)(K - 1)));
          if constexpr (kGamma) gl[gain_slot<BS>(c, K)] = gv[i];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): table and counters written
    __builtin_amdgcn_s_barrier();
    if (grp > 0) {
      while (__hip_atomic_load(&landed[grp - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)kGW)
        __builtin_amdgcn_s_sleep(1);
      load_units_rsrc(x + r0 * K, units, lane, raw);
    }
    __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4): the first 4 of the row's 8 loads are in
    if (lane == 0) atomicAdd(&landed[grp], 1u);
  } else {
    if (pipelined && r < M) load_units(x + r * K, 0, units, lane, raw);
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
      const uint32_t pc = min((uint32_t)perm[c], (uint32_t)(K - 1));
      ps[c] = (uint16_t)(2 * pc);
      if (lds_gamma) gl[gain_slot<BS>(c, K)] = gamma[pc];
    }
    __syncthreads();
  }

  const float s_t = FMT == fp4impl::FMT_NV ? *tensor_scale : 0.0f;
  auto encode = [&](int64_t row, float inv_rms) {
    if constexpr (FMT == fp4impl::FMT_NV) {
      if (kGamma && lds_gamma)
        encode_row<kGamma, kGamma>(xs, ps, row, K, S, lane, inv_rms, gamma, gl, s_t, codes, scales, dbg);
      else
        encode_row<kGamma, false>(xs, ps, row, K, S, lane, inv_rms, gamma, gl, s_t, codes, scales, dbg);
    } else {
      if (kGamma && lds_gamma)
        encode_row_mx<kGamma, kGamma>(xs, ps, row, K, S, lane, inv_rms, gamma, gl, codes, scales, dbg);
      else
        encode_row_mx<kGamma, false>(xs, ps, row, K, S, lane, inv_rms, gamma, gl, codes, scales, dbg);
    }
  };
  if (pipelined) {
    // whole row in one chunk: the next row's loads are in flight while this row is encoded
    for (; r < M; r += stride) {
      const float ss = wave_sum(park_units(raw, 0, units, lane, xs, 0.0f));
      if (r + stride < M) load_units(x + (r + stride) * K, 0, units, lane, raw);
      wave_lds_sync();
      encode(r, inv_rms_of(ss, K, eps));
      wave_lds_sync();                                   // xs is refilled by the next row
    }
  } else {
    for (; r < M; r += stride) {
      const float ss = load_row(x + r * K, units, lane, xs);
      wave_lds_sync();
      encode(r, inv_rms_of(ss, K, eps));
      wave_lds_sync();
    }
  }
}

// Waves per workgroup: one LDS row each plus the shared permutation, within 144 KiB.
int waves_for(int64_t K) {
  int64_t w = kLdsLimit / (2 * K) - 1;
  return (int)(w > kMaxWaves ? kMaxWaves : (w < 1 ? 1 : w));
}

hipError_t allow_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

struct ArcLaunch {
  int W, Wq;
  unsigned grid, grid_q;
  size_t lds_stats, lds_quant;
};

ArcLaunch arc_launch(int64_t M, int64_t K, bool gamma) {
  ArcLaunch a;
  a.W = waves_for(K);
  const int64_t rows_per_grid = 1024 * (int64_t)a.W;     // at most 1024 workgroups, persistent beyond
  a.grid = (unsigned)(M <= 0 ? 1 : (M < rows_per_grid ? (M + a.W - 1) / a.W : 1024));
  const bool pipelined = K / 8 <= 64 * kUnroll;
  const bool lds_gamma = gamma && pipelined;
  a.Wq = pipelined ? (gamma ? pipe_waves<true>() : pipe_waves<false>()) : a.W;
  const int64_t wq_total = pipelined ? (M < kPipeTotal ? M : kPipeTotal) : (M < rows_per_grid ? M : rows_per_grid);
  a.grid_q = (unsigned)(wq_total <= 0 ? 1 : (wq_total + a.Wq - 1) / a.Wq);
  a.lds_stats = (size_t)2 * K * a.W;
  a.lds_quant = (size_t)2 * K * (a.Wq + 1) + (lds_gamma ? (size_t)4 * K : 0);
  return a;
}

// Enqueue the statistics pass (when `compute`) and the quantizing kernel of format FMT,
// with or without a gain vector.
template <int FMT, bool kGamma>
hipError_t launch_arc(const uint16_t* x, int64_t M, int64_t K, const float* gamma, float eps, const int32_t* perm,
                      int64_t S, uint8_t* codes, uint8_t* scales, float* ts, bool compute, float* dbg,
                      hipStream_t st) {
  const ArcLaunch a = arc_launch(M, K, kGamma);
  hipError_t e = allow_lds(reinterpret_cast<const void*>(k_arcquant<FMT, kGamma>), a.lds_quant);
  if (e == hipSuccess && compute && K / 8 > 64 * kUnroll)
    e = allow_lds(reinterpret_cast<const void*>(k_arc_stats<kGamma>), a.lds_stats);
  if (e != hipSuccess) return e;
  if (compute) {
    k_zero_scalar<<<1, 1, 0, st>>>(ts);
    if (M && K / 8 <= 64 * kUnroll) {
      const int64_t wg = (M + 2 * kMaxWaves - 1) / (2 * kMaxWaves);   // two rows per wave per step
      k_arc_stats_rows<kGamma><<<(unsigned)(wg < kStatsGroups ? wg : kStatsGroups), 64 * kMaxWaves, 0, st>>>(
          x, M, (int)K, gamma, eps, ts);
    } else if (M) {
      k_arc_stats<kGamma><<<a.grid < kStatsGroups ? a.grid : kStatsGroups, 64 * a.W, a.lds_stats, st>>>(
          x, M, (int)K, gamma, eps, ts);
    }
  }
  if (M)
    k_arcquant<FMT, kGamma><<<a.grid_q, 64 * a.Wq, a.lds_quant, st>>>(x, M, (int)K, gamma, eps, perm, (int)S,
                                                                     codes, scales, ts, dbg);
  return hipGetLastError();
}

}  // namespace

namespace fp4impl {

hipError_t launch_residual_quantize(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                                    float eps, const int32_t* perm, int64_t S, uint8_t* codes,
                                    uint8_t* scales, float* ts, bool compute, float* dbg,
                                    hipStream_t st) {
  return gamma ? launch_arc<FMT_NV, true>(x, M, K, gamma, eps, perm, S, codes, scales, ts, compute, dbg, st)
               : launch_arc<FMT_NV, false>(x, M, K, gamma, eps, perm, S, codes, scales, ts, compute, dbg, st);
}

hipError_t launch_residual_quantize_mx(const uint16_t* x, int64_t M, int64_t K, const float* gamma, float eps,
                                       const int32_t* perm, int64_t S, uint8_t* codes, uint8_t* scales,
                                       float* dbg, hipStream_t st) {
  if (!M) return hipSuccess;
  return gamma ? launch_arc<FMT_MX, true>(x, M, K, gamma, eps, perm, S, codes, scales, nullptr, false, dbg, st)
               : launch_arc<FMT_MX, false>(x, M, K, gamma, eps, perm, S, codes, scales, nullptr, false, dbg, st);
}

}  // namespace fp4impl
