// FP4Quant-style micro-grouped dual-scale FP4 pack / unpack with the two-level FWHT.
//
// Source: FP4Quant abstract (paperdot.bitmofang.com): a hybrid two-level FWHT ahead of a
// micro-grouped dual-scale FP4 quantization, and a cooperative sub-byte packing.  In the
// pack a 128-group is spread over the four lanes of a DPP quad, each lane owning 32
// contiguous elements (two 16-element micro-groups, one 16-byte code store):
//   level 1   H_16 inside each micro-group: in-lane butterflies;
//   level 2   H_8 across the 8 micro-groups (index 2 p + h for lane p of the quad and
//             micro-group h of the lane): the h butterfly is in-lane, the two lane-bit
//             butterflies use quad_perm DPP.  Lane p computes own + c * partner with
//             c = +-1, which leaves its result multiplied by (-1)^popcount(p); that sign
//             is folded into the 1/sqrt(128) normalisation.
// Group scale fl32(amax/2688) per 128, E4M3 micro scale per 16, E2M1 codes; the message
// is planar: codes | micro scales | group scales, each section 256-byte aligned.  The
// values are rotated (fp32-rounded), so the scale and element decisions take the fast
// reciprocal-and-convert route.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
template <int CTRL>
__device__ __forceinline__ float quad_max(float m) {
  return fmaxf(m, quad_partner<CTRL>(m));
}

__global__ void __launch_bounds__(kThreads)
k_pack(const uint16_t* x, int64_t nchunks, uint8_t* codes, uint8_t* micro, float* group, float* dbg) {
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;            // nchunks % 4 == 0: whole quads leave together
  const int p = (int)(c & 3);
  float v[32];
  load_bf16<32>(x + c * 32, v);
  quad_two_level_fwht(v, p);
  if (dbg) store_f32<32>(dbg + c * 32, v);
  float m = absmax<32>(v);
  m = quad_max<kQuadXor1>(m);
  m = quad_max<kQuadXor2>(m);
  const float s_g = m / 2688.0f;       // correctly rounded fp32 division (stored)
  const float inv6s = recip_fast(6.0f * s_g);
  uint2 w[2];
  uint32_t sm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sm[h] = nvfp4_block_scale_fast(absmax<16>(v + 16 * h), inv6s);
    w[h] = nvfp4_encode16_fast(v + 16 * h, recip_fast(e4m3_value(sm[h]) * s_g));
  }
  store_out(reinterpret_cast<uint4*>(codes) + c, make_uint4(w[0].x, w[0].y, w[1].x, w[1].y));
  store_out(reinterpret_cast<uint16_t*>(micro) + c, (uint16_t)(sm[0] | (sm[1] << 8)));
  if (p == 0) store_out(group + (c >> 2), s_g);
}

// Unpack by groups of 16 lanes: lane g of a group owns elements 8 g .. 8 g + 7 of one
// 128-group (one 4-byte code word), so a wave's bf16 stores are 1 KiB contiguous; the
// two-level FWHT finishes with DPP butterflies across the 16 lanes.
constexpr int kUnpackUnits = 4;

__global__ void __launch_bounds__(kThreads)
k_unpack(const uint8_t* codes, const uint8_t* micro, const float* group, int64_t n8, uint16_t* y) {
  const int64_t base = (int64_t)blockIdx.x * (kUnpackUnits * kThreads) + threadIdx.x;
  const int g = threadIdx.x & 15;
  uint32_t cw[kUnpackUnits], sm[kUnpackUnits];
  float sg[kUnpackUnits];
#pragma unroll
  for (int u = 0; u < kUnpackUnits; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    const bool ok = i < n8;
    cw[u] = ok ? reinterpret_cast<const uint32_t*>(codes)[i] : 0u;
    sm[u] = ok ? (uint32_t)micro[i >> 1] : 0u;
    sg[u] = ok ? group[i >> 4] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kUnpackUnits; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    float v[8];
    e2m1_decode8(cw[u], 1.0f, v);
    const float smv = e4m3_value(sm[u]);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (v[j] * smv) * sg[u];     // V s_m exact
    group16_two_level_fwht8(v, g);                               // every lane takes part
    if (i < n8) store_bf16_out<8>(y + i * 8, v);
  }
}

}  // namespace

namespace fp4impl {

PackLayout pack_layout(int64_t M, int64_t K) {
  auto align = [](size_t n) { return (n + 255) / 256 * 256; };
  size_t n = (size_t)M * (size_t)K;
  PackLayout L;
  L.off_micro = align(n / 2);
  L.off_group = align(L.off_micro + n / 16);
  L.total = align(L.off_group + 4 * (n / 128));
  return L;
}

hipError_t launch_pack(const uint16_t* x, int64_t M, int64_t K, uint8_t* packed, float* dbg,
                       hipStream_t st) {
  int64_t n = M * K / 32;
  if (!n) return hipSuccess;
  PackLayout L = pack_layout(M, K);
  k_pack<<<dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st>>>(
      x, n, packed, packed + L.off_micro, reinterpret_cast<float*>(packed + L.off_group), dbg);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t M, int64_t K, uint16_t* y, hipStream_t st) {
  const int64_t n8 = M * K / 8, per_block = (int64_t)kUnpackUnits * kThreads;
  if (!n8) return hipSuccess;
  PackLayout L = pack_layout(M, K);
  k_unpack<<<dim3((unsigned)((n8 + per_block - 1) / per_block)), dim3(kThreads), 0, st>>>(
      packed, packed + L.off_micro, reinterpret_cast<const float*>(packed + L.off_group), n8, y);
  return hipGetLastError();
}

}  // namespace fp4impl
