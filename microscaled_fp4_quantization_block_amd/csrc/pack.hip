// FP4Quant-style micro-grouped dual-scale FP4 pack / unpack with the two-level FWHT.
//
// Source: FP4Quant abstract (paperdot.bitmofang.com): a hybrid two-level FWHT ahead of a
// micro-grouped dual-scale FP4 quantization, and a cooperative sub-byte packing.  Here a
// 128-group is spread over the four lanes of a DPP quad, each lane owning 32 contiguous
// elements (two 16-element micro-groups, one 16-byte code store):
//   level 1   H_16 inside each micro-group: in-lane butterflies;
//   level 2   H_8 across the 8 micro-groups (index 2 p + h for lane p of the quad and
//             micro-group h of the lane): the h butterfly is in-lane, the two lane-bit
//             butterflies use quad_perm DPP.  Lane p computes own + c * partner with
//             c = +-1, which leaves its result multiplied by (-1)^popcount(p); that sign
//             is folded into the 1/sqrt(128) normalisation.
// Group scale fl32(amax/2688) per 128, E4M3 micro scale per 16, E2M1 codes; the message
// is planar: codes | micro scales | group scales, each section 256-byte aligned.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_partner(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ float quad_max(float m) {
  return fmaxf(m, quad_partner<CTRL>(m));
}

// Two-level FWHT of a 128-group spread over a quad (see file comment), normalised.
__device__ __forceinline__ void quad_two_level_fwht(float* v, int p) {
  fwht_inplace<16>(v);                 // level 1, micro-group h = 0
  fwht_inplace<16>(v + 16);            // level 1, micro-group h = 1
#pragma unroll
  for (int j = 0; j < 16; ++j) {       // level 2, in-lane bit (h)
    float a = v[j], b = v[16 + j];
    v[j] = a + b;
    v[16 + j] = a - b;
  }
  const float c1 = (p & 1) ? -1.0f : 1.0f;
  const float c2 = (p & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = fmaf(quad_partner<kQuadXor1>(v[i]), c1, v[i]);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = fmaf(quad_partner<kQuadXor2>(v[i]), c2, v[i]);
  const float norm = (__popc(p) & 1) ? -InvSqrt<128>::v : InvSqrt<128>::v;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= norm;
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
  const float s_g = m / 2688.0f;       // correctly rounded fp32 division
  uint2 w[2];
  uint32_t sm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sm[h] = nvfp4_block_scale(absmax<16>(v + 16 * h), s_g);
    float S32 = e4m3_value(sm[h]) * s_g;
    float E = S32 > 0.0f ? 1.0f / S32 : 0.0f;
    w[h] = nvfp4_encode16_fast(v + 16 * h, E);
  }
  reinterpret_cast<uint4*>(codes)[c] = make_uint4(w[0].x, w[0].y, w[1].x, w[1].y);
  reinterpret_cast<uint16_t*>(micro)[c] = (uint16_t)(sm[0] | (sm[1] << 8));
  if (p == 0) group[c >> 2] = s_g;
}

__global__ void __launch_bounds__(kThreads)
k_unpack(const uint8_t* codes, const uint8_t* micro, const float* group, int64_t nchunks, uint16_t* y) {
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= nchunks) return;
  const int p = (int)(c & 3);
  uint4 w = reinterpret_cast<const uint4*>(codes)[c];
  uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t sm2 = reinterpret_cast<const uint16_t*>(micro)[c];
  const float s_g = group[c >> 2];
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) e2m1_decode8(ws[i], 1.0f, v + 8 * i);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float sm = e4m3_value((sm2 >> (8 * h)) & 0xFFu);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[16 * h + i] = (v[16 * h + i] * sm) * s_g;   // V s_m exact
  }
  quad_two_level_fwht(v, p);
  store_bf16<32>(y + c * 32, v);
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
  int64_t n = M * K / 32;
  if (!n) return hipSuccess;
  PackLayout L = pack_layout(M, K);
  k_unpack<<<dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st>>>(
      packed, packed + L.off_micro, reinterpret_cast<const float*>(packed + L.off_group), n, y);
  return hipGetLastError();
}

}  // namespace fp4impl
