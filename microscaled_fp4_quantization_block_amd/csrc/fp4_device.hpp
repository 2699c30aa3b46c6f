// Device-side building blocks shared by the gfx950 kernels: bf16 widening, in-register
// fast Walsh-Hadamard transforms, E2M1 / E4M3 / E8M0 encoding and wave reductions.
//
// Format definitions follow OCP MX v1.0 (E2M1 elements, E8M0 scales) and OCP FP8 (E4M3
// scales); the pages name the formats (ARCQuant summary, gist.science: NVFP4 blocks of 16
// with E2M1 elements; MR-GPTQ abstract, hyper.ai: power-of-two MXFP4 scales) but give no
// bit layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

// --------------------------------------------------------------------------- bf16 / fp32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest-even fp32 -> bf16 for finite values.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two values to a packed bf16 pair, nearest-even (gfx950 v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Load N consecutive elements (N % 8 == 0) as fp32 with 16-byte loads.
template <int N>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float* v) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w = q[i];
    v[8 * i + 0] = bf16_lo(w.x); v[8 * i + 1] = bf16_hi(w.x);
    v[8 * i + 2] = bf16_lo(w.y); v[8 * i + 3] = bf16_hi(w.y);
    v[8 * i + 4] = bf16_lo(w.z); v[8 * i + 5] = bf16_hi(w.z);
    v[8 * i + 6] = bf16_lo(w.w); v[8 * i + 7] = bf16_hi(w.w);
  }
}

template <int N>
__device__ __forceinline__ void load_f32(const float* p, float* v) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    float4 w = q[i];
    v[4 * i + 0] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
  }
}

template <int N>
__device__ __forceinline__ void store_f32(float* p, const float* v) {
  float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

template <int N>
__device__ __forceinline__ void store_bf16(uint16_t* p, const float* v) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w;
    w.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
    w.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
    w.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
    w.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
    q[i] = w;
  }
}

// Output stores.  Codes, scales and dequantized values are written once and read, if at
// all, by a later launch: non-temporal stores stream them out without allocating in L2 or
// the Infinity Cache, where a write stream of a working set's size only evicts what the
// loads still need (bf16 4096 x 4096 dequantization: 9.6 us -> 7.2 us).
typedef unsigned int out_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int out_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_out(uint4* p, uint4 w) {
  __builtin_nontemporal_store(out_u32x4{w.x, w.y, w.z, w.w}, reinterpret_cast<out_u32x4*>(p));
}
__device__ __forceinline__ void store_out(uint2* p, uint2 w) {
  __builtin_nontemporal_store(out_u32x2{w.x, w.y}, reinterpret_cast<out_u32x2*>(p));
}
template <typename T>
__device__ __forceinline__ void store_out(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

template <int N>
__device__ __forceinline__ void store_f32_out(float* p, const float* v) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    store_out(q + i, make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                                __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])));
}

template <int N>
__device__ __forceinline__ void store_bf16_out(uint16_t* p, const float* v) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    uint4 w;
    w.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
    w.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
    w.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
    w.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
    store_out(q + i, w);
  }
}

// --------------------------------------------------------------------------- Hadamard

// Unnormalised Sylvester-ordered Walsh-Hadamard transform of v[0..N) in registers:
// log2(N) butterfly stages of N/2 add/sub pairs.  Result = (sqrt(N) H_N) v.
template <int N>
__device__ __forceinline__ void fwht_inplace(float* v) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// 1/sqrt(n) rounded to fp32 (n = 16 is exact).
template <int N> struct InvSqrt;
template <> struct InvSqrt<16> { static constexpr float v = 0.25f; };
template <> struct InvSqrt<32> { static constexpr float v = 0.17677669529663688f; };
template <> struct InvSqrt<128> { static constexpr float v = 0.08838834764831845f; };

// Orthonormal H_B on every contiguous B-block of v[0..N).
template <int N, int B>
__device__ __forceinline__ void block_hadamard(float* v) {
  if constexpr (B > 1) {
#pragma unroll
    for (int b = 0; b < N; b += B) fwht_inplace<B>(v + b);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] *= InvSqrt<B>::v;
  }
}

// Two-level FWHT of one 128-group held in registers (index 16 g + j): H_16 inside each
// micro-group g, then H_8 across the micro-groups at each position j, normalised once.
__device__ __forceinline__ void two_level_fwht128(float* v) {
#pragma unroll
  for (int g = 0; g < 8; ++g) fwht_inplace<16>(v + 16 * g);     // level 1
#pragma unroll
  for (int h = 16; h < 128; h <<= 1) {                            // level 2: strides 16, 32, 64
#pragma unroll
    for (int i = 0; i < 128; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 128; ++i) v[i] *= InvSqrt<128>::v;
}

// --------------------------------------------------------------------------- E2M1

// Round-to-nearest-even E2M1 codes of v[i] / scale for 32 values, scale a power of two
// (gfx950 v_cvt_scalef32_pk_fp4_f32; only the exponent of `scale` is used, and the
// result is the exact RNE decision of the quotient, saturating at +-6, sign kept on 0).
__device__ __forceinline__ uint4 e2m1_encode32(const float* v, float scale) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 0], v[8 * i + 1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 2], v[8 * i + 3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 4], v[8 * i + 5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 6], v[8 * i + 7], scale, 3);
    w[i] = r;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint2 e2m1_encode16(const float* v, float scale) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 0], v[8 * i + 1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 2], v[8 * i + 3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 4], v[8 * i + 5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * i + 6], v[8 * i + 7], scale, 3);
    w[i] = r;
  }
  return make_uint2(w[0], w[1]);
}

// Decode the 8 codes of one packed word: V(code) * scale for a power-of-two scale.
__device__ __forceinline__ void e2m1_decode8(uint32_t w, float scale, float* v) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
}

// Binary32 value whose RNE rounding to E2M1 equals the RNE rounding of the float64 q:
// q is clamped to [2^-10, 6] (which changes no E2M1 decision), truncated to binary32 and
// its last bit set when the truncation was inexact ("round to odd").  Rounding to odd
// into a format with at least two more bits than the target keeps the final
// round-to-nearest-even exact (Boldo & Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", IEEE TC 2008).
__device__ __forceinline__ float round_to_odd_f32(double q) {
  q = fmin(fmax(q, 0x1p-10), 6.0);
  uint64_t b = (uint64_t)__double_as_longlong(q);
  uint32_t hi = (uint32_t)(b >> 32) - (896u << 20);    // rebias exponent 1023 -> 127
  uint32_t lo = (uint32_t)b;
  uint32_t f = __builtin_amdgcn_alignbit(hi, lo, 29);  // 8-bit exponent | top 23 mantissa bits
  f |= (lo & 0x1FFFFFFFu) ? 1u : 0u;
  return __uint_as_float(f);
}

// Exact NVFP4 element codes of 16 values: RNE(|x| / S) for S = s_b s_t (exact in
// float64), sign kept; S = 0 gives sign-only codes.  Each quotient is a correctly rounded
// float64 division: a quotient that is an E2M1 midpoint comes out as that midpoint exactly,
// and any other lies at least 2^-31 (relative) from every midpoint (|x| has 24 significant
// bits, the midpoint times S at most 31), far beyond the division's 2^-53.  A product with
// a rounded reciprocal 1/S would not do: at a tie it can land an ulp off the midpoint,
// which rounding to odd then turns into a rounding away from the even code.
__device__ __forceinline__ uint2 nvfp4_encode16_exact(const float* v, double S) {
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    double a = S > 0.0 ? fabs((double)v[i]) / S : 0.0;
    q[i] = copysignf(round_to_odd_f32(a), v[i]);
  }
  return e2m1_encode16(q, 1.0f);
}

// Fast NVFP4 element codes: RNE(fl32(x * E)) with E = fl32(1 / fl32(s_b s_t)).  Used where
// the values themselves carry fp32 rounding (rotated or normalised inputs).
__device__ __forceinline__ uint2 nvfp4_encode16_fast(const float* v, float E) {
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = v[i] * E;
  return e2m1_encode16(q, 1.0f);
}

// --------------------------------------------------------------------------- E4M3

// E4M3 (OCP FP8 "FN") code of r >= 0: nearest finite value, ties to the even code,
// saturating at 448 (code 0x7E).  Evaluated in float64 on a float64 argument.
__device__ __forceinline__ uint32_t e4m3_rne(double r) {
  if (r >= 448.0) return 0x7Eu;
  if (r < 0x1p-6) return (uint32_t)rint(r * 512.0);     // subnormals: multiples of 2^-9
  int e2;
  (void)frexp(r, &e2);                                   // r = f 2^e2, f in [0.5, 1)
  int E = e2 - 1;                                        // floor(log2 r), -6..8
  uint32_t m = (uint32_t)rint(ldexp(r, 3 - E));          // 8..16 (16 carries into E + 1)
  uint32_t code = (uint32_t)((E + 7) << 3) + m - 8u;
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of an E4M3 code (OCP E4M3FN: 2^(e-7) (1 + m/8), subnormals m 2^-9) by the
// hardware convert, exact for every code; the byte is the low one of `code`.  The same
// instruction family encodes the scales (v_cvt_pk_fp8_f32), so both ends use the same
// format on gfx950.
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// NVFP4 block scale decision for block maximum amax under tensor scale s_t:
// E4M3(amax / (6 s_t)) of the float64 quotient (6 s_t is exact in float64; the quotient
// is within 2^-53 of the real one, which cannot move a decision: a non-tie argument is
// at least 2^-33 away from an E4M3 midpoint and a tie divides exactly).
__device__ __forceinline__ uint32_t nvfp4_block_scale(float amax, float s_t) {
  if (!(s_t > 0.0f)) return 0u;
  return e4m3_rne((double)amax / (6.0 * (double)s_t));
}

// Fast scale arithmetic for paths whose inputs already carry fp32 rounding (rotated or
// normalised values): decisions may move only where the exact argument lies within a
// few binary32 ulps of a boundary.
//   recip_fast       1/x by v_rcp_f32 (about 1 ulp), 0 for x <= 0
//   e4m3_fast        E4M3 code of q >= 0 by the hardware convert (OCP E4M3, nearest-even;
//                    matches the float64 rule on every value up to 448), clamped at 448
//   nvfp4_block_scale_fast   E4M3(amax * inv6s) with inv6s = recip_fast(6 s)
__device__ __forceinline__ float recip_fast(float x) { return x > 0.0f ? __builtin_amdgcn_rcpf(x) : 0.0f; }

__device__ __forceinline__ uint32_t e4m3_fast(float q) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(q, 448.0f), 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ uint32_t nvfp4_block_scale_fast(float amax, float inv6s) {
  return e4m3_fast(amax * inv6s);
}

// Exact decisions without float64 in the common case.  The exact NVFP4 path needs
// RNE_E4M3(amax / (6 s_t)) and RNE_E2M1(x / (s_b s_t)) of the real quotients.  In binary32,
// q = a * fl32(rcp(fl32(d))) with d = 6 s_t or s_b s_t lies within 2^-22 (relative) of the
// real quotient a / d, for d normal: one rounding of d (2^-24), the 1-ulp reciprocal
// (2^-23), one rounding of the product (2^-24).  If q (1 - 2^-19) and q (1 + 2^-19), each
// rounded once more, still round to the same code, the real quotient lies between them
// and, the rounding being monotone, rounds to that code too.  Otherwise (a quotient
// within about 2^-19 of a rounding boundary: ties, near-ties) the caller takes the
// float64 decision.  A quotient below the binary32 normal range is far below the first
// E2M1 / E4M3 boundary and needs no bound; a saturated one gives equal codes at both ends.
constexpr float kBelow = 1.0f - 0x1p-19f, kAbove = 1.0f + 0x1p-19f;

// A divisor d for which the bound above holds: normal and finite.
__device__ __forceinline__ bool checked_divisor(float d) { return d >= 0x1p-126f && d <= 0x1p+126f; }

// E4M3 code of amax * inv6s (inv6s = recip_fast(6 s_t)); false if it may differ from the
// code of the real quotient.
__device__ __forceinline__ bool nvfp4_block_scale_checked(float amax, float inv6s, uint32_t& code) {
  const float r = amax * inv6s;
  code = e4m3_fast(r);
  return e4m3_fast(r * kBelow) == e4m3_fast(r * kAbove);
}

// E2M1 codes of v * E (E = recip_fast(s_b s_t)); false if any may differ from the code of
// the real quotient.
__device__ __forceinline__ bool nvfp4_encode16_checked(const float* v, float E, uint2& w) {
  float q[16], lo[16], hi[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    q[i] = v[i] * E;
    lo[i] = q[i] * kBelow;
    hi[i] = q[i] * kAbove;
  }
  w = e2m1_encode16(q, 1.0f);
  const uint2 a = e2m1_encode16(lo, 1.0f), b = e2m1_encode16(hi, 1.0f);
  return a.x == b.x && a.y == b.y;
}

// --------------------------------------------------------------------------- E8M0

// MX scale code of a block maximum: floor(log2 amax) - 2 + 127, clamped to [0, 254];
// 0 for an all-zero block.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  if (!(amax > 0.0f)) return 0u;
  int e2;
  (void)frexpf(amax, &e2);                   // amax = f 2^e2, f in [0.5, 1)
  int e = e2 - 1 - 2;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return (uint32_t)(e + 127);
}

// 2^(code - 127) as a binary32 (code 0 is the subnormal 2^-127; 0xFF is the format's NaN,
// never produced by e8m0_from_amax).
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  const float v = code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
  return code == 0xFFu ? __uint_as_float(0x7FC00000u) : v;
}

// --------------------------------------------------------------------------- DPP quads

constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]: value of lane ^ 1
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]: value of lane ^ 2

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ float quad_partner(float v) {
  return dpp_move<CTRL>(v);
}

// Walsh-Hadamard butterflies across lane pairs, in signed form: every lane computes
// own + s partner with s = +1 on the lower lane of the pair (bit clear) and -1 on the upper
// one.  The lower lane gets a + b as the in-lane butterfly does; the upper lane gets
// b - a = -(a - b), the butterfly's output negated.  Negation commutes with rounding, so
// after several stages a lane holds its true value times the product of its stage signs,
// and the caller folds that sign into the final normalisation: every nonzero result is
// bit for bit the plain butterflies' result.  An exact zero is the one exception: an
// exactly cancelling sum rounds to +0 whatever the lane's sign, so after the fold it can
// come out as -0 where the plain butterflies give +0 (equal as numbers).
//
// Eight signed butterflies across lane pairs ^X at once: v[j] += v[j](lane ^ X) * s, as
// v_fmac_f32 with a DPP source (the compiler keeps the DPP move separate).  X = 1, 2 read
// the partner through one quad permutation; X = 4, 8 first move v[j] through a row
// mirror into a temporary and read the temporary through a second permutation (4: half
// mirror then quad reverse, (i ^ 7) ^ 3; 8: mirror then half mirror, (i ^ 15) ^ 7).  The
// leading s_nop 1 provides the two wait states a DPP read needs after a VALU write of its
// source; inside the block every DPP source was written at least eight instructions
// earlier.  Each fma rounds once: own + s partner exactly, then one rounding.
#define FP4_FMAC8(CTRL, S0, S1, S2, S3, S4, S5, S6, S7)                                       \
  "v_fmac_f32_dpp %0, " S0 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %1, " S1 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %2, " S2 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %3, " S3 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %4, " S4 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %5, " S5 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %6, " S6 ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                  \
  "v_fmac_f32_dpp %7, " S7 ", %16 " CTRL " row_mask:0xf bank_mask:0xf"
#define FP4_MOV8(CTRL)                                                                      \
  "v_mov_b32_dpp %8, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                            \
  "v_mov_b32_dpp %9, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                            \
  "v_mov_b32_dpp %10, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_mov_b32_dpp %11, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_mov_b32_dpp %12, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_mov_b32_dpp %13, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_mov_b32_dpp %14, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_mov_b32_dpp %15, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"

template <int X>
__device__ __forceinline__ void lane_butterflies8_signed(float* v, float s) {
  float t[8];
#define FP4_OPERANDS                                                                        \
  : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),    \
    "+v"(v[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]),           \
    "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])                                                    \
  : "v"(s)
  if constexpr (X == 1) {
    asm volatile("s_nop 1\n\t" FP4_FMAC8("quad_perm:[1,0,3,2]", "%0", "%1", "%2", "%3", "%4", "%5", "%6", "%7")
                 FP4_OPERANDS);
  } else if constexpr (X == 2) {
    asm volatile("s_nop 1\n\t" FP4_FMAC8("quad_perm:[2,3,0,1]", "%0", "%1", "%2", "%3", "%4", "%5", "%6", "%7")
                 FP4_OPERANDS);
  } else if constexpr (X == 4) {
    asm volatile("s_nop 1\n\t" FP4_MOV8("row_half_mirror")
                 FP4_FMAC8("quad_perm:[3,2,1,0]", "%8", "%9", "%10", "%11", "%12", "%13", "%14", "%15")
                 FP4_OPERANDS);
  } else {
    static_assert(X == 8, "lane distance 1, 2, 4 or 8");
    asm volatile("s_nop 1\n\t" FP4_MOV8("row_mirror")
                 FP4_FMAC8("row_half_mirror", "%8", "%9", "%10", "%11", "%12", "%13", "%14", "%15")
                 FP4_OPERANDS);
  }
#undef FP4_OPERANDS
}
#undef FP4_FMAC8
#undef FP4_MOV8

// Orthonormal H_B over a block spread as 8 contiguous elements per lane across B / 8
// consecutive lanes of a quad (lane p = position within the quad): the in-lane stages
// first (index bits 0-2), then the lane bits, then the 1/sqrt(B) scaling -- the same
// stage order, hence the same roundings, as block_hadamard on the whole block.
template <int B>
__device__ __forceinline__ void quad_hadamard8(float (&v)[8], int p) {
  if constexpr (B >= 16) {
    fwht_inplace<8>(v);
    const float s1 = (p & 1) ? -1.0f : 1.0f;
    lane_butterflies8_signed<1>(v, s1);
    float norm = s1 * InvSqrt<B>::v;
    if constexpr (B == 32) {
      const float s2 = (p & 2) ? -1.0f : 1.0f;
      lane_butterflies8_signed<2>(v, s2);
      norm *= s2;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= norm;
  }
}

// Two-level FWHT of a 128-group spread as 8 contiguous elements per lane over 16
// consecutive lanes (lane g of the group holds elements 8 g .. 8 g + 7): level 1 is H_16
// inside each micro-group (in-lane bits, then lane bit 0), level 2 is H_8 across the
// micro-groups (lane bits 1-3); normalised once at the end.  Same stage order as
// two_level_fwht128 on the whole group.
__device__ __forceinline__ void group16_two_level_fwht8(float (&v)[8], int g) {
  fwht_inplace<8>(v);
  const float s1 = (g & 1) ? -1.0f : 1.0f, s2 = (g & 2) ? -1.0f : 1.0f;
  const float s4 = (g & 4) ? -1.0f : 1.0f, s8 = (g & 8) ? -1.0f : 1.0f;
  lane_butterflies8_signed<1>(v, s1);
  lane_butterflies8_signed<2>(v, s2);
  lane_butterflies8_signed<4>(v, s4);
  lane_butterflies8_signed<8>(v, s8);
  const float norm = (__popc(g & 15) & 1) ? -InvSqrt<128>::v : InvSqrt<128>::v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= norm;
}

// Two-level FWHT of a 128-group spread over the four lanes of a DPP quad, lane p holding
// elements 32 p .. 32 p + 31 (micro-groups 2 p and 2 p + 1): level 1 is H_16 inside each
// micro-group (in-lane), level 2 is H_8 across the 8 micro-groups, whose index 2 p + h has
// the in-lane bit h and the two lane bits of p.  The lane-bit butterflies are the signed
// form above, so lane p's result carries the sign (-1)^popcount(p), folded into the
// 1/sqrt(128) normalisation.  Same stage order as two_level_fwht128 on the whole group.
// All four lanes of the quad must be active.
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
  for (int q = 0; q < 4; ++q) lane_butterflies8_signed<1>(v + 8 * q, c1);
#pragma unroll
  for (int q = 0; q < 4; ++q) lane_butterflies8_signed<2>(v + 8 * q, c2);
  const float norm = (__popc(p) & 1) ? -InvSqrt<128>::v : InvSqrt<128>::v;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= norm;
}

// Rotation of a lane's 32-element chunk before quantization: none (H = 0), H_16 / H_32 on
// whole blocks in-lane, or the two-level 128 transform across the chunk's quad
// (chunk index % 4 = position in its 128-group; the quad's four lanes must be active).
template <int H>
__device__ __forceinline__ void chunk_rotate(float* v, int64_t chunk) {
  if constexpr (H == 128)
    quad_two_level_fwht(v, (int)(chunk & 3));
  else
    block_hadamard<32, H>(v);
}

// Inverse rotation of 8 contiguous dequantized values per lane (the transforms are
// their own inverses): H_16 / H_32 across 2 / 4 lanes of a quad (p = lane % 4), or the
// two-level 128 transform across 16 lanes (g = lane % 16).  Every lane of the span takes
// part.
template <int H>
__device__ __forceinline__ void unit_rotate8(float (&v)[8], int lane) {
  if constexpr (H == 128)
    group16_two_level_fwht8(v, lane & 15);
  else
    quad_hadamard8<H>(v, lane & 3);
}

// --------------------------------------------------------------------------- reductions

template <int N>
__device__ __forceinline__ float absmax(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// One DPP step: v plus the value of the lane that dpp_ctrl kCtrl selects.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the wave, the same value in every lane, in a fixed order: partner sums within
// each row of 16 lanes by DPP (lane ^ 1, lane ^ 2, the half-row mirror, the row mirror --
// each pairs every lane with one partner, and a + b = b + a, so the lanes of a row agree),
// then (row 0 + row 1) + (row 2 + row 3) from lanes 0, 16, 32, 48.  No LDS round trip.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);   // row_half_mirror
  v = dpp_add<0x140>(v);   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Running maximum of non-negative floats through their bit patterns (monotone for >= 0).
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

}  // namespace fp4dev
