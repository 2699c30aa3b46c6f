// W4A4 MXFP4 GEMM on CDNA4 scaled MFMA: C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulate.
//
// Sources: MR-GPTQ abstract (hyper.ai, Résumé): FP4 GEMM kernels with the rotation folded
// into the weights and activations quantized on the fly; ARCQuant summary (gist.science,
// Méthodologie item 4): a single GEMM over the reduction axis whose high-precision
// accumulator sums every product.
//
// Design (gfx950):
// - v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 (cbsz = blgp = 4) and one
//   E8M0 scale per lane per operand: lane l supplies row (l % 32) of its operand, the
//   32-element K block (l / 32) of the current 64-element step (16 bytes of codes), and
//   that block's scale byte.  The product is computed as C^T = B A^T so that each lane
//   ends up holding four consecutive output columns of one output row (an 8-byte bf16
//   store) instead of four rows of one column.
// - Workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 MFMA tiles, 256 fp32
//   accumulators per lane), K step 256 elements = 128 bytes per row = one cache line.
// - Global -> register prefetch of the next K step while the current one is multiplied
//   out of LDS; LDS rows padded to 144 bytes so the 16-lane phases of a 16-byte LDS read
//   hit distinct banks.
// - Tiles are assigned XCD-aware: consecutive workgroup ids land on different XCDs, so the
//   id is remapped to give every XCD a contiguous band of tiles, walked in groups of 8
//   tile-rows, keeping each XCD's L2 working set to a few A and B panels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 256;      // BK in elements
constexpr int ROWB = BK / 2;                      // code bytes per row per K step
constexpr int LDS_STRIDE = ROWB + 16;             // padded LDS row
constexpr int kThreads = 256;
constexpr int kChunks = BM * ROWB / 16 / kThreads; // 16-byte chunks per thread per operand (8)
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)

struct Tile { int m0, n0; };

__device__ __forceinline__ Tile tile_of(int id, int tiles_m, int tiles_n) {
  const int total = tiles_m * tiles_n;
  // XCD-aware remap: hardware places workgroup id on XCD (id % 8); give XCD x the
  // contiguous range [x * total / 8, (x + 1) * total / 8) when that divides evenly.
  if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
  const int per_group = kGroupM * tiles_n;
  const int g = id / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = id % per_group;
  Tile t;
  t.m0 = (first_m + r % gm) * BM;
  t.n0 = (r / gm) * BN;
  return t;
}

__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
       const uint8_t* __restrict__ SB, int M, int N, int K, void* __restrict__ C, int ctype) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * LDS_STRIDE];
  __shared__ uint2 sSA[BM];
  __shared__ uint2 sSB[BN];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const Tile tile = tile_of(blockIdx.x, tiles_m, tiles_n);
  const uint32_t rowbytes = (uint32_t)K / 2, rowscales = (uint32_t)K / 32;
  const int nk = (K + BK - 1) / BK;
  const bool ragged = (K % BK) != 0;              // last K step holds only 128 elements

  // Buffer resources: out-of-range offsets read as 0 and never fault, so rows past M / N
  // need no clamping (they only feed outputs that are never stored).
  const uint32_t kOOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(rowbytes * (uint32_t)M), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, (int)(rowbytes * (uint32_t)N), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)SA, 0, (int)(rowscales * (uint32_t)M), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rSB = __builtin_amdgcn_make_buffer_rsrc((void*)SB, 0, (int)(rowscales * (uint32_t)N), kRsrcWord3);

  // loader mapping: chunk i of thread tid -> row (tid / 8) + 32 i, 16-byte column tid % 8
  const int lrow = tid >> 3, lcol = (tid & 7) * 16;
  uint32_t offA[kChunks], offB[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int am = tile.m0 + lrow + 32 * i, bn = tile.n0 + lrow + 32 * i;
    offA[i] = am < M ? (uint32_t)am * rowbytes + lcol : kOOB;
    offB[i] = bn < N ? (uint32_t)bn * rowbytes + lcol : kOOB;
  }
  const uint32_t offSA = tile.m0 + tid < M ? (uint32_t)(tile.m0 + tid) * rowscales : kOOB;
  const uint32_t offSB = tile.n0 + tid < N ? (uint32_t)(tile.n0 + tid) * rowscales : kOOB;

  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x4 ra[kChunks], rb[kChunks];
  u32x2 rsa, rsb;
  auto gload = [&](int kb) {
    const int soff = kb * ROWB;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, offA[i], soff, 0);
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, offB[i], soff, 0);
    }
    rsa = __builtin_amdgcn_raw_buffer_load_b64(rSA, offSA, kb * (BK / 32), 0);
    rsb = __builtin_amdgcn_raw_buffer_load_b64(rSB, offSB, kb * (BK / 32), 0);
    if (ragged && kb == nk - 1) {                   // keep only the first 128 elements
      if (lcol >= ROWB / 2) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) { ra[i] = u32x4{0, 0, 0, 0}; rb[i] = u32x4{0, 0, 0, 0}; }
      }
      rsa[1] = 0x7F7F7F7Fu;
      rsb[1] = 0x7F7F7F7Fu;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<u32x4*>(sA + row * LDS_STRIDE + lcol) = ra[i];
      *reinterpret_cast<u32x4*>(sB + row * LDS_STRIDE + lcol) = rb[i];
    }
    sSA[tid] = make_uint2(rsa[0], rsa[1]);
    sSB[tid] = make_uint2(rsb[0], rsb[1]);
  };

  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int r32 = lane & 31, khalf = lane >> 5;     // row within a 32-tile, K block in a step
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  gload(0);
  lstore();
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) gload(kb + 1);
    uint2 sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = sSA[wm + 32 * i + r32];
#pragma unroll
    for (int j = 0; j < 4; ++j) sb[j] = sSB[wn + 32 * j + r32];
#pragma unroll
    for (int s = 0; s < BK / 64; ++s) {
      const int off = s * 32 + khalf * 16;
      const int sh = 16 * (s & 1) + 8 * khalf;
      v8i fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = *reinterpret_cast<const uint4*>(sB + (wn + 32 * j + r32) * LDS_STRIDE + off);
        fb[j] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 w = *reinterpret_cast<const uint4*>(sA + (wm + 32 * i + r32) * LDS_STRIDE + off);
        const v8i fa = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        const int scale_a = (int)(((s < 2) ? sa[i].x : sa[i].y) >> sh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int scale_b = (int)(((s < 2) ? sb[j].x : sb[j].y) >> sh);
          // C^T tile = B-rows x A-rows^T: instruction operand A <- B codes, operand B <- A codes
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[j], fa, acc[i][j], 4, 4, 0, scale_b, 0, scale_a);
        }
      }
    }
    __syncthreads();
    if (kb + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // epilogue: lane holds C[m][n0 .. n0+3] for m = row r32 of A-tile i, n0 = 8 g + 4 khalf in B-tile j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tile.m0 + wm + 32 * i + r32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = tile.n0 + wn + 32 * j + 8 * g + 4 * khalf;
        const float c0 = acc[i][j][4 * g], c1 = acc[i][j][4 * g + 1];
        const float c2 = acc[i][j][4 * g + 2], c3 = acc[i][j][4 * g + 3];
        if (ctype == fp4impl::DT_BF16) {
          uint16_t* cp = reinterpret_cast<uint16_t*>(C) + (int64_t)m * N + n0;
          if (n0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2*>(cp) = make_uint2(fp4dev::pack_bf16x2(c0, c1), fp4dev::pack_bf16x2(c2, c3));
          } else {
            if (n0 < N) cp[0] = (uint16_t)fp4dev::bf16_bits_rne(c0);
            if (n0 + 1 < N) cp[1] = (uint16_t)fp4dev::bf16_bits_rne(c1);
            if (n0 + 2 < N) cp[2] = (uint16_t)fp4dev::bf16_bits_rne(c2);
            if (n0 + 3 < N) cp[3] = (uint16_t)fp4dev::bf16_bits_rne(c3);
          }
        } else {
          float* cp = reinterpret_cast<float*>(C) + (int64_t)m * N + n0;
          if (n0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<float4*>(cp) = make_float4(c0, c1, c2, c3);
          } else {
            if (n0 < N) cp[0] = c0;
            if (n0 + 1 < N) cp[1] = c1;
            if (n0 + 2 < N) cp[2] = c2;
            if (n0 + 3 < N) cp[3] = c3;
          }
        }
      }
    }
  }
}

}  // namespace

namespace fp4impl {

hipError_t launch_gemm(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, void* c, int ctype, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm<<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(a, sa, b, sb, (int)M, (int)N, (int)K, c, ctype);
  return hipGetLastError();
}

}  // namespace fp4impl
