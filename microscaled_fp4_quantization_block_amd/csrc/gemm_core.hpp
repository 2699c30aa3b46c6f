#pragma once
// W4A4 MXFP4 GEMM on CDNA4 scaled MFMA: C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulate.
// The kernel body, shared by the library's GEMM (gemm.hip: A arrives quantized) and the
// fused-quantization experiment (gemm_fused.hip: A arrives as bf16 and every tile rotates
// and quantizes its A panel into LDS itself, see fill_a).
//
// Sources: MR-GPTQ abstract (hyper.ai, Résumé): FP4 GEMM kernels with the rotation folded
// into the weights and activations quantized on the fly; ARCQuant summary (gist.science,
// Méthodologie item 4): a single GEMM over the reduction axis whose high-precision
// accumulator sums every product.
//
// Design (gfx950):
// - v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 (cbsz = blgp = 4) and one
//   E8M0 scale per lane per operand: lane l supplies row (l % 32) of its operand, the
//   32-element K block (l / 32) of the current 64-element sub-step (16 bytes of codes),
//   and that block's scale byte.  The product is computed as C^T = B A^T so that each
//   lane ends up holding four consecutive output columns of one output row (an 8-byte
//   bf16 store) instead of four rows of one column.
// - Workgroup tile 256 x 256, 8 waves in a 4 x 2 grid of 64 x 128 (2 x 4 MFMA tiles, 128
//   fp32 accumulators per lane).  Two waves per SIMD: one wave's LDS reads and barrier
//   waits hide behind the other's MFMAs.
// - K advances in buffers of 256 elements: 128 code bytes per row (one cache line) per
//   operand.  Codes go global -> LDS directly (buffer_load ... lds, 16 bytes per lane,
//   eight lanes per row), double-buffered: buffer p + 2 is issued into the slot of
//   buffer p right after the barrier that ends buffer p's reads, so each load has a whole
//   buffer of MFMAs (64 per wave) to land.  Scales travel the same way in groups of 16
//   bytes per row (512 K elements), double-buffered per group.  No VGPR staging, no LDS
//   write instructions.
// - Per buffer, one barrier, placed before the last 64-element sub-step: that sub-step's
//   MFMAs run while the next buffer's first fragments and scales are read and the refill
//   is issued.  The barrier is a bare s_barrier after an explicit wait for the wave's own
//   loads; no memory fence, which would drain every load in flight.
// - Each 128-byte LDS row holds its eight 16-byte chunks XOR-swizzled by (row / 2) % 8, so
//   the sixteen lanes that share an LDS pass (one chunk of sixteen consecutive rows)
//   touch sixteen distinct 16-byte bank groups.
// - Buffer resources are built per tile: rows past M or N fall outside the resource and
//   read as zero (never fault), and only feed outputs that are not stored.
// - Tiles are assigned XCD-aware: consecutive workgroup ids land on different XCDs, so the
//   id is remapped to give every XCD a contiguous band of tiles, walked in groups of 8
//   tile-rows, keeping each XCD's L2 working set to a few A and B panels.
// - When K is a multiple of 256, tiles in odd tile columns start their walk over K one
//   scale group (two buffers) in and wrap around within the whole scale groups (an odd
//   last buffer, half a group, stays last): the tiles that share a B panel stay in step
//   (one stream of B per panel through L2), while neighbouring columns read different K
//   columns of their A panels at any moment.  Only the fp32 summation order
//   changes, and it depends on the parity of the tile column alone, so a GEMM over an
//   even number of 256-column tiles of B gives the same bits as those columns of a wider
//   product.
// - bf16 output (N % 8 == 0) leaves through LDS: the accumulators are written as bf16 into
//   the drained code buffers (16-byte chunks XOR-swizzled by row), then every wave stores
//   two full 512-byte tile rows per instruction, instead of 8 bytes per lane scattered
//   over 32 rows.  C stores are non-temporal.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256;
constexpr int BKP = 256;                           // K elements per LDS buffer ("pair" of 128-steps)
constexpr int ROWB = BKP / 2;                      // code bytes per row per buffer (128, one line)
constexpr int kCodeBytes = BM * ROWB;              // 32 KiB per operand per buffer
constexpr int kBufBytes = 2 * kCodeBytes;          // A + B codes
constexpr int kScaleRow = 16;                      // scale bytes per row per group (2 buffers = 512 K)
constexpr int kScaleBytes = BM * kScaleRow;        // 4 KiB per operand per group
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;             // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;             // offset past every resource: reads 0

// Wave arrangement: NW waves as WM x WN, each owning TI x TJ MFMA blocks of 32 x 32.
template <int NW> struct Cfg;
template <> struct Cfg<8> { static constexpr int WM = 4, WN = 2, TI = 2, TJ = 4; };

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

// C is written once and never read back by this kernel: non-temporal stores keep it from
// displacing operand panels in L2.
template <typename V>
__device__ __forceinline__ void store_streaming(void* p, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// LDS slot of 16-byte chunk c of code row r: c ^ ((r / 2) % 8).  A 16-byte LDS read
// serves 16 lanes per pass over 64 four-byte banks (256 bytes = two 128-byte rows); the
// fragment reads of 16 consecutive rows at one chunk then touch 16 distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Raw buffer descriptor over [base, base + bytes): stride 0, 32-bit data format.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS at lds + 16 lane
// (one wait state between the M0 write and the load that reads it).
// Written as one asm statement (M0 set and the load issued together; it has no register
// results) so the compiler neither sees nor waits on the LDS write: every wait for these
// loads is the explicit vmcnt(0) before a workgroup barrier.
__device__ __forceinline__ void dma16(const u32x4& rsrc, const uint8_t* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Per-thread loader state.  Per buffer and operand, 32 code instructions (8 rows x 128
// bytes = 1 KiB each) are split over the waves, QW = 32 / NW each; per scale group and
// operand, 4 instructions (64 rows x 16 bytes), SW = 8 / NW per wave over both operands.
template <int NW, bool FA = false>
struct Loader {
  static constexpr int QW = 32 / NW;
  static constexpr int SW = 8 / NW;
  u32x4 rA, rB, rSA, rSB;   // buffer descriptors (wave-uniform, SGPRs); rA, rSA unused when FA
  const uint16_t* a16;    // FA: the tile's first A row, bf16, rows of lda elements
  int arows, lda;         // FA: A rows of the tile inside the matrix; row length
  uint32_t code_off[2];   // lane offset of instruction 0 (even) / 1 (odd); +8 q rows per q
  uint32_t row_step;      // 8 rows in bytes
  uint32_t scale_off[SW];
  int wave;
  int rot, ne, np;        // walk offset (even), buffers it rotates over (even), buffer count
  int vcol_buf;           // buffer whose code loads carry the column in the VGPR offset (-1: none)
};

// Buffer that the tile processes at step p: p + rot wrapped into [0, ne) for the first ne
// steps, p itself after them.  ne is even and rot is even, so the two steps of a scale
// group stay one group; an odd last buffer (a half scale group) stays last.
template <int NW, bool FA>
__device__ __forceinline__ int rotated(const Loader<NW, FA>& L, int p) {
  if (p >= L.ne) return p;
  const int q = p + L.rot;
  return q >= L.ne ? q - L.ne : q;
}

// Issue buffer p (K elements 256 p ..) of both operands into `dst`.  Code instruction g
// fills bytes [g KiB, +1 KiB): lane l lands at byte 16 l = row 8 g + l / 8, slot l % 8,
// holding global chunk (l % 8) ^ swz(row) (which depends on g only through g % 2).
// `valid` false issues the instructions with every offset out of range (no memory
// traffic), keeping the control flow straight.
template <int NW, bool FA>
__device__ __forceinline__ void issue_codes(const Loader<NW, FA>& L, int p, bool valid, uint8_t* dst) {
  const int buf = rotated(L, p);
  // The half last buffer of a ragged K (K % 256 == 128) carries its column in the VGPR
  // offset, which the range check covers: its chunks past the operand's last row read
  // zeros.  Every other buffer keeps the column in the SGPR offset.  Both are wave-uniform.
  const uint32_t col = (uint32_t)(buf * ROWB);
  const uint32_t vcol = buf == L.vcol_buf ? col : 0u, scol = col - vcol;
#pragma unroll
  for (int q = 0; q < Loader<NW, FA>::QW; ++q) {
    uint8_t* blk = dst + (Loader<NW, FA>::QW * L.wave + q) * 1024;
    const uint32_t off = (valid ? L.code_off[q & 1] + (uint32_t)(q & ~1) * L.row_step : kOOB) + vcol;
    if constexpr (!FA) dma16(L.rA, blk, off, scol);
    dma16(L.rB, blk + kCodeBytes, off, scol);
  }
}

// Issue scale group h (16 scale bytes per row: K elements 512 h .., counted from the
// tile's starting buffer) into `dst` ([A rows][16 B] then [B rows][16 B]); instruction t
// covers rows 64 (t % 4) + l of operand t / 4.  rot and ne are even, so a group never
// straddles the wrap.  The group's column goes into the VGPR offset, which the
// descriptor's range check covers: when K % 512 != 0 the last group is half a group, and
// at the operand's last row its second 8 bytes lie past the end; they read as zeros (and
// are never used).
template <int NW, bool FA>
__device__ __forceinline__ void issue_scales(const Loader<NW, FA>& L, int h, bool valid, uint8_t* dst) {
  const uint32_t col = (uint32_t)((rotated(L, 2 * h) >> 1) * kScaleRow);
#pragma unroll
  for (int q = 0; q < Loader<NW, FA>::SW; ++q) {
    const int t = Loader<NW, FA>::SW * L.wave + q;
    uint8_t* blk = dst + (t >> 2) * kScaleBytes + (t & 3) * 1024;
    if (!FA || (t >> 2)) dma16((t >> 2) ? L.rSB : L.rSA, blk, (valid ? L.scale_off[q] : kOOB) + col, 0u);
  }
}

// Fused A path (FA): buffer q of the tile's 256 A rows (256 K elements, bf16 in memory),
// rotated by H_32 and quantized to MXFP4 by the workgroup itself, straight into the LDS
// code slot `dst` (the swizzled layout the DMA would write) and into half q % 2 of the
// scale group slot `sdst`.  Thread t takes the 8 columns 8 (t % 32) .. of rows
// 16 i + t / 32, i = 0..15: a 32-column block spans the four lanes of a quad, so H_32 ends
// with DPP butterflies across the quad (the same stages, hence the same roundings, as the
// in-lane transform of fp4_quantize) and the block maximum is a quad maximum.  Rows past
// the matrix read zeros.  Needs K % 256 == 0.
template <int NW, bool FA>
__device__ __forceinline__ void fill_a(const Loader<NW, FA>& L, int q, bool valid, uint8_t* dst, uint8_t* sdst) {
  if constexpr (FA) {
    if (!valid) return;
    int tid = threadIdx.x;
    // opaque per call: keeps the compiler from hoisting the 16 row addresses out of the
    // K loop and holding them in registers for the whole walk
    asm volatile("" : "+v"(tid));
    const int c8 = tid & 31, p4 = tid & 3, blk = c8 >> 2;
    const int col = rotated(L, q) * BKP + 8 * c8;
    constexpr int kBatch = 4;                       // loads in flight per lane
#pragma unroll 1
    for (int i0 = 0; i0 < 16; i0 += kBatch) {
      uint4 raw[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int row = 16 * (i0 + j) + (tid >> 5);
        raw[j] = row < L.arows ? *reinterpret_cast<const uint4*>(L.a16 + (size_t)row * L.lda + col)
                               : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int row = 16 * (i0 + j) + (tid >> 5);
        const uint32_t w4[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = fp4dev::bf16_lo(w4[k]);
          v[2 * k + 1] = fp4dev::bf16_hi(w4[k]);
        }
        fp4dev::quad_hadamard8<32>(v, p4);
        float m = fp4dev::absmax<8>(v);
        m = fmaxf(m, fp4dev::quad_partner<fp4dev::kQuadXor1>(m));
        m = fmaxf(m, fp4dev::quad_partner<fp4dev::kQuadXor2>(m));
        const uint32_t e = fp4dev::e8m0_from_amax(m);
        const float sc = fp4dev::e8m0_value(e);
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], sc, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], sc, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], sc, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], sc, 3);
        *reinterpret_cast<uint32_t*>(dst + row * ROWB + ((blk ^ swz(row)) << 4) + 4 * p4) = w;
        if (p4 == 0) sdst[row * kScaleRow + 8 * (q & 1) + blk] = (uint8_t)e;
      }
    }
  }
}

template <int NW>
struct Frags {
  v8i a[Cfg<NW>::TI], b[Cfg<NW>::TJ];
};

// Fragments of sub-step t (0..3, 64 K elements each) of the buffer `src`.
template <int NW>
__device__ __forceinline__ void read_codes(const uint8_t* src, int t, int wm, int wn, int r32,
                                           int khalf, Frags<NW>& f) {
  const int slot = ((2 * t + khalf) ^ swz(r32)) * 16;
#pragma unroll
  for (int j = 0; j < Cfg<NW>::TJ; ++j) {
    u32x4 w = *reinterpret_cast<const u32x4*>(src + kCodeBytes + (wn + 32 * j + r32) * ROWB + slot);
    f.b[j] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < Cfg<NW>::TI; ++i) {
    u32x4 w = *reinterpret_cast<const u32x4*>(src + (wm + 32 * i + r32) * ROWB + slot);
    f.a[i] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  }
}

// The 8 scale bytes of buffer p (blocks 8 (p % 2) .. of its group) for this lane's rows.
// For a buffer that ends after 128 elements (`half`), the scales of the four blocks past
// the end are set to 2^-127 on both operands: whatever (finite) codes lie there then
// contribute 2^-254 times at most 36, which is exactly zero in fp32.
template <int NW>
__device__ __forceinline__ void read_scales(const uint8_t* sgrp, int p, bool half, int wm, int wn,
                                            int r32, u32x2 (&sa)[Cfg<NW>::TI], u32x2 (&sb)[Cfg<NW>::TJ]) {
  const int off = 8 * (p & 1);
#pragma unroll
  for (int i = 0; i < Cfg<NW>::TI; ++i) {
    sa[i] = *reinterpret_cast<const u32x2*>(sgrp + (wm + 32 * i + r32) * kScaleRow + off);
    sa[i][1] = half ? 0u : sa[i][1];
  }
#pragma unroll
  for (int j = 0; j < Cfg<NW>::TJ; ++j) {
    sb[j] = *reinterpret_cast<const u32x2*>(sgrp + kScaleBytes + (wn + 32 * j + r32) * kScaleRow + off);
    sb[j][1] = half ? 0u : sb[j][1];
  }
}

// MFMAs of sub-step t: the lane's scale byte is block 2 t + khalf of the buffer.
template <int NW>
__device__ __forceinline__ void mfma_substep(v16f (&acc)[Cfg<NW>::TI][Cfg<NW>::TJ], const Frags<NW>& f,
                                             const u32x2 (&sa)[Cfg<NW>::TI], const u32x2 (&sb)[Cfg<NW>::TJ],
                                             int t, int khalf) {
  const int sh = 8 * (2 * (t & 1) + khalf);
#pragma unroll
  for (int i = 0; i < Cfg<NW>::TI; ++i) {
    const int scale_a = (int)(sa[i][t >> 1] >> sh);
#pragma unroll
    for (int j = 0; j < Cfg<NW>::TJ; ++j) {
      const int scale_b = (int)(sb[j][t >> 1] >> sh);
      // C^T tile = B-rows x A-rows^T: instruction operand A <- B codes, operand B <- A codes
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 4, 4, 0,
                                                                  scale_b, 0, scale_a);
    }
  }
}

// Interleave R LDS reads with F MFMAs in the current scheduling region: group k holds
// one read and F / R MFMAs, one more for the first F % R groups.
template <int k, int R, int F>
__device__ __forceinline__ void interleave_groups() {
  if constexpr (k < R) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, F / R + (k < F % R ? 1 : 0), 0);  // MFMA
    interleave_groups<k + 1, R, F>();
  }
}
template <int NW>
__device__ __forceinline__ void interleave_reads() {
  interleave_groups<0, Cfg<NW>::TI + Cfg<NW>::TJ, Cfg<NW>::TI * Cfg<NW>::TJ>();
}

// One buffer (4 sub-steps).  On entry f[0] holds sub-step 0 of buffer p (in `cur`) and
// sa/sb its scales.  Sub-steps 0..2 each run their MFMAs while the next sub-step's
// fragments are read.  Then every wave waits for its DMA of buffer p + 1 and meets the
// barrier: buffer p + 1 is complete and every read of `cur` is done, so `cur` is refilled
// with buffer p + 2 while sub-step 3 runs and the first fragments of buffer p + 1 are
// read.  Steps with p even also refill `sgrp_refill` with the scale group that starts at
// buffer p + 2.  Past the end the loads go out of range: they move no data but still
// write zeros to LDS, into slots that are dead by then (`cur` after its last read, and a
// scale slot whose group was last read two steps earlier).
template <int NW, bool kRefillScales, bool FA>
__device__ __forceinline__ void run_buffer(v16f (&acc)[Cfg<NW>::TI][Cfg<NW>::TJ], Frags<NW> (&f)[2],
                                           u32x2 (&sa)[Cfg<NW>::TI], u32x2 (&sb)[Cfg<NW>::TJ],
                                           const Loader<NW, FA>& L, int p, int np, bool ragged,
                                           uint8_t* cur, const uint8_t* next,
                                           uint8_t* sgrp_refill, const uint8_t* sgrp_next,
                                           int wm, int wn, int r32, int khalf) {
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    read_codes<NW>(cur, t + 1, wm, wn, r32, khalf, f[(t + 1) & 1]);
    mfma_substep<NW>(acc, f[t & 1], sa, sb, t, khalf);
    interleave_reads<NW>();
    __builtin_amdgcn_sched_barrier(0);
  }
  // own DMA of buffer p + 1 landed and own reads of `cur` done; then the workgroup
  // barrier (no memory fence: the waits above are the ordering this step needs)
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  // FA: quantize A's buffer p + 2 into `cur`; its scales go to the slot of scale group
  // (p + 2) / 2, the refill slot on even steps and the next-buffer slot on odd ones (the
  // half that buffer p + 1 does not read).  Waited for at the next step's barrier.
  if constexpr (FA) {
    __builtin_amdgcn_sched_barrier(0);             // no fragment read hoisted above it
    fill_a(L, p + 2, p + 2 < np, cur, kRefillScales ? sgrp_refill : const_cast<uint8_t*>(sgrp_next));
    __builtin_amdgcn_sched_barrier(0);
  }
  u32x2 na[Cfg<NW>::TI], nb[Cfg<NW>::TJ];
  read_scales<NW>(sgrp_next, p + 1, ragged && p + 1 == np - 1, wm, wn, r32, na, nb);
  read_codes<NW>(next, 0, wm, wn, r32, khalf, f[0]);
  const int q = p + 2;
  if constexpr (kRefillScales) issue_scales<NW>(L, q >> 1, q < np, sgrp_refill);
  issue_codes<NW>(L, q, q < np, cur);
  mfma_substep<NW>(acc, f[1], sa, sb, 3, khalf);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < Cfg<NW>::TI; ++i) sa[i] = na[i];
#pragma unroll
  for (int j = 0; j < Cfg<NW>::TJ; ++j) sb[j] = nb[j];
}

// The whole walk over K.  Code buffer p lives in c[p % 2] and scale group h in s[h % 2];
// the loop is unrolled by four so that every access names its slot statically.  All four
// slots arrive as restrict pointers of this one function, so the compiler knows for the
// whole loop that a DMA into one slot never overlaps reads of another and adds no waits
// of its own (the loop-carried DMA would otherwise cost a full drain per buffer).
template <int NW, bool FA>
__device__ __forceinline__ void k_loop(v16f (&acc)[Cfg<NW>::TI][Cfg<NW>::TJ], const Loader<NW, FA>& L, int np,
                                       bool ragged, uint8_t* __restrict__ c0, uint8_t* __restrict__ c1,
                                       uint8_t* __restrict__ s0, uint8_t* __restrict__ s1, int wm, int wn,
                                       int r32, int khalf) {
  // prologue: buffers 0 and 1 and scale group 0 in flight (FA: A quantized into place first)
  if constexpr (FA) {
    fill_a(L, 0, true, c0, s0);
    fill_a(L, 1, np > 1, c1, s0);
  }
  issue_scales<NW>(L, 0, true, s0);
  issue_codes<NW>(L, 0, true, c0);
  issue_codes<NW>(L, 1, np > 1, c1);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  Frags<NW> f[2];
  u32x2 sa[Cfg<NW>::TI], sb[Cfg<NW>::TJ];
  read_scales<NW>(s0, 0, ragged && np == 1, wm, wn, r32, sa, sb);
  read_codes<NW>(c0, 0, wm, wn, r32, khalf, f[0]);
  for (int p = 0; p < np; p += 4) {
    run_buffer<NW, true>(acc, f, sa, sb, L, p, np, ragged, c0, c1, s1, s0, wm, wn, r32, khalf);
    if (p + 1 < np) run_buffer<NW, false>(acc, f, sa, sb, L, p + 1, np, ragged, c1, c0, s0, s1, wm, wn, r32, khalf);
    if (p + 2 < np) run_buffer<NW, true>(acc, f, sa, sb, L, p + 2, np, ragged, c0, c1, s0, s1, wm, wn, r32, khalf);
    if (p + 3 < np) run_buffer<NW, false>(acc, f, sa, sb, L, p + 3, np, ragged, c1, c0, s1, s0, wm, wn, r32, khalf);
  }
}

// FA false: A is MXFP4 codes [M][K/2] and scales SA [M][K/32].  FA true: A is bf16
// [M][K] (passed as bytes) quantized on the fly, SA unused, K % 256 == 0.
template <int NW, bool FA = false>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
k_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
       const uint8_t* __restrict__ SB, int M, int N, int K, void* __restrict__ C, int ctype) {
  // device-only body (buffer resources and MFMA builtins have no host form)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int TI = Cfg<NW>::TI, TJ = Cfg<NW>::TJ;
  __shared__ __attribute__((aligned(1024))) uint8_t codes[2][kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t scales[2][2 * kScaleBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const Tile tile = tile_of(blockIdx.x, tiles_m, tiles_n);
  const uint32_t rowbytes = (uint32_t)K / 2, rowscales = (uint32_t)K / 32;
  const int np = (K + BKP - 1) / BKP;              // K % 128 == 0
  const bool ragged = (K % BKP) != 0;              // last buffer holds 128 elements

  Loader<NW, FA> L;
  {
    const uint32_t rows_a = (uint32_t)min(BM, M - tile.m0), rows_b = (uint32_t)min(BN, N - tile.n0);
    if constexpr (FA) {
      L.a16 = reinterpret_cast<const uint16_t*>(A) + (size_t)tile.m0 * K;
      L.arows = (int)rows_a;
      L.lda = K;
    } else {
      L.rA = make_rsrc(A + (size_t)tile.m0 * rowbytes, rows_a * rowbytes);
    }
    L.rB = make_rsrc(B + (size_t)tile.n0 * rowbytes, rows_b * rowbytes);
    if constexpr (!FA) L.rSA = make_rsrc(SA + (size_t)tile.m0 * rowscales, rows_a * rowscales);
    L.rSB = make_rsrc(SB + (size_t)tile.n0 * rowscales, rows_b * rowscales);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 8 * (Loader<NW, FA>::QW * wave + q) + (lane >> 3);
      L.code_off[q] = (uint32_t)row * rowbytes + 16u * (uint32_t)((lane & 7) ^ swz(row));
    }
    L.row_step = 8u * rowbytes;
#pragma unroll
    for (int q = 0; q < Loader<NW, FA>::SW; ++q) {
      const int t = Loader<NW, FA>::SW * wave + q;
      L.scale_off[q] = (uint32_t)(64 * (t & 3) + lane) * rowscales;
    }
    L.wave = wave;
    L.np = np;
    L.ne = ragged ? 0 : (np & ~1);                 // a ragged last buffer keeps the walk unrotated
    L.rot = L.ne >= 4 ? 2 * ((tile.n0 / BN) & 1) : 0;
    L.vcol_buf = ragged ? np - 1 : -1;
  }

  const int wm = (wave / Cfg<NW>::WN) * (32 * TI), wn = (wave % Cfg<NW>::WN) * (32 * TJ);
  const int r32 = lane & 31, khalf = lane >> 5;   // row within a 32-block, K block in a sub-step
  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  k_loop<NW>(acc, L, np, ragged, codes[0], codes[1], scales[0], scales[1], wm, wn, r32, khalf);

  // epilogue: lane holds C[m][n0 .. n0+3] for m = row r32 of A-block i, n0 = 8 g + 4 khalf in B-block j
  if (ctype == fp4impl::DT_BF16 && (N & 7) == 0) {
    // every LDS DMA (including the out-of-range ones past the end) has landed and every
    // wave is done with the code buffers
    __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    uint8_t* ct = codes[0];                      // [256 rows][512 bytes] of bf16, 128 KiB
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int m = wm + 32 * i + r32;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int byte = 2 * (wn + 32 * j + 8 * g + 4 * khalf);
          const int pos = (((byte >> 4) ^ (m & 15)) << 4) | (byte & 15);
          *reinterpret_cast<uint2*>(ct + m * 512 + pos) =
              make_uint2(fp4dev::pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                         fp4dev::pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
        }
      }
    }
    __syncthreads();
    // thread t: 16-byte chunk t % 32 of rows t / 32 + (2 NW) k
    const int c = tid & 31;
    uint16_t* C16 = reinterpret_cast<uint16_t*>(C);
#pragma unroll
    for (int k = 0; k < BM / (2 * NW); ++k) {
      const int m = (tid >> 5) + 2 * NW * k;
      const uint4 v = *reinterpret_cast<const uint4*>(ct + m * 512 + ((c ^ (m & 15)) << 4));
      const int gm = tile.m0 + m, gn = tile.n0 + 8 * c;
      if (gm < M && gn < N) store_streaming(C16 + (int64_t)gm * N + gn, u32x4{v.x, v.y, v.z, v.w});
    }
    return;
  }
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int m = tile.m0 + wm + 32 * i + r32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = tile.n0 + wn + 32 * j + 8 * g + 4 * khalf;
        const float c0 = acc[i][j][4 * g], c1 = acc[i][j][4 * g + 1];
        const float c2 = acc[i][j][4 * g + 2], c3 = acc[i][j][4 * g + 3];
        if (ctype == fp4impl::DT_BF16) {
          uint16_t* cp = reinterpret_cast<uint16_t*>(C) + (int64_t)m * N + n0;
          if (vec_ok && n0 + 3 < N) {
            store_streaming(cp, u32x2{fp4dev::pack_bf16x2(c0, c1), fp4dev::pack_bf16x2(c2, c3)});
          } else {
            if (n0 < N) cp[0] = (uint16_t)fp4dev::bf16_bits_rne(c0);
            if (n0 + 1 < N) cp[1] = (uint16_t)fp4dev::bf16_bits_rne(c1);
            if (n0 + 2 < N) cp[2] = (uint16_t)fp4dev::bf16_bits_rne(c2);
            if (n0 + 3 < N) cp[3] = (uint16_t)fp4dev::bf16_bits_rne(c3);
          }
        } else {
          float* cp = reinterpret_cast<float*>(C) + (int64_t)m * N + n0;
          if (vec_ok && n0 + 3 < N) {
            store_streaming(cp, u32x4{__float_as_uint(c0), __float_as_uint(c1), __float_as_uint(c2), __float_as_uint(c3)});
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
#endif
}

}  // namespace

