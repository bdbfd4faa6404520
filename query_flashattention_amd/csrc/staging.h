// Row staging and synchronisation helpers shared by the matrix-core attention
// kernels: direct global -> LDS row transfers, LDS-only barriers, explicit
// vector-memory waits, and the LDS tile geometry.
#pragma once

#include "mfma_common.h"

namespace ds4attn {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef int int2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (byte i = element i) to float16, exactly (every finite E4M3
// value is a float16 value; the conversion's scale operand is 1).
__device__ __forceinline__ half8 e4m3x8_to_half8(uint2 w) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.x, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.x, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.y, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w.y, 1.0f, true);
  const half4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const half4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E4M3 x E4M3 products on the matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4):
// operand lane l holds row (column) l % 16 and 32 codes of the 128-long k range;
// A and B pair their codes by lane group and byte, so any k order both operands
// share gives the same sums (the hardware takes bytes 0-15 of group G as k = 16G..
// and bytes 16-31 as k = 64 + 16G..).  Both operands are scaled by 2^(SB - 127) on
// the B side only (uniform E8M0 scale, byte 0 of the scale register).
typedef int int8v __attribute__((ext_vector_type(8)));
template <int SB>
__device__ __forceinline__ floatx4 mfma_e4m3(const int8v &a, const int8v &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, SB);
}

// A float16 query row as two E4M3 terms for those matrix cores: with s = 2^(E - 7),
// where 2^(E - 1) <= max |q| < 2^E over the head (E at least -8), hi = RN(q / s) and
// lo = RN((q - s hi) / (s / 16)), so that q = s (hi + lo / 16) to within 2^-8 |q|
// or 2^-14 s, whichever is larger (s <= 2^-6 max |q|).  Every term stays below 128
// (the E4M3 encoding has no saturation: beyond 448 it gives NaN), and s hi is
// exact in float16 for E >= -8, so the residual is exact too.  `q` holds this
// lane's NC x 32 elements (chunk c, elements 8j .. 8j + 7 in q[c][j]); element e
// of a chunk goes to byte e of the chunk's 32-byte operand.  `amax` is the max |q|
// over every element the factor covers (all lanes concerned agree).  Returns s.
template <int NC>
__device__ __forceinline__ float split_e4m3(const half8 (&q)[NC][4], float amax, int8v (&hi)[NC],
                                            int8v (&lo)[NC]) {
  typedef short short2_t __attribute__((ext_vector_type(2)));
  int e = (int)(__float_as_uint(amax) >> 23) - 126;   // amax = m 2^e, m in [0.5, 1)
  e = e < -8 ? -8 : e;
  const float s = __uint_as_float((uint32_t)(e - 7 + 127) << 23), s16 = s * 0.0625f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const half8 &v = q[c][d >> 1];
      const half2v x0 = {v[4 * (d & 1)], v[4 * (d & 1) + 1]};
      const half2v x1 = {v[4 * (d & 1) + 2], v[4 * (d & 1) + 3]};
      short2_t t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(short2_t{0, 0}, x0, s, false);
      t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(t, x1, s, true);
      const int h = __builtin_bit_cast(int, t);
      const half2v r0 = x0 - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h, s, false);
      const half2v r1 = x1 - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h, s, true);
      short2_t u = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(short2_t{0, 0}, r0, s16, false);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(u, r1, s16, true);
      hi[c][d] = h;
      lo[c][d] = __builtin_bit_cast(int, u);
    }
  }
  return s;
}

// One row: 16 bytes per lane from `row` + 16 * lane (`row` uniform) into LDS at
// `lds` + 16 * lane (`lds` uniform).  The row address travels in scalar registers
// and the lane offset is one shared vector register.  Issued through asm, so the
// compiler's hazard tracking does not see it: the tracking cannot always tell the
// tile buffers from the other LDS arrays and would drain every transfer in flight
// before unrelated LDS reads.  Completion is awaited explicitly (wait_vmcnt)
// before the barrier that publishes a tile, and a buffer is refilled only after
// the barrier that ends its reads.  m0 is written only here in these kernels.
__device__ __forceinline__ void dma16(const char *row, uint32_t lane16, uint32_t lds) {
  // (the builtin returns int: widen each half as unsigned, never sign-extended)
  const uint64_t r = (uint64_t)row;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32));
  const uint64_t ru = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(lane16), "s"(ru), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// A wave-uniform global-memory pointer moved to scalar registers, so that loads
// from it take the scalar-base form with one shared lane offset.  The result is
// typed as global memory: a generic pointer would make them flat loads, which
// also count as LDS operations, so every wait for LDS would wait for them too.
typedef __attribute__((address_space(1))) const char gchar;
__device__ __forceinline__ gchar *uniform_ptr(const char *row) {
  const uint64_t r = (uint64_t)row;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32));
  return (gchar *)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// The same transfer with a per-lane source address: lane i's 16 bytes come from
// `src` (a different row for different lanes) and land at `lds` + 16 * i.  Used
// for FP8 rows, two 512-byte rows per instruction.
__device__ __forceinline__ void dma16_lanes(const char *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 4 bytes per active lane from a per-lane address into LDS at `lds` + 4 * lane.
__device__ __forceinline__ void dma4_lanes(const char *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void *)p;
}

// Source of the rows a mask hides: they arrive in LDS as zeros (from L2).
static __device__ __attribute__((aligned(16))) const char kZeroRow[1024] = {};

// Workgroup barrier for LDS data only: this wave's LDS operations complete, then
// s_barrier.  (The generic barrier also waits for every outstanding global load,
// which would drain the tile transfers kept in flight across it.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N) (other counters untouched), issued through the builtin so
// that the compiler's own wait insertion knows what it has already waited for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// A stage is exactly 16 vector-memory instructions per wave (8 K rows, 8 V rows);
// waiting with vmcnt(16) right after issuing one completes every older stage.
constexpr int kStageOps = 16;

// Visibility masks of list entries live in an LDS ring of 128, filled 64 entries
// at a time, so the half in use is never overwritten.
constexpr int kMaskRing = 128, kMaskChunk = 64;
constexpr int kTable = 256 / kRowsPerBlock;   // dense blocks masked at the start, a row per thread

// Tile rows are padded so that rows start on different banks while every operand
// address stays affine (base + immediate).  Both K and V rows are 1056 bytes apart
// (32 bytes past a multiple of 256): the 16-byte K operand reads of 16 rows and the
// 4 rows x 32 bytes of a V transpose read then meet no bank conflict (rocprofv3
// SQ_LDS_BANK_CONFLICT reads 0).  K rows 1040 bytes apart (16 past a multiple of
// 256) made the K reads conflict: about one stall cycle per LDS instruction.
constexpr int kKRow = 1056, kVRow = 1056;
constexpr int kKTile = 32 * kKRow, kVTile = 32 * kVRow;

// FP8 tiles (512-byte rows of E4M3 codes).  One transfer moves a pair of rows,
// each contiguous (lanes 0-31 the first, 32-63 the second: two contiguous halves
// cost the transfer path about a third less than rows interleaved in 16-byte
// chunks).  Pair p holds row p, then row p + 24 (p < 8) or p + 8 (p >= 8); pairs
// are 1040 bytes apart.  So the 8-byte operand reads of a half-wave touch every
// pair once and fall on distinct banks: K reads rows 0-15 (or 16-31), the 8-bit
// transpose reads rows 0-7 with 16-23 (or 8-15 with 24-31).  A stage is 4 pairs
// of K rows, 4 of V rows and one transfer of 16 scales per wave.
constexpr int kF8Pair = 1040;
__host__ __device__ constexpr int f8_second_row(int p) { return p < 8 ? p + 24 : p + 8; }
__host__ __device__ constexpr int f8_row_off(int r) { return r < 16 ? r * kF8Pair : ((r - 16) ^ 8) * kF8Pair + 512; }
constexpr int kF8Tile = 16 * kF8Pair;
constexpr int kF8StageOps = 9;


}  // namespace ds4attn
