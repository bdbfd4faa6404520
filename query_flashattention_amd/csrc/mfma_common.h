// Helpers shared by the matrix-core attention kernels (decode and prefill).
#pragma once

#include "ds4attn_internal.h"

#include <type_traits>

namespace ds4attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kListCap = 2048;  // non-skipped map blocks a workgroup can list in LDS (65536 rows)

// Buffer descriptors: loads through them take a 32-bit byte offset, and an offset
// at or beyond the descriptor's size returns zero without touching memory.  The
// validity-byte loads use this for rows that have no byte to check.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;   // regions are limited to < 2^31 bytes per sequence

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int buf_load_u8(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const half8 &a, const half8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
// 16 x 16 x 16: operand lane l holds row (column) l % 16, k-slots 4(l / 16) .. +3.
__device__ __forceinline__ floatx4 mfma16k16(const half4v &a, const half4v &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Key slot k (0..31) of an MFMA operand group: slots 8G..8G+3 hold block rows
// 4G..4G+3 and slots 8G+4..8G+7 hold rows 16+4G..16+4G+3, which is exactly the
// set of rows one lane holds in the 16x16 score accumulators of both row tiles.
__device__ __forceinline__ int slot_row(int G, int i) { return i < 4 ? 4 * G + i : 16 + 4 * G + (i - 4); }

// Bits 0..7 of the result: which of the rows slot_row(G, 0..7) are set in `vis`.
__device__ __forceinline__ uint32_t slot_mask(uint32_t vis, int G) {
  return ((vis >> (4 * G)) & 0xfu) | (((vis >> (16 + 4 * G)) & 0xfu) << 4);
}

// Butterfly steps across the four 16-lane groups without the LDS crossbar:
// v_permlane16_swap / v_permlane32_swap with both operands equal hand each lane
// the pair {x[l], x[l ^ 16]} (resp. {x[l], x[l ^ 32]}) in some order, so max and
// sum of the pair are the values of a xor-16 (xor-32) exchange on every lane.
__device__ __forceinline__ float xor_max(float x, int d) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = d == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float xor_sum(float x, int d) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = d == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Maximum over the wave: DPP within rows of 16 lanes (quad swaps, then half-row
// and row mirrors), then the swaps of rows across the halves.
__device__ __forceinline__ float wave_max(float x) {
  auto dpp = [](float v, auto ctrl) __attribute__((always_inline)) {
    constexpr int C = decltype(ctrl)::value;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), C, 0xf, 0xf, false));
  };
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0xb1>{}));    // quad_perm(1, 0, 3, 2): lane ^ 1
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x4e>{}));    // quad_perm(2, 3, 0, 1): lane ^ 2
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x141>{}));   // row_half_mirror: the other quad of 8
  x = fmaxf(x, dpp(x, std::integral_constant<int, 0x140>{}));   // row_mirror: the other half of 16
  x = xor_max(x, 16);
  x = xor_max(x, 32);
  return x;
}

// The online softmax keeps a reference max m per row and rescales the output only
// when a block's max exceeds it by more than this many binary orders of magnitude.
// Below that, P = 2^(s - m) <= 2^8 is exact enough in float16 (11-bit mantissa at
// any magnitude) and l, O accumulate in float32, so the result is the same softmax
// up to rounding while the accumulators are rarely touched outside the MFMAs.
constexpr float kRescaleSlack = 8.f;

// The workgroup lists, in LDS, the map blocks of its query tile that are not SKIP:
// entry = block | status << 14, in block order.  A null map lists every block as
// PARTIAL.  All threads of the workgroup must call it; it always ends with a barrier.
// `cnt` is LDS scratch of NT/64 ints.  `s_first` >= 0 is the status of block
// `threadIdx.x` already loaded by the caller (0 past the end of the row).  The
// barriers order LDS only (lgkmcnt, then s_barrier): a full __syncthreads would
// also wait for every global load in flight, such as the query rows loaded after
// the map row.
template <int NT>
__device__ __forceinline__ int build_block_list(const uint8_t *row, int nbd, uint16_t *list, int *cnt,
                                                int s_first = -1) {
  constexpr int NW = NT / 64;
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int total = 0;
  for (int base = 0; base < nbd; base += NT) {
    const int j = base + tid;
    int s = 0;
    if (base == 0 && s_first >= 0) s = s_first;
    else if (j < nbd) s = row ? (int)row[j] : kPartial;
    const unsigned long long m = __ballot(s != 0);
    if (lane == 0) cnt[wv] = __popcll(m);
    barrier();
    int off = total, sum = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int c = cnt[k];
      off += (k < wv) ? c : 0;
      sum += c;
    }
    if (s != 0) {
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      list[off + rank] = (uint16_t)(j | (s << 14));
    }
    total += sum;
    barrier();
  }
  barrier();  // also orders any LDS writes made before the call when the map is empty
  return total;
}

}  // namespace ds4attn
