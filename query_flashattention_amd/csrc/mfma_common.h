// Helpers shared by the matrix-core attention kernels (decode and prefill).
#pragma once

#include "ds4attn_internal.h"

namespace ds4attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kListCap = 4096;  // non-skipped map blocks a workgroup can list in LDS (131072 rows)

// Buffer descriptors: loads through them take a 32-bit byte offset, and an offset
// at or beyond the descriptor's size returns zero without touching memory.  The
// kernels issue such out-of-range loads where a load must be counted but no data
// is needed, so every loop trip issues the same instructions.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;   // regions are limited to < 2^31 bytes per sequence
typedef int int4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const int4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ int buf_load_u8(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const half8 &a, const half8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Position (in 16-byte units) of the transposed-V chunk holding key slots 8G..8G+7
// of head-dim row d.  Rows and slot groups are swizzled so that both the
// transposing 16-byte stores and the 16-byte operand loads spread over the banks.
__device__ __forceinline__ int vt_index(int d, int G) {
  return ((d ^ ((d >> 3) & 1)) << 2) | (G ^ ((d >> 1) & 3));
}

__device__ __forceinline__ uint32_t word_of(const uint4 &a, int k) {
  return k == 0 ? a.x : (k == 1 ? a.y : (k == 2 ? a.z : a.w));
}

// Half i of a in the low half, half i of b in the high half.
__device__ __forceinline__ uint32_t pair_halves(const uint4 &a, const uint4 &b, int i) {
  const uint32_t wa = word_of(a, i >> 1), wb = word_of(b, i >> 1);
  return (i & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// Key slot k (0..31) of an MFMA operand group: slots 8G..8G+3 hold block rows
// 4G..4G+3 and slots 8G+4..8G+7 hold rows 16+4G..16+4G+3, which is exactly the
// set of rows one lane holds in the 16x16 score accumulators of both row tiles.
__device__ __forceinline__ int slot_row(int G, int i) { return i < 4 ? 4 * G + i : 16 + 4 * G + (i - 4); }

// Transpose 8 rows x 8 halves (rows ordered as slot_row(G, 0..7)) into 8 chunks,
// chunk i = the 8 rows' halves at column i, masked rows zeroed.
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint32_t keep_mask, uint4 (&out)[8]) {
  uint4 vv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vv[i] = ((keep_mask >> i) & 1u) ? in[i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i].x = pair_halves(vv[0], vv[1], i);
    out[i].y = pair_halves(vv[2], vv[3], i);
    out[i].z = pair_halves(vv[4], vv[5], i);
    out[i].w = pair_halves(vv[6], vv[7], i);
  }
}

// Bits 0..7 of the result: which of the rows slot_row(G, 0..7) are set in `vis`.
__device__ __forceinline__ uint32_t slot_mask(uint32_t vis, int G) {
  return ((vis >> (4 * G)) & 0xfu) | (((vis >> (16 + 4 * G)) & 0xfu) << 4);
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
// `cnt` is LDS scratch of NT/64 ints.
template <int NT>
__device__ __forceinline__ int build_block_list(const uint8_t *row, int nbd, uint16_t *list, int *cnt) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int total = 0;
  for (int base = 0; base < nbd; base += NT) {
    const int j = base + tid;
    int s = 0;
    if (j < nbd) s = row ? (int)row[j] : kPartial;
    const unsigned long long m = __ballot(s != 0);
    if (lane == 0) cnt[wv] = __popcll(m);
    __syncthreads();
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
    __syncthreads();
  }
  __syncthreads();  // also orders any LDS staging done before the call when the map is empty
  return total;
}

}  // namespace ds4attn
