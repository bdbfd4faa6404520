// Top-k index selection from given scores: the step that turns an indexer's
// scores into the index list of a ratio-4 layer ([P-DS4] "Architecture Deep
// Dive", Layer Compression: each token attends the top-512 compressed rows).
//
// One workgroup of 256 threads per row of scores.  Scores become unsigned keys
// whose integer order is the total order of the float32 bit patterns.  A
// most-significant-digit-first radix select (four 8-bit digits; LDS histograms,
// one copy per wave so that the four waves do not contend) finds the key T of the
// k-th largest entry and how many entries equal to T are taken; a final pass over
// the row in index order writes the selected indices (key > T, or key == T among
// the first such) at block-wide prefix counts, so the list comes out ascending
// with ties resolved toward the lower index.  Rows of up to kTopkLdsKeys scores
// keep their keys in LDS; longer rows re-read the scores each pass.
//
// [P-DS4] = "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine".
#include "ds4attn_internal.h"

namespace ds4attn {

constexpr int kTopkLdsKeys = 16384;   // 64 KB of keys
constexpr int kHistStride = 257;      // per-wave histogram copies start on different banks

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

template <bool IN_LDS>
__global__ __launch_bounds__(256) void topk_kernel(const char *__restrict__ scores, int64_t s_stride,
                                                   int n, int k, char *__restrict__ out,
                                                   int64_t o_stride) {
  __shared__ uint32_t keys[IN_LDS ? kTopkLdsKeys : 1];
  __shared__ uint32_t hist[4 * kHistStride];
  __shared__ uint32_t pick[2];
  __shared__ uint32_t wcnt[2][4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row = blockIdx.x;
  const float *s = (const float *)(scores + row * s_stride);
  int32_t *o = (int32_t *)(out + row * o_stride);
  auto key_at = [&](int i) -> uint32_t { return IN_LDS ? keys[i] : order_key(s[i]); };
  if (IN_LDS) {
    for (int i = tid; i < n; i += 256) keys[i] = order_key(s[i]);
  }
  const int m = n < k ? n : k;   // entries selected

  // ---- radix select: after the four digits, T = prefix and `krem` entries equal
  // to T are taken (all entries with a larger key are taken too)
  uint32_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)m;
  for (int shift = 24; shift >= 0 && m > 0; shift -= 8) {
    for (int i = tid; i < 4 * kHistStride; i += 256) hist[i] = 0;
    __syncthreads();   // (first pass: also orders the key stores)
    for (int i = tid; i < n; i += 256) {
      const uint32_t kk = key_at(i);
      if ((kk & mask) == prefix) atomicAdd(&hist[w * kHistStride + ((kk >> shift) & 255u)], 1u);
    }
    __syncthreads();
    if (w == 0) {
      // lane l covers digits 255-4l .. 252-4l, highest first; an inclusive scan
      // over the lanes counts the entries at or above each lane's range
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 255 - 4 * lane - q;
        c[q] = hist[d] + hist[kHistStride + d] + hist[2 * kHistStride + d] + hist[3 * kHistStride + d];
        tot += c[q];
      }
      uint32_t inc = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(inc, off);
        if (lane >= off) inc += v;
      }
      const uint32_t exc = inc - tot;
      if (exc < krem && krem <= inc) {   // exactly one lane: the krem-th entry's digit is here
        uint32_t above = exc;
        int dsel = 255 - 4 * lane - 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + c[q] >= krem) {
            dsel = 255 - 4 * lane - q;
            break;
          }
          above += c[q];
        }
        pick[0] = (uint32_t)dsel;
        pick[1] = above;
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= 255u << shift;
    krem -= pick[1];
    __syncthreads();   // pick and hist are rewritten next pass
  }
  const uint32_t T = prefix;

  // ---- write the selection in index order
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  uint32_t eq_run = 0, sel_run = 0;   // totals over the chunks before
  for (int base = 0; base < n && m > 0; base += 256) {
    const int i = base + tid;
    const uint32_t kk = i < n ? key_at(i) : 0u;
    const bool eq = i < n && kk == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wcnt[0][w] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_rank = eq_run + (uint32_t)__popcll(beq & lt);
    for (int ww = 0; ww < w; ++ww) eq_rank += wcnt[0][ww];
    const bool sel = i < n && (kk > T || (eq && eq_rank < krem));
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wcnt[1][w] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t pos = sel_run + (uint32_t)__popcll(bsel & lt);
    for (int ww = 0; ww < w; ++ww) pos += wcnt[1][ww];
    if (sel && pos < (uint32_t)m) o[pos] = i;   // exactly m are selected; the guard only bounds the store
    for (int ww = 0; ww < 4; ++ww) {
      eq_run += wcnt[0][ww];
      sel_run += wcnt[1][ww];
    }
    __syncthreads();   // wcnt is rewritten next chunk
  }
  for (int j = m + tid; j < k; j += 256) o[j] = -1;
}

hipError_t launch_topk(const float *scores, int64_t rows, int n, int64_t s_stride, int k, int32_t *idx,
                       int64_t o_stride, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // one workgroup per row: the grid's total lane count must stay below 2^32
  if (rows > kMaxTopkRows) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows), block(256);
  if (n <= kTopkLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, grid, block, 0, s, (const char *)scores, s_stride, n, k,
                       (char *)idx, o_stride);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, block, 0, s, (const char *)scores, s_stride, n, k,
                       (char *)idx, o_stride);
  return hipGetLastError();
}

}  // namespace ds4attn
