// Top-k index selection from given scores: the step that turns an indexer's
// scores into the index list of a ratio-4 layer ([P-DS4] "Architecture Deep
// Dive", Layer Compression: each token attends the top-512 compressed rows).
//
// One workgroup of 512 threads (8 waves) per row of scores.  Scores become
// unsigned keys whose integer order is the total order of the float32 bit
// patterns.  The row is cut into tiles of CH chunks of 2048 scores; in a chunk,
// thread t holds the four consecutive scores 4t .. 4t+3, so a chunk is one
// coalesced 16-byte load per thread and index order is (chunk, thread, element).
// Rows of up to one tile keep their keys in registers for the whole kernel;
// longer rows re-read their tiles in every pass.  Loads go through a buffer
// resource bounded by the row, so lanes past its end read zeros instead of
// faulting (their keys are never counted).
//
// A most-significant-digit-first radix select over three digits of 11, 11 and
// 10 bits finds the key T of the k-th largest entry and how many of the entries
// equal to T are taken.  Each digit is one pass of LDS atomics into a 2048-bin
// histogram (wide digits spread the bell of real-valued scores over many bins, so
// lanes rarely collide on one counter); each wave then scans one 256-bin segment,
// and after a second barrier every wave finds the segment, lane and digit that
// hold the k-th entry from the segment totals, so the choice needs no broadcast.
// Two histogram sets alternate: the one cleared during a pass was last read
// before that pass's first barrier and is next written after its second.
//
// The write pass counts, per thread and chunk, the entries above T and equal to
// T, prefix-sums both over the workgroup in one packed scan, and places each
// selected index at its rank in an LDS buffer: entries above T all go, entries
// equal to T go while fewer than the remaining count precede them in index
// order.  The list therefore comes out ascending, ties resolved toward the lower
// index, and leaves in one coalesced store with the -1 padding.
//
// [P-DS4] = "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine".
#include "ds4attn_internal.h"
#include "mfma_common.h"

namespace ds4attn {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 4 * kThreads;      // scores per chunk
constexpr int kMaxCh = 8;                 // chunks per tile: rows of up to 16384 stay in registers
constexpr int kBins = 2048;               // histogram bins (the widest digit has 11 bits)

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// Wave-wide inclusive prefix sum over the lanes: DPP row shifts scan each row of
// 16 lanes, then every row adds the totals of the rows below it.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, int lane) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

template <int CH, bool VEC, bool MULTI>
__global__ __launch_bounds__(kThreads) void topk_kernel(const char *__restrict__ scores, int64_t s_stride, int n,
                                                        int k, char *__restrict__ out, int64_t o_stride) {
  constexpr int kTile = CH * kChunk;
  __shared__ __align__(16) uint32_t hist[2][kBins];
  __shared__ __align__(16) uint32_t lane_inc[kWaves][64];   // per segment: inclusive counts over its lanes
  __shared__ __align__(16) uint32_t seg_tot[kWaves];
  __shared__ uint32_t wtot[2][CH][kWaves];
  __shared__ int32_t obuf[kMaxTopkK];                      // the selection, staged for one coalesced store
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row = blockIdx.x;
  const char *srow = scores + row * s_stride;
  int32_t *o = (int32_t *)(out + row * o_stride);
  const int m = n < k ? n : k;   // entries selected

  if (n <= k) {   // everything is selected
    for (int j = tid; j < k; j += kThreads) o[j] = j < n ? j : -1;
    return;
  }

  const rsrc_t rs = make_rsrc(srow, (uint32_t)n * 4u);
  uint32_t key[CH][4];
  auto load_tile = [&](int t0) {
    float4 x[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t off = 4u * (uint32_t)(t0 + c * kChunk + 4 * tid);
      if (VEC && t0 + (c + 1) * kChunk <= n) {   // the whole chunk is inside the row (uniform)
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        x[c] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
      } else {
        x[c].x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        x[c].y = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 4, 0, 0));
        x[c].z = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 8, 0, 0));
        x[c].w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off + 12, 0, 0));
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      key[c][0] = order_key(x[c].x);
      key[c][1] = order_key(x[c].y);
      key[c][2] = order_key(x[c].z);
      key[c][3] = order_key(x[c].w);
    }
  };
  const int ntiles = MULTI ? (n + kTile - 1) / kTile : 1;
  if (!MULTI) load_tile(0);
  ((uint4 *)hist[0])[tid] = make_uint4(0, 0, 0, 0);   // 512 threads x 4 bins

  // ---- radix select: after the three digits, T = prefix, and `krem` of the
  // entries equal to T are taken together with every entry above T
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)m;
  __syncthreads();   // set 0 is clear
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    uint32_t *h = hist[pass & 1];
#pragma unroll 1
    for (int t = 0; t < ntiles; ++t) {
      const int t0 = t * kTile;
      if (MULTI) load_tile(t0);
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kk = key[c][e];
          if (t0 + c * kChunk + 4 * tid + e < n && (kk & mask) == prefix)
            atomicAdd(&h[(kk >> shift) & dmask], 1u);
        }
    }
    __syncthreads();
    // wave w scans segment w, highest digit first: digits 2047-256w .. 1792-256w,
    // lane l the four digits 255-4l .. 252-4l of it
    const uint4 v = *(const uint4 *)&h[kBins - 256 * (w + 1) + 252 - 4 * lane];
    const uint32_t inc = wave_inclusive_sum(v.x + v.y + v.z + v.w, lane);
    lane_inc[w][lane] = inc;
    if (lane == 63) seg_tot[w] = inc;
    // the other set was last read before the barrier above and is next written
    // after the one below
    ((uint4 *)hist[(pass + 1) & 1])[tid] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    // every wave finds the segment, then the lane, then the digit holding the
    // krem-th entry in the same way
    const uint4 s0 = *(const uint4 *)&seg_tot[0], s1 = *(const uint4 *)&seg_tot[4];
    const uint32_t st[kWaves] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t cum = 0, cum_sel = 0;
    int jsel = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      if (!found && cum + st[j] >= krem) {
        found = true;
        jsel = j;
        cum_sel = cum;
      }
      cum += st[j];
    }
    const uint4 hv = *(const uint4 *)&h[kBins - 256 * (jsel + 1) + 252 - 4 * lane];
    const uint32_t hi = cum_sel + lane_inc[jsel][lane], lo = hi - (hv.x + hv.y + hv.z + hv.w);
    const uint64_t bal = __ballot(lo < krem && krem <= hi);
    const int sl = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(bal));
    uint32_t above = lo, dsel = 0;
    const uint32_t cq[4] = {hv.w, hv.z, hv.y, hv.x};   // digits 255-4l .. 252-4l of the segment
    bool got = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!got && above + cq[q] >= krem) {
        got = true;
        dsel = (uint32_t)(kBins - 256 * jsel - 1 - 4 * lane - q);
      } else if (!got) {
        above += cq[q];
      }
    }
    dsel = (uint32_t)__builtin_amdgcn_readlane((int)dsel, sl);
    above = (uint32_t)__builtin_amdgcn_readlane((int)above, sl);
    prefix |= dsel << shift;
    mask |= dmask << shift;
    krem -= above;
  }
  const uint32_t T = prefix;

  // ---- rank the selection in index order, staged in LDS
  uint32_t run_gt = 0, run_eq = 0;   // totals over the tiles before
#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * kTile, wb = t & 1;
    if (MULTI) load_tile(t0);
    // per chunk: entries above T in the low half, entries equal to T in the high
    // half (a tile holds at most 16384 entries, so the halves cannot carry)
    uint32_t own[CH], inc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t v = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = t0 + c * kChunk + 4 * tid + e < n;
        v += (ok && key[c][e] > T) ? 1u : 0u;
        v += (ok && key[c][e] == T) ? 0x10000u : 0u;
      }
      own[c] = v;
      inc[c] = wave_inclusive_sum(v, lane);
      if (lane == 63) wtot[wb][c][w] = inc[c];
    }
    __syncthreads();   // (wtot[wb] was last read two tiles ago, before the previous barrier)
    uint32_t run = 0;  // packed totals of the chunks before c in this tile
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const uint32_t v = wtot[wb][c][ww];
        before += ww < w ? v : 0u;
        total += v;
      }
      const uint32_t ex = run + before + inc[c] - own[c];
      run += total;
      uint32_t g = run_gt + (ex & 0xffffu), q = run_eq + (ex >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = t0 + c * kChunk + 4 * tid + e < n;
        const bool gt = ok && key[c][e] > T, eq = ok && key[c][e] == T;
        // an entry above T has g + min(q, krem) selected entries before it; one
        // equal to T is taken while q < krem, after g + q of them
        const uint32_t pos = g + (q < krem ? q : krem);
        if ((gt || (eq && q < krem)) && pos < (uint32_t)m)   // exactly m are taken; the test bounds the store
          obuf[pos] = t0 + c * kChunk + 4 * tid + e;
        g += gt ? 1u : 0u;
        q += eq ? 1u : 0u;
      }
    }
    run_gt += run & 0xffffu;
    run_eq += run >> 16;
  }
  __syncthreads();
  for (int j = tid; j < k; j += kThreads) o[j] = j < m ? obuf[j] : -1;
}

template <int CH, bool MULTI>
void launch_one(bool vec, dim3 grid, hipStream_t s, const float *scores, int64_t s_stride, int n, int k,
                int32_t *idx, int64_t o_stride) {
  if (vec)
    hipLaunchKernelGGL((topk_kernel<CH, true, MULTI>), grid, dim3(kThreads), 0, s, (const char *)scores,
                       s_stride, n, k, (char *)idx, o_stride);
  else
    hipLaunchKernelGGL((topk_kernel<CH, false, MULTI>), grid, dim3(kThreads), 0, s, (const char *)scores,
                       s_stride, n, k, (char *)idx, o_stride);
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t rows, int n, int64_t s_stride, int k, int32_t *idx,
                       int64_t o_stride, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // one workgroup per row: the grid's total lane count must stay below 2^32
  if (rows > kMaxTopkRows) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows);
  // 16-byte loads need every row start 16-byte aligned
  const bool vec = ((uintptr_t)scores & 15u) == 0 && (s_stride & 15) == 0;
  if (n <= 1 * kChunk)
    launch_one<1, false>(vec, grid, s, scores, s_stride, n, k, idx, o_stride);
  else if (n <= 2 * kChunk)
    launch_one<2, false>(vec, grid, s, scores, s_stride, n, k, idx, o_stride);
  else if (n <= 4 * kChunk)
    launch_one<4, false>(vec, grid, s, scores, s_stride, n, k, idx, o_stride);
  else if (n <= kMaxCh * kChunk)
    launch_one<kMaxCh, false>(vec, grid, s, scores, s_stride, n, k, idx, o_stride);
  else
    launch_one<kMaxCh, true>(vec, grid, s, scores, s_stride, n, k, idx, o_stride);
  return hipGetLastError();
}

}  // namespace ds4attn
