// Padding and block-map kernels.
//
// pad: a KV region becomes whole 32-row blocks -- live rows copied bit for bit,
// the tail rows zero, and a validity byte per row ([P-Metal] "KV-Cache
// Management on Metal Device Buffers"; "FlashAttention Kernel Architecture",
// the pad kernel).
//
// blockmap: one status byte per (query tile, 32-row key block) -- skip, partial or
// full -- so the attention kernel can pass over fully masked blocks ([P-Metal]
// "Mask Handling and Block Skipping").
#include "ds4attn_internal.h"

namespace ds4attn {

// One thread per 16-byte chunk of one row in [row_lo, npad) of each sequence.
__global__ __launch_bounds__(256) void pad_rows_kernel(
    const char *__restrict__ k, const char *__restrict__ v, int64_t in_sb, int64_t in_sr,
    char *__restrict__ kp, char *__restrict__ vp, int64_t out_sb, int64_t out_sr, int n,
    int row_lo, int nrows_out, int chunks_per_row, int64_t total, bool copy_k, bool copy_v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t per_seq = (int64_t)nrows_out * chunks_per_row;
  const int b = (int)(i / per_seq);
  const int64_t rem = i - (int64_t)b * per_seq;
  const int row = row_lo + (int)(rem / chunks_per_row);
  const int c = (int)(rem % chunks_per_row);
  const int64_t src = (int64_t)b * in_sb + (int64_t)row * in_sr + 16 * c;
  const int64_t dst = (int64_t)b * out_sb + (int64_t)row * out_sr + 16 * c;
  if (row < n) {
    if (copy_k) *(uint4 *)(kp + dst) = *(const uint4 *)(k + src);
    if (copy_v) *(uint4 *)(vp + dst) = *(const uint4 *)(v + src);
  } else {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    *(uint4 *)(kp + dst) = z;
    *(uint4 *)(vp + dst) = z;
  }
}

// Validity rows [row_lo, npad) of every sequence (row_lo = n when the output is the
// input buffer: only the tail is written).
__global__ __launch_bounds__(256) void pad_valid_kernel(const uint8_t *__restrict__ valid,
                                                        int64_t valid_sb, uint8_t *__restrict__ validp,
                                                        int64_t validp_sb, int n, int row_lo, int npad,
                                                        int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int per_seq = npad - row_lo;
  const int b = (int)(i / per_seq);
  const int row = row_lo + (int)(i - (int64_t)b * per_seq);
  uint8_t x = 0;
  if (row < n) x = valid ? valid[(int64_t)b * valid_sb + row] : (uint8_t)1;
  validp[(int64_t)b * validp_sb + row] = x;
}

hipError_t launch_pad(const void *k, const void *v, const uint8_t *valid, int64_t in_sb,
                      int64_t in_sr, int64_t valid_sb, void *kp, void *vp, uint8_t *validp,
                      int64_t out_sb, int64_t out_sr, int64_t validp_sb, int B, int n, int npad,
                      int row_bytes, bool copy_k, bool copy_v, bool copy_valid, hipStream_t s) {
  const int row_lo = (copy_k || copy_v) ? 0 : n;
  const int nrows_out = npad - row_lo;
  const int cpr = row_bytes / 16;
  const int64_t total = (int64_t)B * nrows_out * cpr;
  if (total > 0) {
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const char *)k, (const char *)v, in_sb, in_sr, (char *)kp, (char *)vp,
                       out_sb, out_sr, n, row_lo, nrows_out, cpr, total, copy_k, copy_v);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (validp) {
    const int vrow_lo = copy_valid ? 0 : n;
    const int64_t tv = (int64_t)B * (npad - vrow_lo);
    if (tv > 0) {
      hipLaunchKernelGGL(pad_valid_kernel, dim3((unsigned)((tv + 255) / 256)), dim3(256), 0, s,
                         valid, valid_sb, validp, validp_sb, n, vrow_lo, npad, tv);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

// What the map reads, packed so that one burst of scalar loads brings it in (the
// full attention parameter block made the kernel wait on a chain of dependent
// argument loads).
struct BlkParams {
  const uint8_t *valid0, *valid1;
  uint8_t *blk;
  int64_t valid0_sb, valid1_sb;
  int64_t qk_delta;          // q_pos0 - k_pos0
  uint32_t total, nbd, ntiles;
  int T, bq, nb0, n0, n1, window;
};

// One wave per (sequence, query tile, key block).  Lane r (mod 32) owns row r of
// the block; lanes 0-31 take the tile's even tokens, lanes 32-63 the odd ones.
// The block is SKIP when no lane saw a visible pair, FULL when every lane saw
// only visible pairs (all 32 rows for every token), PARTIAL otherwise.  Index
// arithmetic is 32-bit: the map has fewer than 2^31 entries.
__global__ __launch_bounds__(256) void blockmap_kernel(const BlkParams p) {
  asm volatile("" ::"s"(p.valid0), "s"(p.bq));   // both lines of the block in one burst
  const int lane = threadIdx.x & 63;
  const uint32_t wid = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (wid >= p.total) return;  // whole wave exits together
  const int j = (int)(wid % p.nbd);
  const uint32_t bt = wid / p.nbd;
  const int tile = (int)(bt % p.ntiles);
  const int b = (int)(bt / p.ntiles);
  const int r = lane & 31;
  const int t0 = tile * p.bq;
  const int t1 = min(p.T, t0 + p.bq);
  bool any = false, all = true;
  if (j < p.nb0) {
    const int row = j * kRowsPerBlock + r;
    bool live = row < p.n0;
    if (live && p.valid0) live = p.valid0[b * p.valid0_sb + row] != 0;
    for (int t = t0 + (lane >> 5); t < t1; t += 2) {
      bool vis = live;
      if (p.window > 0) {
        const int64_t d = p.qk_delta + t - row;
        vis = vis && d >= 0 && d < p.window;
      }
      any |= vis;
      all &= vis;
    }
  } else {
    // dense region 1: visibility does not depend on the token
    const int c = (j - p.nb0) * kRowsPerBlock + r;
    bool vis = c < p.n1;
    if (vis && p.valid1) vis = p.valid1[b * p.valid1_sb + c] != 0;
    if (t0 + (lane >> 5) < t1) {
      any = vis;
      all = vis;
    }
  }
  const unsigned long long many = __ballot(any);
  const unsigned long long mall = __ballot(all);
  if (lane == 0) p.blk[wid] = (uint8_t)(many == 0ull ? kSkip : (mall == ~0ull ? kFull : kPartial));
}

hipError_t launch_blockmap(const AttnParams &p, uint8_t *blk, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.ntiles * p.nbd;
  if (total == 0) return hipSuccess;
  BlkParams q;
  q.valid0 = p.valid0;
  q.valid1 = p.valid1;
  q.blk = blk;
  q.valid0_sb = p.valid0_sb;
  q.valid1_sb = p.valid1_sb;
  q.qk_delta = p.qk_delta;
  q.total = (uint32_t)total;
  q.nbd = (uint32_t)p.nbd;
  q.ntiles = (uint32_t)p.ntiles;
  q.T = p.T;
  q.bq = p.bq;
  q.nb0 = p.nb0;
  q.n0 = p.n0;
  q.n1 = p.n1;
  q.window = p.window;
  hipLaunchKernelGGL(blockmap_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, q);
  return hipGetLastError();
}

}  // namespace ds4attn
