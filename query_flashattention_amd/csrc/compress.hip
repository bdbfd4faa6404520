// Compressor step of a compressed layer: raw K/V rows and their scores join the
// rolling state of the incomplete group; every complete group of `ratio` rows
// becomes one compressed row, and the trailing rows become the new state
// ([P-DS4] "Architecture Deep Dive", Layer Compression and KV Cache Design: the
// compressor keeps rolling KV/score state and appends pooled rows at ratio
// boundaries).  The pooling is a softmax over the group's rows, per element, of
// the given scores, weighting the rows' values.
//
// Memory-bound: per raw row, head_dim float16 values and head_dim float32 scores
// are read (the scores twice, the second time from L2), and per group one float16
// row is written.  A thread owns two adjacent elements of one compressed row
// (4-byte and 8-byte loads, coalesced across the row).  Short groups: one thread
// walks the whole group, and threads of a workgroup cover consecutive element
// pairs, rows and sequences.  Long groups: the group's rows are split over eight
// thread slices of a workgroup, combined through LDS.
#include "ds4attn_internal.h"

namespace ds4attn {

namespace {

struct CompressArgs {
  const char *state_kv;    // float16 rows, read (rows [0, n_state))
  const char *state_score; // float32 rows, read
  const char *kv_new;
  const char *score_new;
  char *comp;              // float16 output rows
  int64_t state_kv_sb, state_score_sb, kv_new_sb, score_new_sb, comp_sb;
  int32_t D, ratio, n_state, n_out, batch;
};

// Row r of the stream (state rows, then new rows) of sequence b: its value and
// score pairs at element pair e.
__device__ __forceinline__ void stream_row(const CompressArgs &a, int b, int r, int e, const __half2 **kv,
                                           const float2 **sc) {
  if (r < a.n_state) {
    *kv = (const __half2 *)(a.state_kv + b * a.state_kv_sb + (int64_t)r * 2 * a.D) + e;
    *sc = (const float2 *)(a.state_score + b * a.state_score_sb + (int64_t)r * 4 * a.D) + e;
  } else {
    const int q = r - a.n_state;
    *kv = (const __half2 *)(a.kv_new + b * a.kv_new_sb + (int64_t)q * 2 * a.D) + e;
    *sc = (const float2 *)(a.score_new + b * a.score_new_sb + (int64_t)q * 4 * a.D) + e;
  }
}

__global__ __launch_bounds__(256) void compress_pool_kernel(const CompressArgs a, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int pairs = a.D >> 1;
  const int e = (int)(i % pairs);
  const int64_t bc = i / pairs;
  const int c = (int)(bc % a.n_out);
  const int b = (int)(bc / a.n_out);
  const int r0 = c * a.ratio;
  // pass 1: the group's largest score, per element
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll 8
  for (int k = 0; k < a.ratio; ++k) {
    const __half2 *kv;
    const float2 *sc;
    stream_row(a, b, r0 + k, e, &kv, &sc);
    const float2 s = *sc;
    m0 = fmaxf(m0, s.x);
    m1 = fmaxf(m1, s.y);
  }
  // pass 2: weights exp(s - max) (base 2 on the scaled difference), their sum and
  // the weighted sum of the values
  constexpr float kLog2e = 1.4426950408889634f;
  float l0 = 0.f, l1 = 0.f, acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
  for (int k = 0; k < a.ratio; ++k) {
    const __half2 *kv;
    const float2 *sc;
    stream_row(a, b, r0 + k, e, &kv, &sc);
    const float2 s = *sc;
    const float2 v = __half22float2(*kv);
    const float w0 = __builtin_amdgcn_exp2f((s.x - m0) * kLog2e);
    const float w1 = __builtin_amdgcn_exp2f((s.y - m1) * kLog2e);
    l0 += w0;
    l1 += w1;
    acc0 = fmaf(w0, v.x, acc0);
    acc1 = fmaf(w1, v.y, acc1);
  }
  __half2 out;
  out.x = __float2half_rn(acc0 / l0);
  out.y = __float2half_rn(acc1 / l1);
  *((__half2 *)(a.comp + b * a.comp_sb + (int64_t)c * 2 * a.D) + e) = out;
}

// Long groups (ratio >= kSplitRatio): the group's rows are split over RS thread
// slices.  A workgroup owns one group and P = 256 / RS element pairs; slice rs takes
// rows rs, rs + RS, ...  The slices' maxima, then their sums and weighted sums,
// meet in LDS and are combined in slice order (the same order on every call).
constexpr int kSplitRatio = 32;
template <int RS>
__global__ __launch_bounds__(256) void compress_pool_rows_kernel(const CompressArgs a) {
  constexpr int P = 256 / RS;
  __shared__ float2 smax[RS][P];
  __shared__ float4 ssum[RS][P];
  const int el = threadIdx.x % P, rs = threadIdx.x / P;
  const int nchunk = (a.D >> 1) / P;
  const int chunk = (int)(blockIdx.x % (unsigned)nchunk);
  const int bc = (int)(blockIdx.x / (unsigned)nchunk);
  const int c = bc % a.n_out, b = bc / a.n_out;
  const int e = chunk * P + el;
  const int r0 = c * a.ratio;
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll 4
  for (int k = rs; k < a.ratio; k += RS) {
    const __half2 *kv;
    const float2 *sc;
    stream_row(a, b, r0 + k, e, &kv, &sc);
    const float2 s = *sc;
    m0 = fmaxf(m0, s.x);
    m1 = fmaxf(m1, s.y);
  }
  smax[rs][el] = make_float2(m0, m1);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RS; ++q) {
    const float2 x = smax[q][el];
    m0 = fmaxf(m0, x.x);
    m1 = fmaxf(m1, x.y);
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float l0 = 0.f, l1 = 0.f, acc0 = 0.f, acc1 = 0.f;
#pragma unroll 4
  for (int k = rs; k < a.ratio; k += RS) {
    const __half2 *kv;
    const float2 *sc;
    stream_row(a, b, r0 + k, e, &kv, &sc);
    const float2 s = *sc;
    const float2 v = __half22float2(*kv);
    const float w0 = __builtin_amdgcn_exp2f((s.x - m0) * kLog2e);
    const float w1 = __builtin_amdgcn_exp2f((s.y - m1) * kLog2e);
    l0 += w0;
    l1 += w1;
    acc0 = fmaf(w0, v.x, acc0);
    acc1 = fmaf(w1, v.y, acc1);
  }
  ssum[rs][el] = make_float4(l0, l1, acc0, acc1);
  __syncthreads();
  if (rs == 0) {
    float4 t = ssum[0][el];
#pragma unroll
    for (int q = 1; q < RS; ++q) {
      const float4 x = ssum[q][el];
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
    }
    __half2 out;
    out.x = __float2half_rn(t.z / t.x);
    out.y = __float2half_rn(t.w / t.y);
    *((__half2 *)(a.comp + b * a.comp_sb + (int64_t)c * 2 * a.D) + e) = out;
  }
}

// The new state: rows [n_out * ratio, n_state + n_new) of the stream.  With a
// complete group (n_out > 0) they are all new rows; otherwise the pending rows
// stay where they are and the new rows follow them.  16 bytes per thread.
__global__ __launch_bounds__(256) void compress_state_kernel(char *state_kv, char *state_score,
                                                             const char *kv_new, const char *score_new,
                                                             int64_t state_kv_sb, int64_t state_score_sb,
                                                             int64_t kv_new_sb, int64_t score_new_sb, int D,
                                                             int first_new, int dst0, int rows, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  // per row: D/8 chunks of values (8 float16) and D/4 chunks of scores (4 float32)
  const int vchunks = D >> 3, schunks = D >> 2, per_row = vchunks + schunks;
  const int64_t per_seq = (int64_t)rows * per_row;
  const int b = (int)(i / per_seq);
  const int64_t rem = i - (int64_t)b * per_seq;
  const int k = (int)(rem / per_row);
  const int ch = (int)(rem % per_row);
  const int src = first_new + k, dst = dst0 + k;
  if (ch < vchunks) {
    const uint4 x = *((const uint4 *)(kv_new + b * kv_new_sb + (int64_t)src * 2 * D) + ch);
    *((uint4 *)(state_kv + b * state_kv_sb + (int64_t)dst * 2 * D) + ch) = x;
  } else {
    const int cs = ch - vchunks;
    const uint4 x = *((const uint4 *)(score_new + b * score_new_sb + (int64_t)src * 4 * D) + cs);
    *((uint4 *)(state_score + b * state_score_sb + (int64_t)dst * 4 * D) + cs) = x;
  }
}

}  // namespace

hipError_t launch_compress(void *state_kv, float *state_score, int64_t state_kv_sb, int64_t state_score_sb,
                           int n_state, const void *kv_new, const float *score_new, int64_t kv_new_sb,
                           int64_t score_new_sb, int n_new, int B, int D, int ratio, void *comp,
                           int64_t comp_sb, hipStream_t s) {
  const int n_out = (n_state + n_new) / ratio;
  if (n_out > 0) {
    CompressArgs a;
    a.state_kv = (const char *)state_kv;
    a.state_score = (const char *)state_score;
    a.kv_new = (const char *)kv_new;
    a.score_new = (const char *)score_new;
    a.comp = (char *)comp;
    a.state_kv_sb = state_kv_sb;
    a.state_score_sb = state_score_sb;
    a.kv_new_sb = kv_new_sb;
    a.score_new_sb = score_new_sb;
    a.comp_sb = comp_sb;
    a.D = D;
    a.ratio = ratio;
    a.n_state = n_state;
    a.n_out = n_out;
    a.batch = B;
    if (ratio >= kSplitRatio) {
      constexpr int RS = 8;
      const int64_t blocks = (int64_t)B * n_out * ((D / 2) / (256 / RS));
      hipLaunchKernelGGL(compress_pool_rows_kernel<RS>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    } else {
      const int64_t total = (int64_t)B * n_out * (D / 2);
      hipLaunchKernelGGL(compress_pool_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                         total);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // state rows to write: the new rows that are not pooled
  const int consumed = n_out * ratio;                 // stream rows pooled
  const int n_next = n_state + n_new - consumed;      // rows of the new state
  const int first_new = consumed > n_state ? consumed - n_state : 0;   // first new row kept
  const int dst0 = consumed > n_state ? 0 : n_state;  // where it goes
  const int rows = n_new - first_new;
  if (rows > 0 && n_next > 0) {
    const int64_t total = (int64_t)B * rows * (D / 8 + D / 4);
    hipLaunchKernelGGL(compress_state_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       (char *)state_kv, (char *)state_score, (const char *)kv_new, (const char *)score_new,
                       state_kv_sb, state_score_sb, kv_new_sb, score_new_sb, D, first_new, dst0, rows,
                       total);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ds4attn
