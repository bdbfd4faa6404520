// Internal declarations shared by the ds4attn HIP sources (not part of the ABI).
//
// [P-Metal] = page "How DeepSeek V4 Flash Model Inference Works on Apple Silicon
//             with Metal Backend";
// [P-DS4]   = page "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine".
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4attn {

constexpr int kRowsPerBlock = 32;   // [P-Metal] KV-Cache Management: 32-row padding
constexpr int kNumXcd = 8;          // MI355X: 8 accelerator dies, workgroups dealt round-robin
constexpr int kNumCus = 256;        // compute units (32 per die)
constexpr int kIdxCap = 2048;       // largest index list held in LDS by the matrix-core kernel

enum : int { kSkip = 0, kPartial = 1, kFull = 2 };

// Everything a kernel needs, resolved on the host from ds4attn_args.
// Division by a run-time divisor d >= 1 of indices n < 2^31, exact: with
// l = ceil(log2 d) and m = ceil(2^(31+l) / d) < 2^32, n / d = (n * m) >> (31 + l)
// (the rounding error of m adds less than n / 2^(31+l) < 1/d to n/d, which never
// crosses the next integer).  Built on the host by make_fast_div.
struct FastDiv {
  uint32_t m;
  uint32_t shift;   // 31 + l
};
inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t pow = 1ull << (31 + l);
  return FastDiv{(uint32_t)((pow + d - 1) / d), 31 + l};
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.shift);
}

struct AttnParams {
  const char *q;
  char *o;
  int64_t q_sb, q_st, q_sh;
  int64_t o_sb, o_st, o_sh;
  int B, T, H, D;
  float scale_log2;        // scale * log2(e): softmax runs in base 2
  int window;              // 0 = no positional mask on region 0
  int64_t qk_delta;        // q_pos0 - k_pos0
  // region 0 (raw rows)
  const char *k0, *v0;
  int64_t kv0_sb, kv0_sr;
  const uint8_t *valid0;
  int64_t valid0_sb;
  int n0, nb0;             // live rows, 32-row blocks
  // region 1 (compressed rows)
  const char *k1, *v1;
  int64_t kv1_sb, kv1_sr;
  const uint8_t *valid1;
  int64_t valid1_sb;
  int n1, nb1;             // live rows; blocks in the key space (dense: ceil32(n1)/32,
                           // indexed: ceil(r1_k/32), 0 when n1 == 0)
  const int32_t *idx;      // [B][T][r1_k] or null
  int r1_k;
  int indexed;
  // FP8 rows: E4M3 codes, one float32 scale per K row and per V row
  int fp8;
  const char *ks0, *vs0, *ks1, *vs1;   // scales of row r of sequence b at b * s*_sb + 4r
  int64_t s0_sb, s1_sb;
  // split decode: each token's block list divided over nsplit workgroups per head
  // group, partial results in ws (one kSplitRecord per (b, t, head group, split))
  int nsplit;              // 1 = no split
  int decode_split;        // decode work split: 0 = chosen by the library, 1 = DIMS, 2 = KEYS,
                           // 3 = DIMS over 32 heads per workgroup
  char *ws;
  // block map
  const uint8_t *blk;      // [B][ntiles][nbd] or null (every block treated as PARTIAL)
  int bq;
  int64_t ntiles;
  int nbd;                 // blocks covered by the map: nb0 (+ nb1 when not indexed)
  // the matrix-core kernels' index divisions by run-time values, as multiply and
  // shift (see fast_div): by H/16, H/32, H/64, T and bq
  FastDiv div_g16, div_g32, div_g64, div_t, div_bq;
};

// Bound on the length of a token's block list: the dense blocks of region 0 its
// window can reach (all of them without a window: 128 rows span at most 5
// blocks, window / 32 + 2 is an upper bound), plus the blocks of region 1 (dense
// blocks, or gathered blocks of 32 index entries).
inline int64_t list_bound(const AttnParams &p) {
  int64_t r0 = p.nb0;
  if (p.window > 0 && (int64_t)p.window / kRowsPerBlock + 2 < r0) r0 = (int64_t)p.window / kRowsPerBlock + 2;
  return r0 + p.nb1;
}

// ----------------------------------------------------------------------------- device helpers

// Workgroups are dealt to the dies round-robin; give each die a contiguous run of
// logical work items so neighbours (head groups of one token, adjacent tokens)
// share that die's L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ uint32_t xcd_remap32(uint32_t i, uint32_t n) {
  const uint32_t x = i % kNumXcd, k = i / kNumXcd;
  const uint32_t per = n / kNumXcd, rem = n % kNumXcd;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
}
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
  const int64_t x = i % kNumXcd, k = i / kNumXcd;
  const int64_t per = n / kNumXcd, rem = n % kNumXcd;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
}

// Visibility of region-0 row `row` for token t (the allowed-row rule of the header).
__device__ __forceinline__ bool r0_visible(const AttnParams &p, int b, int t, int row) {
  if (row >= p.n0) return false;
  if (p.valid0 && p.valid0[(int64_t)b * p.valid0_sb + row] == 0) return false;
  if (p.window > 0) {
    const int64_t d = p.qk_delta + t - row;
    if (d < 0 || d >= p.window) return false;
  }
  return true;
}

// Visibility of region-1 row c (dense or gathered through the index list).
__device__ __forceinline__ bool r1_visible(const AttnParams &p, int b, int c) {
  if (c < 0 || c >= p.n1) return false;
  if (p.valid1 && p.valid1[(int64_t)b * p.valid1_sb + c] == 0) return false;
  return true;
}

// Status of key block j for the token's query tile: map entries for the dense
// blocks, PARTIAL for gathered blocks (their rows differ per token).
// Wave-uniform: returns the first block >= j that is not SKIP (or nbt), and its status.
__device__ __forceinline__ int next_block(const uint8_t *row, int nbd, int nbt, int j, int lane,
                                          int &status) {
  while (j < nbt) {
    if (j >= nbd) {
      status = kPartial;
      return j;
    }
    const int jj = j + lane;
    int s = 0;
    if (jj < nbt) s = (jj < nbd) ? (row ? (int)row[jj] : kPartial) : kPartial;
    const unsigned long long m = __ballot(s != 0);
    if (m) {
      const int k = __ffsll((unsigned long long)m) - 1;
      status = __builtin_amdgcn_readfirstlane(__shfl(s, k));
      return j + k;
    }
    j += 64;
  }
  status = kSkip;
  return nbt;
}

// ----------------------------------------------------------------------------- launchers

hipError_t launch_pad(const void *k, const void *v, const uint8_t *valid, int64_t in_sb,
                      int64_t in_sr, int64_t valid_sb, void *kp, void *vp, uint8_t *validp,
                      int64_t out_sb, int64_t out_sr, int64_t validp_sb, int B, int n, int npad,
                      int row_bytes, bool copy_k, bool copy_v, bool copy_valid, hipStream_t s);
hipError_t launch_blockmap(const AttnParams &p, uint8_t *blk, hipStream_t s);
hipError_t launch_attn_generic(const AttnParams &p, int elem_bytes, hipStream_t s);
// Matrix-core kernels (head dim 512, float16): decode splits a token's heads over
// workgroups of 16; prefill keeps 64 heads of a token in one workgroup.
hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s);
// Split decode: the partial pass (p.nsplit > 1, p.ws set) then the combine pass.
// A partial record: the part's normalised O of 16 heads x 512 dims (float32,
// head-major), then the 16 running maxima (base-2 scores) and the 16 sums.
constexpr int kMaxSplits = 64;
constexpr int64_t kSplitRecord = 16 * 512 * 4 + 16 * 4 * 2;
hipError_t launch_attn_decode_split(const AttnParams &p, hipStream_t s);
hipError_t launch_attn_prefill(const AttnParams &p, hipStream_t s);
// FP8 quantize step: one wave per row of head_dim elements (elem_bytes 2 or 4).
hipError_t launch_quant_fp8(const void *x, int elem_bytes, int B, int n, int D, int64_t x_sb, int64_t x_sr,
                            uint8_t *codes, int64_t c_sb, int64_t c_sr, float *scales, int64_t s_sb,
                            hipStream_t s);
// Top-k index selection, one workgroup per row of scores.
constexpr int64_t kMaxTopkRows = 1LL << 24;   // rows of one top-k launch (one workgroup each)
constexpr int32_t kMaxTopkN = (1 << 30) - 1;  // scores per row (row bytes fit a 32-bit buffer range)
constexpr int kMaxTopkK = 2048;               // selected entries per row (staged in LDS)
hipError_t launch_topk(const float *scores, int64_t rows, int n, int64_t s_stride, int k, int32_t *idx,
                       int64_t o_stride, hipStream_t s);
// Compressor step: pool every complete group of `ratio` stream rows (state rows,
// then new rows) into a float16 row of comp, then keep the trailing rows as the state.
constexpr int kMaxCompressRatio = 1024;
hipError_t launch_compress(void *state_kv, float *state_score, int64_t state_kv_sb, int64_t state_score_sb,
                           int n_state, const void *kv_new, const float *score_new, int64_t kv_new_sb,
                           int64_t score_new_sb, int n_new, int B, int D, int ratio, void *comp,
                           int64_t comp_sb, hipStream_t s);

}  // namespace ds4attn
