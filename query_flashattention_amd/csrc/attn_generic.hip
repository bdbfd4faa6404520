// Generic attention kernel: the vector-ALU path for any supported head size and
// element type ([P-Metal] "Vector vs Non-Vector Execution Paths": a path that
// handles arbitrary head sizes correctly at lower bandwidth).
//
// One wave per (sequence, token, head).  Lane l holds elements d = l + 64*i of
// q and of the running output.  Key blocks come from the skip map; inside a
// block the visible rows are taken one at a time: score by a wave reduction,
// then the online-softmax update m' = max(m, s), o = o*2^(m-m') + 2^(s-m') v,
// l = l*2^(m-m') + 2^(s-m') ([P-Metal] "FlashAttention Kernel Architecture":
// dot product, softmax and weighted value sum fused in one dispatch).
#include "ds4attn_internal.h"

namespace ds4attn {

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  return (float)x;
}

template <typename T, int DPL>
__global__ __launch_bounds__(64) void attn_generic_kernel(const AttnParams p) {
  const int lane = threadIdx.x;
  const int64_t L = blockIdx.x;
  const int h = (int)(L % p.H);
  const int64_t bt = L / p.H;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);

  const T *qrow = (const T *)(p.q + b * p.q_sb + t * p.q_st + h * p.q_sh);
  float q[DPL], o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    q[i] = to_f32(qrow[lane + 64 * i]);
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const uint8_t *blkrow =
      p.blk ? p.blk + ((int64_t)b * p.ntiles + t / p.bq) * p.nbd : nullptr;
  const int nbt = p.nb0 + p.nb1;
  const int32_t *idx = p.indexed ? p.idx + ((int64_t)b * p.T + t) * p.r1_k : nullptr;

  int status;
  int j = next_block(blkrow, p.nbd, nbt, 0, lane, status);
  while (j < nbt) {
    // visible rows of this block: bit r of `vis`; row ids for gathered blocks
    const int r = lane & 31;
    bool vis;
    int row;
    const char *kb, *vb;
    int64_t sr;
    if (j < p.nb0) {
      row = j * kRowsPerBlock + r;
      vis = (status == kFull) || r0_visible(p, b, t, row);
      kb = p.k0 + b * p.kv0_sb;
      vb = p.v0 + b * p.kv0_sb;
      sr = p.kv0_sr;
    } else {
      const int e = (j - p.nb0) * kRowsPerBlock + r;
      if (p.indexed) row = (e < p.r1_k) ? idx[e] : -1;
      else row = e;
      vis = (status == kFull) || r1_visible(p, b, row);
      kb = p.k1 + b * p.kv1_sb;
      vb = p.v1 + b * p.kv1_sb;
      sr = p.kv1_sr;
    }
    const uint32_t mask = (uint32_t)__ballot(vis);
    for (int rr = 0; rr < kRowsPerBlock; ++rr) {
      if (!((mask >> rr) & 1u)) continue;
      const int rid = __shfl(row, rr);
      const T *krow = (const T *)(kb + rid * sr);
      const T *vrow = (const T *)(vb + rid * sr);
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) s += q[i] * to_f32(krow[lane + 64 * i]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      s *= p.scale_log2;
      const float mn = fmaxf(m, s);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      const float pw = __builtin_amdgcn_exp2f(s - mn);
      l = l * alpha + pw;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] = o[i] * alpha + pw * to_f32(vrow[lane + 64 * i]);
      m = mn;
    }
    j = next_block(blkrow, p.nbd, nbt, j + 1, lane, status);
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *orow = (float *)(p.o + b * p.o_sb + t * p.o_st + h * p.o_sh);
#pragma unroll
  for (int i = 0; i < DPL; ++i) orow[lane + 64 * i] = o[i] * inv;
}

template <typename T>
static hipError_t launch_typed(const AttnParams &p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.T * p.H;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)n), block(64);
  switch (p.D) {
    case 64: hipLaunchKernelGGL((attn_generic_kernel<T, 1>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((attn_generic_kernel<T, 2>), grid, block, 0, s, p); break;
    case 256: hipLaunchKernelGGL((attn_generic_kernel<T, 4>), grid, block, 0, s, p); break;
    case 512: hipLaunchKernelGGL((attn_generic_kernel<T, 8>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_generic(const AttnParams &p, int elem_bytes, hipStream_t s) {
  return elem_bytes == 2 ? launch_typed<_Float16>(p, s) : launch_typed<float>(p, s);
}

}  // namespace ds4attn
