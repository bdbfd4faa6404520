// Matrix-core attention kernel for head dim 512, float16 inputs, float32 output.
//
// The fused step of [P-Metal] "FlashAttention Kernel Architecture" (Q.K^T,
// softmax and value-weighted sum in one dispatch), over 32-row key blocks that
// the skip map leaves in ([P-Metal] "Mask Handling and Block Skipping"), for
// multi-query attention: all query heads of a token share each K/V row
// ([P-DS4] "Architecture Deep Dive", Fixed Model Shape).  Both contractions are
// dense per block (HG heads x 512 dims x 32 rows) and run on
// v_mfma_f32_16x16x32_f16 with float32 accumulation.
//
// Work decomposition (one workgroup = one token x HG heads, 4 waves):
//   * wave w owns head-dim quarter [128w, 128w+128) of the output for all HG heads;
//   * per block, each wave forms the partial score tile S^T = K_q . Q_q^T over its
//     quarter (rows r of the block x heads h), the four partials meet in LDS and
//     every wave adds them in the same order, so all waves hold the identical full
//     S^T for the block;
//   * the S^T accumulator layout (lane = head, 8 rows per lane) makes the softmax
//     row reductions mostly in-lane (two cross-lane steps) and is already the
//     B operand P^T of the P.V product -- no reshuffle of P;
//   * V is the A operand V^T of O^T = V^T P^T, so its rows are transposed through a
//     per-wave LDS tile (8x8 register transpose, then 16-byte stores);
//   * K and V fragments are loaded straight from global memory into registers one
//     block ahead (each wave reads only its quarter, so a K/V byte crosses the
//     L2->CU path once per workgroup), and the output accumulator stays in
//     registers until a single float32 store per element.
// The online softmax runs in base 2: m' = max(m, rowmax s), alpha = 2^(m - m'),
// p = 2^(s - m'), l = alpha l + sum p, O = alpha O + P V, and O/l at the end.
#include "ds4attn_internal.h"

namespace ds4attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// K fragments, raw V rows and visibility of one 32-row key block.
template <int NHT>
struct BlockRegs {
  half8 k[2][4];   // A operand of S^T: row r = 16*rt + (lane & 15), dims 128w + 32ks + 8g .. +7
  uint4 v[8];      // V rows {4*(lane&3) + i, 16 + 4*(lane&3) + i} x dims 128w + 8*(lane>>2) .. +7
  uint32_t vis;    // bit r: row r of the block is visible to this token
};

// Index (in 16-byte units) of the transposed-V chunk holding slots 8G..8G+7 of
// head-dim row d (0..127) in a wave's tile.  Rows and slot groups are swizzled so
// both the transposing stores and the operand loads spread over the LDS banks.
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

template <int HG, bool INDEXED>
__global__ __launch_bounds__(256) void attn_mfma_kernel(const AttnParams p) {
  constexpr int NHT = HG / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;        // head-dim quarter of this wave
  const int g = lane >> 4;       // lane group: operand k-slots 8g..8g+7
  const int c16 = lane & 15;     // MFMA row/column of this lane
  const int wg4 = lane & 3;      // slot group this lane writes in the V transpose
  const int wc = lane >> 2;      // 8-dim chunk this lane loads in the V transpose

  const int ngroups = p.H / HG;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = (int)(L % ngroups);
  const int64_t bt = L / ngroups;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);

  __shared__ floatx4 xs[2][4][2][NHT][64];   // partial S^T exchange, double-buffered
  __shared__ uint4 vts[4][128 * 4];          // per-wave transposed V quarter
  __shared__ int idx_s[INDEXED ? kIdxCap : 1];

  // Q^T operand fragments: head h = hg*HG + 16*ht + c16, dims 128w + 32ks + 8g .. +7
  half8 qf[NHT][4];
  {
    const char *qb = p.q + b * p.q_sb + t * p.q_st;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[ht][ks] = *(const half8 *)(qb + (int64_t)(hg * HG + 16 * ht + c16) * p.q_sh +
                                      2 * (128 * w + 32 * ks + 8 * g));
  }
  if (INDEXED) {
    const int32_t *src = p.idx + ((int64_t)b * p.T + t) * p.r1_k;
    for (int e = tid; e < p.r1_k; e += 256) idx_s[e] = src[e];
    __syncthreads();
  }

  floatx4 o[NHT][8];
  float m[NHT], l[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    m[ht] = -INFINITY;
    l[ht] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ht][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t *blkrow = p.blk ? p.blk + ((int64_t)b * p.ntiles + t / p.bq) * p.nbd : nullptr;
  const int nbt = p.nb0 + p.nb1;

  // Issue the loads of key block j (K fragments, V rows) and its visibility mask.
  auto load_block = [&](int j, int status, BlockRegs<NHT> &br) {
    const char *kb, *vb;
    int64_t sr;
    int rk[2], rv[8];
    bool vis_lane;
    const int r = lane & 31;
    if (j < p.nb0) {
      const int base = j * kRowsPerBlock;
      kb = p.k0 + b * p.kv0_sb;
      vb = p.v0 + b * p.kv0_sb;
      sr = p.kv0_sr;
      rk[0] = base + c16;
      rk[1] = base + 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rv[i] = base + 4 * wg4 + i;
        rv[4 + i] = base + 16 + 4 * wg4 + i;
      }
      vis_lane = (status == kFull) || r0_visible(p, b, t, base + r);
    } else {
      const int base = (j - p.nb0) * kRowsPerBlock;
      kb = p.k1 + b * p.kv1_sb;
      vb = p.v1 + b * p.kv1_sb;
      sr = p.kv1_sr;
      if (INDEXED) {
        // gathered rows: entry e of the token's list; unused entries read row 0
        auto rid = [&](int e) {
          const int c = (e < p.r1_k) ? idx_s[e] : -1;
          return (c >= 0 && c < p.n1) ? c : 0;
        };
        rk[0] = rid(base + c16);
        rk[1] = rid(base + 16 + c16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rv[i] = rid(base + 4 * wg4 + i);
          rv[4 + i] = rid(base + 16 + 4 * wg4 + i);
        }
        const int e = base + r;
        vis_lane = (e < p.r1_k) && r1_visible(p, b, idx_s[e]);
      } else {
        rk[0] = base + c16;
        rk[1] = base + 16 + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rv[i] = base + 4 * wg4 + i;
          rv[4 + i] = base + 16 + 4 * wg4 + i;
        }
        vis_lane = (status == kFull) || r1_visible(p, b, base + r);
      }
    }
    br.vis = (uint32_t)__ballot(vis_lane);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        br.k[rt][ks] = *(const half8 *)(kb + rk[rt] * sr + 2 * (128 * w + 32 * ks + 8 * g));
#pragma unroll
    for (int i = 0; i < 8; ++i) br.v[i] = *(const uint4 *)(vb + rv[i] * sr + 2 * (128 * w + 8 * wc));
  };

  int status;
  int j = next_block(blkrow, p.nbd, nbt, 0, lane, status);
  BlockRegs<NHT> cur;
  if (j < nbt) load_block(j, status, cur);
  int buf = 0;
  uint4 *vt = vts[w];

  while (j < nbt) {
    int nstatus;
    const int jn = next_block(blkrow, p.nbd, nbt, j + 1, lane, nstatus);
    BlockRegs<NHT> nxt;
    if (jn < nbt) load_block(jn, nstatus, nxt);

    const bool full = (status == kFull);
    // ---- V^T tile: masked rows become zero, then an 8x8 transpose of halves
    {
      uint4 vv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (i < 4) ? 4 * wg4 + i : 16 + 4 * wg4 + (i - 4);
        const bool keep = full || ((cur.vis >> row) & 1u);
        vv[i] = keep ? cur.v[i] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint4 out;
        out.x = pair_halves(vv[0], vv[1], i);
        out.y = pair_halves(vv[2], vv[3], i);
        out.z = pair_halves(vv[4], vv[5], i);
        out.w = pair_halves(vv[6], vv[7], i);
        vt[vt_index(8 * wc + i, wg4)] = out;
      }
    }
    // ---- partial S^T over this wave's head-dim quarter
    floatx4 sp[2][NHT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.k[rt][ks], qf[ht][ks], acc, 0, 0, 0);
        sp[rt][ht] = acc;
      }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) xs[buf][w][rt][ht][lane] = sp[rt][ht];
    __syncthreads();
    // ---- full scores, the same sum order in every wave
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        floatx4 s = xs[buf][0][rt][ht][lane];
        s += xs[buf][1][rt][ht][lane];
        s += xs[buf][2][rt][ht][lane];
        s += xs[buf][3][rt][ht][lane];
        sp[rt][ht] = s;
      }
    // ---- online softmax; lane holds rows {4g+i, 16+4g+i} of head c16 (+16 ht)
    half8 pf[NHT];
    float alpha[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = sp[0][ht][i] * p.scale_log2;
        sv[4 + i] = sp[1][ht][i] * p.scale_log2;
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = (i < 4) ? 4 * g + i : 16 + 4 * g + (i - 4);
          if (!((cur.vis >> row) & 1u)) sv[i] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[ht], mx);
      const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
      alpha[ht] = __builtin_amdgcn_exp2f(m[ht] - msafe);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(sv[i] - msafe);
        pf[ht][i] = ph;
        psum += (float)ph;
      }
      l[ht] = alpha[ht] * l[ht] + psum;
      m[ht] = mnew;
    }
    // ---- O^T = alpha O^T + V^T P^T over this wave's 128 dims
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const half8 vf = *(const half8 *)&vt[vt_index(16 * dt + c16, g)];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[ht], o[ht][dt] * alpha[ht], 0, 0, 0);
    }

    cur = nxt;
    status = nstatus;
    j = jn;
    buf ^= 1;
  }

  // ---- epilogue: O = O / l, float32 stores (4 consecutive dims per lane)
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    float lt = l[ht];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float *ob = (float *)(p.o + b * p.o_sb + t * p.o_st +
                          (int64_t)(hg * HG + 16 * ht + c16) * p.o_sh) + 128 * w + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(floatx4 *)(ob + 16 * dt) = o[ht][dt] * inv;
  }
}

hipError_t launch_attn_mfma(const AttnParams &p, int hg, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.T * (p.H / hg);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(256);
  if (p.indexed) {
    switch (hg) {
      case 16: hipLaunchKernelGGL((attn_mfma_kernel<16, true>), grid, block, 0, s, p); break;
      case 32: hipLaunchKernelGGL((attn_mfma_kernel<32, true>), grid, block, 0, s, p); break;
      case 64: hipLaunchKernelGGL((attn_mfma_kernel<64, true>), grid, block, 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (hg) {
      case 16: hipLaunchKernelGGL((attn_mfma_kernel<16, false>), grid, block, 0, s, p); break;
      case 32: hipLaunchKernelGGL((attn_mfma_kernel<32, false>), grid, block, 0, s, p); break;
      case 64: hipLaunchKernelGGL((attn_mfma_kernel<64, false>), grid, block, 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace ds4attn
