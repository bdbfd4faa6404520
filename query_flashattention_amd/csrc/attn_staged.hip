// Matrix-core attention kernels for head dim 512, float16 inputs, float32 output.
//
// The fused step of [P-Metal] "FlashAttention Kernel Architecture" (Q.K^T,
// softmax and value-weighted sum in one dispatch) over the 32-row key blocks the
// skip map leaves in ([P-Metal] "Mask Handling and Block Skipping"), for
// multi-query attention: all query heads of a token share each K/V row
// ([P-DS4] "Architecture Deep Dive", Fixed Model Shape).  Both contractions are
// dense per block and run on v_mfma_f32_16x16x32_f16 with float32 accumulation.
//
// One workgroup = one token x HG heads, 4 waves.  Common structure:
//   * the workgroup first lists its non-skipped blocks in LDS (one read of its
//     map row), so the block sequence is known before any K/V transfer starts;
//   * each key block is staged once in LDS and read by all four waves: K and V
//     rows travel global -> LDS directly (16 bytes per lane, a whole 1 KiB row per
//     instruction, no registers), into tiles whose padded row strides keep the
//     operand reads on distinct banks; tiles are double-buffered, so block i+1 is
//     in flight while block i is consumed;
//   * S^T = K Q^T: A operand = 16 K rows from LDS, B operand = Q^T in registers;
//     in the S^T accumulator layout a lane holds 8 rows of one head, so the
//     softmax max is in-lane plus two cross-lane steps and the float16 P values
//     are already the B operand P^T of O^T += V^T P^T;
//   * the V^T operand comes from the row-major V tile through ds_read_b64_tr_b16
//     (two per 16 x 16 operand: key slots 0-3 and 4-7 of the lane's group);
//   * masked V rows are zeroed in LDS before use, so whatever a masked row holds
//     never reaches the output; masked scores are -inf;
//   * the softmax reference max moves lazily (see kRescaleSlack), so O is rescaled
//     only when a block raises a row's max by more than 2^8.
// Two ways of splitting the work over the four waves:
//   HEADS (HG = 64, prefill): wave w owns heads 16w..16w+15 over the full head
//         dimension; no cross-wave exchange; one workgroup per token fetches each
//         key block once for all 64 heads.
//   DIMS  (HG = 16, decode): wave w owns head-dim quarter [128w, 128w+128) for all
//         16 heads; the four partial score tiles meet in LDS and every wave sums
//         them in the same order; 4 workgroups per 64-head token fill the chip
//         for small decode batches.
#include "mfma_common.h"

namespace ds4attn {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

enum : int { kSplitHeads = 0, kSplitDims = 1 };

// 16 bytes per lane, global -> LDS at byte address `lds` (uniform) + 16 * lane.
// Issued through asm so that the compiler does not order LDS reads of the other
// tile buffer behind it; completion is awaited explicitly (s_waitcnt vmcnt(0))
// before the barrier that publishes the tile.  m0 is not used by anything else in
// these kernels.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void *)p;
}

// Tile rows are padded so that rows start on different banks while every operand
// address stays affine (base + immediate): K rows every 1040 bytes (the 16 rows of
// an A operand spread over 16-byte bank groups), V rows every 1056 bytes (the 4
// rows x 32 bytes of a transpose read spread over 8-byte bank groups).
constexpr int kKRow = 1040, kVRow = 1056;
constexpr int kKTile = 32 * kKRow, kVTile = 32 * kVRow;

struct StageInfo {
  int vis_arith;   // lane's row (lane & 31): inside the region and the window
  int use_byte;    // whether `vbyte` (the row's validity byte) decides visibility
  int vbyte;
  int full;
};

template <int MODE, bool INDEXED>
__global__ __launch_bounds__(256) void attn_staged_kernel(const AttnParams p) {
  constexpr int HG = MODE == kSplitHeads ? 64 : 16;   // heads per workgroup
  constexpr int NKS = MODE == kSplitHeads ? 16 : 4;    // 32-dim k-steps of S per wave
  constexpr int NDT = MODE == kSplitHeads ? 32 : 8;    // 16-dim output tiles per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;       // lane group: operand k-slots 8g..8g+7
  const int c16 = lane & 15;     // MFMA row/column of this lane

  const int ngroups = p.H / HG;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = (int)(L % ngroups);
  const int64_t bt = L / ngroups;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  // this lane's head and the first head dim of this wave's operands
  const int h = hg * HG + (MODE == kSplitHeads ? 16 * w : 0) + c16;
  const int d0 = MODE == kSplitHeads ? 0 : 128 * w;

  // Two tile buffers as separate LDS objects.
  __shared__ __attribute__((aligned(16))) char kt0[kKTile], kt1[kKTile];
  __shared__ __attribute__((aligned(16))) char vt0[kVTile], vt1[kVTile];
  __shared__ floatx4 xs[MODE == kSplitDims ? 4 * 2 * 64 : 1];   // partial S^T exchange
  __shared__ uint16_t blist[kListCap];
  __shared__ int cnt[4];
  __shared__ int idx_s[INDEXED ? kIdxCap : 1];

  // Q^T operand fragments: head h, dims d0 + 32ks + 8g .. +7
  half8 qf[NKS];
  const char *qrow = p.q + b * p.q_sb + t * p.q_st + (int64_t)h * p.q_sh;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const half8 *)(qrow + 2 * (d0 + 32 * ks + 8 * g));
  if (INDEXED) {
    const int32_t *src = p.idx + ((int64_t)b * p.T + t) * p.r1_k;
    for (int e = tid; e < p.r1_k; e += 256) idx_s[e] = src[e];
  }
  const uint8_t *blkrow = p.blk ? p.blk + ((int64_t)b * p.ntiles + t / p.bq) * p.nbd : nullptr;
  const int ndense = build_block_list<256>(blkrow, p.nbd, blist, cnt);   // ends with a barrier
  const int nlist = ndense + (INDEXED ? p.nb1 : 0);

  auto entry = [&](int i, int &j, int &status) {
    if (i < ndense) {
      const int e = blist[i];
      j = e & 0x3fff;
      status = e >> 14;
    } else {
      j = p.nb0 + (i - ndense);
      status = kPartial;
    }
  };
  // validity arrays of this sequence (size 0 when absent: every load out of range)
  const rsrc_t rb0 = make_rsrc(p.valid0 + (int64_t)b * p.valid0_sb, p.valid0 ? (uint32_t)p.n0 : 0u);
  const rsrc_t rb1 = make_rsrc(p.valid1 + (int64_t)b * p.valid1_sb, p.valid1 ? (uint32_t)p.n1 : 0u);
  // gathered row of index entry e (unused entries read row 0; they are masked)
  auto rid = [&](int e) {
    const int c = (e < p.r1_k) ? idx_s[e] : -1;
    return (c >= 0 && c < p.n1) ? c : 0;
  };

  // Start the transfers of list entry i into tiles kt / vt (wave w moves rows
  // 8w..8w+7 of K and of V, one row per instruction) and load the visibility
  // inputs.  Past the end of the list nothing is transferred.
  auto stage = [&](int i, const char *kt, const char *vt, StageInfo &st) {
    int j = 0, status = kFull;
    const bool real = i < nlist;
    if (real) entry(i, j, status);
    st.full = status == kFull;
    const int r = lane & 31;
    st.vis_arith = 1;
    st.use_byte = 0;
    uint32_t offb = kOutOfRange;   // lane's validity byte offset (out of range when unused)
    const char *kb = p.q, *vb = p.q;
    int64_t sr = 0;
    int base = 0;
    bool gathered = false;
    if (!real) {
      // nothing to stage
    } else if (j < p.nb0) {
      base = j * kRowsPerBlock;
      kb = p.k0 + b * p.kv0_sb;
      vb = p.v0 + b * p.kv0_sb;
      sr = p.kv0_sr;
      if (!st.full) {
        const int row = base + r;
        bool ok = row < p.n0;
        if (p.window > 0) {
          const int64_t d = p.qk_delta + t - row;
          ok = ok && d >= 0 && d < p.window;
        }
        st.vis_arith = ok;
        if (p.valid0 && row < p.n0) {
          offb = row;
          st.use_byte = 1;
        }
      }
    } else {
      base = (j - p.nb0) * kRowsPerBlock;
      kb = p.k1 + b * p.kv1_sb;
      vb = p.v1 + b * p.kv1_sb;
      sr = p.kv1_sr;
      if (INDEXED) {
        gathered = true;
        const int e = base + r;
        const int c = (e < p.r1_k) ? idx_s[e] : -1;
        const bool ok = c >= 0 && c < p.n1;
        st.vis_arith = ok;
        if (p.valid1 && ok) {
          offb = c;
          st.use_byte = 1;
        }
      } else if (!st.full) {
        const int c = base + r;
        st.vis_arith = c < p.n1;
        if (p.valid1 && c < p.n1) {
          offb = c;
          st.use_byte = 1;
        }
      }
    }
    // the validity byte: an out-of-range (zero, no traffic) load when unused
    st.vbyte = buf_load_u8(real && j >= p.nb0 ? rb1 : rb0, offb);
    if (!real) return;
    const uint32_t kbase = lds_addr(kt), vbase = lds_addr(vt);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rr = 8 * w + q;
      const int row = gathered ? rid(base + rr) : base + rr;
      const uint32_t koff = __builtin_amdgcn_readfirstlane(kbase + rr * kKRow);
      const uint32_t voff = __builtin_amdgcn_readfirstlane(vbase + rr * kVRow);
      dma16(kb + row * sr + 16 * lane, koff);
      dma16(vb + row * sr + 16 * lane, voff);
    }
  };

  // Wait for the transfers, resolve visibility, zero masked V rows.  Returns the
  // block's visibility mask (bit r = row r visible; all ones for a FULL block).
  auto commit = [&](char *vt, const StageInfo &st) -> uint32_t {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (st.full) return 0xffffffffu;
    const uint32_t vis = (uint32_t)__ballot(st.vis_arith && (!st.use_byte || st.vbyte != 0));
    // each wave clears the masked rows among the ones its own transfers wrote
    // (rows 8w..8w+7): its vmcnt wait above covers exactly those transfers
    uint32_t masked = (~vis >> (8 * w)) & 0xffu;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    while (masked) {
      const int r = 8 * w + __ffs(masked) - 1;
      masked &= masked - 1;
      *(uint4 *)(vt + r * kVRow + 16 * lane) = z;
    }
    return vis;
  };

  floatx4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // transpose-read roles: this lane points at row slot_row(g, e) of the V tile,
  // 4 dims starting at 16dt + 4a, for the lanes 16g + 4a + (0..3) to receive
  // (ds_read_b64_tr_b16 hands element b of lane 16g + 4e + a to lane 16g + 4a + b)
  const int tr_e = (lane >> 2) & 3, tr_a = lane & 3;
  const int tr_r0 = 4 * g + tr_e;   // slot rows 0-3 of group g; rows 16 + ... for slots 4-7

  StageInfo st;
  stage(0, kt0, vt0, st);
  uint32_t vis_cur = commit(vt0, st);
  int full_cur = st.full;
  __syncthreads();

  // One block: start the transfers of list position i+1 into the other buffers,
  // consume block i, then wait for the transfers and publish them.
  auto iteration = [&](int i, const char *ktc, const char *vtc, char *ktn, char *vtn) {
    stage(i + 1, ktn, vtn, st);

    // ---- S^T = K Q^T over this wave's head dims (operand loads one step ahead)
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const char *krow0 = ktc + c16 * kKRow + 2 * (d0 + 8 * g), *krow1 = krow0 + 16 * kKRow;
    uint4 a0 = *(const uint4 *)krow0;
    uint4 a1 = *(const uint4 *)krow1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 n0 = a0, n1 = a1;
      if (ks + 1 < NKS) {
        n0 = *(const uint4 *)(krow0 + 64 * (ks + 1));
        n1 = *(const uint4 *)(krow1 + 64 * (ks + 1));
      }
      s0 = mfma16(*(const half8 *)&a0, qf[ks], s0);
      s1 = mfma16(*(const half8 *)&a1, qf[ks], s1);
      a0 = n0;
      a1 = n1;
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    if (MODE == kSplitDims) {
      // partial tiles meet in LDS; every wave adds them in the same order
      xs[(w * 2 + 0) * 64 + lane] = s0;
      xs[(w * 2 + 1) * 64 + lane] = s1;
      __syncthreads();
      s0 = xs[0 * 64 + lane];
      s1 = xs[1 * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        s0 += xs[(ww * 2 + 0) * 64 + lane];
        s1 += xs[(ww * 2 + 1) * 64 + lane];
      }
    }
    // ---- online softmax: this lane holds rows slot_row(g, 0..7) of head h
    float sv[8];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      sv[i2] = s0[i2] * p.scale_log2;
      sv[4 + i2] = s1[i2] * p.scale_log2;
    }
    if (!full_cur) {
      const uint32_t sm = slot_mask(vis_cur, g);
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2)
        if (!((sm >> i2) & 1u)) sv[i2] = -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i2 = 1; i2 < 8; ++i2) mx = fmaxf(mx, sv[i2]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool grow = mx > m + kRescaleSlack;
    const float mref = grow ? mx : m;
    const float msafe = (mref == -INFINITY) ? 0.f : mref;
    const float alpha = __builtin_amdgcn_exp2f(m - msafe);
    half8 pf;
    float psum = 0.f;
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(sv[i2] - msafe);
      pf[i2] = ph;
      psum += (float)ph;
    }
    l = alpha * l + psum;
    m = mref;
    if (__ballot(grow)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    // ---- O^T += V^T P^T; V^T operand = two transpose reads (slots 0-3, 4-7)
    const lds_char *vrow0 = (const lds_char *)(__attribute__((address_space(3))) const void *)vtc +
                            tr_r0 * kVRow + 2 * d0 + 8 * tr_a;
    const lds_char *vrow1 = vrow0 + 16 * kVRow;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t *)(vrow0 + 32 * dt));
      const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t *)(vrow1 + 32 * dt));
      // whole-vector casts: slots 0-3 from the first read, 4-7 from the second
      const half8 vf = __builtin_shufflevector(__builtin_bit_cast(half4, lo),
                                               __builtin_bit_cast(half4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = mfma16(vf, pf, o[dt]);
      // keep the scheduler from hoisting every operand read ahead of the MFMAs
      if ((dt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }

    const uint32_t vis_next = commit(vtn, st);
    const int full_next = st.full;
    __syncthreads();   // publishes tiles i+1; also orders the next exchange after these reads
    vis_cur = vis_next;
    full_cur = full_next;
  };

  for (int i = 0; i < nlist; i += 2) {
    iteration(i, kt0, vt0, kt1, vt1);
    if (i + 1 < nlist) iteration(i + 1, kt1, vt1, kt0, vt0);
  }

  // ---- epilogue: O = O / l, float32 stores (4 consecutive dims per lane)
  float lt = l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float *ob = (float *)(p.o + b * p.o_sb + t * p.o_st + (int64_t)h * p.o_sh) + d0 + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *(floatx4 *)(ob + 16 * dt) = o[dt] * inv;
}

template <int MODE>
static hipError_t launch_staged(const AttnParams &p, hipStream_t s) {
  constexpr int HG = MODE == kSplitHeads ? 64 : 16;
  const int64_t n = (int64_t)p.B * p.T * (p.H / HG);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(256);
  if (p.indexed) hipLaunchKernelGGL((attn_staged_kernel<MODE, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_staged_kernel<MODE, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s) {
  return launch_staged<kSplitDims>(p, s);
}
hipError_t launch_attn_prefill(const AttnParams &p, hipStream_t s) {
  return launch_staged<kSplitHeads>(p, s);
}

}  // namespace ds4attn
