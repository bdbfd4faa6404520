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
//     operand reads on distinct banks; with two tile pairs, blocks i+1 and i+2
//     are in flight while block i is consumed;
//   * S^T = K Q^T: A operand = 16 K rows from LDS, B operand = Q^T in registers;
//     in the S^T accumulator layout a lane holds 8 rows of one head, so the
//     softmax max is in-lane plus two cross-lane steps and the float16 P values
//     are already the B operand P^T of O^T += V^T P^T;
//   * the V^T operand comes from the row-major V tile through ds_read_b64_tr_b16
//     (two per 16 x 16 operand: key slots 0-3 and 4-7 of the lane's group);
//   * masked V rows are zeroed in LDS before use, so whatever a masked row holds
//     never reaches the output; masked scores are -inf;
//   * the softmax reference max moves lazily (see kRescaleSlack), so O is rescaled
//     only when a block raises a row's max by more than 2^8;
//   * O leaves through non-temporal (streaming) stores: nothing reads it back in
//     the launch, and cached stores would evict K/V rows other workgroups reuse.
// Two ways of splitting the work over the four waves:
//   HEADS (HG = 64, prefill): wave w owns heads 16w..16w+15 over the full head
//         dimension; no cross-wave exchange; one workgroup per token fetches each
//         key block once for all 64 heads.
//   DIMS  (HG = 16, decode): wave w owns head-dim quarter [128w, 128w+128) for all
//         16 heads; the four partial score tiles meet in LDS and every wave sums
//         them in the same order; 4 workgroups per 64-head token fill the chip
//         for small decode batches.
//   KEYS  (HG = 16, decode): the waves take different key rows.  Wave w consumes
//         units w, w+4, w+8, ... of the list (half-blocks of 16 float16 rows, or
//         whole blocks of FP8 rows) for all 16 heads over the full head dimension,
//         with its own running max, sum and output; the four partial results are
//         merged in LDS at the end (the log-sum-exp rule).  Its rows travel
//         global -> registers (1 KiB per load, a unit two rounds ahead of its
//         use) -> the wave's own K and V tiles, so no wave waits for another
//         inside the key loop and the vector-memory path stays busy.
#include "staging.h"

#include <algorithm>
#include <type_traits>

namespace ds4attn {

// (kDimsWide: DIMS over 32 heads per workgroup, see DIMS below)
enum : int { kSplitHeads = 0, kSplitDims = 1, kSplitKeys = 2, kDimsWide = 3 };

// Stores a float32 tile of 16 heads x 16 N dims held in accumulator layout (lane
// 16g + c16 holds head c16, dims 16dt + 4g .. +3 in acc[dt]), times `sc` (this
// lane's head's factor), to the rows at `dst` (head c at dst + c * stride bytes).
// A cross-lane permutation first gives lane l head l >> 2, dims 16dt + 4(l & 3),
// so that four adjacent lanes write 64 contiguous bytes: the address path
// coalesces adjacent lanes only, and 16-byte accesses in the accumulator's lane
// order (a row per lane, a row's four pieces 16 lanes apart) cost it about 3.4
// times as long (measured with loads of the same shape from L2).
template <int N, bool NONTEMPORAL>
__device__ __forceinline__ void store_acc_rows(char *dst, int64_t stride, const floatx4 *acc, float sc,
                                               int lane) {
  typedef int int4v __attribute__((ext_vector_type(4)));
  const int src = 4 * (16 * (lane & 3) + (lane >> 2));   // byte address of the source lane
  floatx4 *row = (floatx4 *)(dst + (int64_t)(lane >> 2) * stride) + (lane & 3);
#pragma unroll
  for (int dt = 0; dt < N; ++dt) {
    // (whole-vector casts: a cast of one element of a vector value is not safe here)
    const int4v v = __builtin_bit_cast(int4v, acc[dt] * sc);
    int4v ri;
#pragma unroll
    for (int k = 0; k < 4; ++k) ri[k] = __builtin_amdgcn_ds_bpermute(src, v[k]);
    const floatx4 r = __builtin_bit_cast(floatx4, ri);
    if constexpr (NONTEMPORAL) __builtin_nontemporal_store(r, row + 4 * dt);
    else row[4 * dt] = r;
  }
}

// FP8 rows (E4M3 codes, a float32 scale per row): the rows travel to LDS as codes
// (half the bytes), two rows per transfer.  Scores: in HEADS the K codes go to the
// E4M3 matrix cores as they are, against Q carried as two E4M3 terms; in DIMS and
// KEYS they are converted to float16 (exact) where the operands are read.  Either
// way the K rows' scales multiply the float32 scores.  V codes come through an
// 8-bit transpose read and are converted to float16 (exact); the V rows' scales
// are folded into P (DIMS, HEADS) or multiply the converted codes in float16
// (KEYS).  The accumulators are float32 as for float16 rows.
// PARTS (decode only): the launch is a split decode; each workgroup takes one part
// of its token's block list and leaves a record for the combine pass.
template <int MODE, bool INDEXED, bool FP8, bool PARTS = false>
__global__ __launch_bounds__(MODE == kSplitDims || MODE == kDimsWide ? 512 : 256, MODE == kSplitHeads ? 2 : 1)
void attn_staged_kernel(const AttnParams p) {
  constexpr bool KEYS = MODE == kSplitKeys;
  // DIMS over 16 heads, or over 32 (kDimsWide: each computing wave carries two
  // 16-head tiles, which share every K and V operand read; half the workgroups
  // per token, so a large batch pulls each key block into half as many CUs)
  constexpr bool DIMS = MODE == kSplitDims || MODE == kDimsWide;
  constexpr int HT = MODE == kDimsWide ? 2 : 1;   // 16-head tiles per computing wave
  static_assert(!(MODE == kDimsWide && (PARTS || INDEXED)), "wide DIMS: no split parts, no index list");
  // KEYS units: float16 rows go in half-blocks of 16 rows, FP8 rows in whole blocks
  // (the FP8 tiles of a block take the space of a float16 half-block, and the
  // 8-bit transpose read hands out 8 keys per lane)
  constexpr int UPE = FP8 ? 1 : 2;   // KEYS units per list entry
  constexpr int HG = MODE == kSplitHeads ? 64 : 16 * HT;   // heads per workgroup
  constexpr int NKS = DIMS ? 4 : 16;    // 32-dim k-steps of S per wave
  constexpr int NDT = DIMS ? 8 : 32;    // 16-dim output tiles per wave (and head tile)
  // Tile buffers: DIMS double-buffers (block i+1 and i+2 in flight while block i
  // is consumed); HEADS keeps one block so that two workgroups share a CU and one
  // computes while the other's transfers are in flight.
  // (FP8 tiles are half the size: DIMS keeps four blocks in flight)
  constexpr int NBUF = MODE == kSplitHeads ? 1 : (FP8 ? 4 : 2);
  // DIMS runs eight waves: waves 0-3 compute, waves 4-7 ("producers") only move
  // key blocks into the tiles.  A wave that issues a block
  // transfer stalls while the vector-memory path drains (about 0.6 us per 64 KiB
  // block and CU), so the computing waves no longer issue any: they meet the
  // producers only at the workgroup barriers.  The producers stage a block's K rows
  // as soon as the score exchange has freed the K tile and its V rows once P.V has
  // freed the V tile; they publish its K rows at the barrier that ends the block
  // before it and its V rows, which only P.V reads, at its own score exchange.
  // FP8 rows (half the bytes, four buffers) are staged a whole block at a time once
  // the end of the block four before has freed its buffer, and published whole by
  // the end of the block before it.  Only the producers' counters see the transfers, so the computing
  // waves' waits for their own loads (Q, the map row, validity bytes) wait for
  // nothing else.
  constexpr bool SPLITKV = DIMS;
  // List entries whose transfers start before the map row is read (guessed).  The
  // float16 producers guess only the first: the prologue's barriers (block list,
  // masks) would otherwise wait while they issue a second block, and with every CU
  // busy the vector-memory path takes about 1 us per block.  They stage the second
  // once the list is known (see the producers' prologue).
  constexpr int kGuessed = SPLITKV && !FP8 ? 1 : NBUF;
  constexpr int kLateVMaxEntries = 5;   // see the producers' prologue
  constexpr int KPD = KEYS ? 4 : 2;   // K operand reads in flight (k-steps)
  // FP8 rows: the V rows' scales are folded into P, and V codes enter P.V as they
  // are: P'[h, r] = fp16(P[h, r] sv[r] vfac), one rounding.  vfac is a power of two
  // that the workgroup (KEYS: each wave) takes from the first block's largest V
  // scale and lowers, rescaling O exactly, only when a later block's largest scale
  // times vfac passes 2^7; O gets 1 / vfac back at the end.  So P' < 2^15 (P <=
  // 2^8 by the rescale slack) and, whatever the rows' magnitude, the largest
  // weights keep float16's full precision instead of sinking into its subnormals.
  // The sums l take P itself.
  constexpr bool FOLDV = FP8;
  // FP8 HEADS: the scores run on the E4M3 matrix cores, K codes against Q carried
  // as two E4M3 terms (split_e4m3) with a power-of-two factor per head; the K rows'
  // scales then multiply the scores with the softmax scale.  No K code is
  // converted.  (The same in DIMS, where each wave's 128 dims are one chunk with a
  // factor of their own, measured no faster than converting: decode_swa 10.6-10.7
  // us either way.)
  constexpr bool F8S = FP8 && MODE == kSplitHeads;
  constexpr int NQC = DIMS ? 1 : 4;   // F8S: 128-dim chunks per wave
  // V operand reads in flight (output tiles); FP8 rows in HEADS take one fewer,
  // which keeps their conversions within 256 registers without spilling
  constexpr int VPD = KEYS ? 8 : (MODE == kSplitHeads && FP8 ? 3 : 4);
  // One field of every 64-byte line of the parameter block is read here, so that
  // the block arrives in one burst of scalar loads; the code below then finds each
  // field in the scalar cache instead of waiting one memory round trip per line in
  // the order it first needs them (four to five serial rounds before the first
  // key-block transfer otherwise).
  asm volatile("" ::"s"(p.q), "s"(p.B), "s"(p.valid0), "s"(p.valid1_sb), "s"(p.vs1), "s"(p.nbd));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index (uniform); SPLITKV: 0-3 within the computing or the producing waves
  const bool producer = SPLITKV && tid >= 256;
  const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  // float16 rows a wave transfers per key block, K and V each (also the transfers
  // it issues per part)
  constexpr int RPW = 8;
  const int g = lane >> 4;       // lane group: operand k-slots 8g..8g+7
  const int c16 = lane & 15;     // MFMA row/column of this lane
  const uint32_t lane16 = 16u * lane;   // this lane's byte offset in a transferred row

  const int ngroups = p.H / HG;
  // split decode: consecutive workgroups share (token, head group) and take
  // consecutive parts of its block list
  static_assert(!(PARTS && MODE == kSplitHeads), "split parts are a decode launch");
  const int nsplit = PARTS ? p.nsplit : 1;
  // (32-bit unsigned arithmetic: the grid is below 2^31 workgroups, and 64-bit
  // divisions by values known only at run time cost hundreds of instructions)
  const uint32_t L0 = xcd_remap32(blockIdx.x, gridDim.x);
  const int split = (int)(L0 % (uint32_t)nsplit);
  const uint32_t L = L0 / (uint32_t)nsplit;
  // (indices below 2^31: multiply-shift divisions by the run-time H/HG and T)
  const uint32_t bt = fast_div(L, HG == 16 ? p.div_g16 : (HG == 32 ? p.div_g32 : p.div_g64));
  const int hg = (int)(L - bt * (uint32_t)ngroups);
  const uint32_t bb = fast_div(bt, p.div_t);
  const int t = (int)(bt - bb * (uint32_t)p.T);
  const int b = (int)bb;
  const int tile = (int)fast_div((uint32_t)t, p.div_bq);   // the token's query tile in the map
  // this lane's head and the first head dim of this wave's operands
  const int h = hg * HG + (MODE == kSplitHeads ? 16 * w : 0) + c16;
  const int d0 = DIMS ? 128 * w : 0;

  // Two tile buffers as separate LDS objects (FP8: codes, plus the blocks' row scales).
  constexpr int KT = KEYS ? 16 : (FP8 ? kF8Tile : kKTile), VT = KEYS ? 16 : (FP8 ? kF8Tile : kVTile);
  // KEYS: each wave's K tile and V tile (16 float16 rows each, or 32 FP8 rows each
  // plus their 64 scales); at the end the same memory holds the waves' partial
  // outputs, and mlw their maxima and sums
  constexpr int kWaveTile = 16 * kKRow + 16 * kVRow;
  static_assert(2 * kF8Tile + 64 * 4 <= kWaveTile, "FP8 tiles fit in a wave's space");
  static_assert(4 * kWaveTile >= 4 * 32 * 64 * 16, "the partial outputs fit in the tiles");
  __shared__ __attribute__((aligned(16))) char wt[KEYS ? 4 * kWaveTile : 16];
  __shared__ float mlw[KEYS ? 2 * 4 * 16 : 1];
  __shared__ __attribute__((aligned(16))) char kt0[KT], kt1[NBUF >= 2 ? KT : 16];
  __shared__ __attribute__((aligned(16))) char kt2[NBUF >= 4 ? KT : 16], kt3[NBUF >= 4 ? KT : 16];
  __shared__ __attribute__((aligned(16))) char vt0[VT], vt1[NBUF >= 2 ? VT : 16];
  __shared__ __attribute__((aligned(16))) char vt2[NBUF >= 4 ? VT : 16], vt3[NBUF >= 4 ? VT : 16];
  // scales of block rows 8w'..8w'+7: K at [16w' + q], V at [16w' + 8 + q]
  __shared__ __attribute__((aligned(16))) float sc0[FP8 ? 64 : 4], sc1[FP8 && NBUF >= 2 ? 64 : 4];
  __shared__ __attribute__((aligned(16))) float sc2[FP8 && NBUF >= 4 ? 64 : 4], sc3[FP8 && NBUF >= 4 ? 64 : 4];
  __shared__ floatx4 xs[DIMS ? 4 * 2 * HT * 64 : 1];   // partial S^T exchange
  __shared__ uint16_t blist[kListCap];
  __shared__ int cnt[4];
  __shared__ int nd_s;   // SPLITKV: the list length, for the producers
  __shared__ __attribute__((aligned(16))) int idx_s[INDEXED ? kIdxCap : 4];
  __shared__ uint32_t vmask[kMaskRing];   // bit r: row r of the entry's block is visible
  __shared__ uint32_t dmask[kTable];      // the same for dense blocks 0..kTable-1

  // Tile buffer pair 0 or 1, chosen at compile time so the compiler can tell the
  // transfers into one pair from the reads of the other.
  auto ktile = [&](auto buf) -> char * {
    constexpr int B = decltype(buf)::value;
    return B == 0 ? kt0 : (B == 1 ? kt1 : (B == 2 ? kt2 : kt3));
  };
  auto vtile = [&](auto buf) -> char * {
    constexpr int B = decltype(buf)::value;
    return B == 0 ? vt0 : (B == 1 ? vt1 : (B == 2 ? vt2 : vt3));
  };
  auto stile = [&](auto buf) -> float * {
    constexpr int B = decltype(buf)::value;
    return B == 0 ? sc0 : (B == 1 ? sc1 : (B == 2 ? sc2 : sc3));
  };
  // f(Buf<0>), ..., f(Buf<NBUF-1>) with compile-time buffer indices
  auto for_bufs = [&](auto f) __attribute__((always_inline)) {
    f(std::integral_constant<int, 0>{});
    if constexpr (NBUF >= 2) f(std::integral_constant<int, 1>{});
    if constexpr (NBUF >= 4) {
      f(std::integral_constant<int, 2>{});
      f(std::integral_constant<int, 3>{});
    }
  };

  // Float16 rows of key block j (uniform) for this wave's transfers: the region's K
  // and V rows of this sequence, the row stride, the wave's RPW rows RPW w .. (a
  // gathered entry reads its row from the list; unused entries read row 0) and the
  // visibility mask `vm`.  issue_row starts the transfer of one of them (K or V):
  // rows whose bit in `vm` is clear arrive as zeros and are not read from memory.
  struct RowSet {
    const char *kb, *vb;
    int64_t sr;
    int rows[RPW];
    uint32_t vm;
  };
  auto row_set = [&](int j, uint32_t vm) __attribute__((always_inline)) -> RowSet {
    RowSet rs;
    rs.vm = vm;
    int base;
    if (j < p.nb0) {
      rs.kb = p.k0 + b * p.kv0_sb;
      rs.vb = p.v0 + b * p.kv0_sb;
      rs.sr = p.kv0_sr;
      base = j * kRowsPerBlock;
    } else {
      rs.kb = p.k1 + b * p.kv1_sb;
      rs.vb = p.v1 + b * p.kv1_sb;
      rs.sr = p.kv1_sr;
      base = (j - p.nb0) * kRowsPerBlock;
    }
    if (INDEXED && j >= p.nb0) {
      // the wave's list entries in 16-byte LDS reads (entries past r1_k hold -1)
      const int4 *src = (const int4 *)&idx_s[base + RPW * w];
      int cs[RPW];
#pragma unroll
      for (int q4 = 0; q4 < RPW / 4; ++q4) {
        const int4 c4 = src[q4];
        cs[4 * q4] = c4.x;
        cs[4 * q4 + 1] = c4.y;
        cs[4 * q4 + 2] = c4.z;
        cs[4 * q4 + 3] = c4.w;
      }
#pragma unroll
      for (int q = 0; q < RPW; ++q) {
        const int c = __builtin_amdgcn_readfirstlane(cs[q]);
        rs.rows[q] = (c >= 0 && c < p.n1) ? c : 0;
      }
    } else {
#pragma unroll
      for (int q = 0; q < RPW; ++q) rs.rows[q] = base + RPW * w + q;
    }
    return rs;
  };
  auto issue_row = [&](const RowSet &rs, int q, uint32_t tile, int stride, auto is_v)
      __attribute__((always_inline)) {
    const int rr = RPW * w + q;
    const bool shown = (rs.vm >> rr) & 1u;
    const char *src = decltype(is_v)::value ? rs.vb : rs.kb;
    dma16(shown ? src + rs.rows[q] * rs.sr : kZeroRow, lane16, tile + rr * stride);
  };

  // Start the transfers of key block j (uniform) into buffer pair `buf`: wave w
  // moves rows RPW w .. RPW w + RPW - 1 of K and of V (FP8: pairs 4w..4w+3), one
  // 1 KiB row per instruction.  Rows whose bit in `vm` is clear arrive as zeros (and are
  // not read from memory); with vm = all ones every row is transferred (gathered
  // entries that are unused read row 0) and hidden rows are cleared afterwards.
  // `part` (float16 rows): 0 = K and V rows, 1 = K rows only, 2 = V rows only.
  auto stage_rows = [&](int j, uint32_t vm, auto buf, auto part) __attribute__((always_inline)) {
    constexpr int PART = decltype(part)::value;
    const uint32_t kbase = lds_addr(ktile(buf)), vbase = lds_addr(vtile(buf));
    const char *kb, *vb, *ksb = nullptr, *vsb = nullptr;
    int64_t sr;
    int base, nlive;
    if (j < p.nb0) {
      kb = p.k0 + b * p.kv0_sb;
      vb = p.v0 + b * p.kv0_sb;
      sr = p.kv0_sr;
      base = j * kRowsPerBlock;
      nlive = p.n0;
      if (FP8) {
        ksb = p.ks0 + b * p.s0_sb;
        vsb = p.vs0 + b * p.s0_sb;
      }
    } else {
      kb = p.k1 + b * p.kv1_sb;
      vb = p.v1 + b * p.kv1_sb;
      sr = p.kv1_sr;
      base = (j - p.nb0) * kRowsPerBlock;
      nlive = p.n1;
      if (FP8) {
        ksb = p.ks1 + b * p.s1_sb;
        vsb = p.vs1 + b * p.s1_sb;
      }
    }
    if constexpr (FP8) {
      // wave w moves pairs 4w..4w+3: lanes 0-31 the pair's first row, lanes 32-63
      // its second, 16 bytes each.  Each lane resolves its own row (a gathered entry
      // is read from the list; unused entries read row 0, masked).
      auto lane_row = [&](int rr) -> int {
        int row = base + rr;
        if (INDEXED && j >= p.nb0) {
          const int c = idx_s[row];
          row = (c >= 0 && c < p.n1) ? c : 0;
        }
        return row;
      };
      const int half = lane >> 5;
      const int64_t chunk = 16 * (lane & 31);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int pr = 4 * w + pp;
        const int rr = half ? f8_second_row(pr) : pr;
        const int row = lane_row(rr);
        const bool shown = (vm >> rr) & 1u;
        const uint32_t off = (uint32_t)(pr * kF8Pair);
        dma16_lanes(shown ? kb + row * sr + chunk : kZeroRow + chunk, kbase + off);
        dma16_lanes(shown ? vb + row * sr + chunk : kZeroRow + chunk, vbase + off);
      }
      // the eight rows' scales: lanes 0-3 K of the pairs' first rows, 4-7 K of their
      // second rows, 8-11 and 12-15 the same for V (rows past the region's live
      // rows have none and read zero)
      if (lane < 16) {
        const int pr = 4 * w + (lane & 3);
        const int rr = (lane & 4) ? f8_second_row(pr) : pr;
        const int row = lane_row(rr);
        const bool shown = ((vm >> rr) & 1u) && row < nlive;
        dma4_lanes(shown ? (lane < 8 ? ksb : vsb) + 4 * (int64_t)row : kZeroRow,
                   lds_addr(stile(buf)) + 64u * w);
      }
    } else {
      const RowSet rs = row_set(j, vm);
#pragma unroll
      for (int q = 0; q < RPW; ++q) {
        if (PART != 2) issue_row(rs, q, kbase, kKRow, std::false_type{});
        if (PART != 1) issue_row(rs, q, vbase, kVRow, std::true_type{});
      }
    }
  };
  using Masked = std::integral_constant<bool, true>;
  using Unmasked = std::integral_constant<bool, false>;
  using BothParts = std::integral_constant<int, 0>;
  using KPart = std::integral_constant<int, 1>;
  using VPart = std::integral_constant<int, 2>;

  // KEYS: a unit's rows travel global -> this wave's staging registers, one
  // contiguous 1 KiB per load (one float16 row, or two FP8 rows: lanes 0-31 the
  // first, 32-63 the second, in the FP8 tile's pair order), K rows then, later, V
  // rows.  `rows_of` resolves the rows of unit `hf` of key block j (uniform):
  // region descriptors and offsets (gathered entries that are unused read row 0;
  // every row is read, and the rows a mask hides are dealt with where they are
  // used).  FP8 rows bring their scales: this lane's K and V scale of row lane & 31
  // (rows past the region's live rows read 0).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // (float16: two staging sets, a wave's units alternating between them, so its
  // rows are requested two rounds before they are used; FP8 keeps one, for the
  // registers its conversions need: rows come a round ahead)
  constexpr int NSET = FP8 ? 1 : 2;
  u32x4 stk0[KEYS ? 16 : 1], stv0[KEYS ? 16 : 1];
  u32x4 stk1[KEYS && NSET == 2 ? 16 : 1], stv1[KEYS && NSET == 2 ? 16 : 1];
  float sck0 = 0.f, scv0 = 0.f, sck1 = 0.f, scv1 = 0.f;
  struct HalfRows {
    rsrc_t k, v, ks, vs;  // the region's K and V rows (and FP8 scales) of this sequence
    int32_t off[16];      // byte offsets of the 16 rows (FP8: of the first rows of the 16 pairs)
    int32_t dif[FP8 ? 16 : 1];   // FP8: second row's offset minus the first's, per pair
    int32_t soff;         // FP8: this lane's scale offset
  };
  auto rows_of = [&](int j, int hf) __attribute__((always_inline)) -> HalfRows {
    HalfRows hr;
    if constexpr (KEYS) {
      int rb, nlive;
      bool gath = false;
      const char *kb, *vb, *ksb = nullptr, *vsb = nullptr;
      int64_t sr, span;
      if (j < p.nb0) {
        kb = p.k0 + b * p.kv0_sb;
        vb = p.v0 + b * p.kv0_sb;
        sr = p.kv0_sr;
        span = (int64_t)p.nb0 * kRowsPerBlock * sr;
        rb = j * kRowsPerBlock + (32 / UPE) * hf;
        nlive = p.n0;
        if (FP8) {
          ksb = p.ks0 + b * p.s0_sb;
          vsb = p.vs0 + b * p.s0_sb;
        }
      } else {
        kb = p.k1 + b * p.kv1_sb;
        vb = p.v1 + b * p.kv1_sb;
        sr = p.kv1_sr;
        // (gathered rows are any of the region's n1 rows; dense ones fill whole blocks)
        span = (INDEXED ? (int64_t)p.n1 : (int64_t)p.nb1 * kRowsPerBlock) * sr;
        rb = (j - p.nb0) * kRowsPerBlock + (32 / UPE) * hf;
        nlive = p.n1;
        gath = INDEXED;
        if (FP8) {
          ksb = p.ks1 + b * p.s1_sb;
          vsb = p.vs1 + b * p.s1_sb;
        }
      }
      // (a sequence's rows span less than 2^31 bytes; loads past the span read 0)
      const uint32_t bytes = (uint32_t)(span < 0x7fffffff ? span : 0x7fffffff);
      hr.k = make_rsrc(kb, bytes);
      hr.v = make_rsrc(vb, bytes);
      const int32_t sr32 = (int32_t)sr;
      if constexpr (FP8) {
        hr.ks = make_rsrc(ksb, 4u * (uint32_t)nlive);
        hr.vs = make_rsrc(vsb, 4u * (uint32_t)nlive);
        int rr[32];
        if (gath) {
          const int4 *src = (const int4 *)&idx_s[rb];
#pragma unroll
          for (int q4 = 0; q4 < 8; ++q4) {
            const int4 c4 = src[q4];
            const int cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = __builtin_amdgcn_readfirstlane(cs[q]);
              rr[4 * q4 + q] = (c >= 0 && c < p.n1) ? c : 0;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 32; ++q) rr[q] = rb + q;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          hr.off[q] = rr[q] * sr32;
          hr.dif[q] = (rr[f8_second_row(q)] - rr[q]) * sr32;
        }
        int myrow = rb + (lane & 31);
        if (gath) {
          const int c = idx_s[rb + (lane & 31)];
          myrow = (c >= 0 && c < p.n1) ? c : 0;
        }
        hr.soff = 4 * myrow;
      } else {
        hr.ks = hr.vs = hr.k;
        hr.soff = 0;
        if (gath) {
          const int4 *src = (const int4 *)&idx_s[rb];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int4 c4 = src[q4];
            const int cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = __builtin_amdgcn_readfirstlane(cs[q]);
              hr.off[4 * q4 + q] = ((c >= 0 && c < p.n1) ? c : 0) * sr32;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) hr.off[q] = (rb + q) * sr32;
        }
      }
    }
    return hr;
  };
  // nothing to read: loads through it return zeros without touching memory
  auto no_rows = [&]() __attribute__((always_inline)) -> HalfRows {
    HalfRows hr;
    hr.k = hr.v = hr.ks = hr.vs = make_rsrc(p.k0, 0u);
#pragma unroll
    for (int q = 0; q < 16; ++q) hr.off[q] = 0;
    if constexpr (FP8) {
#pragma unroll
      for (int q = 0; q < 16; ++q) hr.dif[q] = 0;
    }
    hr.soff = 0;
    return hr;
  };
  // (the row offset is a scalar and the lane offset a shared register; FP8 lanes
  // 32-63 add the distance to the pair's second row)
  const uint32_t lane16lo = 16u * (lane & 31);
  auto load_k = [&](const HalfRows &hr, auto set) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      u32x4 *dst = (NSET == 2 && decltype(set)::value) ? stk1 : stk0;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        dst[q] = __builtin_bit_cast(
            u32x4, FP8 ? __builtin_amdgcn_raw_buffer_load_b128(hr.k, lane16lo + (lane >= 32 ? hr.dif[q] : 0), hr.off[q], 0)
                       : __builtin_amdgcn_raw_buffer_load_b128(hr.k, lane16, hr.off[q], 0));
      if constexpr (FP8) {
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(hr.ks, hr.soff, 0, 0));
        if (decltype(set)::value) sck1 = sc;
        else sck0 = sc;
      }
    }
  };
  auto load_v = [&](const HalfRows &hr, auto set) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      u32x4 *dst = (NSET == 2 && decltype(set)::value) ? stv1 : stv0;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        dst[q] = __builtin_bit_cast(
            u32x4, FP8 ? __builtin_amdgcn_raw_buffer_load_b128(hr.v, lane16lo + (lane >= 32 ? hr.dif[q] : 0), hr.off[q], 0)
                       : __builtin_amdgcn_raw_buffer_load_b128(hr.v, lane16, hr.off[q], 0));
      if constexpr (FP8) {
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(hr.vs, hr.soff, 0, 0));
        if (decltype(set)::value) scv1 = sc;
        else scv0 = sc;
      }
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // The first kGuessed list entries are guessed before the map row arrives, and
  // their transfers start at once: without a map (or for the token's own tile) the
  // list starts at the first block the window reaches.  A wrong guess is redone
  // below.
  int jlo = 0;
  if (p.blk && p.window > 0) {
    const int64_t lo = p.qk_delta + (int64_t)tile * p.bq - p.window + 1;   // tile's first row
    jlo = lo <= 0 ? 0 : (int)(lo / kRowsPerBlock < p.nb0 ? lo / kRowsPerBlock : p.nb0);
  }
  // a split's list part starts at its share of the dense blocks from jlo on
  const int ndguess = p.nbd > jlo ? p.nbd - jlo : 0;
  const int e0_guess = (int)((uint32_t)(ndguess * split) / (uint32_t)nsplit);
  const int n_guess = (int)((uint32_t)(ndguess * (split + 1)) / (uint32_t)nsplit) - e0_guess;   // the part's length
  auto spec = [&](int e) -> int {   // guess for the part's entry e
    return e < n_guess && jlo + e0_guess + e < p.nbd ? jlo + e0_guess + e : -1;
  };
  // KEYS issues its map row load first, so that waiting for it does not wait for
  // the rows loaded behind it (vector loads complete in order).  Its loads are
  // issued unconditionally where it matters (through buffer descriptors of size 0
  // when there is nothing to read): the compiler's wait counts assume the fewest
  // loads any path issues, so a load skipped on some path makes the common path
  // wait for everything in flight.
  const uint8_t *blkrow = p.blk ? p.blk + ((int64_t)b * p.ntiles + tile) * p.nbd : nullptr;
  int s_first = -1;
  if constexpr (KEYS) {
    const int sraw = buf_load_u8(make_rsrc(blkrow, blkrow ? (uint32_t)p.nbd : 0u), (uint32_t)tid);
    s_first = tid < p.nbd ? (blkrow ? sraw : kPartial) : 0;
  }
  if (!KEYS && (!SPLITKV || producer)) {
    for_bufs([&](auto E) {
      if (E < kGuessed && spec(E) >= 0) {
        if constexpr (SPLITKV && !FP8) {
          // (K rows first: an entry's K rows are published before its V rows)
          stage_rows(spec(E), 0xffffffffu, E, KPart{});
          stage_rows(spec(E), 0xffffffffu, E, VPart{});
        } else {
          stage_rows(spec(E), 0xffffffffu, E, BothParts{});
        }
      }
    });
  }

  // This workgroup's part of the list, entries [e0, e1), once the list has been
  // built (ndense dense entries).
  int ndense = 0, e0 = 0, e1 = 0;
  auto part_bounds = [&](int nd) __attribute__((always_inline)) {
    const int nlist = nd + (INDEXED ? p.nb1 : 0);
    // (nlist <= kListCap + kIdxCap / 32 and split < kMaxSplits: 32-bit products)
    e0 = (int)((uint32_t)(nlist * split) / (uint32_t)nsplit);
    e1 = (int)((uint32_t)(nlist * (split + 1)) / (uint32_t)nsplit);
  };
  // List entry i: key block j (dense blocks of both regions, then the gathered
  // blocks of an indexed region) and its map status.
  auto entry_at = [&](int i, int &j, int &status) {
    if (i < ndense) {
      const int e = blist[i];
      j = e & 0x3fff;
      status = e >> 14;
    } else {
      j = p.nb0 + (i - ndense);
      status = kPartial;
    }
  };

  // Start the transfers of list entry i (< nlist) into buffer pair `buf`, with the
  // entry's mask (MASKED) or unmasked.
  auto stage = [&](int i, auto buf, auto masked, auto part) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    int j, status;
    entry_at(i, j, status);
    const uint32_t vm = MASKED ? __builtin_amdgcn_readfirstlane(vmask[i & (kMaskRing - 1)]) : 0xffffffffu;
    stage_rows(__builtin_amdgcn_readfirstlane(j), vm, buf, part);
  };

  // Clear the V rows of entry i that its mask hides, among this wave's own rows
  // (its own completed transfers wrote them).
  auto clear_masked = [&](int i, auto buf) __attribute__((always_inline)) {
    if (i >= e1) return;
    const uint32_t vmi = vmask[i & (kMaskRing - 1)];
    char *vt = vtile(buf);
    if constexpr (FP8) {
      // this wave's rows are the rows of its pairs 4w..4w+3: slot q < 4 the first
      // row of pair 4w + q, slot q >= 4 the second row of pair 4w + q - 4
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int pr = 4 * w + (q & 3);
        const int rr = q < 4 ? pr : f8_second_row(pr);
        if (!((vmi >> rr) & 1u)) {
          // the row's 512 bytes, and its V scale
          if (lane < 32) *(uint4 *)(vt + f8_row_off(rr) + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
          if (lane == 0) stile(buf)[16 * w + 8 + q] = 0.f;
        }
      }
    } else {
      uint32_t hidden = (~vmi >> (RPW * w)) & ((1u << RPW) - 1u);
      while (hidden) {
        const int rr = RPW * w + __ffs(hidden) - 1;
        hidden &= hidden - 1;
        *(uint4 *)(vt + rr * kVRow + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  // The guessed first entries against the list: a wrong guess is staged again,
  // unmasked (its hidden rows are cleared once it has landed).  Returns whether any
  // entry was staged again.
  auto check_guesses = [&]() __attribute__((always_inline)) -> bool {
    bool hit[NBUF], all = true;
    for_bufs([&](auto E) {
      int j = -1, st;
      if (e1 > e0 + E) entry_at(e0 + E, j, st);
      j = __builtin_amdgcn_readfirstlane(j);
      hit[E] = e1 <= e0 + E || E >= kGuessed || j == spec(E);
      all = all && hit[E];
    });
    if (!all) {
      wait_vmcnt<0>();   // the guessed transfers land before their buffers are refilled
      for_bufs([&](auto E) {
        if (!hit[E]) stage(e0 + E, E, Unmasked{}, BothParts{});
      });
    }
    return !all;
  };

  // SPLITKV producers: their whole program.  It meets the computing waves' barriers
  // in the same order: the block list's (two per 256 map entries and a final one),
  // the first-block mask table's, the masks', entry e0's, then per entry i the
  // score exchange, a mask refill when entry i + NBUF starts a chunk, and the end of
  // the entry while another follows.  It branches off before the
  // computing waves load anything through the compiler, so that no wait of theirs
  // (nor one for registers their loads would write) lands in this path.
  if constexpr (SPLITKV) {
    if (producer) {
      // (float16: whether entry e0 + 1's V rows are staged late, and masked; set in
      // the prologue below)
      bool v_late = false;
      // An entry's K rows are published by the barrier that ends the entry before
      // it, its V rows (needed only from P.V on) by its own score exchange.  In
      // issue order: K rows of entry nx after the exchange of entry i, its V rows
      // after the end of entry i.
      auto produce16 = [&](int i, auto buf) __attribute__((always_inline)) {
        const int nx = i + NBUF;
        // entry i's V rows landed: only entry i + 1's transfers may be in flight;
        // entry e0 (guessed) and, unless staged masked, entry e0 + 1 arrived
        // unmasked: clear their hidden V rows
        if (i + 1 < e1) wait_vmcnt<2 * RPW>();
        else wait_vmcnt<0>();
        if (i == e0 || (i == e0 + 1 && !v_late)) clear_masked(i, buf);
        lds_barrier();   // score exchange of entry i: its V rows ready, K tile B free
        if (nx < e1 && (nx & (kMaskChunk - 1)) == 0) lds_barrier();   // masks of entries nx..
        if (nx < e1) stage(nx, buf, Masked{}, KPart{});
        if (i + 1 < e1) {
          // entry i + 1's K rows landed: only its V rows and the K rows of entry nx
          // may be in flight
          if (nx < e1) wait_vmcnt<2 * RPW>();
          else wait_vmcnt<RPW>();
          lds_barrier();   // end of entry i: entry i + 1's K rows ready, V tile B free
          if (nx < e1) stage(nx, buf, Masked{}, VPart{});
        }
      };
      // FP8 rows: entry nx is staged whole (kF8StageOps transfers) after the end of
      // entry i, and entry i + 1 is published whole by the end of entry i.  Entries
      // i + 2 and i + 3, where they exist, were staged after entry i + 1 (by the
      // prologue's guesses or after the ends of entries i - 2 and i - 1); counting
      // only those keeps the wait safe when a guessed entry past the list is in
      // flight too.
      auto produce8 = [&](int i, auto buf) __attribute__((always_inline)) {
        constexpr int B = decltype(buf)::value;
        const int nx = i + NBUF;
        lds_barrier();   // score exchange of entry i
        if (nx < e1 && (nx & (kMaskChunk - 1)) == 0) lds_barrier();   // masks of entries nx..
        if (i + 1 < e1) {
          const int later = (i + 3 < e1 - 1 ? i + 3 : e1 - 1) - (i + 1);
          if (later >= 2) wait_vmcnt<2 * kF8StageOps>();
          else if (later == 1) wait_vmcnt<kF8StageOps>();
          else wait_vmcnt<0>();
          // (the first NBUF entries were staged unmasked, as guessed: FP8 guesses all)
          if (i + 1 < e0 + NBUF) clear_masked(i + 1, std::integral_constant<int, (B + 1) % NBUF>{});
          lds_barrier();   // end of entry i: entry i + 1 ready, buffer B free
          if (nx < e1) stage(nx, buf, Masked{}, BothParts{});
        }
      };
      const int nbar = 2 * ((p.nbd + 255) / 256) + 1;
      for (int k = 0; k < nbar; ++k) lds_barrier();   // the block list
      lds_barrier();                                  // the first-block mask table
      ndense = nd_s;
      part_bounds(ndense);
      const bool redo = check_guesses();
      // Float16: entry e0 + 1, now known.  Its K rows go at once (unmasked; the
      // mask hides them in the scores).  Its V rows go now too (unmasked, cleared
      // once landed), except for a short list (a window's blocks) with every CU
      // busy: there the prologue is a large part of the chain, and they go (masked)
      // after entry e0's barrier, so that the barriers before it do not wait for
      // them to be issued.  (Measured, 64 sequences: a 4-block window 10.6 -> 10.0
      // us with the late V rows; 12-block lists 20.3 us with early, 20.6 with late
      // V rows; a single sequence split in 16 workgroups 11.8 early, 12.0 late.)
      const bool second = !FP8 && e0 + 1 < e1;
      v_late = gridDim.x >= (uint32_t)kNumCus && e1 - e0 <= kLateVMaxEntries;
      if constexpr (!FP8) {
        if (second) {
          stage(e0 + 1, std::integral_constant<int, 1>{}, Unmasked{}, KPart{});
          if (!v_late) stage(e0 + 1, std::integral_constant<int, 1>{}, Unmasked{}, VPart{});
        }
      }
      lds_barrier();   // masks visible
      if constexpr (FP8) {
        // entry e0 landed: only the guessed entries after it may be in flight (after
        // a redo the order is not known: wait for everything, as for an empty list)
        if (redo || e0 >= e1) wait_vmcnt<0>();
        else if (spec(3) >= 0) wait_vmcnt<3 * kF8StageOps>();
        else if (spec(2) >= 0) wait_vmcnt<2 * kF8StageOps>();
        else if (spec(1) >= 0) wait_vmcnt<kF8StageOps>();
        else wait_vmcnt<0>();
        clear_masked(e0, std::integral_constant<int, 0>{});
        lds_barrier();   // entry e0 ready
      } else {
        // entry e0's K rows landed: only its V rows (after a redo, which stages the
        // entry whole: none of its rows) and entry e0 + 1's rows may be in flight
        const int later = second ? (v_late ? RPW : 2 * RPW) : 0;   // e0 + 1's transfers
        if (redo) {
          if (later == 2 * RPW) wait_vmcnt<2 * RPW>();
          else if (later == RPW) wait_vmcnt<RPW>();
          else wait_vmcnt<0>();
        } else {
          if (later == 2 * RPW) wait_vmcnt<3 * RPW>();
          else if (later == RPW) wait_vmcnt<2 * RPW>();
          else wait_vmcnt<RPW>();
        }
        lds_barrier();   // entry e0's K rows ready
        if (second && v_late) stage(e0 + 1, std::integral_constant<int, 1>{}, Masked{}, VPart{});
      }
      for (int i = e0; i < e1; i += NBUF) {
        for_bufs([&](auto E) {
          if (i + E < e1) {
            if constexpr (FP8) produce8(i + E, E);
            else produce16(i + E, E);
          }
        });
      }
      wait_vmcnt<0>();   // nothing in flight when the workgroup ends
      return;
    }
  }

  // validity arrays of this sequence (size 0 when absent: every load out of range)
  const rsrc_t rb0 = make_rsrc(p.valid0 + (int64_t)b * p.valid0_sb, p.valid0 ? (uint32_t)p.n0 : 0u);
  const rsrc_t rb1 = make_rsrc(p.valid1 + (int64_t)b * p.valid1_sb, p.valid1 ? (uint32_t)p.n1 : 0u);
  // Row r of key block j for this token: `ok` = visible by the arithmetic rules
  // (inside the region, the window, a used index entry); off0 / off1 = the
  // validity byte that must also be nonzero (out of range when none applies).
  // Gathered blocks read the index list, so they are resolved only after it is
  // in LDS.
  auto row_rule = [&](int j, int r, int &ok, uint32_t &off0, uint32_t &off1)
      __attribute__((always_inline)) {
    off0 = off1 = kOutOfRange;
    if (j < p.nb0) {
      const int row = j * kRowsPerBlock + r;
      bool v = row < p.n0;
      if (p.window > 0) {
        const int64_t d = p.qk_delta + t - row;
        v = v && d >= 0 && d < p.window;
      }
      ok = v;
      if (p.valid0 && row < p.n0) off0 = row;
    } else {
      const int e = (j - p.nb0) * kRowsPerBlock + r;
      const int c = INDEXED ? ((e < p.r1_k) ? idx_s[e] : -1) : e;
      const bool v = c >= 0 && c < p.n1;
      ok = v;
      if (p.valid1 && v) off1 = c;
    }
  };
  // The masks of the first kTable dense blocks (one row per thread) are loaded
  // together with the map row, so short lists need no second round trip.
  const int tj = tid >> 5;
  int tok = 0;
  uint32_t toff0 = kOutOfRange, toff1 = kOutOfRange;
  if (tj < p.nbd) row_rule(tj, tid & 31, tok, toff0, toff1);
  // (a region without a validity array needs no load: a load, even out of range,
  // is a full round trip queued behind the block transfers)
  // (KEYS loads both unconditionally: the loads go out before the rows, and a
  // conditional load makes the compiler wait for everything in flight)
  const int tv0 = (KEYS || p.valid0) ? buf_load_u8(rb0, toff0) : 0;
  const int tv1 = (KEYS || p.valid1) ? buf_load_u8(rb1, toff1) : 0;
  // The first 512 index entries into registers before Q and the rows are loaded
  // (loads complete in order: waiting for these then waits for nothing behind them)
  int ia = -1, ib = -1;
  if (INDEXED) {
    const rsrc_t ri = make_rsrc(p.idx + ((int64_t)b * p.T + t) * p.r1_k, 4u * (uint32_t)p.r1_k);
    const int va = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, 4u * tid, 0, 0);
    const int vb = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, 4u * (tid + 256), 0, 0);
    ia = tid < p.r1_k ? va : -1;
    ib = tid + 256 < p.r1_k ? vb : -1;
  }

  // The computing waves' map row (its first 256 entries), for the same reason
  // (KEYS loaded it before its rows)
  if constexpr (!KEYS) {
    const int sraw = buf_load_u8(make_rsrc(blkrow, blkrow ? (uint32_t)p.nbd : 0u), (uint32_t)tid);
    s_first = tid < p.nbd ? (blkrow ? sraw : kPartial) : 0;
  }

  // Q^T operand fragments: head h, dims d0 + 32ks + 8g .. +7 (F8S: the two E4M3
  // terms of head h, dims 128c + 32g .. +31 in chunk c, and the head's factor)
  half8 qf[F8S ? 1 : NKS];
  int8v qhi[NQC], qlo[NQC];
  float qsc = 1.f;
  half8 qf2[HT == 2 ? NKS : 1];   // kDimsWide: Q^T fragments of heads h + 16
  u32x4 qst[KEYS ? 4 : 1];
  if constexpr (KEYS) {
    // Q rows of heads 16hg + 4w .. +3, one contiguous 1 KiB row per load (they reach
    // the operand registers through LDS: operand-shaped loads touch 16 rows each)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      qst[q] = *(__attribute__((address_space(1))) const u32x4 *)(
          uniform_ptr(p.q + b * p.q_sb + t * p.q_st + (int64_t)(hg * HG + 4 * w + q) * p.q_sh) + lane16);
    // each wave's first two units (u = w and w + 4: entries u / UPE, unit u % UPE
    // within its entry) as guessed
    {
      const HalfRows hr = spec(w / UPE) >= 0 ? rows_of(spec(w / UPE), w % UPE) : no_rows();
      load_k(hr, Set0{});
      load_v(hr, Set0{});
    }
    // Q rows into the first wave tile (free until the key loop starts)
#pragma unroll
    for (int q = 0; q < 4; ++q) *(u32x4 *)(wt + (4 * w + q) * kKRow + lane16) = qst[q];
    if constexpr (NSET == 2) {
      const HalfRows hr = spec((w + 4) / UPE) >= 0 ? rows_of(spec((w + 4) / UPE), w % UPE) : no_rows();
      load_k(hr, Set1{});
      load_v(hr, Set1{});
    }
  } else {
    const char *qrow = p.q + b * p.q_sb + t * p.q_st + (int64_t)h * p.q_sh;
    if constexpr (F8S) {
      half8 qv[NQC][4];
#pragma unroll
      for (int c = 0; c < NQC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[c][j] = *(const half8 *)(qrow + 2 * (d0 + 128 * c + 32 * g + 8 * j));
      // max |q| over the head's dims of this wave: this lane's elements, then the
      // head's four lanes
      half2v mx = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
      for (int c = 0; c < NQC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            mx = __builtin_elementwise_max(mx, __builtin_elementwise_abs(half2v{qv[c][j][e], qv[c][j][e + 1]}));
      float amax = fmaxf((float)mx[0], (float)mx[1]);
      amax = xor_max(amax, 16);
      amax = xor_max(amax, 32);
      qsc = split_e4m3(qv, amax, qhi, qlo);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const half8 *)(qrow + 2 * (d0 + 32 * ks + 8 * g));
    }
    if constexpr (HT == 2) {
      const char *qrow2 = qrow + 16 * p.q_sh;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf2[ks] = *(const half8 *)(qrow2 + 2 * (d0 + 32 * ks + 8 * g));
    }
  }
  if (INDEXED) {
    // the token's index list; entries up to the end of its last 32-entry block
    // that lie past r1_k read as unused (-1)
    const int32_t *src = p.idx + ((int64_t)b * p.T + t) * p.r1_k;
    const int padded = p.nb1 * kRowsPerBlock;
    if (tid < padded) idx_s[tid] = ia;
    if (tid + 256 < padded) idx_s[tid + 256] = ib;
    for (int e = tid + 512; e < padded; e += 256) idx_s[e] = e < p.r1_k ? src[e] : -1;
  }
  ndense = build_block_list<256>(blkrow, p.nbd, blist, cnt, s_first);   // ends with a barrier
  {
    const bool vis = tok && (toff0 == kOutOfRange || tv0 != 0) && (toff1 == kOutOfRange || tv1 != 0);
    const uint64_t bal = __ballot(vis);
    if ((lane & 31) == 0) dmask[tj] = (uint32_t)(bal >> (lane & 32));
  }
  if (SPLITKV && tid == 0) nd_s = ndense;
  lds_barrier();
  part_bounds(ndense);

  // Visibility masks of list entries [c0, c0 + n) into the ring, K rounds of 8
  // entries per batch of loads: half-wave (w, lane >> 5) takes entry 8k + 2w + (lane >> 5)
  // of a round, lane & 31 its row.  Dense blocks below kTable come from the table.
  // Every thread must call it (ballots, LDS writes).
  auto build_masks = [&](int c0, int n, auto rounds) __attribute__((always_inline)) {
    constexpr int K = decltype(rounds)::value;
    const int r = lane & 31, half = lane >> 5;
    for (int e0 = 0; e0 < n; e0 += 8 * K) {
      int ok[K], full[K], tab[K];
      uint32_t off0[K], off1[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int el = e0 + 8 * k + 2 * w + half;
        ok[k] = 0;
        full[k] = 0;
        tab[k] = -1;
        off0[k] = off1[k] = kOutOfRange;
        if (el < n) {
          int j, status;
          entry_at(c0 + el, j, status);
          full[k] = status == kFull;
          if (j < kTable && !(INDEXED && j >= p.nb0)) tab[k] = j;
          else if (!full[k]) row_rule(j, r, ok[k], off0[k], off1[k]);
        }
      }
      // the validity bytes: loaded and used inside the branch of a region that has
      // them, so that the wait for them is there too (a wait after the branch
      // would also wait for every row transfer in flight when there is none)
      bool okv[K];
#pragma unroll
      for (int k = 0; k < K; ++k) okv[k] = ok[k];
      if (p.valid0) {
        int vb[K];
#pragma unroll
        for (int k = 0; k < K; ++k) vb[k] = buf_load_u8(rb0, off0[k]);
#pragma unroll
        for (int k = 0; k < K; ++k) okv[k] = okv[k] && (off0[k] == kOutOfRange || vb[k] != 0);
      }
      if (p.valid1) {
        int vb[K];
#pragma unroll
        for (int k = 0; k < K; ++k) vb[k] = buf_load_u8(rb1, off1[k]);
#pragma unroll
        for (int k = 0; k < K; ++k) okv[k] = okv[k] && (off1[k] == kOutOfRange || vb[k] != 0);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int el = e0 + 8 * k + 2 * w + half;
        const bool vis = okv[k];
        const uint64_t bal = __ballot(vis);
        if (el < n && r == 0)
          vmask[(c0 + el) & (kMaskRing - 1)] =
              full[k] ? 0xffffffffu : (tab[k] >= 0 ? dmask[tab[k]] : (uint32_t)(bal >> (32 * half)));
      }
    }
  };

  // The masks of the part's first entries (up to `cap` of them), in as few rounds of
  // eight entries as the list needs: the unrolled rounds of a long batch cost about
  // 0.8 us when the list has only a few entries.
  auto build_masks_first = [&](int cap) __attribute__((always_inline)) {
    const int n = e1 - e0 < cap ? e1 - e0 : cap;
    if (n <= 8) build_masks(e0, n, std::integral_constant<int, 1>{});
    else if (n <= 16) build_masks(e0, n, std::integral_constant<int, 2>{});
    else if (n <= 32) build_masks(e0, n, std::integral_constant<int, 4>{});
    else build_masks(e0, n, std::integral_constant<int, 8>{});
  };



  floatx4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  // kDimsWide: output, running max and sum of the second head tile
  floatx4 o2[HT == 2 ? NDT : 1];
#pragma unroll
  for (int dt = 0; dt < (HT == 2 ? NDT : 1); ++dt) o2[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY, l2 = 0.f;
  // FOLDV: the V scales' running power-of-two factor vfac = 2^-vexp (0 until a
  // block has a nonzero V scale), and its update for a block whose V row scales
  // (this lane's eight slot rows) are in vr: afterwards vr holds the folded factors
  // sv vfac, and the result is the factor (a power of two, 1 if unchanged) the
  // outputs must take, which the softmax applies with its own rescale (vfold_update
  // only moves the factor).  The update sits on each block's chain from its scales
  // to P': about 0.5 us of a 4-block FP8 decode and 3 % of the FP8 prefill, the
  // same wherever it was placed (at the block's start, behind a vote, on scalar
  // registers) -- the price of full precision at any V magnitude.
  int vexp = 0;
  bool vset = false;
  auto vfold_update = [&](const float (&vr)[8]) __attribute__((always_inline)) -> float {
    // the block's largest V scale: the four lane groups hold its 32 rows (the
    // lanes of a group the same eight), as the score max does
    float mx = fmaxf(fmaxf(fmaxf(vr[0], vr[1]), fmaxf(vr[2], vr[3])), fmaxf(fmaxf(vr[4], vr[5]), fmaxf(vr[6], vr[7])));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    // mx = f 2^e with f in [0.5, 1), e taken within [-125, 126] so that 2^-e and 2^e
    // are normal floats (a subnormal mx counts as 2^-125; a finite mx of 2^126 or
    // more gives mx vfac < 4).  A new factor 2^-e when none is set yet, or when mx
    // vfac may pass 2^7 (e - vexp > 7), so that P' < 2^8 * 2^7.  Selects only: a
    // branch here makes the wave wait for the scales before anything else.
    const uint32_t mb = __float_as_uint(mx);
    int e = (int)((mb >> 23) & 0xffu) - 126;
    e = e > -125 ? (e < 126 ? e : 126) : -125;
    const bool upd = (mb != 0u) & (!vset | (e - vexp > 7));
    // the outputs' factor 2^(vexp - e) (at least 2^-126: blocks so much smaller
    // than the new one no longer matter)
    const int dd = vexp - e;
    const int d = (upd & vset) ? (dd > -126 ? dd : -126) : 0;
    vexp = upd ? e : vexp;
    vset = vset | upd;
    return __uint_as_float((uint32_t)(127 + d) << 23);
  };
  auto vfold = [&](float (&vr)[8]) __attribute__((always_inline)) -> float {
    const float r = vfold_update(vr);
    const float vfac = vset ? __uint_as_float((uint32_t)(127 - vexp) << 23) : 0.f;
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) vr[i2] *= vfac;
    return r;
  };

  // transpose-read roles: this lane points at row slot_row(g, e) of the V tile,
  // 4 dims starting at 16dt + 4a, for the lanes 16g + 4a + (0..3) to receive
  // (ds_read_b64_tr_b16 hands element b of lane 16g + 4e + a to lane 16g + 4a + b)
  const int tr_e = (lane >> 2) & 3, tr_a = lane & 3;
  const int tr_r0 = 4 * g + tr_e;   // slot rows 0-3 of group g; rows 16 + ... for slots 4-7

  if constexpr (KEYS) {
    // ---- KEYS: wave w consumes units u = w, w + 4, ... of entries [e0, e1)
    // (float16: 16 K rows kKRow apart, then 16 V rows kVRow apart; FP8: the K tile
    // and the V tile of a block in pair order, then 32 K scales and 32 V scales)
    char *ktw = wt + w * kWaveTile;
    char *vtw = ktw + (FP8 ? kF8Tile : 16 * kKRow);
    float *sct = (float *)(ktw + 2 * kF8Tile);
    const int nh = UPE * (e1 - e0);
    // the guessed first two units are loaded again when the list says otherwise
    auto recheck = [&](int e, auto set) __attribute__((always_inline)) {
      if (e0 + e < e1) {
        int j, st;
        entry_at(e0 + e, j, st);
        j = __builtin_amdgcn_readfirstlane(j);
        if (j != spec(e)) {
          const HalfRows hr = rows_of(j, w % UPE);
          load_k(hr, set);
          load_v(hr, set);
        }
      }
    };
    recheck(w / UPE, Set0{});
    if constexpr (NSET == 2) recheck((w + 4) / UPE, Set1{});
    // Q^T operand fragments (head h, dims 32ks + 8g .. +7) from the Q rows in LDS
    // (written before the list barrier; read before the barrier after the masks)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const half8 *)(wt + c16 * kKRow + 64 * ks + 16 * g);
    // masks of the first two chunks of entries (the whole ring)
    build_masks_first(kMaskRing);
    lds_barrier();   // masks visible
    // Round r: wave w takes unit 4r + w, i.e. entries e0 + 4r / UPE .. (two entries
    // of half-blocks, or four blocks).  Every kMaskChunk entries all waves meet and
    // fill the ring slots of the chunk they have left with the masks of the chunk
    // after the next.
    const int nrounds = (nh + 3) >> 2;
    // Rounds in which every wave has a half-block two rounds on ("steady") issue
    // their loads unconditionally; the last rounds test for them.
    auto round = [&](int r, auto set, auto steady) __attribute__((always_inline)) {
      constexpr int S = decltype(set)::value;
      constexpr bool STEADY = decltype(steady)::value;
      u32x4 *stk = (NSET == 2 && S) ? stk1 : stk0;
      u32x4 *stv = (NSET == 2 && S) ? stv1 : stv0;
      constexpr int kRoundsPerChunk = kMaskChunk * UPE / 4;
      if (r > 0 && (r & (kRoundsPerChunk - 1)) == 0) {
        const int c0 = e0 + 4 * r / UPE + kMaskChunk;
        lds_barrier();   // every wave is done with the entries below e0 + 4r / UPE
        if (c0 < e1) {
          build_masks(c0, e1 - c0 < kMaskChunk ? e1 - c0 : kMaskChunk, std::integral_constant<int, 1>{});
          lds_barrier();
        }
      }
      const int u = 4 * r + w;
      if (!STEADY && u >= nh) return;
      const int hf = u % UPE;
      const uint32_t vmw = __builtin_amdgcn_readfirstlane(vmask[(e0 + u / UPE) & (kMaskRing - 1)]);
      const uint32_t vm = FP8 ? vmw : (vmw >> (16 * hf)) & 0xffffu;
      // staged K rows -> this wave's K tile (FP8: and the K scales); the K rows of
      // the wave's unit two rounds on start moving into the same staging set
      if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < 16; ++q) *(u32x4 *)(ktw + q * kF8Pair + lane16) = stk[q];
        if (lane < 32) sct[lane] = S ? sck1 : sck0;
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) *(u32x4 *)(ktw + q * kKRow + lane16) = stk[q];
      }
      const bool more = STEADY || u + 4 * NSET < nh;
      HalfRows nx;
      if (STEADY || more) {
        int j, st;
        entry_at(e0 + (u + 4 * NSET) / UPE, j, st);
        nx = rows_of(__builtin_amdgcn_readfirstlane(j), (u + 4 * NSET) % UPE);
        load_k(nx, set);
      }
      // S^T = K Q^T over the 512 dims, K reads KPD steps ahead: float16, one tile of
      // 16 keys x 16 heads; FP8, two tiles (rows c16 and 16 + c16 of the block)
      floatx4 sacc = {0.f, 0.f, 0.f, 0.f}, sacc1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
        const char *krow0 = ktw + f8_row_off(c16) + 8 * g;
        const char *krow1 = ktw + f8_row_off(16 + c16) + 8 * g;
        uint2 ka[KPD], kb[KPD];
#pragma unroll
        for (int u2 = 0; u2 < KPD; ++u2) {
          ka[u2] = *(const uint2 *)(krow0 + 32 * u2);
          kb[u2] = *(const uint2 *)(krow1 + 32 * u2);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          sacc = mfma16(e4m3x8_to_half8(ka[ks % KPD]), qf[ks], sacc);
          sacc1 = mfma16(e4m3x8_to_half8(kb[ks % KPD]), qf[ks], sacc1);
          if (ks + KPD < NKS) {
            ka[ks % KPD] = *(const uint2 *)(krow0 + 32 * (ks + KPD));
            kb[ks % KPD] = *(const uint2 *)(krow1 + 32 * (ks + KPD));
          }
          __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMAs, then the reads they free
        }
      } else {
        const char *krow = ktw + c16 * kKRow + 16 * g;
        uint4 ka[KPD];
#pragma unroll
        for (int u2 = 0; u2 < KPD; ++u2) ka[u2] = *(const uint4 *)(krow + 64 * u2);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          sacc = mfma16(*(const half8 *)&ka[ks % KPD], qf[ks], sacc);
          if (ks + KPD < NKS) ka[ks % KPD] = *(const uint4 *)(krow + 64 * (ks + KPD));
          __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMA, then the read it frees
        }
      }
      // staged V rows -> this wave's V tile, the rows the mask hides as zeros (FP8:
      // with zero scales); the next unit's V rows start moving
      if constexpr (FP8) {
        // transfer q: lanes 0-31 row q, lanes 32-63 row f8_second_row(q)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rq = lane < 32 ? q : f8_second_row(q);
          *(u32x4 *)(vtw + q * kF8Pair + lane16) = ((vm >> rq) & 1u) ? stv[q] : u32x4{0u, 0u, 0u, 0u};
        }
        if (lane >= 32) sct[lane] = ((vm >> (lane & 31)) & 1u) ? (S ? scv1 : scv0) : 0.f;
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          *(u32x4 *)(vtw + q * kVRow + lane16) = ((vm >> q) & 1u) ? stv[q] : u32x4{0u, 0u, 0u, 0u};
      }
      if (STEADY || more) load_v(nx, set);
      if constexpr (FP8) {
        // online softmax: this lane holds rows slot_row(g, 0..7) of head h; K row
        // scales of slot rows 4g..4g+3 and 16+4g..16+4g+3
        const float4 klo = *(const float4 *)(sct + 4 * g);
        const float4 khi = *(const float4 *)(sct + 16 + 4 * g);
        const float kq[8] = {klo.x, klo.y, klo.z, klo.w, khi.x, khi.y, khi.z, khi.w};
        float sv[8];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          sv[i2] = sacc[i2] * (p.scale_log2 * kq[i2]);
          sv[4 + i2] = sacc1[i2] * (p.scale_log2 * kq[4 + i2]);
        }
        if (vm != 0xffffffffu) {
          const uint32_t sm = slot_mask(vm, g);
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2)
            if (!((sm >> i2) & 1u)) sv[i2] = -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int i2 = 1; i2 < 8; ++i2) mx = fmaxf(mx, sv[i2]);
        mx = xor_max(mx, 16);
        mx = xor_max(mx, 32);
        const bool grow = mx > m + kRescaleSlack;
        const float mref = grow ? mx : m;
        const float msafe = (mref == -INFINITY) ? 0.f : mref;
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);
        // the V rows' scales of the same slot rows, folded into P
        const float4 vlo = *(const float4 *)(sct + 32 + 4 * g);
        const float4 vhi = *(const float4 *)(sct + 48 + 4 * g);
        float vr[8] = {vlo.x, vlo.y, vlo.z, vlo.w, vhi.x, vhi.y, vhi.z, vhi.w};
        const float vrs = vfold(vr);
        half8 pf;
        float psum = 0.f;
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          const float e = __builtin_amdgcn_exp2f(sv[i2] - msafe);
          pf[i2] = (_Float16)(e * vr[i2]);
          psum += e;
        }
        l = alpha * l + psum;
        m = mref;
        if (__ballot(grow || vrs != 1.f)) {
          const float f = alpha * vrs;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= f;
        }
        // O^T += V^T P^T, 32 keys per MFMA: the 8-bit transpose read hands lane
        // 16g + c dim 16dt + c of its group's eight slot rows (this lane supplies
        // row slot_row(g, (lane & 15) >> 1), dims 16dt + 8(lane & 1) .. +7)
        const int trk = (lane & 15) >> 1;
        const int trow = trk < 4 ? 4 * g + trk : 16 + 4 * g + (trk - 4);
        const lds_char *vsrc = (const lds_char *)(__attribute__((address_space(3))) const void *)vtw +
                               f8_row_off(trow) + 8 * (lane & 1);
        auto vload = [&](int dt) __attribute__((always_inline)) -> uint2 {
          const int2v rv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) int2v *)(vsrc + 16 * dt));
          return make_uint2((uint32_t)rv.x, (uint32_t)rv.y);
        };
        uint2 vq[VPD];
#pragma unroll
        for (int u2 = 0; u2 < VPD; ++u2) vq[u2] = vload(u2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          o[dt] = mfma16(e4m3x8_to_half8(vq[dt % VPD]), pf, o[dt]);
          if (dt + VPD < NDT) vq[dt % VPD] = vload(dt + VPD);
          __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMA, then the read it frees
        }
      } else {
        // online softmax: this lane holds keys 4g .. 4g+3 of head h
        float sv[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          sv[i2] = sacc[i2] * p.scale_log2;
          if (!((vm >> (4 * g + i2)) & 1u)) sv[i2] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = xor_max(mx, 16);
        mx = xor_max(mx, 32);
        const bool grow = mx > m + kRescaleSlack;
        const float mref = grow ? mx : m;
        const float msafe = (mref == -INFINITY) ? 0.f : mref;
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);
        half4 pf;
        float psum = 0.f;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
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
        // O^T += V^T P^T, 16 keys per MFMA; one transpose read per output tile hands
        // this lane dim 16dt + (lane & 15) of rows 4g .. 4g+3
        const lds_char *vsrc = (const lds_char *)(__attribute__((address_space(3))) const void *)vtw +
                               (4 * g + tr_e) * kVRow + 8 * tr_a;
        auto vload = [&](int dt) __attribute__((always_inline)) -> half4 {
          return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                               (__attribute__((address_space(3))) short4_t *)(vsrc + 32 * dt)));
        };
        half4 vq[VPD];
#pragma unroll
        for (int u2 = 0; u2 < VPD; ++u2) vq[u2] = vload(u2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          o[dt] = mfma16k16(vq[dt % VPD], pf, o[dt]);
          if (dt + VPD < NDT) vq[dt % VPD] = vload(dt + VPD);
          __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMA, then the read it frees
        }
      }
    };
    using Steady = std::integral_constant<bool, true>;
    using Tail = std::integral_constant<bool, false>;
    // steady rounds: 4r + 3 + 4 NSET < nh (a multiple of NSET of them), then the rest
    constexpr int kAhead = 3 + 4 * NSET;
    const int rsteady = (nh > kAhead ? (nh - kAhead + 3) >> 2 : 0) & ~(NSET - 1);
    int r = 0;
    if constexpr (NSET == 2) {
      for (; r < rsteady; r += 2) {
        round(r, Set0{}, Steady{});
        round(r + 1, Set1{}, Steady{});
      }
      for (; r < nrounds; r += 2) {
        round(r, Set0{}, Tail{});
        if (r + 1 < nrounds) round(r + 1, Set1{}, Tail{});
      }
    } else {
      for (; r < rsteady; ++r) round(r, Set0{}, Steady{});
      for (; r < nrounds; ++r) round(r, Set0{}, Tail{});
    }

    // ---- merge the four waves: with M = max_w m_w and f_w = 2^(m_w - M), the
    // result is sum_w f_w O_w / sum_w f_w l_w (zero when no wave saw a row)
    float lw = l;
    lw = xor_sum(lw, 16);
    lw = xor_sum(lw, 32);
    lds_barrier();   // every wave is done with its tiles
    if (g == 0) {
      mlw[w * 16 + c16] = m;
      mlw[64 + w * 16 + c16] = lw;
    }
    lds_barrier();
    float mall = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mall = fmaxf(mall, mlw[ww * 16 + c16]);
    float lall = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = mlw[ww * 16 + c16];
      lall += (mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mall)) * mlw[64 + ww * 16 + c16];
    }
    // Each wave's share of the normalised output, so that no sum exceeds the V
    // rows' own magnitude: 2^(m - mall) / lall, times this wave's V factor (FP8; a
    // wave whose V scales were all zero has O = 0).
    const float f = m == -INFINITY || !(lall > 0.f)
                        ? 0.f
                        : (FP8 ? (vset ? __uint_as_float((uint32_t)(127 + vexp) << 23) : 0.f) : 1.f) *
                              (__builtin_amdgcn_exp2f(m - mall) / lall);
    // wave w finishes output tiles 8w .. 8w+7 (dims 128w .. 128w+127); the others
    // hand it theirs through LDS: xo[wave][tile][lane].  Instantiated per wave
    // index, so that the tile selection is resolved at compile time.
    floatx4 *xo = (floatx4 *)wt;
    floatx4 acc[8];
    auto merge = [&](auto wc) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        if ((dt >> 3) != W) xo[(W * NDT + dt) * 64 + lane] = o[dt] * f;
      lds_barrier();
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = o[8 * W + k] * f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        if (ww != W) {
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] += xo[(ww * NDT + 8 * W + k) * 64 + lane];
        }
    };
    if (w == 0) merge(std::integral_constant<int, 0>{});
    else if (w == 1) merge(std::integral_constant<int, 1>{});
    else if (w == 2) merge(std::integral_constant<int, 2>{});
    else merge(std::integral_constant<int, 3>{});
    if constexpr (PARTS) {
      // partial record of this split: its normalised O, then the maxima and the sums
      char *rec = p.ws + ((int64_t)L * nsplit + split) * kSplitRecord;
      store_acc_rows<8, false>(rec + 512 * w, 512 * 4, acc, 1.f, lane);
      if (w == 0 && g == 0) {
        ((float *)(rec + 16 * 512 * 4))[c16] = mall;
        ((float *)(rec + 16 * 512 * 4))[16 + c16] = lall;
      }
      return;
    }
    store_acc_rows<8, true>(p.o + b * p.o_sb + t * p.o_st + (int64_t)(hg * HG) * p.o_sh + 512 * w, p.o_sh, acc,
                            1.f, lane);
    return;
  }

  // Pipeline: blocks i+1 .. i+NBUF are in flight while block i is consumed.
  //   prologue: entry e -> buffer e unmasked for e < NBUF (already in flight when
  //             guessed right), meanwhile compute the masks of the first entries;
  //             clear the hidden rows of those entries
  //   block i (buffer B = i mod NBUF): consume from B; barrier (B free); stage
  //             i+NBUF -> B masked; wait for this wave's transfers of i+1; barrier
  //             (publishes i+1)
  // SPLITKV: the producers stage; the computing waves only meet them at barriers,
  //   the score exchange of block i (which publishes its V rows, and after which
  //   its K tile takes entry i + 2) and the end of block i (which publishes entry
  //   i + 1's K rows, and after which block i's V tile takes entry i + 2).  Block
  //   e0's K rows are published as soon as they have landed.
  if constexpr (SPLITKV) {
    build_masks_first(kMaskChunk);
    lds_barrier();   // masks visible
    lds_barrier();   // entry e0's K rows ready (the producers publish them)
  } else {
    check_guesses();
    build_masks_first(kMaskChunk);
    wait_vmcnt<0>();
    lds_barrier();   // masks visible
    for_bufs([&](auto E) { clear_masked(e0 + E, E); });
    lds_barrier();   // blocks 0 and 1 ready
  }

  // (buffer B below: `buf`, the entry's tile buffer)
  auto iteration = [&](int i, auto buf) __attribute__((always_inline)) {
    // ---- S^T = K Q^T over this wave's head dims; operand reads run KPD steps ahead
    // (kDimsWide: t0, t1 for the second head tile, from the same K operands)
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    floatx4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    const char *ktc = ktile(buf), *vtc = vtile(buf);
    uint32_t kdep = 0;   // FP8: a register of the last K operand read (see the scale tile below)
    if constexpr (F8S) {
      // rows c16 and 16 + c16, dims 128c + 32g .. +31: 32 codes per operand; each K
      // operand meets the two Q terms (lo weighted 2^-4 by the B-side scale)
      const char *krow0 = ktc + f8_row_off(c16) + d0 + 32 * g;
      const char *krow1 = ktc + f8_row_off(16 + c16) + d0 + 32 * g;
      auto kload = [&](const char *row, int c) __attribute__((always_inline)) -> int8v {
        const uint4 x = *(const uint4 *)(row + 128 * c), y = *(const uint4 *)(row + 128 * c + 16);
        return int8v{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      };
      constexpr int KP8 = 1;   // chunks of K operands read ahead
      int8v ka[KP8], kb[KP8];
#pragma unroll
      for (int u = 0; u < KP8; ++u) {
        ka[u] = kload(krow0, u);
        kb[u] = kload(krow1, u);
      }
#pragma unroll
      for (int c = 0; c < NQC; ++c) {
        s0 = mfma_e4m3<127>(ka[c % KP8], qhi[c], s0);
        s1 = mfma_e4m3<127>(kb[c % KP8], qhi[c], s1);
        s0 = mfma_e4m3<123>(ka[c % KP8], qlo[c], s0);
        s1 = mfma_e4m3<123>(kb[c % KP8], qlo[c], s1);
        if (c + KP8 < NQC) {
          ka[c % KP8] = kload(krow0, c + KP8);
          kb[c % KP8] = kload(krow1, c + KP8);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMAs, then the reads they free
      }
      s0 *= qsc;   // the Q terms' factor
      s1 *= qsc;
    } else if constexpr (FP8) {
      // rows c16 and 16 + c16, dims d0 + 32ks + 8g .. +7: 8 codes
      const char *krow0 = ktc + f8_row_off(c16) + d0 + 8 * g;
      const char *krow1 = ktc + f8_row_off(16 + c16) + d0 + 8 * g;
      uint2 ka[KPD], kb[KPD];
#pragma unroll
      for (int u = 0; u < KPD; ++u) {
        ka[u] = *(const uint2 *)(krow0 + 32 * u);
        kb[u] = *(const uint2 *)(krow1 + 32 * u);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const half8 kah = e4m3x8_to_half8(ka[ks % KPD]), kbh = e4m3x8_to_half8(kb[ks % KPD]);
        s0 = mfma16(kah, qf[ks], s0);
        s1 = mfma16(kbh, qf[ks], s1);
        if constexpr (HT == 2) {
          t0 = mfma16(kah, qf2[ks], t0);
          t1 = mfma16(kbh, qf2[ks], t1);
        }
        if (ks + KPD < NKS) {
          ka[ks % KPD] = *(const uint2 *)(krow0 + 32 * (ks + KPD));
          kb[ks % KPD] = *(const uint2 *)(krow1 + 32 * (ks + KPD));
        }
        __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMAs, then the reads they free
      }
      kdep = kb[(NKS - 1) % KPD].y;
    } else {
      const char *krow0 = ktc + c16 * kKRow + 2 * (d0 + 8 * g), *krow1 = krow0 + 16 * kKRow;
      uint4 ka[KPD], kb[KPD];
#pragma unroll
      for (int u = 0; u < KPD; ++u) {
        ka[u] = *(const uint4 *)(krow0 + 64 * u);
        kb[u] = *(const uint4 *)(krow1 + 64 * u);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s0 = mfma16(*(const half8 *)&ka[ks % KPD], qf[ks], s0);
        s1 = mfma16(*(const half8 *)&kb[ks % KPD], qf[ks], s1);
        if constexpr (HT == 2) {
          t0 = mfma16(*(const half8 *)&ka[ks % KPD], qf2[ks], t0);
          t1 = mfma16(*(const half8 *)&kb[ks % KPD], qf2[ks], t1);
        }
        if (ks + KPD < NKS) {
          ka[ks % KPD] = *(const uint4 *)(krow0 + 64 * (ks + KPD));
          kb[ks % KPD] = *(const uint4 *)(krow1 + 64 * (ks + KPD));
        }
        __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMAs, then the reads they free
      }
    }
    if constexpr (DIMS) {
      // partial tiles meet in LDS; every wave adds them in the same order
      constexpr int XT = 2 * HT;   // partial tiles per wave
      xs[(w * XT + 0) * 64 + lane] = s0;
      xs[(w * XT + 1) * 64 + lane] = s1;
      if constexpr (HT == 2) {
        xs[(w * XT + 2) * 64 + lane] = t0;
        xs[(w * XT + 3) * 64 + lane] = t1;
      }
      lds_barrier();
      s0 = xs[0 * 64 + lane];
      s1 = xs[1 * 64 + lane];
      if constexpr (HT == 2) {
        t0 = xs[2 * 64 + lane];
        t1 = xs[3 * 64 + lane];
      }
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        s0 += xs[(ww * XT + 0) * 64 + lane];
        s1 += xs[(ww * XT + 1) * 64 + lane];
        if constexpr (HT == 2) {
          t0 += xs[(ww * XT + 2) * 64 + lane];
          t1 += xs[(ww * XT + 3) * 64 + lane];
        }
      }
    }
    const int nx = i + NBUF;   // the entry buffer B takes next
    if constexpr (SPLITKV) {
      // the exchange barrier ended every wave's K reads: the producers stage entry
      // nx into the K tile, after the next chunk of masks when nx starts one
      // (entries i and i + 1 sit in the other half of the ring)
      if (nx < e1 && (nx & (kMaskChunk - 1)) == 0) {
        const int n = e1 - nx;
        build_masks(nx, n < kMaskChunk ? n : kMaskChunk, std::integral_constant<int, 1>{});
        lds_barrier();
      }
    }
    // ---- online softmax: this lane holds rows slot_row(g, 0..7) of head h (and,
    // kDimsWide, of head h + 16): the scores' factors (softmax scale, and FP8: the
    // K rows' scales), then one pass per head tile
    float kq[8];
    // FP8: the scale tile's address is tied to the last K operand read (DIMS), so
    // that its loads and the V factor below go out after the score phase's reads,
    // while its last MFMAs run (scheduled at the top of the block, their wait held
    // back the K reads), or to the scores (HEADS: during the last MFMAs their
    // registers push the query terms out to scratch)
    typedef __attribute__((address_space(3))) const float lds_float;
    uint32_t sca = lds_addr(stile(buf));
    if constexpr (F8S) asm volatile("" : "+v"(sca) : "v"(s0[0]), "v"(s1[0]));
    else if constexpr (FP8) asm volatile("" : "+v"(sca) : "v"(kdep));
    lds_float *sct8 = (lds_float *)(size_t)sca;
    if constexpr (FP8) {
      // K row scales of slot rows 4g..4g+3 (first rows of wave g's pairs) and
      // 16+4g..16+4g+3 (second rows of wave (g ^ 2)'s pairs)
      lds_float *sc = sct8;
      typedef __attribute__((address_space(3))) const floatx4 lds_f4;
      const floatx4 klo = *(lds_f4 *)(sc + 16 * g);
      const floatx4 khi = *(lds_f4 *)(sc + 16 * (g ^ 2) + 4);
      const float kr[8] = {klo[0], klo[1], klo[2], klo[3], khi[0], khi[1], khi[2], khi[3]};
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) kq[i2] = p.scale_log2 * kr[i2];
    } else {
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) kq[i2] = p.scale_log2;
    }
    // FOLDV: the V rows' scales of the same slot rows (V at [16w' + 8 + q]) times
    // the V factor
    float vr[FOLDV ? 8 : 1];
    float vrs = 1.f;   // FOLDV: the outputs' factor from the V factor's update
    if constexpr (FOLDV) {
      typedef __attribute__((address_space(3))) const floatx4 lds_f4;
      const floatx4 vlo = *(lds_f4 *)(sct8 + 16 * g + 8);
      const floatx4 vhi = *(lds_f4 *)(sct8 + 16 * (g ^ 2) + 12);
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        vr[i2] = vlo[i2];
        vr[4 + i2] = vhi[i2];
      }
      vrs = vfold(vr);
    }
    const uint32_t vis = __builtin_amdgcn_readfirstlane(vmask[i & (kMaskRing - 1)]);
    const uint32_t sm = slot_mask(vis, g);
    auto softmax = [&](const floatx4 &a0, const floatx4 &a1, float &mm, float &ll, floatx4 *oo)
        __attribute__((always_inline)) -> half8 {
      float sv[8];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        sv[i2] = a0[i2] * kq[i2];
        sv[4 + i2] = a1[i2] * kq[4 + i2];
      }
      if (vis != 0xffffffffu) {
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2)
          if (!((sm >> i2) & 1u)) sv[i2] = -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int i2 = 1; i2 < 8; ++i2) mx = fmaxf(mx, sv[i2]);
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const bool grow = mx > mm + kRescaleSlack;
      const float mref = grow ? mx : mm;
      const float msafe = (mref == -INFINITY) ? 0.f : mref;
      const float alpha = __builtin_amdgcn_exp2f(mm - msafe);
      half8 pp;
      float psum = 0.f;
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) {
        if constexpr (FOLDV) {
          const float e = __builtin_amdgcn_exp2f(sv[i2] - msafe);
          pp[i2] = (_Float16)(e * vr[i2]);
          psum += e;
        } else {
          const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(sv[i2] - msafe);
          pp[i2] = ph;
          psum += (float)ph;
        }
      }
      ll = alpha * ll + psum;
      mm = mref;
      if (__ballot(grow || vrs != 1.f)) {
        const float f = alpha * vrs;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oo[dt] *= f;
      }
      return pp;
    };
    const half8 pf = softmax(s0, s1, m, l, o);
    half8 pf2 = pf;
    if constexpr (HT == 2) pf2 = softmax(t0, t1, m2, l2, o2);
    // ---- O^T += V^T P^T; V^T operand = two transpose reads (slots 0-3, 4-7), VPD
    // output tiles ahead
    if constexpr (FP8) {
      // 8-bit transpose read (lane 16G + 8H + B receives byte B of lanes 16G + H + 2k,
      // k = 0..7, measured on the device): this lane supplies row slot_row(g, k),
      // k = (lane & 15) >> 1, dims 16dt + 8(lane & 1) .. +7, so lane 16g + c
      // receives dim 16dt + c of its group's eight slot rows
      const int trk = (lane & 15) >> 1;
      const int trow = trk < 4 ? 4 * g + trk : 16 + 4 * g + (trk - 4);
      const lds_char *vsrc = (const lds_char *)(__attribute__((address_space(3))) const void *)vtc +
                             f8_row_off(trow) + d0 + 8 * (lane & 1);
      // (the V rows' scales are in P: FOLDV)
      auto vload = [&](int dt) __attribute__((always_inline)) -> uint2 {
        const int2v r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) int2v *)(vsrc + 16 * dt));
        return make_uint2((uint32_t)r.x, (uint32_t)r.y);
      };
      uint2 vq[VPD];
#pragma unroll
      for (int u = 0; u < VPD; ++u) vq[u] = vload(u);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const half8 vop = e4m3x8_to_half8(vq[dt % VPD]);
        o[dt] = mfma16(vop, pf, o[dt]);
        if constexpr (HT == 2) o2[dt] = mfma16(vop, pf2, o2[dt]);
        if (dt + VPD < NDT) vq[dt % VPD] = vload(dt + VPD);
        __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMA, then the reads it frees
      }
    } else {
      const lds_char *vrow0 = (const lds_char *)(__attribute__((address_space(3))) const void *)vtc +
                              tr_r0 * kVRow + 2 * d0 + 8 * tr_a;
      const lds_char *vrow1 = vrow0 + 16 * kVRow;
      auto vload = [&](int dt) __attribute__((always_inline)) -> half8 {
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t *)(vrow0 + 32 * dt));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t *)(vrow1 + 32 * dt));
        // whole-vector casts: slots 0-3 from the first read, 4-7 from the second
        return __builtin_shufflevector(__builtin_bit_cast(half4, lo), __builtin_bit_cast(half4, hi), 0,
                                       1, 2, 3, 4, 5, 6, 7);
      };
      half8 vq[VPD];
#pragma unroll
      for (int u = 0; u < VPD; ++u) vq[u] = vload(u);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[dt] = mfma16(vq[dt % VPD], pf, o[dt]);
        if constexpr (HT == 2) o2[dt] = mfma16(vq[dt % VPD], pf2, o2[dt]);
        if (dt + VPD < NDT) vq[dt % VPD] = vload(dt + VPD);
        __builtin_amdgcn_sched_barrier(0);   // keep this order: MFMA, then the reads it frees
      }
    }

    if constexpr (SPLITKV) {
      // every read of buffer B is done; the producers publish entry i + 1
      if (i + 1 < e1) lds_barrier();
      return;
    }
    lds_barrier();   // every wave is done with buffer B
    // HEADS (two workgroups per CU): a wave issuing its block's transfers runs at
    // raised priority, so the other workgroup's MFMA phase yields issue slots to it
    if constexpr (MODE == kSplitHeads) __builtin_amdgcn_s_setprio(1);
    if (nx < e1) {
      if ((nx & (kMaskChunk - 1)) == 0) {
        // next chunk of masks (one batch of loads per 8 entries; drains the transfers)
        const int n = e1 - nx;
        build_masks(nx, n < kMaskChunk ? n : kMaskChunk, std::integral_constant<int, 1>{});
        lds_barrier();
      }
      stage(nx, buf, Masked{}, BothParts{});
      // block i+1 (staged earlier) landed: only the NBUF - 1 newer stages may be in flight
      if constexpr (NBUF >= 2) wait_vmcnt<(NBUF - 1) * (FP8 ? kF8StageOps : kStageOps)>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    if constexpr (MODE == kSplitHeads) __builtin_amdgcn_s_setprio(0);
    lds_barrier();   // publishes block i+1
  };

  for (int i = e0; i < e1; i += NBUF) {
    for_bufs([&](auto E) {
      if (i + E < e1) iteration(i + E, E);
    });
  }

  // ---- epilogue: O = O / l, float32 stores (4 consecutive dims per lane)
  float lt = l;
  lt = xor_sum(lt, 16);
  lt = xor_sum(lt, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // FP8: the V scales' factor comes off (O = 0 if it was never set)
  const float ivf = !FP8 ? 1.f : (vset ? __uint_as_float((uint32_t)(127 + vexp) << 23) : 0.f);
  if constexpr (DIMS) {
    // DIMS: wave w writes dims 128w .. 128w + 127 of the workgroup's 16 (kDimsWide:
    // 32) heads, or, for a split part, of its partial record (normalised like an
    // output, so that it never exceeds the V rows' magnitude; read back by the
    // combine pass: cached stores)
    if constexpr (PARTS) {
      char *rec = p.ws + ((int64_t)L * nsplit + split) * kSplitRecord;
      store_acc_rows<NDT, false>(rec + 4 * d0, 512 * 4, o, inv * ivf, lane);
      if (w == 0 && g == 0) {
        // then the maxima and the sums
        ((float *)(rec + 16 * 512 * 4))[c16] = m;
        ((float *)(rec + 16 * 512 * 4))[16 + c16] = lt;
      }
    } else {
      char *orow = p.o + b * p.o_sb + t * p.o_st + (int64_t)(hg * HG) * p.o_sh + 4 * d0;
      store_acc_rows<NDT, true>(orow, p.o_sh, o, inv * ivf, lane);
      if constexpr (HT == 2) {
        float lt2 = l2;
        lt2 = xor_sum(lt2, 16);
        lt2 = xor_sum(lt2, 32);
        store_acc_rows<NDT, true>(orow + 16 * p.o_sh, p.o_sh, o2, (lt2 > 0.f ? 1.f / lt2 : 0.f) * ivf, lane);
      }
    }
    return;
  }
  if constexpr (MODE == kSplitHeads) {
    // HEADS: the 64 x 512 float32 outputs leave through the free tile buffers, so
    // that every store writes 1 KiB of one row.  Per pass WPP waves write their 16
    // rows; then all four waves store them.  (Stored straight from the accumulators
    // with store_acc_rows, 16 rows x 64 bytes per store, the 128 KiB per token made
    // the prefill kernels slower, the sliding-window chunk 110 -> 119 us.)
    typedef __attribute__((address_space(3))) char lds_w;
    lds_w *kts = (lds_w *)(__attribute__((address_space(3))) void *)kt0;
    lds_w *vts = (lds_w *)(__attribute__((address_space(3))) void *)vt0;
    constexpr int kORow = 2064;         // 512 float32, padded
    constexpr int RPT = KT / kORow;     // rows per tile buffer: float16 16, FP8 8
    static_assert((RPT == 16 || RPT == 8) && RPT * kORow <= VT, "output rows fit the tiles");
    constexpr int WPP = 2 * RPT / 16;   // waves per pass
    auto slot = [&](int sl) __attribute__((always_inline)) -> lds_w * {
      return (sl < RPT ? kts : vts) + (sl % RPT) * kORow;
    };
#pragma unroll
    for (int pass = 0; pass < 4 / WPP; ++pass) {
      const int wj = w - pass * WPP;
      if (wj >= 0 && wj < WPP) {
        lds_w *row = slot(16 * wj + c16) + 16 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *(__attribute__((address_space(3))) floatx4 *)(row + 64 * dt) = o[dt] * (inv * ivf);
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int sl = (RPT / 2) * w + (k >> 1), half = k & 1;
        const int head = hg * HG + 16 * (pass * WPP + sl / 16) + (sl % 16);
        const floatx4 v = *(const __attribute__((address_space(3))) floatx4 *)(slot(sl) + 1024 * half + lane16);
        __builtin_nontemporal_store(v, (floatx4 *)((float *)(p.o + b * p.o_sb + t * p.o_st + (int64_t)head * p.o_sh) + 256 * half + 4 * lane));
      }
      if (pass + 1 < 4 / WPP) lds_barrier();
    }
    return;
  }
}

template <int MODE>
static hipError_t launch_staged(const AttnParams &p, hipStream_t s) {
  constexpr int HG = MODE == kSplitHeads ? 64 : 16;
  const int64_t n = (int64_t)p.B * p.T * (p.H / HG) * (MODE == kSplitHeads ? 1 : p.nsplit);
  if (n == 0) return hipSuccess;
  // (DIMS: four computing and four producing waves)
  const dim3 grid((unsigned)n), block(MODE == kSplitDims ? 512 : 256);
  auto go = [&](auto parts) {
    constexpr bool P = decltype(parts)::value;
    if (p.fp8) {
      if (p.indexed) hipLaunchKernelGGL((attn_staged_kernel<MODE, true, true, P>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((attn_staged_kernel<MODE, false, true, P>), grid, block, 0, s, p);
    } else {
      if (p.indexed) hipLaunchKernelGGL((attn_staged_kernel<MODE, true, false, P>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((attn_staged_kernel<MODE, false, false, P>), grid, block, 0, s, p);
    }
  };
  if constexpr (MODE == kSplitHeads) go(std::false_type{});
  else if (p.nsplit > 1) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

// Decode: lists that can be long take the KEYS split; shorter ones take the DIMS
// split.  The list length is bounded by list_bound, per split part.  Measured per
// launch, DIMS with its producer waves against KEYS: float16 rows, 64 sequences x
// 8 blocks 16.1 us against 19.8 us, x 16 blocks 28.2 against 30.1, about even at
// 32, slower at 64 (16 sequences: 81.5 against 75.6); FP8 rows, 64 sequences x 4
// blocks 11.1 against 11.8 us, x 12 blocks 23.8 against 20.5.
constexpr int64_t kKeysMinEntries = 40, kKeysMinEntriesFp8 = 8;
static bool use_keys(const AttnParams &p) {
  if (p.decode_split) return p.decode_split == 2;
  return list_bound(p) / (p.nsplit > 0 ? p.nsplit : 1) >= (p.fp8 ? kKeysMinEntriesFp8 : kKeysMinEntries);
}
// Wide DIMS (32 heads per workgroup) once the 16-head grid has more workgroups than
// the chip has CUs: it then fits in half the rounds.  Below that its extra work per
// block lengthens every workgroup (measured on the sliding-window decode: 8 / 32 / 64
// sequences 10.8 / 11.4 / 13.0 us wide against 8.2 / 8.9 / 10.6 us; 128 sequences,
// 512 workgroups of 16 heads, 14.8 us against 20.0 us).  No index lists (their LDS
// does not fit beside the wider score exchange), no split parts.
constexpr int64_t kWideAboveGroups = kNumCus;
static bool use_wide(const AttnParams &p) {
  if (p.indexed || p.nsplit > 1 || p.H % 32 != 0) return false;
  if (p.decode_split) return p.decode_split == 3;
  return (int64_t)p.B * p.T * (p.H / 16) > kWideAboveGroups;
}
static hipError_t launch_wide(const AttnParams &p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.T * (p.H / 32);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(512);
  if (p.fp8) hipLaunchKernelGGL((attn_staged_kernel<kDimsWide, false, true, false>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_staged_kernel<kDimsWide, false, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}
hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s) {
  if (use_keys(p)) return launch_staged<kSplitKeys>(p, s);
  if (use_wide(p)) return launch_wide(p, s);
  return launch_staged<kSplitDims>(p, s);
}
// Combine the split partials of one (token, head group): 16 heads x 512 dims over
// 1024 threads, thread = (head, 8 dims).  Each part's record holds its own
// normalised output O_s (its rows' weights summing to one) with the running
// maximum m_s (base 2) and the sum l_s its weights were taken against; with
// M = max m_s and w_s = 2^(m_s - M) l_s the result is sum_s (w_s / sum_t w_t) O_s,
// zero when no split saw a row.  The weights are normalised before the outputs
// meet, so no sum exceeds the V rows' magnitude.  The maxima and sums of all
// parts are staged in LDS, and the parts' outputs are read eight parts at a time,
// so the pass costs a few memory round trips whatever the split count.
__global__ __launch_bounds__(1024) void split_combine_kernel(const AttnParams p) {
  __shared__ float ml[2][16][kMaxSplits];   // [m | l][head][part]
  const int ngroups = p.H / 16;
  const int64_t L = blockIdx.x;
  const int hg = (int)(L % ngroups);
  const int64_t bt = L / ngroups;
  const int t = (int)(bt % p.T), b = (int)(bt / p.T);
  // (lane l: dims 4l .. 4l + 3 and 256 + 4l .. 256 + 4l + 3, so that adjacent
  // lanes read and write adjacent 16 bytes)
  const int tid = threadIdx.x, hh = tid >> 6, dq = (tid & 63) * 4;
  const int ns = p.nsplit;
  const char *rec0 = p.ws + L * ns * kSplitRecord;
  floatx4 v0[8], v1[8];
  // (every load below is unconditional -- parts past the last re-read the last
  // part's record, whose copies are never used -- so that the compiler's wait
  // counts know how many loads are younger than each one and need not drain them)
  auto load8 = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = s0 + u < ns ? s0 + u : ns - 1;
      const floatx4 *src = (const floatx4 *)((const float *)(rec0 + sp * kSplitRecord) + hh * 512 + dq);
      v0[u] = src[0];
      v1[u] = src[64];
    }
  };
  // The maxima and sums of all parts go to LDS, padded to a multiple of eight
  // parts with m = -inf and l = 0 so that they are reduced eight independent reads
  // at a time.  Each thread stages at most two of them (32 x 64 entries at most);
  // they are loaded before the first eight parts' outputs, so that waiting for
  // them leaves the outputs in flight through the reductions (one memory round
  // trip for the whole pass when there are at most eight parts).
  const int ns8 = (ns + 7) & ~7;
  float st[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 1024 * i, sp = e >> 5, k = e & 31;   // part, then 0..15 maxima, 16..31 sums
    const float x = ((const float *)(rec0 + (sp < ns ? sp : ns - 1) * kSplitRecord + 16 * 512 * 4))[k];
    st[i] = sp < ns ? x : (k < 16 ? -INFINITY : 0.f);
  }
  load8(0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 1024 * i, sp = e >> 5, k = e & 31;
    if (sp < ns8) ml[k >> 4][k & 15][sp] = st[i];
  }
  lds_barrier();
  float mmax = -INFINITY;
  for (int s0 = 0; s0 < ns8; s0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) mmax = fmaxf(mmax, ml[0][hh][s0 + u]);
  }
  auto weight = [&](int sp) {   // (both read first: a select, not a branch per part)
    const float ms = ml[0][hh][sp], ls = ml[1][hh][sp];
    const float x = __builtin_amdgcn_exp2f(ms - mmax) * ls;
    return ms == -INFINITY ? 0.f : x;
  };
  float w8[8], lsum = 0.f;   // (the first eight parts' weights stay in registers)
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    w8[u] = weight(u);
    lsum += w8[u];
  }
  for (int s0 = 8; s0 < ns8; s0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) lsum += weight(s0 + u);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (mmax != -INFINITY) {
    // normalised weights: no sum exceeds the V rows' magnitude
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < ns) {
        acc0 += (w8[u] * inv) * v0[u];
        acc1 += (w8[u] * inv) * v1[u];
      }
    }
    for (int s0 = 8; s0 < ns; s0 += 8) {
      load8(s0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < ns) {
          const float wgt = weight(s0 + u) * inv;
          acc0 += wgt * v0[u];
          acc1 += wgt * v1[u];
        }
      }
    }
  }
  float *ob = (float *)(p.o + b * p.o_sb + t * p.o_st + (int64_t)(hg * 16 + hh) * p.o_sh) + dq;
  *(floatx4 *)ob = acc0;
  *(floatx4 *)(ob + 256) = acc1;
}

hipError_t launch_attn_decode_split(const AttnParams &p, hipStream_t s) {
  hipError_t e = use_keys(p) ? launch_staged<kSplitKeys>(p, s) : launch_staged<kSplitDims>(p, s);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)p.B * p.T * (p.H / 16);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)n), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnParams &p, hipStream_t s) {
  return launch_staged<kSplitHeads>(p, s);
}

}  // namespace ds4attn
