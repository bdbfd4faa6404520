// C ABI of libds4attn: argument checks, parameter resolution and kernel dispatch.
// Every check runs on the host before anything is enqueued (see include/ds4attn.h).
#include "ds4attn.h"
#include "ds4attn_internal.h"

#include <algorithm>
#include "mfma_common.h"

#include <cmath>
#include <mutex>

using namespace ds4attn;

namespace {

constexpr int kMaxIndexK = kIdxCap;

inline int64_t ceil32(int64_t n) { return (n + 31) / 32 * 32; }
inline bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }
inline bool stride16(int64_t s) { return s >= 0 && (s & 15) == 0; }
inline int elem_bytes(int32_t dtype) { return dtype == DS4ATTN_F16 ? 2 : (dtype == DS4ATTN_E4M3 ? 1 : 4); }
inline bool aligned4(const void *ptr) { return ((uintptr_t)ptr & 3u) == 0; }

// FP8 regions with live rows need both scale arrays, holding n_rows floats per sequence.
int check_scales(const ds4attn_region &r, int32_t batch) {
  if (r.n_rows == 0 || batch == 0) return DS4ATTN_OK;
  if (!r.k_scale || !r.v_scale || !aligned4(r.k_scale) || !aligned4(r.v_scale)) return DS4ATTN_E_INVAL;
  if (r.scale_stride_b < 0 || (r.scale_stride_b & 3)) return DS4ATTN_E_INVAL;
  if (batch > 1 && r.scale_stride_b < 4LL * r.n_rows) return DS4ATTN_E_INVAL;
  return DS4ATTN_OK;
}
inline bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// A region with n_rows > 0 needs K, V and strides that hold whole padded rows.
int check_region(const ds4attn_region &r, int32_t batch, int row_bytes, bool need_kv) {
  if (r.n_rows < 0) return DS4ATTN_E_INVAL;
  if (r.n_rows == 0 || batch == 0) return DS4ATTN_OK;
  if (r.valid && (batch > 1 && r.valid_stride_b < r.n_rows)) return DS4ATTN_E_INVAL;
  if (!need_kv) return DS4ATTN_OK;
  if (!r.k || !r.v || !aligned16(r.k) || !aligned16(r.v)) return DS4ATTN_E_INVAL;
  if (!stride16(r.stride_row) || r.stride_row < row_bytes || !stride16(r.stride_b))
    return DS4ATTN_E_INVAL;
  if (batch > 1 && r.stride_b < ceil32(r.n_rows) * r.stride_row) return DS4ATTN_E_INVAL;
  return DS4ATTN_OK;
}

// Mask-side checks shared by blockmap and attention; fills the mask fields of P.
int resolve_mask(const ds4attn_args *a, int row_bytes, bool need_kv, AttnParams &P) {
  if (!a) return DS4ATTN_E_INVAL;
  if (a->batch < 0 || a->n_tok < 0 || a->n_head < 1) return DS4ATTN_E_INVAL;
  if (a->window < 0) return DS4ATTN_E_INVAL;
  int st = check_region(a->r0, a->batch, row_bytes, need_kv);
  if (st) return st;
  st = check_region(a->r1, a->batch, row_bytes, need_kv);
  if (st) return st;
  if (a->r1_index && (a->r1_k < 1 || a->r1_k > kMaxIndexK)) return DS4ATTN_E_INVAL;
  P = AttnParams{};
  P.B = a->batch;
  P.T = a->n_tok;
  P.H = a->n_head;
  P.D = a->head_dim;
  P.window = a->window;
  P.qk_delta = a->q_pos0 - a->k_pos0;
  P.k0 = (const char *)a->r0.k;
  P.v0 = (const char *)a->r0.v;
  P.kv0_sb = a->r0.stride_b;
  P.kv0_sr = a->r0.stride_row;
  P.valid0 = a->r0.valid;
  P.valid0_sb = a->r0.valid_stride_b;
  P.n0 = a->r0.n_rows;
  P.nb0 = (int)(ceil32(a->r0.n_rows) / 32);
  P.k1 = (const char *)a->r1.k;
  P.v1 = (const char *)a->r1.v;
  P.kv1_sb = a->r1.stride_b;
  P.kv1_sr = a->r1.stride_row;
  P.valid1 = a->r1.valid;
  P.valid1_sb = a->r1.valid_stride_b;
  P.n1 = a->r1.n_rows;
  P.indexed = a->r1_index != nullptr;
  P.idx = a->r1_index;
  P.r1_k = P.indexed ? a->r1_k : 0;
  if (P.n1 == 0) P.nb1 = 0;
  else P.nb1 = P.indexed ? (P.r1_k + 31) / 32 : (int)(ceil32(P.n1) / 32);
  P.nbd = P.nb0 + (P.indexed ? 0 : P.nb1);
  P.nsplit = 1;
  P.decode_split = 0;
  return DS4ATTN_OK;
}

bool ranges_overlap(const void *a, int64_t alen, const void *b, int64_t blen) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)blen && b0 < a0 + (uintptr_t)alen;
}

int64_t split_workspace_bytes(const ds4attn_args *a, int32_t splits) {
  return splits > 1 ? (int64_t)a->batch * a->n_tok * (a->n_head / 16) * splits * kSplitRecord : 0;
}

// An attention call resolved on the host: kernel parameters (pointers not yet
// set), which kernel family applies, and whether there is any work.
struct Resolved {
  AttnParams P;
  bool mfma;     // the matrix-core kernels apply
  bool empty;    // B * T == 0: nothing to launch
  int eb;        // element bytes of Q (and of plain K/V rows)
};

// Every check that needs only *a: shapes, strides, regions, formats, flags.
int resolve_args(const ds4attn_args *a, bool prefill, Resolved &R) {
  if (!a) return DS4ATTN_E_INVAL;
  if (a->dtype != DS4ATTN_F16 && a->dtype != DS4ATTN_F32) return DS4ATTN_E_INVAL;
  if (a->head_dim <= 0) return DS4ATTN_E_INVAL;
  if (!head_dim_ok(a->head_dim)) return DS4ATTN_E_UNSUPPORTED;
  if (!std::isfinite(a->scale)) return DS4ATTN_E_INVAL;
  if (a->kv_format != DS4ATTN_KV_PLAIN && a->kv_format != DS4ATTN_KV_FP8_E4M3) return DS4ATTN_E_INVAL;
  const bool fp8 = a->kv_format == DS4ATTN_KV_FP8_E4M3;
  R.eb = elem_bytes(a->dtype);
  const int row_bytes = a->head_dim * R.eb;                     // Q rows
  const int kv_row_bytes = fp8 ? a->head_dim : row_bytes;       // K/V rows
  AttnParams &P = R.P;
  int st = resolve_mask(a, kv_row_bytes, true, P);
  if (st) return st;
  if (fp8) {
    if ((st = check_scales(a->r0, a->batch)) || (st = check_scales(a->r1, a->batch))) return st;
    P.fp8 = 1;
    P.ks0 = (const char *)a->r0.k_scale;
    P.vs0 = (const char *)a->r0.v_scale;
    P.s0_sb = a->r0.scale_stride_b;
    P.ks1 = (const char *)a->r1.k_scale;
    P.vs1 = (const char *)a->r1.v_scale;
    P.s1_sb = a->r1.scale_stride_b;
  }
  const int64_t work = (int64_t)a->batch * a->n_tok;
  R.empty = work == 0;
  if (R.empty) {
    R.mfma = false;
    return DS4ATTN_OK;
  }
  if (!stride16(a->q_stride_b) || !stride16(a->q_stride_t) || !stride16(a->q_stride_h) ||
      !stride16(a->o_stride_b) || !stride16(a->o_stride_t) || !stride16(a->o_stride_h))
    return DS4ATTN_E_INVAL;
  if (a->n_head > 1 && (a->q_stride_h < row_bytes || a->o_stride_h < a->head_dim * 4))
    return DS4ATTN_E_INVAL;
  if (work * a->n_head > 0x7fffffffLL) return DS4ATTN_E_UNSUPPORTED;
  // The matrix-core kernels list the token's non-skipped map blocks in LDS (up to
  // kListCap of them) and address each sequence's K/V region with 32-bit offsets
  // (< 2^31 bytes); longer dense regions run on the vector-ALU kernel.
  const int64_t rows1 = P.indexed ? ceil32(P.n1) : (int64_t)P.nb1 * 32;
  const bool fits32 = (int64_t)P.nb0 * 32 * P.kv0_sr < 0x80000000LL && rows1 * P.kv1_sr < 0x80000000LL;
  R.mfma = a->dtype == DS4ATTN_F16 && a->head_dim == 512 && a->n_head % 16 == 0 &&
           !(a->flags & DS4ATTN_FLAG_GENERIC) && P.nbd <= kListCap && fits32;
  // FP8 rows are dequantized inside the matrix-core kernels only
  if (fp8 && !R.mfma) return DS4ATTN_E_UNSUPPORTED;
  const bool want_dims = a->flags & DS4ATTN_FLAG_DECODE_DIMS, want_keys = a->flags & DS4ATTN_FLAG_DECODE_KEYS;
  const bool want_wide = a->flags & DS4ATTN_FLAG_DECODE_WIDE;
  if ((int)want_dims + (int)want_keys + (int)want_wide > 1) return DS4ATTN_E_INVAL;
  if (want_dims || want_keys || want_wide) {
    // a chosen decode split: the matrix-core decode kernel
    if (!R.mfma || (prefill && a->n_head % 64 == 0)) return DS4ATTN_E_UNSUPPORTED;
    // the wide split: 32 heads per workgroup, no index list
    if (want_wide && (P.indexed || a->n_head % 32 != 0)) return DS4ATTN_E_UNSUPPORTED;
    P.decode_split = want_keys ? 2 : (want_wide ? 3 : 1);
  }
  return DS4ATTN_OK;
}

// The split the library picks for a decode call ([P-DS4] "Architecture Deep
// Dive", Whole-Model Graph Execution: the attention path is chosen by layer type
// and batch size).  A decode workgroup covers one token's 16 heads; a batch with
// fewer than 128 such groups leaves most of the 256 CUs idle, so each token's
// block list is divided over up to 256 / groups workgroups, at least two key
// blocks per part and at most 8 parts (the combine pass reads eight parts' records
// per memory round trip), then over as few parts as keep the longest part that
// short; lists of up to 5 blocks stay whole (the combine pass costs more than the
// split saves).  Measured on one sequence (µs, parts in brackets): a 4-block
// window 7.9 [1], 9.4 [2]; 8 dense blocks 11.8 [2], 10.4 [4]; 12 blocks of the
// ratio-128 layer 13.3 [3], 12.5 [4], 11.9 [6], 13.6 [12]; 16 dense blocks 12.6
// [4], 11.9 [8], 13.1 [11]; the ratio-4 layer's 20 blocks 15.6 [6], 14.1 [7],
// 14.3 [8], 14.5 [10]; 32 dense blocks 13.8 [8], 15.6 [10].  64-sequence batches
// only lose from splitting.
int plan_splits(const Resolved &R, bool prefill) {
  // (a chosen wide split has no split parts)
  if (prefill || R.empty || !R.mfma || R.P.decode_split == 3) return 1;
  const AttnParams &P = R.P;
  const int64_t groups = (int64_t)P.B * P.T * (P.H / 16);
  if (groups >= 128) return 1;
  const int64_t lb = list_bound(P);
  if (lb <= 5) return 1;
  const int64_t cap = std::min<int64_t>({lb / 2, 8, 256 / groups, (int64_t)kMaxSplits});
  if (cap <= 1) return 1;
  const int64_t per = (lb + cap - 1) / cap;   // blocks in the longest part
  return (int)((lb + per - 1) / per);
}

// Pointer checks and the launch of a resolved call with `splits` parts (> 1: the
// records go to `ws`, which must hold split_workspace_bytes).
int launch_resolved(const ds4attn_args *a, Resolved &R, const void *q, const uint8_t *blk, int32_t bq,
                    float *o, bool prefill, int32_t splits, void *ws, int64_t ws_bytes, void *stream) {
  if (R.empty) return DS4ATTN_OK;
  if (!q || !o || !aligned16(q) || !aligned16(o)) return DS4ATTN_E_INVAL;
  if (blk && bq < 1) return DS4ATTN_E_INVAL;
  AttnParams &P = R.P;
  P.q = (const char *)q;
  P.o = (char *)o;
  P.q_sb = a->q_stride_b;
  P.q_st = a->q_stride_t;
  P.q_sh = a->q_stride_h;
  P.o_sb = a->o_stride_b;
  P.o_st = a->o_stride_t;
  P.o_sh = a->o_stride_h;
  P.scale_log2 = a->scale * 1.4426950408889634f;
  P.blk = blk;
  // a tile longer than the chunk is the whole chunk (same map, same tile of every token)
  P.bq = blk ? (int)std::min<int64_t>(bq, std::max(1, a->n_tok)) : 1;
  P.ntiles = ((int64_t)a->n_tok + P.bq - 1) / P.bq;
  P.div_g16 = make_fast_div((uint32_t)std::max(1, a->n_head / 16));
  P.div_g32 = make_fast_div((uint32_t)std::max(1, a->n_head / 32));
  P.div_g64 = make_fast_div((uint32_t)std::max(1, a->n_head / 64));
  P.div_t = make_fast_div((uint32_t)std::max(1, a->n_tok));
  P.div_bq = make_fast_div((uint32_t)P.bq);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (splits > 1) {
    // split decode runs on the matrix-core decode kernel only, 16 heads per part
    if (!R.mfma || prefill || R.P.decode_split == 3) return DS4ATTN_E_UNSUPPORTED;
    const int64_t work = (int64_t)a->batch * a->n_tok;
    if (work * (a->n_head / 16) * splits > 0x7fffffffLL) return DS4ATTN_E_UNSUPPORTED;
    const int64_t need = split_workspace_bytes(a, splits);
    if (!ws || !aligned16(ws)) return DS4ATTN_E_INVAL;
    if (ws_bytes < need) return DS4ATTN_E_WORKSPACE;
    const int64_t o_len = (a->batch - 1) * a->o_stride_b + (a->n_tok - 1) * a->o_stride_t +
                          (a->n_head - 1) * a->o_stride_h + 4LL * a->head_dim;
    if (ranges_overlap(ws, need, o, o_len)) return DS4ATTN_E_INVAL;
    P.nsplit = splits;
    P.ws = (char *)ws;
    e = launch_attn_decode_split(P, s);
    return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
  }
  if (R.mfma && prefill && a->n_head % 64 == 0) e = launch_attn_prefill(P, s);
  else if (R.mfma) e = launch_attn_decode(P, s);
  else e = launch_attn_generic(P, R.eb, s);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

// ---------------------------------------------------------------------------- static scratch
// The split records of ds4attn_decode_noalloc live in this array: each device the
// library runs on holds its own copy until the process ends.  The decode plan
// splits only batches of fewer than 128 groups of 16 heads, into at most 256 /
// groups parts, so a call never needs more than 256 records.
constexpr int64_t kScratchRecords = 256;
constexpr int64_t kScratchBytes = kScratchRecords * kSplitRecord;
static __device__ __align__(256) char scratch[kScratchBytes];

// The device address of this device's `scratch`, looked up once per device (the
// array's name is a host-side stand-in; only this address may reach a kernel).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_of_device(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return DS4ATTN_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DS4ATTN_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DS4ATTN_OK;
}

// ds4attn_decode / ds4attn_prefill: the library's plan, run in the caller's workspace.
int run_planned(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq, float *o, void *ws,
                int64_t ws_bytes, void *stream, bool prefill) {
  if (ws_bytes < 0) return DS4ATTN_E_INVAL;
  Resolved R;
  int st = resolve_args(a, prefill, R);
  if (st) return st;
  const int splits = plan_splits(R, prefill);
  // no workspace: the call runs unsplit
  const int use = (splits > 1 && ws) ? splits : 1;
  return launch_resolved(a, R, q, blk, bq, o, prefill, use, ws, ws_bytes, stream);
}


}  // namespace

extern "C" {

int ds4attn_pad(const ds4attn_region *in, int32_t batch, int32_t head_dim, int32_t dtype,
                void *k_pad, void *v_pad, int64_t out_stride_b, int64_t out_stride_row,
                uint8_t *valid_pad, int64_t valid_pad_stride_b, void *stream) {
  if (!in || batch < 0 || in->n_rows < 0) return DS4ATTN_E_INVAL;
  if (dtype != DS4ATTN_F16 && dtype != DS4ATTN_F32 && dtype != DS4ATTN_E4M3) return DS4ATTN_E_INVAL;
  if (head_dim <= 0 || (head_dim * elem_bytes(dtype)) % 16) return DS4ATTN_E_INVAL;
  const int row_bytes = head_dim * elem_bytes(dtype);
  const int64_t n = in->n_rows, npad = ceil32(n);
  if (batch == 0 || npad == 0) return DS4ATTN_OK;
  if (!k_pad || !v_pad || !aligned16(k_pad) || !aligned16(v_pad)) return DS4ATTN_E_INVAL;
  if (!stride16(out_stride_row) || out_stride_row < row_bytes || !stride16(out_stride_b))
    return DS4ATTN_E_INVAL;
  if (batch > 1 && out_stride_b < npad * out_stride_row) return DS4ATTN_E_INVAL;
  if (n > 0) {
    if (!in->k || !in->v || !aligned16(in->k) || !aligned16(in->v)) return DS4ATTN_E_INVAL;
    if (!stride16(in->stride_row) || in->stride_row < row_bytes || !stride16(in->stride_b))
      return DS4ATTN_E_INVAL;
    if (batch > 1 && in->stride_b < n * in->stride_row) return DS4ATTN_E_INVAL;
  }
  if (valid_pad && batch > 1 && valid_pad_stride_b < npad) return DS4ATTN_E_INVAL;
  if (in->valid && batch > 1 && in->valid_stride_b < n) return DS4ATTN_E_INVAL;
  if (npad > 0x7fffffffLL) return DS4ATTN_E_UNSUPPORTED;
  const bool same_layout = in->stride_b == out_stride_b && in->stride_row == out_stride_row;
  const bool inplace_k = n > 0 && k_pad == in->k && same_layout;
  const bool inplace_v = n > 0 && v_pad == in->v && same_layout;
  const int64_t out_len = (batch - 1) * out_stride_b + (npad - 1) * out_stride_row + row_bytes;
  if (n > 0) {
    const int64_t in_len = (batch - 1) * in->stride_b + (n - 1) * in->stride_row + row_bytes;
    if (!inplace_k && ranges_overlap(k_pad, out_len, in->k, in_len)) return DS4ATTN_E_INVAL;
    if (!inplace_v && ranges_overlap(v_pad, out_len, in->v, in_len)) return DS4ATTN_E_INVAL;
    if (!inplace_k && ranges_overlap(k_pad, out_len, in->v, in_len) && in->k != in->v)
      return DS4ATTN_E_INVAL;
    if (!inplace_v && ranges_overlap(v_pad, out_len, in->k, in_len) && in->k != in->v)
      return DS4ATTN_E_INVAL;
  }
  // K and V outputs may be one buffer only when K and V inputs are one buffer too.
  if (ranges_overlap(k_pad, out_len, v_pad, out_len) && !(k_pad == v_pad && in->k == in->v))
    return DS4ATTN_E_INVAL;
  // Validity in place: the output is the input buffer with the same stride.
  const bool inplace_valid = valid_pad && in->valid == valid_pad &&
                             (batch == 1 || in->valid_stride_b == valid_pad_stride_b);
  if (valid_pad && in->valid && !inplace_valid && n > 0) {
    const int64_t vout_len = (batch - 1) * valid_pad_stride_b + npad;
    const int64_t vin_len = (batch - 1) * in->valid_stride_b + n;
    if (ranges_overlap(valid_pad, vout_len, in->valid, vin_len)) return DS4ATTN_E_INVAL;
  }
  // Nothing to write: every output is its input and there is no tail.
  if (npad == n && (n == 0 || (inplace_k && inplace_v)) && (!valid_pad || inplace_valid))
    return DS4ATTN_OK;
  hipError_t e = launch_pad(in->k, in->v, in->valid, in->stride_b, in->stride_row,
                            in->valid_stride_b, k_pad, v_pad, valid_pad, out_stride_b,
                            out_stride_row, valid_pad_stride_b, batch, (int)n, (int)npad,
                            row_bytes, !inplace_k, !inplace_v, !inplace_valid,
                            (hipStream_t)stream);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

int ds4attn_blockmap_dims(const ds4attn_args *a, int32_t bq, int64_t *n_tiles, int32_t *n_blocks) {
  if (!a || bq < 1 || !n_tiles || !n_blocks) return DS4ATTN_E_INVAL;
  if (a->n_tok < 0 || a->r0.n_rows < 0 || a->r1.n_rows < 0) return DS4ATTN_E_INVAL;
  *n_tiles = ((int64_t)a->n_tok + bq - 1) / bq;
  int64_t nb = ceil32(a->r0.n_rows) / 32;
  if (!a->r1_index) nb += ceil32(a->r1.n_rows) / 32;
  *n_blocks = (int32_t)nb;
  return DS4ATTN_OK;
}

int ds4attn_blockmap(const ds4attn_args *a, int32_t bq, uint8_t *blk, void *stream) {
  if (!a || bq < 1) return DS4ATTN_E_INVAL;
  AttnParams P;
  // Only the mask side is read: sizes, window, positions, validity, index presence.
  int st = resolve_mask(a, 16, false, P);
  if (st) return st;
  // a tile longer than the chunk is the whole chunk (the same map)
  P.bq = (int)std::min<int64_t>(bq, std::max(1, a->n_tok));
  P.ntiles = ((int64_t)a->n_tok + P.bq - 1) / P.bq;
  const int64_t total = (int64_t)P.B * P.ntiles * P.nbd;
  if (total == 0) return DS4ATTN_OK;
  if (!blk) return DS4ATTN_E_INVAL;
  if (total > 0x7fffffffLL) return DS4ATTN_E_UNSUPPORTED;   // 32-bit entry indices
  hipError_t e = launch_blockmap(P, blk, (hipStream_t)stream);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

int ds4attn_decode(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq, float *o,
                   void *workspace, int64_t workspace_bytes, void *stream) {
  return run_planned(a, q, blk, bq, o, workspace, workspace_bytes, stream, false);
}

int ds4attn_prefill(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq, float *o,
                    void *workspace, int64_t workspace_bytes, void *stream) {
  return run_planned(a, q, blk, bq, o, workspace, workspace_bytes, stream, true);
}

int ds4attn_decode_noalloc(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq, float *o,
                           void *stream) {
  Resolved R;
  int st = resolve_args(a, false, R);
  if (st) return st;
  const int splits = plan_splits(R, false);
  if (splits <= 1) return launch_resolved(a, R, q, blk, bq, o, false, 1, nullptr, 0, stream);
  if (split_workspace_bytes(a, splits) > kScratchBytes) return DS4ATTN_E_WORKSPACE;
  // the array of the device the kernels run on, which must be the current device
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DS4ATTN_E_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return DS4ATTN_E_HIP;
    if (sdev != dev) return DS4ATTN_E_INVAL;
  }
  void *ws = nullptr;
  if ((st = scratch_of_device(dev, &ws))) return st;
  return launch_resolved(a, R, q, blk, bq, o, false, splits, ws, kScratchBytes, stream);
}

int ds4attn_workspace_bytes(const ds4attn_args *a, int32_t is_prefill, int64_t *bytes) {
  if (!bytes) return DS4ATTN_E_INVAL;
  Resolved R;
  const int st = resolve_args(a, is_prefill != 0, R);
  if (st) return st;
  *bytes = split_workspace_bytes(a, plan_splits(R, is_prefill != 0));
  return DS4ATTN_OK;
}

int ds4attn_decode_workspace_bytes(const ds4attn_args *a, int32_t splits, int64_t *bytes) {
  if (!a || !bytes || splits < 1 || splits > kMaxSplits) return DS4ATTN_E_INVAL;
  if (a->batch < 0 || a->n_tok < 0 || a->n_head < 1) return DS4ATTN_E_INVAL;
  if (splits > 1 && a->n_head % 16) return DS4ATTN_E_UNSUPPORTED;
  *bytes = split_workspace_bytes(a, splits);
  return DS4ATTN_OK;
}

int ds4attn_decode_split(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq, float *o,
                         int32_t splits, void *workspace, int64_t workspace_bytes, void *stream) {
  if (splits < 1 || splits > kMaxSplits || workspace_bytes < 0) return DS4ATTN_E_INVAL;
  Resolved R;
  const int st = resolve_args(a, false, R);
  if (st) return st;
  return launch_resolved(a, R, q, blk, bq, o, false, splits, workspace, workspace_bytes, stream);
}

int32_t ds4attn_prefill_bq(void) { return 16; }

int ds4attn_topk(const float *scores, int64_t rows, int32_t n, int64_t score_stride, int32_t k,
                 int32_t *idx, int64_t idx_stride, void *stream) {
  static_assert(kMaxTopkK <= kMaxIndexK, "a selection must be a valid index list");
  if (rows < 0 || n < 0 || k < 1 || k > kMaxTopkK) return DS4ATTN_E_INVAL;
  if (rows > kMaxTopkRows || n > kMaxTopkN) return DS4ATTN_E_UNSUPPORTED;
  if (rows == 0) return DS4ATTN_OK;
  auto aligned4 = [](const void *ptr) { return ((uintptr_t)ptr & 3u) == 0; };
  if (!idx || !aligned4(idx) || (idx_stride & 3) || idx_stride < 0) return DS4ATTN_E_INVAL;
  if (n > 0 && (!scores || !aligned4(scores))) return DS4ATTN_E_INVAL;
  if ((score_stride & 3) || score_stride < 0) return DS4ATTN_E_INVAL;
  if (rows > 1 && (idx_stride < 4LL * k || score_stride < 4LL * n)) return DS4ATTN_E_INVAL;
  const int64_t out_len = (rows - 1) * idx_stride + 4LL * k;
  const int64_t in_len = (rows - 1) * score_stride + 4LL * n;
  if (n > 0 && ranges_overlap(idx, out_len, scores, in_len)) return DS4ATTN_E_INVAL;
  const hipError_t e = launch_topk(scores, rows, n, score_stride, k, idx, idx_stride, (hipStream_t)stream);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

int ds4attn_quantize_fp8(const void *x, int32_t dtype, int32_t batch, int32_t n_rows, int32_t head_dim,
                         int64_t x_stride_b, int64_t x_stride_row, uint8_t *codes,
                         int64_t code_stride_b, int64_t code_stride_row, float *scales,
                         int64_t scale_stride_b, void *stream) {
  if (dtype != DS4ATTN_F16 && dtype != DS4ATTN_F32) return DS4ATTN_E_INVAL;
  if (batch < 0 || n_rows < 0 || head_dim <= 0) return DS4ATTN_E_INVAL;
  if (!head_dim_ok(head_dim)) return DS4ATTN_E_UNSUPPORTED;
  if ((int64_t)batch * n_rows == 0) return DS4ATTN_OK;
  if ((int64_t)batch * n_rows > 0x7fffffffLL) return DS4ATTN_E_UNSUPPORTED;
  const int eb = elem_bytes(dtype);
  const int64_t row_bytes = (int64_t)head_dim * eb;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) || !aligned4(scales))
    return DS4ATTN_E_INVAL;
  if (!stride16(x_stride_row) || !stride16(x_stride_b) || !stride16(code_stride_row) ||
      !stride16(code_stride_b) || scale_stride_b < 0 || (scale_stride_b & 3))
    return DS4ATTN_E_INVAL;
  if (n_rows > 1 && (x_stride_row < row_bytes || code_stride_row < head_dim)) return DS4ATTN_E_INVAL;
  if (batch > 1 && (x_stride_b < (n_rows - 1) * x_stride_row + row_bytes ||
                    code_stride_b < (n_rows - 1) * code_stride_row + head_dim ||
                    scale_stride_b < 4LL * n_rows))
    return DS4ATTN_E_INVAL;
  const int64_t x_len = (batch - 1) * x_stride_b + (n_rows - 1) * x_stride_row + row_bytes;
  const int64_t c_len = (batch - 1) * code_stride_b + (n_rows - 1) * code_stride_row + head_dim;
  const int64_t s_len = (batch - 1) * scale_stride_b + 4LL * n_rows;
  if (ranges_overlap(codes, c_len, x, x_len) || ranges_overlap(scales, s_len, x, x_len) ||
      ranges_overlap(scales, s_len, codes, c_len))
    return DS4ATTN_E_INVAL;
  const hipError_t e = launch_quant_fp8(x, eb, batch, n_rows, head_dim, x_stride_b, x_stride_row, codes,
                                        code_stride_b, code_stride_row, scales, scale_stride_b,
                                        (hipStream_t)stream);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

int ds4attn_compress(int32_t batch, int32_t head_dim, int32_t ratio, int32_t n_state, int32_t n_new,
                     void *state_kv, int64_t state_kv_stride_b, float *state_score, int64_t state_score_stride_b,
                     const void *kv_new, int64_t kv_new_stride_b, const float *score_new,
                     int64_t score_new_stride_b, void *comp, int64_t comp_stride_b, void *stream) {
  if (batch < 0 || n_new < 0 || head_dim <= 0) return DS4ATTN_E_INVAL;
  if (ratio < 1 || n_state < 0 || n_state >= ratio) return DS4ATTN_E_INVAL;
  if (!head_dim_ok(head_dim) || ratio > kMaxCompressRatio) return DS4ATTN_E_UNSUPPORTED;
  if (batch == 0 || n_new == 0) return DS4ATTN_OK;
  const int64_t n_out = ((int64_t)n_state + n_new) / ratio;
  if ((int64_t)n_state + n_new > 0x7fffffffLL || (int64_t)batch * n_out * head_dim > 0x7fffffffLL ||
      (int64_t)batch * n_new * head_dim > 0x7fffffffLL)
    return DS4ATTN_E_UNSUPPORTED;
  const int64_t vrow = 2LL * head_dim, srow = 4LL * head_dim;
  if (!state_kv || !state_score || !kv_new || !score_new || !aligned16(state_kv) || !aligned16(state_score) ||
      !aligned16(kv_new) || !aligned16(score_new))
    return DS4ATTN_E_INVAL;
  if (n_out > 0 && (!comp || !aligned16(comp))) return DS4ATTN_E_INVAL;
  if (!stride16(state_kv_stride_b) || !stride16(state_score_stride_b) || !stride16(kv_new_stride_b) ||
      !stride16(score_new_stride_b) || !stride16(comp_stride_b))
    return DS4ATTN_E_INVAL;
  if (batch > 1 && (state_kv_stride_b < ratio * vrow || state_score_stride_b < ratio * srow ||
                    kv_new_stride_b < n_new * vrow || score_new_stride_b < n_new * srow ||
                    (n_out > 0 && comp_stride_b < n_out * vrow)))
    return DS4ATTN_E_INVAL;
  const int64_t st_kv_len = (batch - 1) * state_kv_stride_b + ratio * vrow;
  const int64_t st_sc_len = (batch - 1) * state_score_stride_b + ratio * srow;
  const int64_t kv_len = (batch - 1) * kv_new_stride_b + n_new * vrow;
  const int64_t sc_len = (batch - 1) * score_new_stride_b + n_new * srow;
  const int64_t c_len = (batch - 1) * comp_stride_b + n_out * vrow;
  // the state is updated in place: it must not overlap the new rows or each other;
  // the compressed rows must not overlap anything read
  if (ranges_overlap(state_kv, st_kv_len, state_score, st_sc_len) ||
      ranges_overlap(state_kv, st_kv_len, kv_new, kv_len) || ranges_overlap(state_kv, st_kv_len, score_new, sc_len) ||
      ranges_overlap(state_score, st_sc_len, kv_new, kv_len) ||
      ranges_overlap(state_score, st_sc_len, score_new, sc_len))
    return DS4ATTN_E_INVAL;
  if (n_out > 0 && (ranges_overlap(comp, c_len, state_kv, st_kv_len) ||
                    ranges_overlap(comp, c_len, state_score, st_sc_len) ||
                    ranges_overlap(comp, c_len, kv_new, kv_len) || ranges_overlap(comp, c_len, score_new, sc_len)))
    return DS4ATTN_E_INVAL;
  const hipError_t e = launch_compress(state_kv, state_score, state_kv_stride_b, state_score_stride_b, n_state,
                                       kv_new, score_new, kv_new_stride_b, score_new_stride_b, n_new, batch,
                                       head_dim, ratio, comp, comp_stride_b, (hipStream_t)stream);
  return e == hipSuccess ? DS4ATTN_OK : DS4ATTN_E_HIP;
}

const char *ds4attn_status_string(int status) {
  switch (status) {
    case DS4ATTN_OK: return "ok";
    case DS4ATTN_E_INVAL: return "invalid argument";
    case DS4ATTN_E_UNSUPPORTED: return "unsupported configuration";
    case DS4ATTN_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
