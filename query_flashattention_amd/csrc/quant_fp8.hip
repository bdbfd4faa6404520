// FP8 KV quantize step: each K or V row becomes E4M3 codes plus one float32
// scale before it is stored in the cache ([P-DS4] "Architecture Deep Dive",
// Whole-Model Graph Execution, where an FP8 KV quantize step precedes the raw KV
// store; the element format and the per-row scale are this library's reading).
//
// Each wave takes four rows, E = D/64 consecutive elements per lane.  In float32:
// amax by a wave reduction, scale = amax / 448, each element x / scale clamped to
// +-448 and rounded to the nearest E4M3 value, ties to even, by v_cvt_pk_fp8_f32
// (two elements per instruction; on values within +-448 it gives the round-to-
// nearest-even code, exact ties and subnormals included, measured against that rule
// on the device), so both the codes and the scale are exactly determined by
// float32 arithmetic.  Each row is read once and written once: 2D or 4D bytes in,
// D + 4 bytes out.
//
// [P-DS4] = "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine".
#include "mfma_common.h"

namespace ds4attn {

namespace {

constexpr float kE4M3Max = 448.0f;

// R rows per wave: their loads are all issued before the first reduction, so a
// wave keeps R row reads in flight instead of one.
template <int E, bool F32, int R>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const char *__restrict__ x, int n, int64_t x_sb,
                                                        int64_t x_sr, char *__restrict__ codes, int64_t c_sb,
                                                        int64_t c_sr, char *__restrict__ scales,
                                                        int64_t s_sb, int rows) {
  const int lane = threadIdx.x & 63;
  // (rows < 2^31: 32-bit index arithmetic)
  const uint32_t r0 = ((uint32_t)blockIdx.x * 4u + (uint32_t)(threadIdx.x >> 6)) * (uint32_t)R;
  if (r0 >= (uint32_t)rows) return;   // whole wave exits together
  float v[R][E];
  int bs[R], rs[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    // (a row past the end reads row r0 again and is not stored: the loads stay
    // unconditional, so that they all go out before the first wait)
    const uint32_t r = r0 + (uint32_t)j < (uint32_t)rows ? r0 + (uint32_t)j : r0;
    bs[j] = (int)(r / (uint32_t)n);
    rs[j] = (int)(r - (uint32_t)bs[j] * (uint32_t)n);
    // the lane's E elements are contiguous and aligned to their size (row starts
    // and strides are multiples of 16 bytes)
    const char *src = x + bs[j] * x_sb + rs[j] * x_sr + (int64_t)lane * E * (F32 ? 4 : 2);
    if constexpr (F32) {
      float t[E];
      __builtin_memcpy(t, __builtin_assume_aligned(src, 4 * E < 16 ? 4 * E : 16), 4 * E);
#pragma unroll
      for (int i = 0; i < E; ++i) v[j][i] = t[i];
    } else {
      _Float16 t[E];
      __builtin_memcpy(t, __builtin_assume_aligned(src, 2 * E < 16 ? 2 * E : 16), 2 * E);
#pragma unroll
      for (int i = 0; i < E; ++i) v[j][i] = (float)t[i];
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (r0 + (uint32_t)j >= (uint32_t)rows) break;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    amax = wave_max(amax);
    const float scale = amax / kE4M3Max;
    // x / scale, correctly rounded, from the correctly rounded reciprocal and one
    // FMA correction (q0 = x y, r = x - s q0 exactly, q = q0 + r y rounded once:
    // Markstein's division step, exact when y is the rounded reciprocal and r is
    // not subnormal); the quotient takes x's sign, zeros included.  Scales below
    // 2^-80 (a residual could be subnormal) or not finite take the division itself.
    // (Checked on the CPU against float32 division: 2e9 pairs, every E4M3 code and
    // every normal quotient equal.)
    const bool fast = scale >= 0x1p-80f && scale <= 3.4028235e38f;
    const float inv = 1.0f / scale;
    float y[E < 2 ? 2 : E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float q = 0.f;   // (a row with scale 0 gets zero codes)
      if (scale != 0.f) {
        if (fast) {
          const float q0 = v[j][i] * inv;
          q = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, scale, v[j][i]), inv, q0), v[j][i]);
        } else {
          q = v[j][i] / scale;
        }
      }
      y[i] = fminf(fmaxf(q, -kE4M3Max), kE4M3Max);   // keeps the sign of zero
    }
    if constexpr (E == 1) y[1] = 0.f;
    // codes of elements 4k .. 4k + 3 in dword k, element 4k in its low byte
    uint32_t w[E < 4 ? 1 : E / 4];
#pragma unroll
    for (int k = 0; k < (E < 4 ? 1 : E / 4); ++k) {
      w[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k], y[4 * k + 1], 0, false);
      if constexpr (E >= 4)
        w[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k + 2], y[4 * k + 3], (int)w[k], true);
    }
    char *dst = codes + bs[j] * c_sb + rs[j] * c_sr + (int64_t)lane * E;
    if constexpr (E == 8) {
      *(uint2 *)dst = make_uint2(w[0], w[1]);
    } else if constexpr (E == 4) {
      *(uint32_t *)dst = w[0];
    } else if constexpr (E == 2) {
      *(uint16_t *)dst = (uint16_t)w[0];
    } else {
      *(uint8_t *)dst = (uint8_t)w[0];
    }
    if (lane == 0) *(float *)(scales + bs[j] * s_sb + 4LL * rs[j]) = scale;
  }
}

constexpr int kRowsPerWave = 4;

template <int E>
hipError_t launch_e(bool f32, const void *x, int B, int n, int64_t x_sb, int64_t x_sr, uint8_t *codes,
                    int64_t c_sb, int64_t c_sr, float *scales, int64_t s_sb, hipStream_t s) {
  const int rows = B * n;
  constexpr int per_block = 4 * kRowsPerWave;
  const dim3 grid((unsigned)((rows + per_block - 1) / per_block)), block(256);
  if (f32)
    hipLaunchKernelGGL((quant_fp8_kernel<E, true, kRowsPerWave>), grid, block, 0, s, (const char *)x, n, x_sb,
                       x_sr, (char *)codes, c_sb, c_sr, (char *)scales, s_sb, rows);
  else
    hipLaunchKernelGGL((quant_fp8_kernel<E, false, kRowsPerWave>), grid, block, 0, s, (const char *)x, n, x_sb,
                       x_sr, (char *)codes, c_sb, c_sr, (char *)scales, s_sb, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const void *x, int elem_bytes, int B, int n, int D, int64_t x_sb, int64_t x_sr,
                            uint8_t *codes, int64_t c_sb, int64_t c_sr, float *scales, int64_t s_sb,
                            hipStream_t s) {
  const bool f32 = elem_bytes == 4;
  switch (D) {
    case 64: return launch_e<1>(f32, x, B, n, x_sb, x_sr, codes, c_sb, c_sr, scales, s_sb, s);
    case 128: return launch_e<2>(f32, x, B, n, x_sb, x_sr, codes, c_sb, c_sr, scales, s_sb, s);
    case 256: return launch_e<4>(f32, x, B, n, x_sb, x_sr, codes, c_sb, c_sr, scales, s_sb, s);
    case 512: return launch_e<8>(f32, x, B, n, x_sb, x_sr, codes, c_sb, c_sr, scales, s_sb, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ds4attn
