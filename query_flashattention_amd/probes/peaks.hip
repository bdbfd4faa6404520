// Achievable peaks of the device, measured beside the published ones: a
// streaming read of a buffer much larger than the last-level cache (HBM read
// bandwidth) and a loop of independent float16 MFMA chains with no memory traffic
// (matrix-core throughput, and the shader clock it runs at).  Measurement probes
// only: nothing on the attention path calls them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ds4probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Each thread reads 16-byte words at a grid stride, kUnroll loads in flight, and
// writes one word of their XOR, so that no load can be dropped.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                               uint32_t *__restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Eight independent accumulator chains of v_mfma_f32_16x16x32_f16 per wave.  The
// operands depend on the thread index so that nothing folds away; the wave's
// shader-clock cycles (s_memtime) and 100 MHz reference ticks (s_memrealtime)
// over the loop give the clock the matrix cores ran at.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float *__restrict__ out,
                                                             unsigned long long *__restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (_Float16)(0.001f * (float)((lane + k) & 7));
    b[k] = (_Float16)(0.002f * (float)((lane * 3 + k) & 7));
  }
  floatx4 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = floatx4{0.f, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  floatx4 s = c[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) s += c[k];
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  out[gtid] = s.x + s.y + s.z + s.w;
  if (lane == 0) {
    const int64_t wave = gtid >> 6;
    clocks[2 * wave] = t1 - t0;
    clocks[2 * wave + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int ds4probe_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t grid, void *stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || grid < 1 || ((uintptr_t)buf & 15)) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int ds4probe_mfma_loop(int32_t iters, float *out, unsigned long long *clocks, int32_t grid,
                                  void *stream) {
  if (!out || !clocks || iters < 1 || grid < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, iters, out,
                     clocks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int64_t ds4probe_mfma_loop_flops(int32_t iters, int32_t grid) {
  return (int64_t)grid * (kThreads / 64) * iters * 8 * (2LL * 16 * 16 * 32);
}
