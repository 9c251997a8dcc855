// Achievable-peak microbenchmarks on gfx950, next to the datasheet peaks the layer's kernels
// are measured against. Measurement infrastructure only (libmoe_peak.so, include/moe_peak.h);
// the layer never calls it.
//
//  mfma  every wave of a full grid issues v_mfma_f32_32x32x16_bf16 back to back on register
//        operands (four independent accumulator chains, four operand sets of random bf16
//        rotating so that the multiplier inputs toggle like a GEMM's), no memory traffic:
//        the matrix-core rate the chip sustains under that load, and the shader clock it
//        sustains it at (cycle counter over the 100 MHz real-time counter, per workgroup).
//  lds   every wave reads 16 bytes per lane from LDS back to back (ds_read_b128, addresses
//        spread over all banks), summing what it reads: the LDS read bandwidth per CU.
//  copy  16-byte loads and stores over a buffer (grid-stride, every line read and written
//        once): the HBM stream rate a hand-written kernel reaches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_peak.h"

namespace {

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPeakThreads = 512;   // 8 waves: two per SIMD

__global__ __launch_bounds__(kPeakThreads) void mfma_loop_kernel(const pbf16x8_t *__restrict__ seed,
                                                               float *__restrict__ out,
                                                               uint64_t *__restrict__ clk,
                                                               int iters) {
  const int lane = threadIdx.x & 63;
  pbf16x8_t a0 = seed[lane], a1 = seed[64 + lane], b0 = seed[128 + lane], b1 = seed[192 + lane];
  pf32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c3, 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += (c0[v] + c1[v]) + (c2[v] + c3[v]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

constexpr int kLdsBytes = 64 * 1024;

__global__ __launch_bounds__(kPeakThreads) void lds_read_kernel(float *__restrict__ out, int iters) {
  __shared__ uint4 buf[kLdsBytes / 16];
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += blockDim.x)
    buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  // lane L of wave w reads 16-byte word (w * 64 + L + 512 * j) mod 4096: a wave's 64 reads
  // cover 1 KB of consecutive words, so every access spreads over all banks
  const int base = threadIdx.x;
  uint32_t acc0 = 0, acc1 = 0, acc2 = 0, acc3 = 0;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = buf[(base + 512 * j + 64 * (i & 7)) & (kLdsBytes / 16 - 1)];
      acc0 += v.x; acc1 ^= v.y; acc2 += v.z; acc3 ^= v.w;
    }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc0 + acc1 + acc2 + acc3);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src,
                                                  uint4 *__restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {   // four loads in flight per lane
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a; dst[i + stride] = b; dst[i + 2 * stride] = c; dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int moe_peak_mfma(const void *seed, float *out, uint64_t *clk, int grid, int iters,
                  hipStream_t stream) {
  if (!seed || !out || !clk || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(kPeakThreads), 0, stream,
                     (const pbf16x8_t *)seed, out, clk, iters);
  return (int)hipGetLastError();
}

int moe_peak_lds(float *out, int grid, int iters, hipStream_t stream) {
  if (!out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(lds_read_kernel, dim3(grid), dim3(kPeakThreads), 0, stream, out, iters);
  return (int)hipGetLastError();
}

int moe_peak_copy(const void *src, void *dst, size_t bytes, int grid, hipStream_t stream) {
  if (!src || !dst || (bytes & 15) || (((uintptr_t)src | (uintptr_t)dst) & 15) || grid < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, stream, (const uint4 *)src,
                     (uint4 *)dst, bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
