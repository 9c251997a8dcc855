// Shared device helpers of the MoE layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__
#define MOE_HD __host__ __device__ __forceinline__

typedef uint16_t bf16_t;   // bfloat16 storage

namespace moe {

constexpr int kWave = 64;

MOE_DEV float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// round to nearest even (gfx950's v_cvt_pk_bf16_f32); NaN stays NaN
MOE_DEV bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> MOE_DEV float to_f32(T v);
template <> MOE_DEV float to_f32<float>(float v) { return v; }
template <> MOE_DEV float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> MOE_DEV T from_f32(float v);
template <> MOE_DEV float from_f32<float>(float v) { return v; }
template <> MOE_DEV bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// order-preserving map float -> uint32 (larger float -> larger key); -0.0 maps like +0.0
MOE_DEV uint32_t float_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
MOE_DEV int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves: shifts by 1, 2, 4
// and 8 inside each row of 16 lanes, then the last lane of rows 0 and 2 into rows 1 and 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31); a lane with no source lane
// (or outside the row mask) adds 0
MOE_DEV int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// sum over the 64 lanes of a wave with the DPP scan above (lane 63 holds the total)
MOE_DEV int wave_sum_dpp(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// Block-wide exclusive scan of one int per thread; returns the exclusive prefix and
// writes the block total to *total. `smem` needs blockDim.x/64 + 1 ints. Contains barriers.
MOE_DEV int block_excl_scan(int v, int *smem, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == 63) smem[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) { int t = smem[w]; smem[w] = run; run += t; }
    smem[nw] = run;
  }
  __syncthreads();
  int res = smem[wid] + inc - v;
  *total = smem[nw];
  __syncthreads();
  return res;
}

// N independent exclusive scans over the block at once (thread order), two barriers in
// all. smem: (blockDim.x/64) * N + N ints. total[c] gets the block total of column c.
template <int N>
MOE_DEV void block_excl_scan_vec(int (&v)[N], int *smem, int (&total)[N]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc[N];
#pragma unroll
  for (int c = 0; c < N; ++c) inc[c] = wave_incl_scan(v[c]);
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < N; ++c) smem[wid * N + c] = inc[c];
  __syncthreads();
  if (threadIdx.x < N) {
    const int c = threadIdx.x;
    int run = 0;
    for (int w = 0; w < nw; ++w) { const int t = smem[w * N + c]; smem[w * N + c] = run; run += t; }
    smem[nw * N + c] = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const int ex = smem[wid * N + c] + inc[c] - v[c];
    total[c] = smem[nw * N + c];
    v[c] = ex;
  }
  __syncthreads();
}

MOE_DEV float block_sum(float v, float *smem) {   // smem: blockDim.x/64 floats; contains barriers
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) smem[wid] = v;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < nw; ++w) r += smem[w];      // fixed order: deterministic
  __syncthreads();
  return r;
}
MOE_DEV float block_max(float v, float *smem) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  if (lane == 0) smem[wid] = v;
  __syncthreads();
  float r = smem[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, smem[w]);
  __syncthreads();
  return r;
}

}  // namespace moe
