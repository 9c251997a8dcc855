// Row movement of the MoE layer: the dispatch gather and the gate-weighted combine
// (gfx950). Both are HBM-bound row copies: one wave per row, 16-byte vector accesses,
// contiguous per row, no atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

// x_perm[p] = x[perm_token[p]] for p < offsets[E] (rows are dispatched in expert order).
// Each wave copies one row; a workgroup of 256 threads copies 4 rows.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ x,
                                                          const int32_t *__restrict__ perm_token,
                                                          const int32_t *__restrict__ n_rows_dev,
                                                          uint4 *__restrict__ x_perm,
                                                          int row_vecs, int max_rows) {
  const int n_rows = *n_rows_dev;
  const int lane = threadIdx.x & 63;
  for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < min(n_rows, max_rows); p += gridDim.x * 4) {
    const int t = perm_token[p];
    const uint4 *src = x + (size_t)t * row_vecs;
    uint4 *dst = x_perm + (size_t)p * row_vecs;
    int v = lane;
    for (; v + 192 < row_vecs; v += 256) {   // 4 loads in flight per lane
      const uint4 a = src[v], b = src[v + 64], c = src[v + 128], d = src[v + 192];
      dst[v] = a; dst[v + 64] = b; dst[v + 128] = c; dst[v + 192] = d;
    }
    for (; v < row_vecs; v += 64) dst[v] = src[v];
  }
}

// y[t] = sum_{i in [tok_ptr[t], tok_ptr[t+1])} perm_w[tok_pos[i]] * o[tok_pos[i]] (+ o_shared[t]),
// float32 sum in CSR order (the shared row added last), one rounding into y. One wave per
// token, 4 columns (16 bytes of o) per lane access.
template <typename TY>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const float *__restrict__ o_shared,
                                                      const int32_t *__restrict__ tok_ptr,
                                                      const int32_t *__restrict__ tok_pos,
                                                      const float *__restrict__ perm_w,
                                                      TY *__restrict__ y, int Tn, int d) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int b = tok_ptr[t], e = tok_ptr[t + 1];
  for (int c0 = lane * 4; c0 < d; c0 += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = b; i < e; ++i) {
      const int p = tok_pos[i];
      const float w = perm_w[p];
      const float4 v = *reinterpret_cast<const float4 *>(o + (size_t)p * d + c0);
      acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
    }
    if (o_shared) {
      const float4 v = *reinterpret_cast<const float4 *>(o_shared + (size_t)t * d + c0);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    TY *yp = y + (size_t)t * d + c0;
    if constexpr (sizeof(TY) == 2) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
      *reinterpret_cast<uint2 *>(yp) = pk;
    } else {
      *reinterpret_cast<float4 *>(yp) = acc;
    }
  }
}

hipError_t launch_gather(int elt, const void *x, const int32_t *perm_token,
                         const int32_t *n_rows_dev, void *x_perm, int d, int max_rows,
                         int num_cu, hipStream_t st) {
  const int row_vecs = d * elt / 16;
  int grid = (max_rows + 3) / 4;
  if (grid > num_cu * 16) grid = num_cu * 16;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, st, (const uint4 *)x,
                     perm_token, n_rows_dev, (uint4 *)x_perm, row_vecs, max_rows);
  return hipGetLastError();
}

hipError_t launch_combine(int y_elt, const float *o, const float *o_shared,
                          const int32_t *tok_ptr, const int32_t *tok_pos, const float *perm_w,
                          void *y, int T, int d, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  if (y_elt == 2)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, st, o, o_shared, tok_ptr,
                       tok_pos, perm_w, (bf16_t *)y, T, d);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, st, o, o_shared, tok_ptr,
                       tok_pos, perm_w, (float *)y, T, d);
  return hipGetLastError();
}

}  // namespace moe
