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
// float32 sum in CSR order (the shared row added last), one rounding into y. WPT waves per
// token (more than one when there are few tokens), each taking every WPT-th block of 1024
// columns: the token's row indices and weights sit one per lane and are broadcast; each step
// issues the loads of two rows x CH column chunks (16 bytes of o per lane per chunk) before
// the multiply-adds, so several rows' loads are in flight at once. A missing second row of a
// pair reads the first row again with weight 0, which leaves the sum unchanged
// (fma(0, v, acc) = acc for finite v), so the result equals the row-by-row sum.
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

// 16-byte load of o; streaming (non-temporal) when the rows the combine reads far exceed the
// last-level cache, so they do not push out each other's lines
template <bool NT> MOE_DEV float4 load_o(const float *p) {
  if constexpr (NT) {
    const f32x4v_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t *>(p));
    return make_float4(q.x, q.y, q.z, q.w);
  } else {
    return *reinterpret_cast<const float4 *>(p);
  }
}

template <typename TY, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ o,
                                                      const float *__restrict__ o_shared,
                                                      const int32_t *__restrict__ tok_ptr,
                                                      const int32_t *__restrict__ tok_pos,
                                                      const float *__restrict__ perm_w,
                                                      TY *__restrict__ y, int Tn, int d, int wpt) {
  constexpr int CH = 4;   // 256-column chunks per step
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);   // global wave
  const int t = gw / wpt, part = gw % wpt;
  if (t >= Tn) return;
  const int b = tok_ptr[t], n = tok_ptr[t + 1] - b;
  // uniform over the wave (the shuffles below)
  for (int cb = part * 256 * CH; cb < d; cb += wpt * 256 * CH) {
    const int c0 = cb + lane * 4;
    float4 acc[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int rb = 0; rb < n; rb += 64) {   // rows in blocks of 64, one per lane
    const int m = min(64, n - rb);
    const int my_p = lane < m ? tok_pos[b + rb + lane] : 0;
    const float my_w = lane < m ? perm_w[my_p] : 0.f;
    for (int j = 0; j < m; j += 2) {
      const int p0 = __shfl(my_p, j, 64);
      const float w0 = __shfl(my_w, j, 64);
      const bool two = j + 1 < m;
      const int p1 = two ? __shfl(my_p, j + 1, 64) : p0;
      const float w1 = two ? __shfl(my_w, j + 1, 64) : 0.f;
      float4 v0[CH], v1[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int c = c0 + u * 256;
        if (c < d) {
          v0[u] = load_o<NT>(o + (size_t)p0 * d + c);
          v1[u] = load_o<NT>(o + (size_t)p1 * d + c);
        } else {
          v0[u] = v1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        acc[u].x = fmaf(w0, v0[u].x, acc[u].x); acc[u].y = fmaf(w0, v0[u].y, acc[u].y);
        acc[u].z = fmaf(w0, v0[u].z, acc[u].z); acc[u].w = fmaf(w0, v0[u].w, acc[u].w);
        acc[u].x = fmaf(w1, v1[u].x, acc[u].x); acc[u].y = fmaf(w1, v1[u].y, acc[u].y);
        acc[u].z = fmaf(w1, v1[u].z, acc[u].z); acc[u].w = fmaf(w1, v1[u].w, acc[u].w);
      }
    }
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = c0 + u * 256;
      if (c >= d) break;
      float4 a = acc[u];
      if (o_shared) {
        const float4 v = load_o<NT>(o_shared + (size_t)t * d + c);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      }
      TY *yp = y + (size_t)t * d + c;
      if constexpr (sizeof(TY) == 2) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
        pk.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
        *reinterpret_cast<uint2 *>(yp) = pk;
      } else {
        *reinterpret_cast<float4 *>(yp) = a;
      }
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
                          void *y, int T, int d, int max_rows, hipStream_t st) {
  // few tokens: split each row's 1024-column blocks over several waves (about 1024 waves)
  const int blocks = (d + 1023) / 1024;
  int wpt = (1024 + T - 1) / T;
  if (wpt > blocks) wpt = blocks;
  if (wpt < 1) wpt = 1;
  dim3 grid((unsigned)(((long)T * wpt + 3) / 4));
  // bytes of o the combine may read: past ~320 MB (above the 256 MB MALL) streaming loads
  // measured faster (fine-grained layer, 1 GB of o: 174 -> 131 us); below, plain loads win
  const double obytes = ((double)max_rows + (o_shared ? T : 0)) * d * 4.0;
  const bool nt = obytes > 320e6;
#define MOE_COMB(TYY, NTT) hipLaunchKernelGGL((combine_kernel<TYY, NTT>), grid, dim3(256), 0, st, o, \
                                               o_shared, tok_ptr, tok_pos, perm_w, (TYY *)y, T, d, wpt)
  if (y_elt == 2) { if (nt) MOE_COMB(bf16_t, true); else MOE_COMB(bf16_t, false); }
  else { if (nt) MOE_COMB(float, true); else MOE_COMB(float, false); }
#undef MOE_COMB
  return hipGetLastError();
}

}  // namespace moe
