// Router, selection and dispatch-index kernels of the sparse MoE layer (gfx950).
//
// Steps (problem statement of the pages: T tokens, E experts, top-k, capacity gamma):
//   router          l[t,e] = sum_j x[t,j] W_r[j,e] + b[e]                       (fp32)
//   token choice    k largest logits per token, ties to the lower expert; gates =
//                   softmax over all E renormalised over the picks
//   capacity drop   C = floor(gamma*T*k/E); per expert keep the C candidates with the
//                   highest routing score p32 (ties to the lower token)
//   expert choice   c = floor(k*T/E) largest logits per expert column, ties to the
//                   lower token; weight = softmax over the column's T tokens
//   dispatch        per-expert histogram -> exclusive scan -> stable permutation
//                   (ascending token inside an expert), CSR token -> rows
// Integer decisions never depend on summation order or arrival order: histograms are built
// from bit masks and popcounts or from order-independent LDS integer adds, positions from
// prefix scans and wave ballots.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace moe {

// ----------------------------------------------------------------------------------------
// Routing score p32: Cody & Waite exponential (W. J. Cody, W. Waite, Software Manual for
// the Elementary Functions, 1980) on float32 with every operation rounded separately:
// n = rint(x*log2 e); r = (x - n*LN2_HI) - n*LN2_LO with LN2_HI holding only the top 15
// significant bits of ln 2 (so n*LN2_HI is exact); exp(r) from its degree-7 Taylor
// polynomial as 1 + (r + r*(r*(1/2! + r*(1/3! + ... + r/7!)))); times 2^n built in the
// exponent field. Inputs below -87 give +0. Constants are the float32 roundings of
// log2(e), ln 2 (split), and 1/i!.
MOE_DEV float rexp_spec(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;
  const float kLn2Hi = 0x1.62e4p-1f;
  const float kLn2Lo = 0x1.7f7d1cp-20f;
  const float c2 = 0x1.0p-1f, c3 = 0x1.555556p-3f, c4 = 0x1.555556p-5f, c5 = 0x1.111112p-7f,
              c6 = 0x1.6c16c2p-10f, c7 = 0x1.a01a02p-13f;
  if (x < -87.0f) return 0.0f;
  float n = __builtin_rintf(__fmul_rn(x, kLog2e));
  float r = __fsub_rn(__fsub_rn(x, __fmul_rn(n, kLn2Hi)), __fmul_rn(n, kLn2Lo));
  float p = c7;
  p = __fadd_rn(__fmul_rn(p, r), c6);
  p = __fadd_rn(__fmul_rn(p, r), c5);
  p = __fadd_rn(__fmul_rn(p, r), c4);
  p = __fadd_rn(__fmul_rn(p, r), c3);
  p = __fadd_rn(__fmul_rn(p, r), c2);
  p = __fmul_rn(p, r);
  p = __fmul_rn(p, r);
  p = __fadd_rn(p, r);
  p = __fadd_rn(p, 1.0f);
  const float scale = __uint_as_float((uint32_t)((int)n + 127) << 23);
  return __fmul_rn(p, scale);
}

// ----------------------------------------------------------------------------------------
// SIMT router for float32 x, E <= 8 (bf16 x always takes the matrix-core routers: bf16
// problems have d a multiple of 64). A workgroup of 8 waves streams a run of tokens: lane l of wave w owns VEC
// consecutive columns (w*64 + l)*VEC of a 512*VEC-column pass and keeps their W_r rows in
// registers, so W_r is read once per workgroup (per pass); x is read once. Per batch of 8
// tokens each lane accumulates 8 tokens x 8 experts over its columns; a butterfly
// reduce-scatter leaves lane L with the (token L/8, expert L%8) sum of its wave, and the 8
// wave sums are added in wave order.
template <typename XT>
__global__ __launch_bounds__(512) void router_narrow_kernel(const XT *__restrict__ x,
                                                            const float *__restrict__ w,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits, int T,
                                                            int d, int E, int tok_per_blk) {
  constexpr int VEC = 16 / sizeof(XT);
  constexpr int TOK = 8, EP = 8, NW = 8;
  constexpr int PASS = NW * 64 * VEC;
  __shared__ float part[NW][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t_begin = blockIdx.x * tok_per_blk, t_end = min(T, t_begin + tok_per_blk);
  const int npass = (d + PASS - 1) / PASS;
  float wreg[VEC][EP];
  auto load_w = [&](int pass) {
    const int j0 = pass * PASS + (wv * 64 + lane) * VEC;
    if (E == 8 && j0 + VEC <= d) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float4 *wp = reinterpret_cast<const float4 *>(w + (size_t)(j0 + v) * 8);
        const float4 a = wp[0], b = wp[1];
        wreg[v][0] = a.x; wreg[v][1] = a.y; wreg[v][2] = a.z; wreg[v][3] = a.w;
        wreg[v][4] = b.x; wreg[v][5] = b.y; wreg[v][6] = b.z; wreg[v][7] = b.w;
      }
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v)
#pragma unroll
        for (int e = 0; e < EP; ++e)
          wreg[v][e] = (j0 + v < d && e < E) ? w[(size_t)(j0 + v) * E + e] : 0.f;
    }
  };
  if (npass == 1) load_w(0);
  for (int tb = t_begin; tb < t_end; tb += TOK) {
    float acc[TOK][EP];
#pragma unroll
    for (int i = 0; i < TOK; ++i)
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[i][e] = 0.f;
    for (int pass = 0; pass < npass; ++pass) {
      if (npass > 1) load_w(pass);
      const int j0 = pass * PASS + (wv * 64 + lane) * VEC;
      const bool full = j0 + VEC <= d;
      float xv[TOK][VEC];
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        const int t = tb + i;
        if (t < t_end && full) {
          const XT *xp = x + (size_t)t * d + j0;
          if constexpr (sizeof(XT) == 2) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(xp);
            const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              xv[i][2 * v] = __uint_as_float(r4[v] << 16);
              xv[i][2 * v + 1] = __uint_as_float(r4[v] & 0xffff0000u);
            }
          } else {
            const float4 raw = *reinterpret_cast<const float4 *>(xp);
            xv[i][0] = raw.x; xv[i][1] = raw.y; xv[i][2] = raw.z; xv[i][3] = raw.w;
          }
        } else {
#pragma unroll
          for (int v = 0; v < VEC; ++v)
            xv[i][v] = (t < t_end && j0 + v < d) ? to_f32<XT>(x[(size_t)t * d + j0 + v]) : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < TOK; ++i)
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
          for (int e = 0; e < EP; ++e) acc[i][e] = fmaf(xv[i][v], wreg[v][e], acc[i][e]);
    }
    // butterfly reduce-scatter of the 64 (token, expert) sums across the wave
    float v[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = acc[i / EP][i % EP];
#pragma unroll
    for (int o = 32, n = 64; o > 0; o >>= 1, n >>= 1) {
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float send = up ? v[i] : v[i + n / 2];
        const float keep = up ? v[i + n / 2] : v[i];
        v[i] = keep + __shfl_xor(send, o, 64);
      }
    }
    part[wv][lane] = v[0];
    __syncthreads();
    if (wv == 0) {
      const int t = tb + lane / EP, e = lane % EP;
      float sum = part[0][lane];
#pragma unroll
      for (int q = 1; q < NW; ++q) sum += part[q][lane];
      if (t < t_end && e < E) logits[(size_t)t * E + e] = sum + (bias ? bias[e] : 0.f);
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------
// SIMT router for float32 x, E > 8. One workgroup = 4 waves handles 64 tokens x up to 128
// experts (grid.y
// walks expert blocks of 128). x and W_r tiles of 64 columns are staged in LDS; lane l
// owns experts l and l+64, wave w tokens w*16..w*16+15. Each 64-column chunk is summed
// into a fresh partial before being added to the total (two-level float32 sum).
template <typename XT>
__global__ __launch_bounds__(256) void router_wide_kernel(const XT *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits, int T, int d,
                                                          int E) {
  constexpr int TT = 64, BK = 64, TW = 16;
  __shared__ float xs[TT][BK + 4];
  __shared__ float ws[BK][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * 128;
  float acc[TW][2], part[TW][2];
#pragma unroll
  for (int i = 0; i < TW; ++i) acc[i][0] = acc[i][1] = 0.f;
  for (int k0 = 0; k0 < d; k0 += BK) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < TT * BK; idx += 256) {
      const int r = idx / BK, c = idx % BK, t = t0 + r, j = k0 + c;
      xs[r][c] = (t < T && j < d) ? to_f32<XT>(x[(size_t)t * d + j]) : 0.f;
    }
    for (int idx = threadIdx.x; idx < BK * 128; idx += 256) {
      const int r = idx / 128, c = idx % 128, j = k0 + r, e = e0 + c;
      ws[r][c] = (j < d && e < E) ? w[(size_t)j * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TW; ++i) part[i][0] = part[i][1] = 0.f;
    for (int c = 0; c < BK; c += 4) {
      float w0[4], w1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { w0[u] = ws[c + u][lane]; w1[u] = ws[c + u][lane + 64]; }
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const float4 xv = *reinterpret_cast<const float4 *>(&xs[wv * TW + i][c]);
        part[i][0] = fmaf(xv.x, w0[0], part[i][0]); part[i][1] = fmaf(xv.x, w1[0], part[i][1]);
        part[i][0] = fmaf(xv.y, w0[1], part[i][0]); part[i][1] = fmaf(xv.y, w1[1], part[i][1]);
        part[i][0] = fmaf(xv.z, w0[2], part[i][0]); part[i][1] = fmaf(xv.z, w1[2], part[i][1]);
        part[i][0] = fmaf(xv.w, w0[3], part[i][0]); part[i][1] = fmaf(xv.w, w1[3], part[i][1]);
      }
    }
#pragma unroll
    for (int i = 0; i < TW; ++i) { acc[i][0] += part[i][0]; acc[i][1] += part[i][1]; }
  }
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int t = t0 + wv * TW + i;
    if (t >= T) continue;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = e0 + lane + 64 * h;
      if (e < E) logits[(size_t)t * E + e] = acc[i][h] + (bias ? bias[e] : 0.f);
    }
  }
}

// ----------------------------------------------------------------------------------------
// Router on the matrix cores (bf16 x). W_r (float32) is split exactly into three bf16 parts,
// W = hi + mid + lo (hi = bf16(W), mid = bf16(W - hi), lo = W - hi - mid, which fits in bf16
// because each step removes the leading 8 significant bits of a 24-bit value). Every
// product of a bf16 x and a bf16 part is exact in float32, so
//   l = x.hi + x.mid + x.lo  (float32 accumulation)
// gives float32-accurate logits at MFMA rate. The parts are stored transposed, [3][E_pad][d],
// so both MFMA operands stream along d like the expert GEMMs.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));

// Row stride (elements) of the stored W parts: d plus 32, so that the 64-byte pieces the
// MFMA fragment loads take from 16 rows at one K offset do not all fall on the same L2
// channel (measured: +64 B per row runs the wide router 1.3x faster than a 4 KB or 8 KB
// stride; +128 B and +256 B do not help).
MOE_HD int router_w3_ld(int d) { return d + 32; }

__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ w, int d,
                                                           int E, int E_pad,
                                                           bf16_t *__restrict__ w3) {
  const size_t n = (size_t)E_pad * d;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int e = (int)(i / d), j = (int)(i % d);
    const float v = e < E ? w[(size_t)j * E + e] : 0.f;
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const bf16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    const size_t o = (size_t)e * router_w3_ld(d) + j, pl = (size_t)E_pad * router_w3_ld(d);
    w3[o] = hi;
    w3[pl + o] = mid;
    w3[2 * pl + o] = lo;
  }
}

// Wide router (E > 10). A workgroup of 8 waves takes 64 tokens x 128 experts (grid.y walks
// groups of 128 experts); the 64 x 64 slice of x for each K step of 64 goes global -> LDS
// (gfx950 global_load_lds, a three-stage ring, rows of 128 B with 16-byte chunks XOR-swizzled
// by row/2), and wave w streams the W parts of expert block w (16 experts) straight from
// global memory (L2) into a three-slice register ring, two K steps ahead. A wave owns all
// three parts of its experts, so hi, mid and lo sums meet in its registers:
// v_mfma_f32_16x16x32_bf16 over 4 token blocks x 3 parts per K half.
typedef __attribute__((address_space(3))) void rlds_void_t;
typedef __attribute__((address_space(1))) const void rgbl_void_t;
typedef float rf32x4_t __attribute__((ext_vector_type(4)));

MOE_DEV int rswz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

struct XStage { char b[64 * 128]; };

__global__ __launch_bounds__(512) void router_mfma_kernel(const bf16_t *__restrict__ x,
                                                             const bf16_t *__restrict__ w3,
                                                             const float *__restrict__ bias,
                                                             float *__restrict__ logits, int T,
                                                             int d, int E, int E_pad) {
  __shared__ XStage xs0, xs1, xs2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int t0 = blockIdx.x * 64;
  const int eg = blockIdx.y * 128;                   // first expert of the workgroup
  const int neb_all = (min(E_pad - eg, 128)) / 16;   // expert blocks of the workgroup
  constexpr int NEB = 1;
  const int eb0 = wvu;                               // this wave's expert block
  const int ldw = router_w3_ld(d);
  const size_t plane = (size_t)E_pad * ldw;
  const int nk = d / 64;
  // x copies: wave wv fills rows wv*8 .. +7 of a stage with one 1 KB copy
  const int xrow = wvu * 8 + (lane >> 3);
  const uint32_t xoff = (uint32_t)(min(t0 + xrow, T - 1)) * (uint32_t)d +
                        (((lane & 7) ^ ((xrow >> 1) & 7)) * 8);   // elements
  auto copy_x = [&](XStage &st, int kc) {
    __builtin_amdgcn_global_load_lds((rgbl_void_t *)(x + xoff + kc * 64),
                                     (rlds_void_t *)(st.b + wvu * 1024), 16, 0, 0);
  };
  // W fragments: block (eb, part), K half kh: lane l reads row e = l%16 of the block,
  // columns kc*64 + 32 kh + 8 (l/16) .. + 7. Idle waves (fewer expert blocks than waves)
  // re-read the last block and store nothing.
  const bool live = eb0 < neb_all;
  const bf16_t *wrow[NEB][3];
#pragma unroll
  for (int j = 0; j < NEB; ++j)
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int e = eg + min(eb0 + j, neb_all - 1) * 16 + (lane & 15);
      wrow[j][p] = w3 + p * plane + (size_t)e * ldw + 8 * (lane >> 4);
    }
  rbf16x8_t wb[3][NEB][3][2];   // ring of three K slices of W fragments
  rf32x4_t acc[NEB][3][4];
#pragma unroll
  for (int j = 0; j < NEB; ++j)
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[j][p][tb] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  XStage *xs[3] = {&xs0, &xs1, &xs2};
  auto load_w = [&](auto S, int kc) {
#pragma unroll
    for (int j = 0; j < NEB; ++j)
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wb[S.value][j][p][h] = *reinterpret_cast<const rbf16x8_t *>(wrow[j][p] + kc * 64 + h * 32);
  };
  // Step kc (x slice kc in stage kc % 3, W slice kc in wb[kc % 3]): wait for this wave's
  // copy of slice kc (issued two steps back, before the W loads and copy of slice kc+1:
  // 6 NEB + 1 operations may stay in flight; the W loads of slice kc went out before its
  // copies, so they have landed too), barrier (every wave's copies landed; every wave is
  // done reading slice kc-1's stage), then the W loads and copies of slice kc+2 (past the
  // end: the last slice again) into the ring entries slice kc-1 used, then the MFMAs.
  constexpr int INFLIGHT = 6 * NEB + 1;
  static_assert(INFLIGHT < 64, "vmcnt field");
  auto step = [&](auto S, int kc) {
    constexpr int s = decltype(S)::value, s2 = (s + 2) % 3;
    __builtin_amdgcn_s_waitcnt((INFLIGHT & 15) | ((INFLIGHT >> 4) << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_w(std::integral_constant<int, s2>{}, min(kc + 2, nk - 1));
    copy_x(*xs[s2], min(kc + 2, nk - 1));
    __builtin_amdgcn_sched_barrier(0);   // the prefetch goes out before the MFMAs
    const XStage &cur = *xs[s];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      rbf16x8_t a[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        a[tb] = *reinterpret_cast<const rbf16x8_t *>(cur.b + rswz(tb * 16 + (lane & 15), 4 * h + (lane >> 4)));
#pragma unroll
      for (int j = 0; j < NEB; ++j)
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            acc[j][p][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], wb[s][j][p][h], acc[j][p][tb], 0, 0, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // prologue in the order the steps assume: slice 0 (W, x), then slice 1
  load_w(I0{}, 0);
  copy_x(xs0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(I1{}, min(1, nk - 1));
  copy_x(xs1, min(1, nk - 1));
  __builtin_amdgcn_sched_barrier(0);
  int kc = 0;
  for (; kc + 3 <= nk; kc += 3) {
    step(I0{}, kc);
    step(I1{}, kc + 1);
    step(I2{}, kc + 2);
  }
  if (kc < nk) step(I0{}, kc);
  if (kc + 1 < nk) step(I1{}, kc + 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // the surplus loads and copies of the last steps
  if (!live) return;
  // lane l holds tokens 4*(l/16) + i of each block of 16, expert l%16 of each block
#pragma unroll
  for (int j = 0; j < NEB; ++j) {
    const int e = eg + (eb0 + j) * 16 + (lane & 15);
    if (eb0 + j >= neb_all || e >= E) continue;
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + tb * 16 + 4 * (lane >> 4) + i;
        if (t < T) logits[(size_t)t * E + e] = ((acc[j][0][tb][i] + acc[j][1][tb][i]) + acc[j][2][tb][i]) + b;
      }
  }
}

// Wide router for E_pad a multiple of 128: a workgroup of 8 waves takes 128 tokens x 64
// experts (grid.y walks groups of 64 experts), so a K step moves 16 KB of x and 24 KB of W
// parts into the CU instead of 8 KB and 48 KB (flop per byte 77 instead of 55: the 64-token
// kernel above is bound by the CU's load pipe, and the fine-grained layer's router took 34 us
// with x in the last-level cache, 53 us with x in HBM). Both operands go global -> LDS with
// 16-byte buffer loads into LDS (rows of 128 B, chunks XOR-swizzled by row/2 as above): x in
// a ring of 4 stages issued 3 K steps ahead (it streams from HBM), the W parts in a ring of 3
// issued 2 steps ahead (they stay in L2). Wave w computes tokens 64 (w / 4) .. + 63 against
// expert block w % 4 (16 experts), all three parts, so hi, mid and lo meet in its registers
// and every logit sums its K steps in the same order as the 64-token kernel. Rows past T and
// past E_pad are loads beyond the buffer (zeros, no memory traffic).
constexpr int kRwTM = 128, kRwEN = 64;
constexpr int kRwXBytes = kRwTM * 128;       // one K step of x: 128 rows x 64 bf16
constexpr int kRwWBytes = 3 * kRwEN * 128;   // one K step of W: 3 parts x 64 rows x 64 bf16
constexpr int kRwXStages = 4, kRwWStages = 3;

MOE_DEV void rw_copy(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (rlds_void_t *)lds, 16, (int)voff, 0, 0, 0);
}

__global__ __launch_bounds__(512) void router_mfma128_kernel(const bf16_t *__restrict__ x,
                                                             const bf16_t *__restrict__ w3,
                                                             const float *__restrict__ bias,
                                                             float *__restrict__ logits, int T,
                                                             int d, int E, int E_pad) {
  __shared__ __attribute__((aligned(16))) char lds[kRwXStages * kRwXBytes + kRwWStages * kRwWBytes];
  constexpr uint32_t kOut = 0x80000000u;   // offset beyond either buffer
  const int lane = threadIdx.x & 63;
  const int wvu = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int t0 = blockIdx.x * kRwTM, eg = blockIdx.y * kRwEN;
  const int tq = wvu >> 2, eb = wvu & 3;
  const uint32_t ldw = (uint32_t)router_w3_ld(d), plane = (uint32_t)E_pad * ldw;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(x), (short)0, (int)((uint32_t)T * (uint32_t)d * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(w3), (short)0, (int)(3u * plane * 2u), 0x00020000);
  // byte offsets (K step 0) of this lane's 16-byte chunks: x rows 16 w + 8 c + lane/8 (c < 2),
  // W stage rows 24 w + 8 c + lane/8 (c < 3), stage row R = part * 64 + expert
  uint32_t xo[2], wo[3];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 16 * wvu + 8 * c + (lane >> 3);
    xo[c] = t0 + r < T ? ((uint32_t)(t0 + r) * (uint32_t)d + 8u * ((lane & 7) ^ ((r >> 1) & 7))) * 2u : kOut;
  }
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int R = 24 * wvu + 8 * c + (lane >> 3), p = R >> 6, e = eg + (R & 63);
    wo[c] = e < E_pad ? ((uint32_t)p * plane + (uint32_t)e * ldw + 8u * ((lane & 7) ^ ((R >> 1) & 7))) * 2u : kOut;
  }
  auto issue_x = [&](int kc) {
    char *dst = lds + (kc & 3) * kRwXBytes + wvu * 2048;
#pragma unroll
    for (int c = 0; c < 2; ++c) rw_copy(rx, dst + c * 1024, xo[c] == kOut ? kOut : xo[c] + (uint32_t)kc * 128u);
  };
  auto issue_w = [&](int kc) {
    char *dst = lds + kRwXStages * kRwXBytes + (kc % 3) * kRwWBytes + wvu * 3072;
#pragma unroll
    for (int c = 0; c < 3; ++c) rw_copy(rw, dst + c * 1024, wo[c] == kOut ? kOut : wo[c] + (uint32_t)kc * 128u);
  };
  rf32x4_t acc[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[p][tb] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = d / 64;
  // issue order: x0, x1, x2, W0, W1 here, then at step s W(s+2) and x(s+3). Loads complete in
  // issue order, so at step s, with s >= 2 and s + 2 < nk, the copies issued after W(s) are
  // x(s+1), W(s+1) and x(s+2): waiting until at most 7 are in flight leaves W(s) and x(s)
  // landed. Other steps wait for everything.
  issue_x(0);
  if (nk > 1) issue_x(1);
  if (nk > 2) issue_x(2);
  issue_w(0);
  if (nk > 1) issue_w(1);
  for (int kc = 0; kc < nk; ++kc) {
    if (kc >= 2 && kc + 2 < nk)
      __builtin_amdgcn_s_waitcnt((7 & 15) | (0 << 14) | (7 << 4) | (0xF << 8));
    else
      __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | (7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kc + 2 < nk) issue_w(kc + 2);
    if (kc + 3 < nk) issue_x(kc + 3);
    __builtin_amdgcn_sched_barrier(0);   // the prefetch goes out before the MFMAs
    const char *xs = lds + (kc & 3) * kRwXBytes;
    const char *ws = lds + kRwXStages * kRwXBytes + (kc % 3) * kRwWBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      rbf16x8_t a[4], b[3];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        a[tb] = *reinterpret_cast<const rbf16x8_t *>(xs + rswz(tq * 64 + tb * 16 + (lane & 15), 4 * h + (lane >> 4)));
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[p] = *reinterpret_cast<const rbf16x8_t *>(ws + rswz(p * 64 + eb * 16 + (lane & 15), 4 * h + (lane >> 4)));
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[p][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], b[p], acc[p][tb], 0, 0, 0);
    }
  }
  // lane l holds tokens 4 (l/16) + i of each block of 16, expert l % 16 of the wave's block
  const int e = eg + eb * 16 + (lane & 15);
  if (e >= E) return;
  const float bv = bias ? bias[e] : 0.f;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + tq * 64 + tb * 16 + 4 * (lane >> 4) + i;
      if (t < T) logits[(size_t)t * E + e] = ((acc[0][tb][i] + acc[1][tb][i]) + acc[2][tb][i]) + bv;
    }
}

// ----------------------------------------------------------------------------------------
// Router, bf16 x and E <= 10, on the matrix cores, reading the float32 W_r itself. The three
// bf16 parts of W_r (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid)) form the 3E
// rows of a 32-row B operand: row p*E + e holds part p of column e, rows 3E..31 are zero. A
// workgroup of 8 waves takes 16 tokens (32 when T >= 8192); wave w sums its share of the
// 64-column units of d (units w, w + 8, ...) with v_mfma_f32_16x16x32_bf16 (A: 16 token rows
// of x, B: the two 16-row halves of the part operand). For each unit a wave loads the two
// float32 blocks W_r[j0 .. j0+31][0 .. E) of its 32-column K steps (128 E contiguous bytes
// each, 16 bytes per lane), every lane splits its 4 elements of each once and writes the parts
// into the wave's two LDS tiles in the operand's layout (32 rows of 32 bf16), and each lane
// reads its four fragments back with 16-byte LDS reads: W_r is read as it is, with no separate
// split pass, and one LDS round trip serves a whole unit. The loads run kNarrowRing units ahead
// of the arithmetic in a ring of registers: a slot's next unit is requested as soon as its
// current unit is consumed, so a wave keeps issuing loads while it splits and multiplies
// instead of issuing all of them first (a CU's load pipe takes one 16-byte-per-lane load every
// few cycles, and a wave that issued its whole share up front left its arithmetic waiting
// behind the queue: Mixtral-shaped route stage 28.1 -> 25.1 us with a ring of 2 units; 4 and 6
// units measured slower than 2, and 1 slower still). Rows past T, W_r chunks past the block and
// units past the end are buffer loads beyond the buffer, which return zeros and read nothing.
// The workgroups walk the units in rotated order (workgroup b starts at unit 8 (b mod nu/8)),
// so that they do not all read the same W_r lines from L2 at the same moment. The 8 partial
// 16 x 32 tiles are added in wave order in LDS, then each logit is (hi + mid) + lo + bias;
// every token's sums run in the order its workgroup fixes.
constexpr int kNarrowRows = 32;
constexpr int kNarrowMaxE = 10;
constexpr int kNarrowRing = 2;    // units in flight per wave
constexpr int kNarrowWaves = 8;   // waves per workgroup (16 measured no faster)
constexpr int kBlkMaxE = kBlkCountMaxE;
constexpr int kWtRowBytes = 80;   // LDS row stride of a part tile: 64 B of data + 16 B pad
constexpr int kNarrowTileBytes = kNarrowRows * kWtRowBytes;

// Token-choice top-k of one token on a group of G lanes (G = 8 for E <= 8, else 16), lane gl
// holding expert gl's logit (-inf past E), with topk_kernel's arithmetic for the same E and G:
// k rounds of group argmax by (logit desc, expert asc) in the same butterfly, gate numerators
// exp(l - max) over the first pick's logit, the renormalisation mass of the first kden picks in
// pick order or the full softmax sum in butterfly order, and the routing keys of the capacity
// forms (q_e = rexp_spec(l_e - max), S = q_0 + q_1 + ... left to right, key = q_e / S). Lane r
// of the group keeps pick r and writes it. With cnt (LDS, one int per expert) every pick is
// also counted there; with prow / grow (LDS rows of k entries) the picks and their gates are
// also kept there. Every lane of the group must call this (the butterflies use them all).
template <int G>
MOE_DEV void topk_lanes(float lv, int gl, bool live, int t, int E, const TopkOut &o, int *cnt,
                        int *prow = nullptr, float *grow = nullptr) {
  const int lane = threadIdx.x & 63, g0 = lane - gl;   // first lane of this group
  bool taken = false;
  float mx = 0.f, qsum = 0.f, myq = 0.f;
  int myid = 0;
  for (int r = 0; r < o.k; ++r) {   // o.k is uniform: every lane runs the same rounds
    float bv = (gl < E && !taken) ? lv : -INFINITY;
    int be = (gl < E && !taken) ? gl : 0x7fffffff;
#pragma unroll
    for (int s = G / 2; s > 0; s >>= 1) {
      const float ov = __shfl_xor(bv, s, 64);
      const int oe = __shfl_xor(be, s, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (r == 0) mx = bv;
    if (be == gl) taken = true;
    const float q = expf(bv - mx);
    if (r < o.kden) qsum += q;
    if (gl == r) { myq = q; myid = be; }
    if (gl == r && live && cnt) atomicAdd(&cnt[be], 1);   // LDS integer add: order-free
  }
  float denom = qsum;
  if (!o.renorm) {
    float s = gl < E ? expf(lv - mx) : 0.f;
#pragma unroll
    for (int d = G / 2; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
    denom = s;
  }
  if (gl < o.k && live) {
    o.ids[(size_t)t * o.k + gl] = myid;
    o.gates[(size_t)t * o.k + gl] = myq / denom;
    if (prow) { prow[gl] = myid; grow[gl] = myq / denom; }
  }
  if (o.want_key) {
    const float qv = gl < E ? rexp_spec(__fsub_rn(lv, mx)) : 0.f;
    float S = __shfl(qv, g0, 64);
    for (int e = 1; e < E; ++e) S = __fadd_rn(S, __shfl(qv, g0 + e, 64));
    const float qp = __shfl(qv, g0 + (gl < o.k ? myid : 0), 64);
    if (gl < o.k && live) o.keys[(size_t)t * o.k + gl] = qp / S;
  }
}

template <int TB, int NCH>   // NCH: 16-byte W_r chunks per lane and block (1: E <= 8, 2: E <= 10)
__global__ __launch_bounds__(64 * kNarrowWaves) void router_mfma_narrow_kernel(const bf16_t *__restrict__ x,
                                                                 const float *__restrict__ w,
                                                                 const float *__restrict__ bias,
                                                                 float *__restrict__ logits,
                                                                 int T, int d, int E,
                                                                 TopkOut topk,
                                                                 int32_t *__restrict__ blk_cnt,
                                                                 RouterExtra ex,
                                                                 BlkDispatchOut disp) {
  constexpr int U = kNarrowRing;
  constexpr int TT = 16 * TB;   // tokens per workgroup
  constexpr int NW = kNarrowWaves, NT = 64 * NW;
  __shared__ float part[NW][TT * kNarrowRows];
  __shared__ __attribute__((aligned(16))) char wt[NW][2 * kNarrowTileBytes];   // two per wave
  __shared__ int cnt[kNarrowMaxE];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TT;
  const int kq = 8 * (lane >> 4);   // this lane's 8 columns inside a 32-column MFMA step
  const int nchunk = 8 * E;         // 16-byte chunks of a 32-column block of W_r
  // buffer loads: a lane whose row is past T, whose W_r chunk is past the block, or whose unit
  // is past the end gets an offset beyond the buffer, which returns zeros and reads nothing
  constexpr uint32_t kOut = 0x80000000u;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(x), (short)0, (int)((uint32_t)T * (uint32_t)d * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(w), (short)0, (int)((uint32_t)d * (uint32_t)E * 4u), 0x00020000);
  uint32_t xoff[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int tr = t0 + 16 * b + (lane & 15);
    xoff[b] = tr < T ? ((uint32_t)tr * (uint32_t)d + (uint32_t)kq) * 2u : kOut;
  }
  char *tile = wt[wv];
  // the part rows this lane writes: element i of its chunk(s) is W_r[j0 + f / E][f % E],
  // f = 4 c + i; its part p goes to row p E + f % E, column f / E of the tile
  // rows 3E..31 stay zero: cleared once
  for (int i = lane; i < 2 * kNarrowTileBytes / 4; i += 64)
    reinterpret_cast<uint32_t *>(tile)[i] = 0u;
  if (threadIdx.x < kNarrowMaxE) cnt[threadIdx.x] = 0;
  rf32x4_t acc0[TB], acc1[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) acc0[b] = acc1[b] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nu = d / 64;
  const int rot = (nu % 8 == 0) ? (int)(blockIdx.x % (unsigned)(nu / 8)) * 8 : 0;
  rbf16x8_t a[U][TB][2];
  float4 wr[U][2][NCH];   // raw float32 W_r chunks: [slot][half][chunk lane (+ 64)]
  // loads of unit ui into ring slot v (none past the end: ui >= nu reads nothing)
  auto issue = [&](int v, int ui) {
    const bool live = ui < nu;   // wave-uniform
    const int u = live ? (ui + rot) % nu : 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t o = (uint32_t)u * 64u + (uint32_t)h * 32u;   // first column of the block
#pragma unroll
      for (int b = 0; b < TB; ++b)
        a[v][b][h] = __builtin_bit_cast(rbf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
            rx, live && xoff[b] != kOut ? xoff[b] + o * 2u : kOut, 0, 0));
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        const int c = lane + 64 * c2;
        wr[v][h][c2] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
            rw, live && c < nchunk ? o * (uint32_t)E * 4u + (uint32_t)c * 16u : kOut, 0, 0));
      }
    }
  };
  // split both W_r blocks of slot v into the wave's two tiles, then multiply
  auto consume = [&](int v) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      char *th = tile + h * kNarrowTileBytes;
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        const int c = lane + 64 * c2;
        if (c < nchunk) {
          const float vals[4] = {wr[v][h][c2].x, wr[v][h][c2].y, wr[v][h][c2].z, wr[v][h][c2].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int f = 4 * c + i, col = f / E, e = f - col * E;
            const __bf16 hi = (__bf16)vals[i];
            const float r1 = vals[i] - (float)hi;
            const __bf16 mid = (__bf16)r1;
            const __bf16 lo = (__bf16)(r1 - (float)mid);
            char *at = th + e * kWtRowBytes + col * 2;
            *reinterpret_cast<__bf16 *>(at) = hi;
            *reinterpret_cast<__bf16 *>(at + E * kWtRowBytes) = mid;
            *reinterpret_cast<__bf16 *>(at + 2 * E * kWtRowBytes) = lo;
          }
        }
      }
    }
    // the wave's LDS accesses complete in order: the reads below see the writes above
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    rbf16x8_t p[2], q[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const char *th = tile + h * kNarrowTileBytes;
      p[h] = *reinterpret_cast<const rbf16x8_t *>(th + (lane & 15) * kWtRowBytes + kq * 2);
      q[h] = *reinterpret_cast<const rbf16x8_t *>(th + (16 + (lane & 15)) * kWtRowBytes + kq * 2);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();   // every lane has read before the next blocks land
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        acc0[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[v][b][h], p[h], acc0[b], 0, 0, 0);
        acc1[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[v][b][h], q[h], acc1[b], 0, 0, 0);
      }
  };
#pragma unroll
  for (int v = 0; v < U; ++v) issue(v, wv + NW * v);
  for (int ub = wv; ub < nu; ub += NW * U) {
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const int ui = ub + NW * v;
      if (ui < nu) consume(v);   // wave-uniform
      issue(v, ui + NW * U);
    }
  }
  // lane l holds rows 4*(l/16) + i, column l%16 of each 16 x 16 block
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * b + 4 * (lane >> 4) + i;
      part[wv][r * kNarrowRows + (lane & 15)] = acc0[b][i];
      part[wv][r * kNarrowRows + 16 + (lane & 15)] = acc1[b][i];
    }
  __syncthreads();
  constexpr int NS = (TT * kNarrowRows + NT - 1) / NT;   // sums per thread
  float sum[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int idx = j * NT + threadIdx.x;   // token * 32 + row
    if (idx < TT * kNarrowRows) {
      sum[j] = part[0][idx];
#pragma unroll
      for (int q = 1; q < NW; ++q) sum[j] += part[q][idx];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (j * NT + (int)threadIdx.x < TT * kNarrowRows) part[0][j * NT + threadIdx.x] = sum[j];
  __syncthreads();
  float *lg = &part[1][0];   // [TT][E] final logits for the fused top-k
  for (int i = threadIdx.x; i < TT * E; i += NT) {
    const int r = i / E, e = i % E, t = t0 + r;
    const float *sr = &part[0][r * kNarrowRows];
    const float v = ((sr[e] + sr[E + e]) + sr[2 * E + e]) + (bias ? bias[e] : 0.f);
    lg[i] = v;
    if (t < T) logits[(size_t)t * E + e] = v;
  }
  if (ex.logits_t) {   // expert choice: the same logits transposed, expert-major rows of T
    __syncthreads();
    for (int i = threadIdx.x; i < TT * E; i += NT) {
      const int e = i / TT, r = i - e * TT, t = t0 + r;
      if (t < T) ex.logits_t[(size_t)e * T + t] = lg[r * E + e];
    }
  }
  if (!topk.ids) return;   // block-uniform
  __syncthreads();
  int *cp = blk_cnt ? cnt : nullptr;
  // picks and gates of the workgroup's tokens in LDS when it also does the dispatch
  __shared__ int spick[16 * TB * kNarrowMaxE];
  __shared__ float sgate[16 * TB * kNarrowMaxE];
  const bool own = disp.perm_token != nullptr;   // grid-uniform
  if (E <= 8) {
    const int gi = threadIdx.x / 8, gl = threadIdx.x % 8;
    if (gi < TT)   // whole groups of 8 lanes
      topk_lanes<8>(gl < E ? lg[gi * E + gl] : -INFINITY, gl, t0 + gi < T, t0 + gi, E, topk, cp,
                    own ? spick + gi * topk.k : nullptr, own ? sgate + gi * topk.k : nullptr);
  } else {
    const int gi = threadIdx.x / 16, gl = threadIdx.x % 16;
    if (gi < TT)
      topk_lanes<16>(gl < E ? lg[gi * E + gl] : -INFINITY, gl, t0 + gi < T, t0 + gi, E, topk, cp,
                     own ? spick + gi * topk.k : nullptr, own ? sgate + gi * topk.k : nullptr);
  }
  if (!blk_cnt) return;
  __syncthreads();
  if (threadIdx.x < E) blk_cnt[(size_t)blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
  if (!own) return;
  // The one workgroup holds every token (the launcher checks T <= its tokens): the dispatch of
  // token choice without a capacity limit, as dispatch_blocks_kernel writes it: expert offsets
  // from the counts, pair (t, j) of expert e at offsets[e] + (picks of e by tokens before t),
  // token t owning CSR entries t k .. t k + k - 1.
  __shared__ int soff[kNarrowMaxE];
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      soff[e] = run;
      disp.counts[e] = cnt[e];
      disp.offsets[e] = run;
      run += cnt[e];
    }
    disp.offsets[E] = run;
  }
  __syncthreads();
  const int K = topk.k;
  for (int i = threadIdx.x; i < T * K; i += NT) {
    const int t = i / K, e = spick[i];
    int rank = 0;
    for (int q = 0; q < t * K; ++q) rank += spick[q] == e;
    const int pos = soff[e] + rank;
    disp.perm_token[pos] = t;
    disp.perm_w[pos] = sgate[i];
    disp.tok_pos[i] = pos;
    if (disp.kept) disp.kept[i] = 1;
  }
  for (int t = threadIdx.x; t <= T; t += NT) disp.tok_ptr[t] = t * K;
}

// ----------------------------------------------------------------------------------------
// Token-choice top-k. A group of G lanes (G = power of two >= min(E, 64)) handles one
// token; lane i of the group holds experts i, i+G, i+2G, ... Each round takes the group
// maximum (ties: lower expert index). Gates: exp(l - max) normalised over the picks (or
// over all E). With a capacity limit the float32 routing score of each pick is written:
// q_e = rexp_spec(l_e - max), S = q_0 + q_1 + ... left to right, p32 = q_e / S.
template <int G, int MAXPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int kden, int renorm, int want_key,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ gates,
                                                   float *__restrict__ keys,
                                                   int32_t *__restrict__ blk_cnt) {
  extern __shared__ float qsh[];   // [256/G][E] when want_key
  __shared__ int cnt[kBlkMaxE];    // picks per expert of this workgroup's tokens (blk_cnt)
  const int gl = threadIdx.x % G, gi = threadIdx.x / G;
  if (blk_cnt && threadIdx.x < E) cnt[threadIdx.x] = 0;
  if (blk_cnt) __syncthreads();
  const int t = blockIdx.x * (256 / G) + gi;
  const bool live = t < T;
  const int npl = (E + G - 1) / G;   // logits per lane (<= MAXPL)
  float lv[MAXPL];
  uint32_t taken = 0u;
#pragma unroll
  for (int i = 0; i < MAXPL; ++i) {
    const int e = gl + i * G;
    lv[i] = (live && i < npl && e < E) ? logits[(size_t)t * E + e] : -INFINITY;
  }
  float mx = 0.f, qsum = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
      const int e = gl + i * G;
      if (i < npl && e < E && !((taken >> i) & 1u)) {
        const float v = lv[i];
        if (v > bv || (v == bv && e < be) || be == 0x7fffffff) { bv = v; be = e; }
      }
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (r == 0) mx = bv;
    if ((be % G) == gl) taken |= 1u << (be / G);
    const float q = expf(bv - mx);
    if (r < kden) qsum += q;   // renormalisation mass: the first kden picks
    if (gl == 0 && live) {
      ids[(size_t)t * k + r] = be;
      gates[(size_t)t * k + r] = q;   // numerator for now
      if (blk_cnt) atomicAdd(&cnt[be], 1);   // LDS integer add: order does not matter
    }
  }
  float denom = qsum;
  if (!renorm) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
      const int e = gl + i * G;
      if (i < npl && e < E) s += expf(lv[i] - mx);
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    denom = s;
  }
  if (gl == 0 && live) {
    for (int r = 0; r < k; ++r) gates[(size_t)t * k + r] = gates[(size_t)t * k + r] / denom;
  }
  if (blk_cnt) {   // block-uniform
    __syncthreads();
    if (threadIdx.x < E) blk_cnt[(size_t)blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
  }
  if (want_key) {
    float *qrow = qsh + gi * E;
#pragma unroll
    for (int i = 0; i < MAXPL; ++i) {
      const int e = gl + i * G;
      if (i < npl && e < E) qrow[e] = live ? rexp_spec(__fsub_rn(lv[i], mx)) : 0.f;
    }
    __syncthreads();
    if (gl == 0 && live) {
      float S = qrow[0];
      for (int e = 1; e < E; ++e) S = __fadd_rn(S, qrow[e]);
      for (int r = 0; r < k; ++r) {
        const int e = ids[(size_t)t * k + r];
        keys[(size_t)t * k + r] = qrow[e] / S;
      }
    }
  }
}

// Token-choice top-k for 33..128 experts and k <= 8, by merging instead of k rounds of group
// argmax. A group of 16 lanes handles one token, lane i holding experts i, i+16, ... (8 each).
// A (logit, expert) pair is one 64-bit key, the order-preserving image of the logit above
// the complement of the expert index, so that "larger key" is the total order (logit desc,
// expert asc) and a compare-exchange is one 64-bit compare and two selects (the two zeros
// share a key, as they compare equal). Each lane sorts its 8 keys with a 19-comparator
// network; then, for partner distance 8, 4, 2, 1, it takes the partner's sorted list, keeps
// the larger of A[i] and B[7-i] (a bitonic sequence holding the top 8 of both lists) and
// sorts that with a 12-comparator bitonic merge. The order is total, so after four merges
// every lane of the group holds the same sorted top 8: the picks in order. Gates and routing
// keys follow topk_kernel's arithmetic exactly.
MOE_DEV uint64_t pick_key(float v, int e) {
  return ((uint64_t)float_key(v) << 32) | (uint32_t)~(uint32_t)e;
}
MOE_DEV float pick_value(uint64_t k) {   // the logit back (a zero comes back as +0)
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
MOE_DEV int pick_expert(uint64_t k) { return (int)~(uint32_t)k; }
MOE_DEV void key_ce(uint64_t &a, uint64_t &b) {   // a <- the larger, b <- the smaller
  const bool keep = a > b;
  const uint64_t lo = keep ? b : a;
  a = keep ? a : b;
  b = lo;
}

__global__ __launch_bounds__(256) void topk_merge_kernel(const float *__restrict__ logits, int T,
                                                         int E, int k, int kden, int renorm,
                                                         int want_key, int32_t *__restrict__ ids,
                                                         float *__restrict__ gates,
                                                         float *__restrict__ keys) {
  constexpr int G = 16, PL = 8;
  extern __shared__ float qsh[];   // [16][E] when want_key
  const int gl = threadIdx.x % G, gi = threadIdx.x / G;
  const int t = blockIdx.x * (256 / G) + gi;
  const bool live = t < T;
  float lv[PL];
  uint64_t a[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = gl + i * G;
    lv[i] = (live && e < E) ? logits[(size_t)t * E + e] : -INFINITY;
    a[i] = pick_key(lv[i], e < E ? e : 0x7fffffff);
  }
  // sort the lane's 8 keys, largest first (Batcher's odd-even merge sort)
  key_ce(a[0], a[1]); key_ce(a[2], a[3]); key_ce(a[4], a[5]); key_ce(a[6], a[7]);
  key_ce(a[0], a[2]); key_ce(a[1], a[3]); key_ce(a[4], a[6]); key_ce(a[5], a[7]);
  key_ce(a[1], a[2]); key_ce(a[5], a[6]);
  key_ce(a[0], a[4]); key_ce(a[1], a[5]); key_ce(a[2], a[6]); key_ce(a[3], a[7]);
  key_ce(a[2], a[4]); key_ce(a[3], a[5]);
  key_ce(a[1], a[2]); key_ce(a[3], a[4]); key_ce(a[5], a[6]);
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    uint64_t b[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const uint32_t hi = __shfl_xor((uint32_t)(a[i] >> 32), o, 64);
      const uint32_t lo = __shfl_xor((uint32_t)a[i], o, 64);
      b[i] = ((uint64_t)hi << 32) | lo;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (b[PL - 1 - i] > a[i]) a[i] = b[PL - 1 - i];
#pragma unroll
    for (int dd = PL / 2; dd > 0; dd >>= 1)
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if ((i & dd) == 0) key_ce(a[i], a[i + dd]);
  }
  float av[PL];
#pragma unroll
  for (int r = 0; r < PL; ++r) av[r] = pick_value(a[r]);
  const float mx = av[0];
  float qn[PL], qsum = 0.f;
#pragma unroll
  for (int r = 0; r < PL; ++r) {
    qn[r] = expf(av[r] - mx);
    if (r < k && r < kden) qsum += qn[r];
  }
  float denom = qsum;
  if (!renorm) {
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = gl + i * G;
      if (e < E) sm += expf(lv[i] - mx);
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
    denom = sm;
  }
  if (gl == 0 && live) {
#pragma unroll
    for (int r = 0; r < PL; ++r)
      if (r < k) {
        ids[(size_t)t * k + r] = pick_expert(a[r]);
        gates[(size_t)t * k + r] = qn[r] / denom;
      }
  }
  if (want_key) {
    float *qrow = qsh + gi * E;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = gl + i * G;
      if (e < E) qrow[e] = live ? rexp_spec(__fsub_rn(lv[i], mx)) : 0.f;
    }
    __syncthreads();
    if (gl == 0 && live) {
      float S = qrow[0];
      for (int e = 1; e < E; ++e) S = __fadd_rn(S, qrow[e]);
#pragma unroll
      for (int r = 0; r < PL; ++r)
        if (r < k) keys[(size_t)t * k + r] = qrow[pick_expert(a[r])] / S;
    }
  }
}

// ----------------------------------------------------------------------------------------
// Dispatch of token choice without a capacity limit, in one launch, from the per-block expert
// counts the top-k (inside the narrow router or in topk_kernel) left: blk_cnt[b][e] = picks of
// expert e among tokens [bt*b, bt*b + bt). Workgroup w takes tokens [256w, 256w + 256) (a
// whole number of count blocks, bt dividing 256). It sums the count rows of all blocks, and of
// the blocks before its own, in a fixed order (integer sums), which gives the expert offsets
// (exclusive scan over experts) and where each expert's rows of its blocks start; a token's
// rank inside its count block comes from the picks of the block's earlier tokens. Pair (t, j)
// of expert e goes to offsets[e] + (pairs of e among tokens before t): ascending token inside
// an expert, as the general dispatch does. Every pair is kept, so token t owns CSR entries
// t k .. t k + k - 1 in slot order. Workgroup 0 also writes counts and offsets.
constexpr int kBlkPerWg = 256 / 16;   // count blocks per dispatch workgroup (bt >= 16)

template <int EM>   // experts handled: E <= EM (8 or 16)
__global__ __launch_bounds__(256) void dispatch_blocks_kernel(const int32_t *__restrict__ ids,
                                                              const float *__restrict__ gates,
                                                              int T, int k, int E,
                                                              const int32_t *__restrict__ blk_cnt,
                                                              int bt, BlkDispatchOut o) {
  __shared__ int wsum[256 / 64][2 * EM];
  __shared__ int colc[kBlkPerWg][EM];
  __shared__ int base[kBlkPerWg][EM];
  __shared__ int off[EM];
  __shared__ unsigned long long wball[256 / 64][EM];
  __shared__ int sids[256 * EM];
  __shared__ float sgate[256 * EM];
  const bool cand = o.cand_slot != nullptr;   // candidate lists for the capacity selection
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nblk = (T + bt - 1) / bt;
  const int t0 = blockIdx.x * 256, b0 = t0 / bt;
  const int nb = min(256 / bt, nblk - b0);   // count blocks of this workgroup
  const int t = t0 + threadIdx.x;
  // the first count row of this thread (the rows of every block, written by the top-k just
  // before on any XCD, are the longest wait): its loads go out first, then this workgroup's
  // picks and gates (contiguous rows) and its blocks' count rows, so that the waits overlap
  int c0[EM];
  {
    const int r = threadIdx.x;
#pragma unroll
    for (int e = 0; e < EM; ++e) c0[e] = r < nblk ? blk_cnt[(size_t)r * E + min(e, E - 1)] : 0;
  }
  const int nown = (min(T, t0 + 256) - t0) * k;
  for (int i = threadIdx.x; i < nown; i += 256) {
    sids[i] = ids[(size_t)t0 * k + i];
    sgate[i] = gates[(size_t)t0 * k + i];
  }
  {
    const int eb = threadIdx.x % EM, bb = threadIdx.x / EM;
    if (bb < kBlkPerWg)
      colc[bb][eb] = (eb < E && bb < nb) ? blk_cnt[(size_t)(b0 + bb) * E + eb] : 0;
  }
  // per expert: picks of all blocks (va) and of the blocks before b0 (vp); thread i adds rows
  // i, i + 256, ... (integer sums: the order does not change them)
  int va[EM], vp[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int ce = (e < E && (int)threadIdx.x < nblk) ? c0[e] : 0;
    va[e] = ce;
    vp[e] = (int)threadIdx.x < b0 ? ce : 0;
  }
  for (int r = threadIdx.x + 256; r < nblk; r += 256) {
    int c[EM];
#pragma unroll
    for (int e = 0; e < EM; ++e) c[e] = blk_cnt[(size_t)r * E + min(e, E - 1)];
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      const int ce = e < E ? c[e] : 0;
      va[e] += ce;
      vp[e] += r < b0 ? ce : 0;
    }
  }
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int a = wave_sum_dpp(va[e]), b = wave_sum_dpp(vp[e]);
    if (lane == 0) { wsum[wid][e] = a; wsum[wid][EM + e] = b; }
  }
  __syncthreads();
  // expert offsets (exclusive scan over experts), where this workgroup's blocks start inside
  // every expert, and each wave's expert masks for the ranks; with candidate lists also the
  // capacity-capped counts and offsets of the final rows
  if (threadIdx.x == 0) {
    int run = 0, run_fin = 0;
    for (int e = 0; e < E; ++e) {
      const int all = wsum[0][e] + wsum[1][e] + wsum[2][e] + wsum[3][e];
      off[e] = run;
      if (blockIdx.x == 0) {
        o.counts[e] = all;
        o.offsets[e] = run;
        if (cand) {
          const int kc = min(all, o.C);
          o.cnt_fin[e] = kc;
          o.off_fin[e] = run_fin;
          run_fin += kc;
        }
      }
      run += all;
    }
    if (blockIdx.x == 0) {
      o.offsets[E] = run;
      if (cand) o.off_fin[E] = run_fin;
    }
  }
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    int run = wsum[0][EM + e] + wsum[1][EM + e] + wsum[2][EM + e] + wsum[3][EM + e];
#pragma unroll
    for (int b = 0; b < kBlkPerWg; ++b) {
      base[b][e] = run;
      run += colc[b][e];
    }
  }
  uint32_t mine = 0u;   // experts this token picked
  if (t < T)
    for (int j = 0; j < k; ++j) mine |= 1u << sids[threadIdx.x * k + j];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const unsigned long long m = __ballot((mine >> e) & 1u);
    if (lane == 0) wball[wid][e] = m;
  }
  __syncthreads();
  if (t >= T) return;
  // each pair's position: pairs of its expert among the earlier tokens of its count block
  // (count blocks of 16 or 32 tokens lie inside one wave: a ballot gives them)
  const int lb = threadIdx.x / bt;
  const int first_lane = lane - (threadIdx.x % bt);
  const unsigned long long before = ((1ull << lane) - 1ull) & ~((1ull << first_lane) - 1ull);
  if (!cand) {
    o.tok_ptr[t] = t * k;
    if (t == T - 1) o.tok_ptr[T] = T * k;
  }
  for (int j = 0; j < k; ++j) {
    const int e = sids[threadIdx.x * k + j];
    const int rank = __popcll(wball[wid][e] & before);
    const int pos = off[e] + base[lb][e] + rank;
    o.perm_token[pos] = t;
    o.perm_w[pos] = sgate[threadIdx.x * k + j];
    if (cand) {
      o.cand_slot[pos] = j;
      o.cand_key[pos] = o.keys[(size_t)t * k + j];
    } else {
      o.tok_pos[(size_t)t * k + j] = pos;
      if (o.kept) o.kept[(size_t)t * k + j] = 1;
    }
  }
}

// ----------------------------------------------------------------------------------------
// Dispatch histogram. Block b owns tokens [256b, 256b+256). Each token has a row of S slots
// (expert ids); the pairs taken are the slots in [j0, j1), minus those with kept == 0 when a
// kept array is given, and a pair's bucket is its expert / gs (gs = 1: one bucket per
// expert; gs = E/D: one per group of experts). A token can have up to `mult` pairs in one
// bucket. For every bucket and c < mult a 256-bit mask marks the block's tokens with more
// than c pairs in it (LDS atomicOr of distinct bits, order free), so popcounts give the
// block's per-bucket counts and, in the scatter, each pair's rank: pairs of lower tokens
// first, a token's own pairs in slot order.
struct PairSel {
  const uint8_t *kept;
  int S, j0, j1, gs, mult;
};

constexpr int kMaxSlots = 16;   // pairs of one token in one bucket are tracked up to k <= 16
constexpr int kSlotBatch = 8;   // slots of a token whose loads are issued together

// Buckets of slots j .. j + kSlotBatch - 1 of token t (-1: past j1, or not kept), all loads
// issued before any is used.
MOE_DEV void slot_buckets(const int32_t *ids, const PairSel &f, int t, int j,
                          int (&bk)[kSlotBatch]) {
#pragma unroll
  for (int i = 0; i < kSlotBatch; ++i) {
    int b = -1;
    if (j + i < f.j1) {
      const size_t ij = (size_t)t * f.S + j + i;
      const int id = ids[ij];
      const bool kp = !f.kept || f.kept[ij];
      b = kp ? (f.gs == 1 ? id : id / f.gs) : -1;
    }
    bk[i] = b;
  }
}

MOE_DEV void build_masks(uint32_t *mask, const int32_t *ids, const PairSel &f, int T, int B) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  int bk[kSlotBatch];   // the first batch travels while the masks are cleared
  if (t < T) slot_buckets(ids, f, t, f.j0, bk);
  for (int i = threadIdx.x; i < B * f.mult * 8; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  if (t < T) {
    int seen[kMaxSlots];
    int ns = 0;
    for (int j = f.j0; j < f.j1; j += kSlotBatch) {
      if (j > f.j0) slot_buckets(ids, f, t, j, bk);
#pragma unroll
      for (int i = 0; i < kSlotBatch; ++i) {
        const int b = bk[i];
        if (b < 0) continue;
        int c = 0;
        if (f.mult > 1) {
          for (int q = 0; q < ns; ++q) c += seen[q] == b;
          seen[ns++] = b;
        }
        atomicOr(&mask[(b * f.mult + c) * 8 + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void assign_count_kernel(const int32_t *__restrict__ ids, int T,
                                                           PairSel f, int B,
                                                           int32_t *__restrict__ blk_cnt) {
  extern __shared__ uint32_t mask[];
  build_masks(mask, ids, f, T, B);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    int c = 0;
    for (int m = 0; m < f.mult; ++m)
#pragma unroll
      for (int w = 0; w < 8; ++w) c += __popc(mask[(b * f.mult + m) * 8 + w]);
    blk_cnt[(size_t)blockIdx.x * B + b] = c;
  }
}

// Column scans of the block counts (one thread per bucket, blocks in order), bucket
// totals, exclusive scan over buckets. With a capacity C >= 0 the kept counts are
// min(count, C) and a second offset table is produced for them.
__global__ __launch_bounds__(1024) void assign_scan_kernel(const int32_t *__restrict__ blk_cnt,
                                                           int nblk, int E, int C,
                                                           int32_t *__restrict__ blk_base,
                                                           int32_t *__restrict__ cnt_pre,
                                                           int32_t *__restrict__ off_pre,
                                                           int32_t *__restrict__ cnt_fin,
                                                           int32_t *__restrict__ off_fin) {
  __shared__ int sm[1024 / 64 + 1];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {   // eight independent loads in flight, then the scan
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = blk_cnt[(size_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        blk_base[(size_t)(b + i) * E + e] = run;
        run += c[i];
      }
    }
    for (; b < nblk; ++b) {
      const int c = blk_cnt[(size_t)b * E + e];
      blk_base[(size_t)b * E + e] = run;
      run += c;
    }
    cnt_pre[e] = run;
  }
  int tot;
  const int ex = block_excl_scan(e < E ? run : 0, sm, &tot);
  if (e < E) off_pre[e] = ex;
  if (e == 0) off_pre[E] = tot;
  if (C >= 0) {
    const int kc = (e < E) ? min(run, C) : 0;
    const int ex2 = block_excl_scan(kc, sm, &tot);
    if (e < E) { cnt_fin[e] = kc; off_fin[e] = ex2; }
    if (e == 0) off_fin[E] = tot;
  }
}

// Stable scatter: pair (t, j) of bucket b goes to off[b] + (its rank in the block), off[b]
// being where bucket b's rows of this block start (the bucket's offset plus the rows of the
// earlier blocks in it), held in LDS.
// Candidate mode writes (token, slot, key) lists for cap_select; final mode writes the
// dispatch arrays, and marks the slots in [j0, j1) that were not taken with -1. When every
// slot of every token is kept (no capacity limit), final mode can also write the token ->
// rows CSR directly (csr_ptr, csr_pos non-null): token t owns entries t*S .. t*S+S-1.
// Expects the block's masks (build_masks) in `mask`.
MOE_DEV void scatter_block(const uint32_t *mask, const int32_t *__restrict__ ids,
                           const float *__restrict__ gates, const float *__restrict__ keys, int T,
                           const PairSel &f, const int32_t *off, int candidates,
                           int32_t *__restrict__ out_token, float *__restrict__ out_w,
                           int32_t *__restrict__ out_slot, float *__restrict__ out_key,
                           int32_t *__restrict__ slot_pos, uint8_t *__restrict__ kept_out,
                           int32_t *__restrict__ csr_ptr, int32_t *__restrict__ csr_pos) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (csr_ptr) {   // every pair kept, in slot order: token t's rows are CSR entries t*S ..
    csr_ptr[t] = t * f.S;
    if (t == T - 1) csr_ptr[T] = T * f.S;
  }
  const int word = threadIdx.x >> 5, bit = threadIdx.x & 31;
  const bool want_w = !candidates || out_w;
  int seen[kMaxSlots];
  int ns = 0;
  for (int j = f.j0; j < f.j1; j += kSlotBatch) {
    // the batch's buckets, gates and keys are loaded before any is used
    int bk[kSlotBatch];
    float gv[kSlotBatch], kv[kSlotBatch];
    slot_buckets(ids, f, t, j, bk);
#pragma unroll
    for (int i = 0; i < kSlotBatch; ++i) {
      const size_t ij = (size_t)t * f.S + j + i;
      const bool in = j + i < f.j1;
      gv[i] = (in && want_w) ? gates[ij] : 0.f;
      kv[i] = (in && candidates) ? keys[ij] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kSlotBatch; ++i) {
      if (j + i >= f.j1) break;
      const size_t ij = (size_t)t * f.S + j + i;
      const int b = bk[i];
      if (b < 0) {   // not kept
        if (!candidates) slot_pos[ij] = -1;
        continue;
      }
      int c = 0;
      if (f.mult > 1) {
        for (int q = 0; q < ns; ++q) c += seen[q] == b;
        seen[ns++] = b;
      }
      // rank: pairs of the bucket among the block's earlier tokens (the 8 mask words of the
      // bucket in two 16-byte LDS reads), then the token's own earlier pairs in it
      int rank = c;
      for (int m = 0; m < f.mult; ++m) {
        const uint4 *mk = reinterpret_cast<const uint4 *>(mask + (b * f.mult + m) * 8);
        const uint4 lo = mk[0], hi = mk[1];
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int q = 0; q < 8; ++q)
          rank += q < word ? __popc(w[q]) : (q == word ? __popc(w[q] & ((1u << bit) - 1u)) : 0);
      }
      const int pos = off[b] + rank;
      const int jj = j + i;
      if (candidates) {
        out_token[pos] = t;
        out_slot[pos] = jj;
        out_key[pos] = kv[i];
        if (out_w) out_w[pos] = gv[i];   // the pair's gate rides along with its key
      } else {
        out_token[pos] = t;
        out_w[pos] = gv[i];
        slot_pos[ij] = pos;
        if (kept_out) kept_out[ij] = 1;
        if (csr_pos) csr_pos[ij] = pos;
      }
    }
  }
}

__global__ __launch_bounds__(256) void assign_scatter_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ gates,
    const float *__restrict__ keys, int T, PairSel f, int B, const int32_t *__restrict__ off,
    const int32_t *__restrict__ blk_base, int candidates, int32_t *__restrict__ out_token,
    float *__restrict__ out_w, int32_t *__restrict__ out_slot, float *__restrict__ out_key,
    int32_t *__restrict__ slot_pos, uint8_t *__restrict__ kept_out, int32_t *__restrict__ csr_ptr,
    int32_t *__restrict__ csr_pos) {
  extern __shared__ uint32_t mask[];
  // where each bucket's rows of this block start (bucket offset + the block's base), in LDS;
  // build_masks' barriers order these writes before the scatter reads them
  int32_t *soff = reinterpret_cast<int32_t *>(mask + (size_t)B * f.mult * 8);
  const int32_t *bb = blk_base + (size_t)blockIdx.x * B;
  for (int b = threadIdx.x; b < B; b += blockDim.x) soff[b] = off[b] + bb[b];
  build_masks(mask, ids, f, T, B);
  scatter_block(mask, ids, gates, keys, T, f, soff, candidates, out_token, out_w, out_slot,
                out_key, slot_pos, kept_out, csr_ptr, csr_pos);
}

// All three steps for at most 256 tokens (one block): masks, bucket counts and offsets (as
// assign_scan_kernel computes them for one block, including the capped second table when
// C >= 0), then the scatter. Thread i owns buckets 4i .. 4i+3 for the scans (B <= 1024).
// Dynamic LDS: the masks, then B ints of bucket offsets.
__global__ __launch_bounds__(256) void assign_single_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ gates,
    const float *__restrict__ keys, int T, PairSel f, int B, int C, int32_t *__restrict__ cnt_pre,
    int32_t *__restrict__ off_pre, int32_t *__restrict__ cnt_fin, int32_t *__restrict__ off_fin,
    int candidates, int32_t *__restrict__ out_token, float *__restrict__ out_w,
    int32_t *__restrict__ out_slot, float *__restrict__ out_key, int32_t *__restrict__ slot_pos,
    uint8_t *__restrict__ kept_out, int32_t *__restrict__ csr_ptr, int32_t *__restrict__ csr_pos) {
  extern __shared__ uint32_t mask[];
  int32_t *soff = reinterpret_cast<int32_t *>(mask + (size_t)B * f.mult * 8);
  __shared__ int sm[256 / 64 + 1];
  build_masks(mask, ids, f, T, B);
  int c[4], own = 0, own_fin = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = threadIdx.x * 4 + q;
    c[q] = 0;
    if (b < B)
      for (int m = 0; m < f.mult; ++m)
#pragma unroll
        for (int w = 0; w < 8; ++w) c[q] += __popc(mask[(b * f.mult + m) * 8 + w]);
    own += c[q];
    own_fin += C >= 0 ? min(c[q], C) : 0;
  }
  int tot;
  int run = block_excl_scan(own, sm, &tot);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = threadIdx.x * 4 + q;
    if (b < B) { cnt_pre[b] = c[q]; off_pre[b] = run; soff[b] = run; }
    run += c[q];
  }
  if (threadIdx.x == 0) off_pre[B] = tot;
  if (C >= 0) {
    int run2 = block_excl_scan(own_fin, sm, &tot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = threadIdx.x * 4 + q;
      const int kc = min(c[q], C);
      if (b < B) { cnt_fin[b] = kc; off_fin[b] = run2; }
      run2 += kc;
    }
    if (threadIdx.x == 0) off_fin[B] = tot;
  }
  __syncthreads();
  scatter_block(mask, ids, gates, keys, T, f, soff, candidates, out_token, out_w, out_slot, out_key,
                slot_pos, kept_out, csr_ptr, csr_pos);
}

// Expanded drop, between its two selections: a token that lost some of its first k picks
// offers its extra candidates (kept[j >= k] = 1 marks the offer) ...
__global__ __launch_bounds__(256) void expand_offer_kernel(uint8_t *__restrict__ kept, int T,
                                                           int k, int S) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int have = 0;
  for (int j = 0; j < k; ++j) have += kept[(size_t)t * S + j];
  for (int j = k; j < S; ++j) kept[(size_t)t * S + j] = have < k ? 1 : 0;
}

// ... and after the admission (kept[j >= k] = admitted) keeps its first admitted extra
// pairs in slot order, as many as it lost.
__global__ __launch_bounds__(256) void expand_keep_kernel(uint8_t *__restrict__ kept, int T,
                                                          int k, int S) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int have = 0;
  for (int j = 0; j < k; ++j) have += kept[(size_t)t * S + j];
  for (int j = k; j < S; ++j) {
    uint8_t &v = kept[(size_t)t * S + j];
    if (v && have < k) ++have;
    else v = 0;
  }
}

// ----------------------------------------------------------------------------------------
// Block-wide radix selection (1024 threads): among n uint32 keys, find the want-th largest
// value tau and how many keys equal to tau are needed (need_eq) so that
// {u > tau} + (first need_eq of {u == tau}) is exactly the top `want`. Histograms of one
// byte per pass (LDS integer adds: the counts do not depend on order), one per wave so that
// the many keys sharing a leading byte (scores of similar size) do not all queue on one LDS
// word; the 16 wave histograms are summed bin by bin.
struct SelectResult { uint32_t tau; int need_eq; };
constexpr int kSelWaves = 16;   // waves of a 1024-thread selection block

// bin counts of the pass into hist[wave][bin] -> returns the total of bin 255-b to thread b
MOE_DEV int sum_wave_hists(const int *hist, int b) {
  int h = 0;
  if (b < 256)
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) h += hist[w * 256 + 255 - b];
  return h;
}

template <typename GetKey>
MOE_DEV SelectResult block_radix_select(GetKey get, int n, int want, int *hist, int *sm) {
  uint32_t prefix = 0u, pmask = 0u;
  int *wh = hist + (threadIdx.x >> 6) * 256;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kSelWaves * 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    uint32_t cd = 0u;   // runs of equal digits, one atomic each (see block_radix_select_regs)
    int cc = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t u = get(i);
      if ((u & pmask) == prefix) {
        const uint32_t dg = (u >> shift) & 255u;
        if (cc && dg != cd) {
          atomicAdd(&wh[cd], cc);
          cc = 0;
        }
        cd = dg;
        ++cc;
      }
    }
    if (cc) atomicAdd(&wh[cd], cc);
    __syncthreads();
    // thread b looks at bin 255-b: inclusive scan from the top bin down
    const int b = threadIdx.x;
    const int h = sum_wave_hists(hist, b);
    int tot;
    const int ex = block_excl_scan(h, sm, &tot);
    __shared__ int pick[2];
    if (b < 256 && ex < want && want <= ex + h) { pick[0] = 255 - b; pick[1] = want - ex; }
    __syncthreads();
    prefix |= ((uint32_t)pick[0]) << shift;
    pmask |= 255u << shift;
    want = pick[1];
    __syncthreads();
  }
  return SelectResult{prefix, want};
}

// The same selection over keys held in registers: thread tid owns keys tid + 1024 j.
template <int KPT>
MOE_DEV SelectResult block_radix_select_regs(const uint32_t (&u)[KPT], int n, int want, int *hist,
                                             int *sm) {
  uint32_t prefix = 0u, pmask = 0u;
  int *wh = hist + (threadIdx.x >> 6) * 256;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < kSelWaves * 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    // a thread adds runs of equal digits among its keys with one atomic each: the keys of one
    // bucket share their leading bytes, so in the first passes a thread's keys mostly fall in
    // one bin and 64 lanes adding 1 to the same LDS word, key after key, serialise
    uint32_t cd = 0u;
    int cc = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (threadIdx.x + j * 1024 < n && (u[j] & pmask) == prefix) {
        const uint32_t dg = (u[j] >> shift) & 255u;
        if (cc && dg != cd) {
          atomicAdd(&wh[cd], cc);
          cc = 0;
        }
        cd = dg;
        ++cc;
      }
    if (cc) atomicAdd(&wh[cd], cc);
    __syncthreads();
    const int b = threadIdx.x;
    const int h = sum_wave_hists(hist, b);
    int tot;
    const int ex = block_excl_scan(h, sm, &tot);
    __shared__ int pick[2];
    if (b < 256 && ex < want && want <= ex + h) { pick[0] = 255 - b; pick[1] = want - ex; }
    __syncthreads();
    prefix |= ((uint32_t)pick[0]) << shift;
    pmask |= 255u << shift;
    want = pick[1];
    __syncthreads();
  }
  return SelectResult{prefix, want};
}

// Capacity selection, one workgroup per bucket. The candidates of bucket e sit in their
// rank order (ascending token, then slot) at [off_pre[e], off_pre[e] + cnt), each with its
// key and gate; if more than the bucket's capacity (C, minus used[e] places already taken
// when `used` is given), the ones with the largest (key, then earlier rank) stay. Final mode
// (perm_token given): survivors keep their order and go to off_fin[e] + rank, dropped slots
// get -1. Flag mode: only kept[t, j] = survived.
__global__ __launch_bounds__(1024) void cap_select_kernel(
    const int32_t *__restrict__ cand_token, const int32_t *__restrict__ cand_slot,
    const float *__restrict__ cand_key, const float *__restrict__ cand_w,
    const int32_t *__restrict__ cnt_pre, const int32_t *__restrict__ off_pre,
    const int32_t *__restrict__ off_fin, int C, const int32_t *__restrict__ used, int S,
    int32_t *__restrict__ perm_token, float *__restrict__ perm_w, int32_t *__restrict__ slot_pos,
    uint8_t *__restrict__ kept) {
  constexpr int KPT = 16;   // keys per thread kept in registers (n <= 16384)
  __shared__ int hist[kSelWaves * 256];
  __shared__ int sm[kSelWaves * KPT + KPT];
  const int e = blockIdx.x;
  const int n = cnt_pre[e], base = off_pre[e];
  const int cap = used ? max(C - used[e], 0) : C;
  // capacity 0 keeps nothing: a threshold above every finite key
  SelectResult sr{0xffffffffu, 0};
  const bool drop = n > cap;
  auto emit = [&](int i, bool self, int rank) {
    const int t = cand_token[base + i], j = cand_slot[base + i];
    const size_t ij = (size_t)t * S + j;
    if (perm_token) {
      if (self) {
        const int q = off_fin[e] + rank;
        perm_token[q] = t;
        perm_w[q] = cand_w[base + i];
        slot_pos[ij] = q;
      } else {
        slot_pos[ij] = -1;
      }
    }
    if (kept) kept[ij] = (uint8_t)self;
  };
  if (!drop) {   // every candidate stays, in list order: its rank is its index
    for (int i = threadIdx.x; i < n; i += blockDim.x) emit(i, true, i);
    return;
  }
  // thread tid owns candidates tid + 1024 c (chunk c): keys in registers; the ranks of each
  // chunk come from one vector scan over the block, chunks in order
  auto in_regs = [&](auto kpt) {
    constexpr int K = decltype(kpt)::value;
    uint32_t u[K];
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const int i = threadIdx.x + c * 1024;
      u[c] = (drop && i < n) ? float_key(cand_key[base + i]) : 0u;
    }
    if (drop && cap > 0) sr = block_radix_select_regs<K>(u, n, cap, hist, sm);
    int eq[K], eq_tot[K];
#pragma unroll
    for (int c = 0; c < K; ++c)
      eq[c] = (drop && threadIdx.x + c * 1024 < n && u[c] == sr.tau) ? 1 : 0;
    block_excl_scan_vec<K>(eq, sm, eq_tot);
    int sel[K], sel_tot[K];
    uint32_t selm = 0u;
    int run = 0;
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const bool in = threadIdx.x + c * 1024 < n;
      const bool is_eq = drop && in && u[c] == sr.tau;
      const bool self = in && (!drop || u[c] > sr.tau || (is_eq && run + eq[c] < sr.need_eq));
      run += eq_tot[c];
      sel[c] = self ? 1 : 0;
      selm |= (self ? 1u : 0u) << c;
    }
    block_excl_scan_vec<K>(sel, sm, sel_tot);
    run = 0;
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const int i = threadIdx.x + c * 1024;
      if (i < n) emit(i, (selm >> c) & 1u, run + sel[c]);
      run += sel_tot[c];
    }
  };
  if (n <= 2 * 1024) { in_regs(std::integral_constant<int, 2>{}); return; }
  if (n <= 4 * 1024) { in_regs(std::integral_constant<int, 4>{}); return; }
  if (n <= KPT * 1024) { in_regs(std::integral_constant<int, KPT>{}); return; }
  // many candidates: keys re-read from memory, ranks by 1024-wide chunks in order
  if (drop && cap > 0) {
    auto get = [&](int i) { return float_key(cand_key[base + i]); };
    sr = block_radix_select(get, n, cap, hist, sm);
  }
  int run_eq = 0, run_sel = 0;
  for (int c0 = 0; c0 < n; c0 += blockDim.x) {
    const int i = c0 + threadIdx.x;
    const bool in = i < n;
    uint32_t uu = 0u;
    if (in && drop) uu = float_key(cand_key[base + i]);
    const int eqf = (in && drop && uu == sr.tau) ? 1 : 0;
    int tot;
    const int eq_rank = run_eq + block_excl_scan(eqf, sm, &tot);
    run_eq += tot;
    const int self = in && (!drop || uu > sr.tau || (eqf && eq_rank < sr.need_eq)) ? 1 : 0;
    const int rank = run_sel + block_excl_scan(self, sm, &tot);
    run_sel += tot;
    if (in) emit(i, self, rank);
  }
}

// Expert choice, one workgroup per expert: column max and softmax denominator over all T
// tokens, radix selection of the c largest logits (ties: lower token), then an ordered
// compaction so that the expert's rows hold its tokens in ascending order.
__global__ __launch_bounds__(1024) void ec_select_kernel(const float *__restrict__ logits, int T,
                                                         int E, int c,
                                                         uint32_t *__restrict__ colkeys,
                                                         int32_t *__restrict__ perm_token,
                                                         float *__restrict__ perm_w,
                                                         int32_t *__restrict__ slot_pos,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets) {
  __shared__ int hist[kSelWaves * 256];
  __shared__ int sm[1024 / 64 + 1];
  __shared__ float fsm[1024 / 64];
  const int e = blockIdx.x;
  uint32_t *keys = colkeys + (size_t)e * T;
  float mx = -INFINITY;
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    const float v = logits[(size_t)t * E + e];
    keys[t] = float_key(v);
    mx = fmaxf(mx, v);
  }
  mx = block_max(mx, fsm);
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += blockDim.x) s += expf(logits[(size_t)t * E + e] - mx);
  const float Z = block_sum(s, fsm);
  __syncthreads();   // keys visible to the whole block
  auto get = [&](int i) { return keys[i]; };
  const SelectResult sr = block_radix_select(get, T, c, hist, sm);
  int run_eq = 0, run_sel = 0;
  for (int c0 = 0; c0 < T; c0 += blockDim.x) {
    const int t = c0 + threadIdx.x;
    const bool in = t < T;
    const uint32_t u = in ? keys[t] : 0u;
    const int eqf = (in && u == sr.tau) ? 1 : 0;
    int tot;
    const int eq_rank = run_eq + block_excl_scan(eqf, sm, &tot);
    run_eq += tot;
    const int self = in && (u > sr.tau || (eqf && eq_rank < sr.need_eq)) ? 1 : 0;
    const int rank = run_sel + block_excl_scan(self, sm, &tot);
    run_sel += tot;
    if (in) {
      if (self) {
        const int q = e * c + rank;
        perm_token[q] = t;
        perm_w[q] = expf(logits[(size_t)t * E + e] - mx) / Z;
        slot_pos[(size_t)t * E + e] = q;
      } else {
        slot_pos[(size_t)t * E + e] = -1;
      }
    }
  }
  if (threadIdx.x == 0) {
    counts[e] = c;
    offsets[e] = e * c;
    if (e == E - 1) offsets[E] = E * c;
  }
}

// The same selection with the column held in registers (T <= 1024 KPT): thread tid owns
// tokens tid + 1024 j (chunk j), so ranks taken chunk by chunk, threads in order, follow
// ascending token. One pass reads the column (from the transposed logits when given: one
// contiguous row); the radix selection and the ordered compaction (two vector scans) work on
// registers and LDS only.
template <int KPT>
__global__ __launch_bounds__(1024) void ec_select_regs_kernel(const float *__restrict__ logits,
                                                              int T, int E, int c,
                                                              int32_t *__restrict__ perm_token,
                                                              float *__restrict__ perm_w,
                                                              int32_t *__restrict__ slot_pos,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ offsets,
                                                              const float *__restrict__ logits_t) {
  __shared__ int hist[kSelWaves * 256];
  __shared__ int sm[kSelWaves * KPT + KPT];
  __shared__ float fsm[1024 / 64];
  const int e = blockIdx.x;
  float v[KPT];
  uint32_t u[KPT];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = threadIdx.x + 1024 * j;
    v[j] = t < T ? (logits_t ? logits_t[(size_t)e * T + t] : logits[(size_t)t * E + e]) : -INFINITY;
    u[j] = t < T ? float_key(v[j]) : 0u;
    mx = fmaxf(mx, v[j]);
  }
  mx = block_max(mx, fsm);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (threadIdx.x + 1024 * j < T) sum += expf(v[j] - mx);
  const float Z = block_sum(sum, fsm);
  const SelectResult sr = block_radix_select_regs<KPT>(u, T, c, hist, sm);
  int eq[KPT], eq_tot[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) eq[j] = (threadIdx.x + 1024 * j < T && u[j] == sr.tau) ? 1 : 0;
  block_excl_scan_vec<KPT>(eq, sm, eq_tot);
  int sel[KPT], sel_tot[KPT];
  int run = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool in = threadIdx.x + 1024 * j < T;
    const bool self = in && (u[j] > sr.tau || (u[j] == sr.tau && run + eq[j] < sr.need_eq));
    run += eq_tot[j];
    sel[j] = self ? 1 : 0;
  }
  int flag[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) flag[j] = sel[j];
  block_excl_scan_vec<KPT>(sel, sm, sel_tot);
  run = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int t = threadIdx.x + 1024 * j;
    if (t < T) {
      if (flag[j]) {
        const int q = e * c + run + sel[j];
        perm_token[q] = t;
        perm_w[q] = expf(v[j] - mx) / Z;
        slot_pos[(size_t)t * E + e] = q;
      } else {
        slot_pos[(size_t)t * E + e] = -1;
      }
    }
    run += sel_tot[j];
  }
  if (threadIdx.x == 0) {
    counts[e] = c;
    offsets[e] = e * c;
    if (e == E - 1) offsets[E] = E * c;
  }
}

// ----------------------------------------------------------------------------------------
// CSR over tokens from the slot table slot_pos[T, S] (row index or -1): per-block totals,
// one scan over blocks, then per-token offsets and the row lists in slot order.
__global__ __launch_bounds__(256) void tok_count_kernel(const int32_t *__restrict__ slot_pos, int T,
                                                        int S, int32_t *__restrict__ blk_sum) {
  __shared__ int sm[256 / 64 + 1];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int c = 0;
  if (t < T)
    for (int s = 0; s < S; ++s) c += slot_pos[(size_t)t * S + s] >= 0;
  int tot;
  block_excl_scan(c, sm, &tot);
  if (threadIdx.x == 0) blk_sum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void blk_scan_kernel(const int32_t *__restrict__ in, int n,
                                                        int32_t *__restrict__ out,
                                                        int32_t *__restrict__ total) {
  __shared__ int sm[1024 / 64 + 1];
  int run = 0;
  for (int c0 = 0; c0 < n; c0 += 1024) {
    const int i = c0 + threadIdx.x;
    int tot;
    const int ex = block_excl_scan(i < n ? in[i] : 0, sm, &tot);
    if (i < n) out[i] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0 && total) *total = run;
}

__global__ __launch_bounds__(256) void tok_write_kernel(const int32_t *__restrict__ slot_pos, int T,
                                                        int S, const int32_t *__restrict__ blk_off,
                                                        int32_t *__restrict__ tok_ptr,
                                                        int32_t *__restrict__ tok_pos) {
  __shared__ int sm[256 / 64 + 1];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int c = 0;
  if (t < T)
    for (int s = 0; s < S; ++s) c += slot_pos[(size_t)t * S + s] >= 0;
  int tot;
  const int ex = block_excl_scan(c, sm, &tot);
  if (t < T) {
    int p = blk_off[blockIdx.x] + ex;
    tok_ptr[t] = p;
    for (int s = 0; s < S; ++s) {
      const int v = slot_pos[(size_t)t * S + s];
      if (v >= 0) tok_pos[p++] = v;
    }
    if (t == T - 1) tok_ptr[T] = p;
  }
}

// The scan and the write in one launch when there are at most kCsrFusedBlocks blocks: each
// block adds the totals of the blocks before it itself (integer sums, fixed order per thread,
// then a block-wide sum), instead of a separate scan kernel.
constexpr int kCsrFusedBlocks = 1024;

__global__ __launch_bounds__(256) void tok_write_fused_kernel(const int32_t *__restrict__ slot_pos,
                                                              int T, int S,
                                                              const int32_t *__restrict__ blk_sum,
                                                              int32_t *__restrict__ tok_ptr,
                                                              int32_t *__restrict__ tok_pos) {
  __shared__ int sm[256 / 64 + 1];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int c = 0;
  if (t < T)
    for (int j = 0; j < S; ++j) c += slot_pos[(size_t)t * S + j] >= 0;
  int before = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += 256) before += blk_sum[b];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  before = wave_sum_int(before);
  if (lane == 0) sm[wid] = before;
  __syncthreads();
  const int base = sm[0] + sm[1] + sm[2] + sm[3];
  __syncthreads();
  int tot;
  const int ex = block_excl_scan(c, sm, &tot);
  if (t < T) {
    int p = base + ex;
    tok_ptr[t] = p;
    for (int j = 0; j < S; ++j) {
      const int v = slot_pos[(size_t)t * S + j];
      if (v >= 0) tok_pos[p++] = v;
    }
    if (t == T - 1) tok_ptr[T] = p;
  }
}

// ----------------------------------------------------------------------------------------
// Expert-utilisation statistics. Pass 1: per block of 256 tokens, the sum over its tokens
// of softmax_E(l)[t, e] for every expert (thread e adds its block's tokens in order).
// Pass 2 (one block): fixed-order sums over blocks and the scalar statistics.
__global__ __launch_bounds__(256) void stats_partial_kernel(const float *__restrict__ logits, int T,
                                                            int E, float *__restrict__ part) {
  __shared__ float rmax[256], rinv[256];
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, logits[(size_t)t * E + e]);
    float s = 0.f;
    for (int e = 0; e < E; ++e) s += __expf(logits[(size_t)t * E + e] - m);
    rmax[threadIdx.x] = m;
    rinv[threadIdx.x] = 1.f / s;
  }
  __syncthreads();
  const int nt = min(256, T - blockIdx.x * 256);
  for (int e = threadIdx.x; e < E; e += 256) {
    float a = 0.f;
    for (int i = 0; i < nt; ++i) {
      const int tt = blockIdx.x * 256 + i;
      a += __expf(logits[(size_t)tt * E + e] - rmax[i]) * rinv[i];
    }
    part[(size_t)blockIdx.x * E + e] = a;
  }
}

__global__ __launch_bounds__(1024) void stats_final_kernel(const float *__restrict__ part, int nblk,
                                                           const int32_t *__restrict__ counts,
                                                           const int32_t *__restrict__ offsets,
                                                           int T, int E, int k, int token_choice,
                                                           float *__restrict__ out) {
  __shared__ float fsm[1024 / 64];
  const int rows = offsets[E];
  float fp = 0.f, mxc = 0.f, empty = 0.f;
  for (int e = threadIdx.x; e < E; e += 1024) {
    float P = 0.f;
    for (int b = 0; b < nblk; ++b) P += part[(size_t)b * E + e];
    P /= (float)T;
    const float f = rows > 0 ? (float)counts[e] / (float)rows : 0.f;
    out[e] = f;
    out[E + e] = P;
    fp += f * P;
    mxc = fmaxf(mxc, (float)counts[e]);
    empty += counts[e] == 0 ? 1.f : 0.f;
  }
  fp = block_sum(fp, fsm);
  mxc = block_max(mxc, fsm);
  empty = block_sum(empty, fsm);
  if (threadIdx.x == 0) {
    out[2 * E] = fp;   // sum_i f_i P_i, unscaled
    out[2 * E + 1] = rows > 0 ? mxc / ((float)rows / (float)E) : 0.f;
    out[2 * E + 2] = token_choice ? (float)(T * k - rows) : 0.f;
    out[2 * E + 3] = empty;
  }
}

// ----------------------------------------------------------------------------------------
// host-side launchers

int router_epad(int E) { return E <= 32 ? 32 : E <= 64 ? 64 : ((E + 127) / 128) * 128; }

bool router_narrow_mfma(int dtype, int d, int E) {
  return dtype == 1 && 3 * E <= kNarrowRows && d % 64 == 0;
}

size_t router_w3_bytes(int dtype, int d, int E) {
  if (router_narrow_mfma(dtype, d, E)) return 0;   // splits W_r in LDS itself
  if (dtype == 1 && E > 8 && d % 64 == 0) return 3 * (size_t)router_epad(E) * router_w3_ld(d) * 2;
  return 0;
}

hipError_t launch_router(int dtype, const void *x, const float *w, const float *bias,
                         float *logits, int T, int d, int E, bf16_t *w3, hipStream_t st,
                         const TopkOut *topk, bool *topk_done, int *cnt_block,
                         const RouterExtra *ex, bool *ex_done, const BlkDispatchOut *disp,
                         bool *disp_done) {
  if (topk_done) *topk_done = false;
  if (cnt_block) *cnt_block = 0;
  if (ex_done) *ex_done = false;
  if (disp_done) *disp_done = false;
  if (router_narrow_mfma(dtype, d, E)) {
    const TopkOut tk = topk ? *topk : TopkOut{0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr};
    if (topk && topk_done) *topk_done = true;
    const RouterExtra rx = ex ? *ex : RouterExtra{nullptr};
    if (ex && ex_done) *ex_done = true;
    // one workgroup for every token: it also writes the dispatch (final mode)
    BlkDispatchOut dsp{};
    if (disp && topk && tk.blk_cnt && T <= 16 && disp->perm_token && !disp->cand_slot) {
      dsp = *disp;
      if (disp_done) *disp_done = true;
    }
    const int tb = T >= 16 * 2 * 256 ? 2 : 1;   // two token blocks per workgroup halve the W reads
    if (tk.blk_cnt && cnt_block) *cnt_block = 16 * tb;
#define MOE_NARROW(TBB, NCHH) hipLaunchKernelGGL((router_mfma_narrow_kernel<TBB, NCHH>),          \
                                               dim3((T + 16 * TBB - 1) / (16 * TBB)), dim3(64 * kNarrowWaves), 0, \
                                               st, (const bf16_t *)x, w, bias, logits, T, d, E, tk, \
                                               tk.blk_cnt, rx, dsp)
    if (tb == 2) { if (E <= 8) MOE_NARROW(2, 1); else MOE_NARROW(2, 2); }
    else { if (E <= 8) MOE_NARROW(1, 1); else MOE_NARROW(1, 2); }
#undef MOE_NARROW
    return hipGetLastError();
  }
  if (dtype == 1 && E > 8 && d % 64 == 0) {
    // bf16 activations, wide router: three-part split of W_r on the matrix cores
    const int E_pad = router_epad(E);
    const size_t n = (size_t)E_pad * d;
    int g = (int)((n + 255) / 256);
    if (g > 2048) g = 2048;
    hipLaunchKernelGGL(router_split_kernel, dim3(g), dim3(256), 0, st, w, d, E, E_pad, w3);
    if (E_pad % 128 == 0) {   // same workgroup count as 64 x 128 tiles, fewer bytes per CU
      const dim3 grid((T + kRwTM - 1) / kRwTM, E_pad / kRwEN);
      hipLaunchKernelGGL(router_mfma128_kernel, grid, dim3(512), 0, st, (const bf16_t *)x, w3,
                         bias, logits, T, d, E, E_pad);
    } else {
      const dim3 grid((T + 63) / 64, (E_pad + 127) / 128);
      hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(512), 0, st, (const bf16_t *)x, w3, bias,
                         logits, T, d, E, E_pad);
    }
    return hipGetLastError();
  }
  // SIMT float32 routers (bf16 problems, whose d is a multiple of 64, never get here)
  if (dtype != 0) return hipErrorInvalidValue;
  if (E <= 8) {
    // tokens per workgroup: a multiple of 8, about T / 256 (one workgroup per CU)
    int tpb = ((T + 255) / 256 + 7) / 8 * 8;
    if (tpb < 8) tpb = 8;
    dim3 grid((T + tpb - 1) / tpb);
    hipLaunchKernelGGL(router_narrow_kernel<float>, grid, dim3(512), 0, st, (const float *)x, w,
                       bias, logits, T, d, E, tpb);
  } else {
    dim3 grid((T + 63) / 64, (E + 127) / 128);
    hipLaunchKernelGGL(router_wide_kernel<float>, grid, dim3(256), 0, st, (const float *)x, w,
                       bias, logits, T, d, E);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int kden, int renorm,
                       int want_key, int32_t *ids, float *gates, float *keys, hipStream_t st,
                       int32_t *blk_cnt, int *cnt_block) {
  if (cnt_block) *cnt_block = 0;
  if (E > kBlkMaxE) blk_cnt = nullptr;
  // G lanes per token, each holding up to PL logits: narrow rows keep one logit per lane;
  // up to 128 experts use 16 lanes x 8 (16 tokens per block): merged sorted lists for
  // k = 5..8, else a 4-step butterfly per pick
  int G = 64;
  if (E <= 8) G = 8;
  else if (E <= 16) G = 16;
  else if (E <= 32) G = 32;
  else if (E <= 128) G = 16;
  const int tpb = 256 / G;
  const size_t sh = want_key ? (size_t)tpb * E * sizeof(float) : 0;
  dim3 grid((T + tpb - 1) / tpb);
  if (blk_cnt && cnt_block) *cnt_block = tpb;   // E <= 16: G = 8 or 16, one logit per lane
#define MOE_TOPK(GG, PL) hipLaunchKernelGGL((topk_kernel<GG, PL>), grid, dim3(256), sh, st, logits, \
                                            T, E, k, kden, renorm, want_key, ids, gates, keys, \
                                            blk_cnt)
  if (E <= 8) MOE_TOPK(8, 1);
  else if (E <= 16) MOE_TOPK(16, 1);
  else if (E <= 32) MOE_TOPK(32, 1);
  else if (E <= 128 && k >= 5 && k <= 8)   // merging beats k argmax rounds from k = 5 on
    hipLaunchKernelGGL(topk_merge_kernel, grid, dim3(256), sh, st, logits, T, E, k, kden, renorm,
                       want_key, ids, gates, keys);
  else if (E <= 128) MOE_TOPK(16, 8);
  else MOE_TOPK(64, kMaxExperts / 64);
#undef MOE_TOPK
  return hipGetLastError();
}

namespace {

// histogram + scan + scatter of the pairs `f` selects into B buckets. Candidate mode:
// per-bucket candidate lists in s.cand_* with counts s.cnt_pre and offsets s.off_pre.
// Final mode: counts/offsets and the dispatch arrays.
void assign_pairs(const RouteScratch &s, const int32_t *ids, const float *gates, int T,
                  const PairSel &f, int B, bool candidates, int32_t *perm_token, float *perm_w,
                  uint8_t *kept_out, int32_t *counts, int32_t *offsets, hipStream_t st,
                  int32_t *csr_ptr = nullptr, int32_t *csr_pos = nullptr) {
  const int nblk = (T + 255) / 256;
  const size_t msh = (size_t)B * f.mult * 8 * sizeof(uint32_t);
  const size_t msh_sc = msh + (size_t)B * 4;   // + the bucket starts of the scatter
  int32_t *cnt = candidates ? s.cnt_pre : counts, *off = candidates ? s.off_pre : offsets;
  if (nblk == 1) {   // one launch instead of three
    if (candidates)
      hipLaunchKernelGGL(assign_single_kernel, dim3(1), dim3(256), msh + (size_t)B * 4, st, ids,
                         gates, s.keys, T, f, B, -1, cnt, off, (int32_t *)nullptr,
                         (int32_t *)nullptr, 1, s.cand_token, s.cand_w, s.cand_slot, s.cand_key,
                         (int32_t *)nullptr, (uint8_t *)nullptr, (int32_t *)nullptr,
                         (int32_t *)nullptr);
    else
      hipLaunchKernelGGL(assign_single_kernel, dim3(1), dim3(256), msh + (size_t)B * 4, st, ids,
                         gates, (const float *)nullptr, T, f, B, -1, cnt, off, (int32_t *)nullptr,
                         (int32_t *)nullptr, 0, perm_token, perm_w, (int32_t *)nullptr,
                         (float *)nullptr, s.slot_pos, kept_out, csr_ptr, csr_pos);
    return;
  }
  hipLaunchKernelGGL(assign_count_kernel, dim3(nblk), dim3(256), msh, st, ids, T, f, B, s.blk_cnt);
  hipLaunchKernelGGL(assign_scan_kernel, dim3(1), dim3(1024), 0, st, s.blk_cnt, nblk, B, -1,
                     s.blk_base, cnt, off, (int32_t *)nullptr, (int32_t *)nullptr);
  if (candidates)
    hipLaunchKernelGGL(assign_scatter_kernel, dim3(nblk), dim3(256), msh_sc, st, ids, gates, s.keys,
                       T, f, B, off, s.blk_base, 1, s.cand_token, s.cand_w, s.cand_slot,
                       s.cand_key, (int32_t *)nullptr, (uint8_t *)nullptr, (int32_t *)nullptr,
                       (int32_t *)nullptr);
  else
    hipLaunchKernelGGL(assign_scatter_kernel, dim3(nblk), dim3(256), msh_sc, st, ids, gates,
                       (const float *)nullptr, T, f, B, off, s.blk_base, 0, perm_token, perm_w,
                       (int32_t *)nullptr, (float *)nullptr, s.slot_pos, kept_out, csr_ptr,
                       csr_pos);
}

}  // namespace

hipError_t launch_dispatch_blocks(const int32_t *ids, const float *gates, int T, int k, int E,
                                  const int32_t *blk_cnt, int bt, const BlkDispatchOut &o,
                                  hipStream_t st) {
  if (E > kBlkMaxE || bt < 256 / kBlkPerWg || bt > 64 || 256 % bt != 0)
    return hipErrorInvalidValue;
  if (E <= 8)
    hipLaunchKernelGGL(dispatch_blocks_kernel<8>, dim3((T + 255) / 256), dim3(256), 0, st, ids,
                       gates, T, k, E, blk_cnt, bt, o);
  else
    hipLaunchKernelGGL(dispatch_blocks_kernel<16>, dim3((T + 255) / 256), dim3(256), 0, st, ids,
                       gates, T, k, E, blk_cnt, bt, o);
  return hipGetLastError();
}

hipError_t launch_cap_select_final(const RouteScratch &s, int E, int C, int S, int32_t *perm_token,
                                   float *perm_w, uint8_t *kept, const int32_t *off_fin,
                                   hipStream_t st) {
  hipLaunchKernelGGL(cap_select_kernel, dim3(E), dim3(1024), 0, st, s.cand_token, s.cand_slot,
                     s.cand_key, s.cand_w, s.cnt_pre, s.off_pre, off_fin, C,
                     (const int32_t *)nullptr, S, perm_token, perm_w, s.slot_pos, kept);
  return hipGetLastError();
}

hipError_t launch_token_dispatch(const RouteScratch &s, const int32_t *ids, const float *gates,
                                 int T, int k, int E, int C, int32_t *perm_token, float *perm_w,
                                 uint8_t *kept, int32_t *counts, int32_t *offsets,
                                 int32_t *tok_ptr, int32_t *tok_pos, hipStream_t st) {
  const int nblk = (T + 255) / 256;
  const PairSel all{nullptr, k, 0, k, 1, 1};
  if (C < 0) {
    assign_pairs(s, ids, gates, T, all, E, false, perm_token, perm_w, kept, counts, offsets, st,
                 tok_ptr, tok_pos);
    return hipGetLastError();
  }
  const size_t msh = (size_t)E * 8 * sizeof(uint32_t);
  const size_t msh_sc = msh + (size_t)E * 4;   // + the bucket starts of the scatter
  if (nblk == 1) {   // one launch instead of three
    hipLaunchKernelGGL(assign_single_kernel, dim3(1), dim3(256), msh + (size_t)E * 4, st, ids,
                       gates, s.keys, T, all, E, C, s.cnt_pre, s.off_pre, counts, offsets, 1,
                       s.cand_token, s.cand_w, s.cand_slot, s.cand_key, (int32_t *)nullptr,
                       (uint8_t *)nullptr, (int32_t *)nullptr, (int32_t *)nullptr);
  } else {
    hipLaunchKernelGGL(assign_count_kernel, dim3(nblk), dim3(256), msh, st, ids, T, all, E,
                       s.blk_cnt);
    hipLaunchKernelGGL(assign_scan_kernel, dim3(1), dim3(1024), 0, st, s.blk_cnt, nblk, E, C,
                       s.blk_base, s.cnt_pre, s.off_pre, counts, offsets);
    hipLaunchKernelGGL(assign_scatter_kernel, dim3(nblk), dim3(256), msh_sc, st, ids, gates, s.keys,
                       T, all, E, s.off_pre, s.blk_base, 1, s.cand_token, s.cand_w,
                       s.cand_slot, s.cand_key, (int32_t *)nullptr, (uint8_t *)nullptr,
                       (int32_t *)nullptr, (int32_t *)nullptr);
  }
  hipLaunchKernelGGL(cap_select_kernel, dim3(E), dim3(1024), 0, st, s.cand_token, s.cand_slot,
                     s.cand_key, s.cand_w, s.cnt_pre, s.off_pre, offsets, C, (const int32_t *)nullptr, k,
                     perm_token, perm_w, s.slot_pos, kept);
  return hipGetLastError();
}

hipError_t launch_group_capacity(const RouteScratch &s, const int32_t *ids, const float *gates,
                                 int T, int k, int E, int D, int C_D, int32_t *perm_token,
                                 float *perm_w, uint8_t *kept, int32_t *counts, int32_t *offsets,
                                 hipStream_t st) {
  const int gs = E / D;
  // candidates per group (a token may have up to min(k, E/D) pairs in one group)
  const PairSel grp{nullptr, k, 0, k, gs, k < gs ? k : gs};
  assign_pairs(s, ids, gates, T, grp, D, true, nullptr, nullptr, nullptr, nullptr, nullptr, st);
  hipLaunchKernelGGL(cap_select_kernel, dim3(D), dim3(1024), 0, st, s.cand_token, s.cand_slot,
                     s.cand_key, s.cand_w, s.cnt_pre, s.off_pre, s.off_pre, C_D,
                     (const int32_t *)nullptr, k, (int32_t *)nullptr, (float *)nullptr,
                     (int32_t *)nullptr, kept);
  // dispatch of the kept pairs per expert
  const PairSel fin{kept, k, 0, k, 1, 1};
  assign_pairs(s, ids, gates, T, fin, E, false, perm_token, perm_w, nullptr, counts, offsets, st);
  return hipGetLastError();
}

hipError_t launch_expanded_drop(const RouteScratch &s, const int32_t *ids, const float *gates,
                                int T, int k, int m, int E, int C, int32_t *perm_token,
                                float *perm_w, uint8_t *kept, int32_t *counts, int32_t *offsets,
                                hipStream_t st) {
  const int S = k + m, nblk = (T + 255) / 256;
  const size_t msh = (size_t)E * 8 * sizeof(uint32_t);
  const size_t msh_sc = msh + (size_t)E * 4;   // + the bucket starts of the scatter
  // 1. token drop over the first k slots (flags); counts <- kept top-k pairs per expert
  const PairSel top{nullptr, S, 0, k, 1, 1};
  hipLaunchKernelGGL(assign_count_kernel, dim3(nblk), dim3(256), msh, st, ids, T, top, E,
                     s.blk_cnt);
  hipLaunchKernelGGL(assign_scan_kernel, dim3(1), dim3(1024), 0, st, s.blk_cnt, nblk, E, C,
                     s.blk_base, s.cnt_pre, s.off_pre, counts, offsets);
  hipLaunchKernelGGL(assign_scatter_kernel, dim3(nblk), dim3(256), msh_sc, st, ids, gates, s.keys, T,
                     top, E, s.off_pre, s.blk_base, 1, s.cand_token, s.cand_w,
                     s.cand_slot, s.cand_key, (int32_t *)nullptr, (uint8_t *)nullptr,
                     (int32_t *)nullptr, (int32_t *)nullptr);
  hipLaunchKernelGGL(cap_select_kernel, dim3(E), dim3(1024), 0, st, s.cand_token, s.cand_slot,
                     s.cand_key, s.cand_w, s.cnt_pre, s.off_pre, s.off_pre, C, (const int32_t *)nullptr,
                     S, (int32_t *)nullptr, (float *)nullptr, (int32_t *)nullptr, kept);
  // 2. offers of the tokens that lost picks, admitted into each expert's leftover places
  hipLaunchKernelGGL(expand_offer_kernel, dim3(nblk), dim3(256), 0, st, kept, T, k, S);
  const PairSel ext{kept, S, k, S, 1, 1};
  assign_pairs(s, ids, gates, T, ext, E, true, nullptr, nullptr, nullptr, nullptr, nullptr, st);
  hipLaunchKernelGGL(cap_select_kernel, dim3(E), dim3(1024), 0, st, s.cand_token, s.cand_slot,
                     s.cand_key, s.cand_w, s.cnt_pre, s.off_pre, s.off_pre, C, counts, S,
                     (int32_t *)nullptr, (float *)nullptr, (int32_t *)nullptr, kept);
  // 3. each token keeps as many admitted extra pairs as it lost, in slot order
  hipLaunchKernelGGL(expand_keep_kernel, dim3(nblk), dim3(256), 0, st, kept, T, k, S);
  // 4. dispatch of all kept pairs per expert
  const PairSel fin{kept, S, 0, S, 1, 1};
  assign_pairs(s, ids, gates, T, fin, E, false, perm_token, perm_w, nullptr, counts, offsets, st);
  return hipGetLastError();
}

hipError_t launch_expert_choice(const RouteScratch &s, const float *logits, int T, int E, int c,
                                int32_t *perm_token, float *perm_w, int32_t *counts,
                                int32_t *offsets, hipStream_t st, const float *logits_t) {
  if (T > 16384) logits_t = nullptr;
#define MOE_EC(K) hipLaunchKernelGGL((ec_select_regs_kernel<K>), dim3(E), dim3(1024), 0, st, logits, \
                                     T, E, c, perm_token, perm_w, s.slot_pos, counts, offsets,   \
                                     logits_t)
  if (T <= 2048) MOE_EC(2);
  else if (T <= 4096) MOE_EC(4);
  else if (T <= 8192) MOE_EC(8);
  else if (T <= 16384) MOE_EC(16);
  else
    hipLaunchKernelGGL(ec_select_kernel, dim3(E), dim3(1024), 0, st, logits, T, E, c, s.colkeys,
                       perm_token, perm_w, s.slot_pos, counts, offsets);
#undef MOE_EC
  return hipGetLastError();
}

hipError_t launch_token_csr(const RouteScratch &s, int T, int S, int32_t *tok_ptr,
                            int32_t *tok_pos, hipStream_t st) {
  const int nblk = (T + 255) / 256;
  if (nblk <= kCsrFusedBlocks) {   // two launches instead of three
    hipLaunchKernelGGL(tok_count_kernel, dim3(nblk), dim3(256), 0, st, s.slot_pos, T, S,
                       s.tok_blk);
    hipLaunchKernelGGL(tok_write_fused_kernel, dim3(nblk), dim3(256), 0, st, s.slot_pos, T, S,
                       s.tok_blk, tok_ptr, tok_pos);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(tok_count_kernel, dim3(nblk), dim3(256), 0, st, s.slot_pos, T, S,
                     s.tok_blk);
  hipLaunchKernelGGL(blk_scan_kernel, dim3(1), dim3(1024), 0, st, s.tok_blk, nblk, s.tok_blk_off,
                     (int32_t *)nullptr);
  hipLaunchKernelGGL(tok_write_kernel, dim3(nblk), dim3(256), 0, st, s.slot_pos, T, S,
                     s.tok_blk_off, tok_ptr, tok_pos);
  return hipGetLastError();
}

hipError_t launch_stats(const float *logits, const int32_t *counts, const int32_t *offsets, int T,
                        int E, int k, int token_choice, float *part, float *out, hipStream_t st) {
  const int nblk = (T + 255) / 256;
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(256), 0, st, logits, T, E, part);
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, st, part, nblk, counts, offsets,
                     T, E, k, token_choice, out);
  return hipGetLastError();
}

}  // namespace moe
