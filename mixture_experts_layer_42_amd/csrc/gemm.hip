// Grouped GEMMs of the expert SwiGLU FFN (gfx950).
//
//   gate/up:  h[p, :] = silu(x_perm[p] . W_gate[e]^T) * (x_perm[p] . W_up[e]^T)   [rows_e, d_ff]
//   down:     o[p, :] = h[p] . W_down[e]^T                                       [rows_e, d_model] fp32
// for every expert e over its rows p in [offsets[e], offsets[e+1]), plus one optional
// "shared" group with its own sizes (all T tokens, weight 1). Both operands are
// K-contiguous (weights in [out, in] layout), so A and B tiles stream along K.
//
// bf16 path: persistent workgroups walk a tile list built on the device from the
// per-expert row counts (no host round trip). A tile is 256 rows x 256 columns, K in
// steps of 64; 4 waves in a 2 x 2 layout each own 128 x 128 of the tile as 4 x 4 blocks
// of v_mfma_f32_32x32x16_bf16 with float32 accumulators. A and B K-slices are staged in
// LDS straight from global memory (gfx950 global_load_lds, no register staging), two
// stages so the next K-slice lands while the current one feeds the MFMAs, 16-byte chunks
// XOR-swizzled by row so the MFMA fragment reads hit distinct banks. Tiles of one expert that share a weight column are consecutive in the
// tile list, and consecutive list entries are given to workgroups on the same XCD, so the
// weight slice is fetched into that XCD's L2 once and reused by every row tile.
// For gate/up the B tile interleaves 64 gate rows and the matching 64 up rows per wave,
// so SiLU(gate) * up is formed in registers and only h is written.
//
// float32 path (used when the problem dtype is float32): a plain LDS-tiled SIMT GEMM over
// the same tile list.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct GroupDesc {
  const void *A;      // first row of the group
  const void *B0;     // [N, K] weights (gate or down)
  const void *B1;     // [N, K] up weights (gate/up only)
  void *C;            // first output row
  int rows, N, K, lda, ldc;
};

MOE_DEV GroupDesc group_desc(const GemmArgs &a, int g) {
  GroupDesc d;
  if (g < a.E) {
    const int off = a.offsets[g];
    d.rows = a.counts[g];
    d.A = (const char *)a.A + (size_t)off * a.lda * a.elt;
    d.B0 = (const char *)a.B0 + (size_t)g * a.N * a.K * a.elt;
    d.B1 = a.B1 ? (const char *)a.B1 + (size_t)g * a.N * a.K * a.elt : nullptr;
    d.C = (char *)a.C + (size_t)off * a.ldc * a.c_elt;
    d.N = a.N; d.K = a.K; d.lda = a.lda; d.ldc = a.ldc;
  } else {
    d.rows = a.s_rows;
    d.A = a.sA; d.B0 = a.sB0; d.B1 = a.sB1; d.C = a.sC;
    d.N = a.sN; d.K = a.sK; d.lda = a.s_lda; d.ldc = a.s_ldc;
  }
  return d;
}

// tile prefix over groups in LDS: tstart[g] = first tile of group g, tstart[G] = total
template <int BM, int BNOUT>
MOE_DEV int build_tile_table(const GemmArgs &a, int *tstart, int *sm) {
  const int G = a.E + (a.s_rows > 0 ? 1 : 0);
  int run = 0;
  for (int c0 = 0; c0 < G; c0 += blockDim.x) {
    const int g = c0 + threadIdx.x;
    int nt = 0;
    if (g < G) {
      const GroupDesc d = group_desc(a, g);
      nt = ((d.rows + BM - 1) / BM) * ((d.N + BNOUT - 1) / BNOUT);
    }
    int tot;
    const int ex = block_excl_scan(nt, sm, &tot);
    if (g < G) tstart[g] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) tstart[G] = run;
  __syncthreads();
  return G;
}

MOE_DEV int find_group(const int *tstart, int G, int tile) {
  int lo = 0, hi = G;   // tstart[lo] <= tile < tstart[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= tile) lo = mid; else hi = mid;
  }
  // skip empty groups sharing the same start
  while (lo + 1 < G && tstart[lo + 1] <= tile) ++lo;
  return lo;
}

MOE_DEV int xcd_virtual_block() {
  // workgroups are dispatched round-robin over the 8 XCDs; give consecutive virtual ids
  // to workgroups of the same XCD
  const int n = gridDim.x, b = blockIdx.x;
  if (n % 8 != 0) return b;
  return (b % 8) * (n / 8) + b / 8;
}

// ----------------------------------------------------------------------------------------
// bf16 MFMA kernel
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kLdsTile = BM * BK * 2;   // bytes of one A (or B) K-slice: 256 rows x 128 B

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// LDS byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`: rows of 128 B, chunks
// XOR-swizzled by (row/2) so that the 32 rows one MFMA fragment read touches spread over
// all banks.
MOE_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Direct global -> LDS copy of 16 bytes per lane: lane L of the wave writes LDS bytes
// [lds_base + 16 L, +16). lds_base must be the same in every lane.
MOE_DEV void g2lds16(const void *g, char *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t *)g, (lds_void_t *)lds_base, 16, 0, 0);
}

// Two pipeline stages as separate LDS objects, so loads into one stage are never mistaken
// for writes to the stage being read.
struct Stage { char a[kLdsTile]; char b[kLdsTile]; };

template <bool GATE_UP>
MOE_DEV void mma_stage(const Stage &st, int lane, int wm, int wn, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int chunk = ks * 2 + (lane >> 5);
    bf16x8_t af[4], bfr[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      af[mb] = *reinterpret_cast<const bf16x8_t *>(st.a + swz(wm * 128 + mb * 32 + (lane & 31), chunk));
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bfr[nb] = *reinterpret_cast<const bf16x8_t *>(st.b + swz(wn * 128 + nb * 32 + (lane & 31), chunk));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs args) {
  __shared__ Stage st0, st1;
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int sm[256 / 64 + 1];
  constexpr int BNOUT = GATE_UP ? BN / 2 : BN;
  const int G = build_tile_table<BM, BNOUT>(args, tstart, sm);
  const int total = tstart[G];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  for (int tile = xcd_virtual_block(); tile < total; tile += gridDim.x) {
    const int g = find_group(tstart, G, tile);
    const GroupDesc d = group_desc(args, g);
    const int local = tile - tstart[g];
    const int mt = (d.rows + BM - 1) / BM;
    const int n_tile = local / mt, m_tile = local % mt;
    const int m0 = m_tile * BM;
    // Loader: wave wv fills LDS rows wv*64 .. wv*64+63 of both slices with 8 copies of
    // 1 KB (8 rows) each; lane L fetches row r0 + L/8, physical chunk L%8, i.e. logical
    // K-chunk (L%8) ^ ((row/2)%8). For gate/up the B rows of wave wv are all gate rows
    // (wv even) or all up rows (wv odd): B row r holds h column n_tile*128 + (r/128)*64 + r%64.
    const int wvu = __builtin_amdgcn_readfirstlane(wv);   // wave-uniform, kept in SGPRs
    const char *Ab = (const char *)d.A;
    const char *Bb = (const char *)((GATE_UP && (wvu & 1)) ? d.B1 : d.B0);
    uint32_t aoff[8], boff[8];   // per-lane byte offsets from the (scalar) K-slice bases
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wvu * 64 + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      aoff[i] = ((uint32_t)min(m0 + r, d.rows - 1) * (uint32_t)d.lda + c * 8) * 2u;
      const int n = GATE_UP ? n_tile * (BN / 2) + (r >> 7) * 64 + (r & 63) : n_tile * BN + r;
      boff[i] = ((uint32_t)min(n, d.N - 1) * (uint32_t)d.K + c * 8) * 2u;
    }
    char *const la0 = st0.a + wvu * 8 * 1024, *const lb0 = st0.b + wvu * 8 * 1024;
    char *const la1 = st1.a + wvu * 8 * 1024, *const lb1 = st1.b + wvu * 8 * 1024;
    auto issue = [&](char *la, char *lb, int k0) {
      const char *a = Ab + (size_t)k0 * 2, *b = Bb + (size_t)k0 * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        g2lds16(a + aoff[i], la + i * 1024);
        g2lds16(b + boff[i], lb + i * 1024);
      }
    };
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = d.K / BK;
    issue(la0, lb0, 0);
    // K loop, two slices per trip: each half reads one fixed stage while the next slice
    // lands in the other one (an odd slice count ends with one more stage-0 step).
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      issue(la1, lb1, (kt + 1) * BK);
      mma_stage<GATE_UP>(st0, lane, wm, wn, acc);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt + 2 < nk) issue(la0, lb0, (kt + 2) * BK);
      mma_stage<GATE_UP>(st1, lane, wm, wn, acc);
    }
    if (kt < nk) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      mma_stage<GATE_UP>(st0, lane, wm, wn, acc);
    }
    __syncthreads();   // every wave is done with both stages before the next tile's loads
    // epilogue: h in bf16 (it feeds the next bf16 GEMM), o in float32
    bf16_t *Cb = (bf16_t *)d.C;
    float *Cf = (float *)d.C;
    if (GATE_UP) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n_tile * (BN / 2) + wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = m0 + wm * 128 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (row < d.rows && col < d.N) {
              const float gv = acc[mb][nb][i], uv = acc[mb][nb + 2][i];
              const float h = gv / (1.0f + __expf(-gv)) * uv;
              Cb[(size_t)row * d.ldc + col] = f32_to_bf16(h);
            }
          }
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = n_tile * BN + wn * 128 + nb * 32 + (lane & 31);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = m0 + wm * 128 + mb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (row < d.rows && col < d.N) Cf[(size_t)row * d.ldc + col] = acc[mb][nb][i];
          }
        }
    }
  }
}

// ----------------------------------------------------------------------------------------
// float32 SIMT kernel: 64 x 64 output tile, K step 16, 256 threads with 4 x 4 outputs each
// (gate/up keeps a gate and an up accumulator per output).
template <bool GATE_UP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs args) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[2][TK][TN + 4];
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int sm[256 / 64 + 1];
  const int G = build_tile_table<TM, TN>(args, tstart, sm);
  const int total = tstart[G];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int g = find_group(tstart, G, tile);
    const GroupDesc d = group_desc(args, g);
    const int local = tile - tstart[g];
    const int mt = (d.rows + TM - 1) / TM;
    const int n0 = (local / mt) * TN, m0 = (local % mt) * TM;
    const float *A = (const float *)d.A;
    const float *B0 = (const float *)d.B0, *B1 = (const float *)d.B1;
    float acc[2][4][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][i][j] = 0.f;
    for (int k0 = 0; k0 < d.K; k0 += TK) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < TM * TK; idx += 256) {
        const int r = idx / TK, c = idx % TK, m = m0 + r, k = k0 + c;
        As[c][r] = (m < d.rows && k < d.K) ? A[(size_t)m * d.lda + k] : 0.f;
        const int n = n0 + r;
        const bool ok = n < d.N && k < d.K;
        Bs[0][c][r] = ok ? B0[(size_t)n * d.K + k] : 0.f;
        if (GATE_UP) Bs[1][c][r] = ok ? B1[(size_t)n * d.K + k] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < TK; ++c) {
        float av[4], bv[4], uv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[c][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[j] = Bs[0][c][tx * 4 + j];
          uv[j] = GATE_UP ? Bs[1][c][tx * 4 + j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[0][i][j] = fmaf(av[i], bv[j], acc[0][i][j]);
            if (GATE_UP) acc[1][i][j] = fmaf(av[i], uv[j], acc[1][i][j]);
          }
      }
    }
    float *C = (float *)d.C;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
        if (m < d.rows && n < d.N) {
          float v = acc[0][i][j];
          if (GATE_UP) v = v / (1.0f + expf(-v)) * acc[1][i][j];
          C[(size_t)m * d.ldc + n] = v;
        }
      }
  }
}

int gemm_tiles_upper(const GemmArgs &a, int bm, int bn_out, int max_rows) {
  // every routed row tile: at most ceil(max_rows/bm) + E row tiles over all experts
  long t = (long)((max_rows + bm - 1) / bm + a.E) * ((a.N + bn_out - 1) / bn_out);
  if (a.s_rows > 0) t += (long)((a.s_rows + bm - 1) / bm) * ((a.sN + bn_out - 1) / bn_out);
  return (int)(t > (1 << 30) ? (1 << 30) : t);
}

hipError_t launch_gemm(const GemmArgs &a, bool gate_up, int max_rows, int num_cu,
                       hipStream_t st) {
  if (a.elt == 2) {
    const int bn_out = gate_up ? BN / 2 : BN;
    int grid = gemm_tiles_upper(a, BM, bn_out, max_rows);
    if (grid > num_cu) grid = num_cu;
    if (grid < 1) grid = 1;
    if (gate_up)
      hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  } else {
    int grid = gemm_tiles_upper(a, 64, 64, max_rows);
    if (grid > 4 * num_cu) grid = 4 * num_cu;
    if (grid < 1) grid = 1;
    if (gate_up)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t gemm_setup_attributes() { return hipSuccess; }

}  // namespace moe
