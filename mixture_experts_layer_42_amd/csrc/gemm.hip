// Grouped GEMMs of the expert SwiGLU FFN (gfx950).
//
//   gate/up:  h[p, :] = silu(x_perm[p] . W_gate[e]^T) * (x_perm[p] . W_up[e]^T)   [rows_e, d_ff]
//   down:     o[p, :] = h[p] . W_down[e]^T                                       [rows_e, d_model] fp32
// for every expert e over its rows p in [offsets[e], offsets[e+1]), plus one optional
// "shared" group with its own sizes (all T tokens, weight 1). Both operands are
// K-contiguous (weights in [out, in] layout), so A and B tiles stream along K.
//
// bf16 path: persistent workgroups walk a tile list built on the device from the
// per-expert row counts (no host round trip). A tile is 256 rows x 256 columns (a group's
// last row tile shrinks to 64, 128 or 192 rows when that covers its remaining rows); K goes in
// slices of 64 through two 72 KB LDS stages (one lands while the other feeds the MFMAs; a
// 256 x 256 tile uses 64 KB of each).
// Waves (4 as 2 x 2 of 128 x 128, or 8 as 2 x 4 of 128 x 64) compute with
// v_mfma_f32_32x32x16_bf16 into float32 accumulators. Slices are copied from global memory
// straight into LDS (gfx950 buffer loads into LDS, no register staging); each 1 KB copy covers 8
// rows x 128 B, i.e. whole 128-byte lines, which streams about twice as fast as half-line
// rows. 16-byte chunks are XOR-swizzled by row so the MFMA fragment reads hit distinct banks.
// Tiles of one expert go in bands of 4 weight panels, row tile by row tile inside a band, and
// consecutive list entries are given to workgroups on the same XCD, so the 32 workgroups of an
// XCD share a few weight panels and row tiles through its L2. A group's last row tile of at
// most 64 rows may span two panels (64 x 512, "wide", the down GEMM's default). For gate/up the B tile
// interleaves per wave column the gate rows and the matching up rows, so SiLU(gate) * up is
// formed in registers and only h is written.
//
// float32 path (used when the problem dtype is float32): a plain LDS-tiled SIMT GEMM over
// the same tile list.
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct GroupDesc {
  const void *A;      // first row of the group (or the whole A when rows are mapped)
  const int32_t *amap;  // row map of the group (rows read A[amap[r]]), or null
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
    d.amap = a.a_rows ? a.a_rows + off : nullptr;
    d.A = a.a_rows ? a.A : (const char *)a.A + (size_t)off * a.lda * a.elt;
    d.B0 = (const char *)a.B0 + (size_t)g * a.N * a.K * a.elt;
    d.B1 = a.B1 ? (const char *)a.B1 + (size_t)g * a.N * a.K * a.elt : nullptr;
    d.C = (char *)a.C + (size_t)off * a.ldc * a.c_elt;
    d.N = a.N; d.K = a.K; d.lda = a.lda; d.ldc = a.ldc;
  } else {
    d.rows = a.s_rows;
    d.amap = nullptr;
    d.A = a.sA; d.B0 = a.sB0; d.B1 = a.sB1; d.C = a.sC;
    d.N = a.sN; d.K = a.sK; d.lda = a.s_lda; d.ldc = a.s_ldc;
  }
  return d;
}

// Whether a group of `rows` rows (mt row tiles of 256) takes wide last row tiles (bf16 path,
// see group_tile): its last row tile holds at most 64 rows and N is a whole number of at least
// two column panels of bnout columns, so the second panel of a pair never reaches past N.
MOE_DEV bool group_wide(int rows, int mt, int N, int bnout) {
  return rows > 0 && N % bnout == 0 && N / bnout >= 2 && rows - (mt - 1) * 256 <= 64;
}

// Tiles of a group of `rows` rows and N columns, tiles of TM rows x bnout columns.
template <int TM>
MOE_DEV int group_tiles(int rows, int N, int bnout, bool wide) {
  const int mt = (rows + TM - 1) / TM, ncol = (N + bnout - 1) / bnout;
  if (!wide || !group_wide(rows, mt, N, bnout)) return mt * ncol;
  return (ncol / 2) * (2 * mt - 1) + (ncol & 1) * mt;
}

// tile prefix over groups in LDS: tstart[g] = first tile of group g, tstart[G] = total
template <int BM, int BNOUT>
MOE_DEV int build_tile_table(const GemmArgs &a, int *tstart, int *sm, bool wide = false) {
  const int G = a.E + (a.s_rows > 0 ? 1 : 0);
  int run = 0;
  for (int c0 = 0; c0 < G; c0 += blockDim.x) {
    const int g = c0 + threadIdx.x;
    int nt = 0;
    if (g < G) {
      const GroupDesc d = group_desc(a, g);
      nt = group_tiles<BM>(d.rows, d.N, BNOUT, wide);
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

// Tail split. With P persistent workgroups and `total` tiles, the first r*P tiles (r whole
// rounds) run whole; if the remaining L tiles fill at most half a round, each is cut into
// S = min(8, floor(P / L)) K-parts (part p takes K-slices [p nk / S, (p + 1) nk / S)) so
// that the last round takes about 1/S of a tile's time. Each part keeps at least
// kMinPartSteps slices: a part stores a float32 partial tile (256 KB) that the reduction reads
// back, which shorter parts do not amortise (Mixtral-shaped gate/up GEMM: 5 parts of 12.8
// slices measured 1% slower than 4 of 16; down GEMM: 3 parts of 74.7 slices 4.5% faster than
// 2 of 112). Both the GEMM and the reduction kernel derive
// the same plan from the device-side tile count. P is always kMaxPersistent (one workgroup
// per CU of a full MI355X), whatever grid actually runs: which tiles are split, and so the
// order of every float32 sum, does not depend on how many CUs the launch gets.
struct SplitPlan { int full, L, S; };
constexpr int kMinPartSteps = 16;

MOE_DEV SplitPlan split_plan(int total, int P, int nk, int ok) {
  SplitPlan sp{total, 0, 1};
  const int r = total / P, L = total - r * P;
  if (!ok || L == 0 || 2 * L > P) return sp;
  int S = P / L;
  if (S > 8) S = 8;
  while (S > 1 && nk / S < kMinPartSteps) --S;
  if (S < 2) return sp;
  sp.full = r * P; sp.L = L; sp.S = S;
  return sp;
}

// ----------------------------------------------------------------------------------------
// bf16 MFMA kernel. A tile is 256 rows x 256 B-columns, K in slices of 64 staged through two
// 64 KB LDS buffers. W waves share it: W = 4 as 2 x 2 waves of 128 x 128 (one wave per
// SIMD, 256 accumulators each), W = 8 as 2 x 4 waves of 128 x 64 (two waves per SIMD, so
// one wave's LDS reads and barrier waits overlap the other's MFMAs).
constexpr int BM = 256, BN = 256, BK = 64, NSTAGE = 2;
constexpr int kRowBytes = BK * 2;                 // 128 B: 8 chunks of 16 B
constexpr int kSub = BK / 16;                     // k=16 MFMA sub-steps per slice
constexpr int kMaxWaves = 8;

template <int W> struct Cfg {
  static constexpr int WN = W / 2;                // wave columns (two wave rows of 128)
  static constexpr int WCOLS = BN / WN;           // B columns per wave
  static constexpr int NB = WCOLS / 32;           // 32-column MFMA blocks per wave
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int A_DMA = A_BYTES / 1024 / W, B_DMA = B_BYTES / 1024 / W;   // per wave
  static constexpr int DMA = A_DMA + B_DMA;       // 1 KB copies per wave per slice
  static constexpr int PART_WAVE = 4 * NB * 16 * 64;     // floats of one wave's accumulators
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// LDS byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`: rows of 128 B, chunks
// XOR-swizzled by (row/2) % 8, so that the 16 rows a quarter-wave of an MFMA fragment read
// touches (same logical chunk) cover all 64 banks exactly once.
MOE_DEV int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Direct global -> LDS copy of 16 bytes per lane: lane L of the wave writes LDS bytes
// [lds_base + 16 L, +16). lds_base must be the same in every lane.
MOE_DEV void g2lds16(const void *g, char *lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t *)g, (lds_void_t *)lds_base, 16, 0, 0);
}

// The same copy through a buffer resource: lane L writes LDS bytes [lds_base + 16 L, +16)
// from byte voff + soff of the resource (soff wave-uniform). Buffer copies count only
// against the vector-memory counter, while global copies into LDS also count as LDS events
// for the compiler's wait insertion, which then has to wait for every outstanding LDS read
// (lgkmcnt(0)) before each MFMA sub-step instead of only the fragments that sub-step needs.
MOE_DEV void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 16, (int)voff, soff, 0, 0);
}

// Buffer resource over an operand with the whole 32-bit byte range (operand byte offsets
// stay below 4 GiB: the entry points reject larger panels).
MOE_DEV __amdgpu_buffer_rsrc_t operand_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, -1, 0x00020000);
}

// The pipeline stages are separate LDS objects, so loads into one stage are never mistaken
// for writes to the stage being read. A wide tile (kWideMB) puts its 64 A rows at the start of
// the stage and its 512 B rows right after them (8 KB + 64 KB), hence the longer b.
constexpr int kWideA = 64 * kRowBytes;
struct Stage { char a[BM * kRowBytes]; char b[BN * kRowBytes + kWideA]; };
static_assert(sizeof(Stage) == kWideA + 2 * BN * kRowBytes, "wide layout fills the stage");
MOE_DEV const char *stage_b(const Stage &st, bool wide) {
  return wide ? reinterpret_cast<const char *>(&st) + kWideA : st.b;
}
MOE_DEV char *stage_b(Stage &st, bool wide) {
  return wide ? reinterpret_cast<char *>(&st) + kWideA : st.b;
}

// Row tiles. A group's rows go in tiles of 256; its last tile, holding rem = rows - m0 rows,
// shrinks to 64 * MB rows with MB = 1 (rem <= 64), 2 (rem <= 128), 3 (rem <= 192) or 4, so a
// ragged group end costs MFMAs for at most 63 padding rows instead of up to 255. Wave row wm
// of a tile owns rows wm * 32 MB .. + 32 MB - 1 as MB blocks of 32.
MOE_DEV int tile_mb(int rem) { return rem > 192 ? 4 : (rem > 128 ? 3 : (rem > 64 ? 2 : 1)); }

// Wide last row tiles. A 64-row tile costs a quarter of a full tile's MFMAs but, bound by the
// latency of its copies landing, about 70% of its time. When a group's last row tile holds at
// most 64 rows and the group has at least two column panels, its column panels go in pairs:
// the full row tiles of panel 2q, those of panel 2q+1, then one 64-row tile spanning both
// panels (512 B-columns, mb = kWideMB), which reads its rows once for the pair and keeps the
// MFMAs of 8 waves busy with 64 x 64 each; an odd last panel keeps its own row tiles. The
// tiles that share a weight panel stay next to each other in the list. Groups without wide
// tiles go in bands of `band` panels, row tile by row tile inside a band (each row tile's
// panels of the band in order); band <= 1 or a single row tile: panel by panel.
constexpr int kWideMB = 5;
struct TileLoc { int n_tile, m0, mb; };   // n_tile: first column panel of the tile

MOE_DEV TileLoc group_tile(int rows, int N, int bnout, bool wide, int local, int band = 1) {
  const int mt = (rows + BM - 1) / BM, ncol = (N + bnout - 1) / bnout;
  TileLoc t;
  if (!wide || !group_wide(rows, mt, N, bnout)) {
    if (band > 1 && mt > 1) {
      // bands of `band` panels; inside a band row tile by row tile, its panels in order
      const int b = local / (mt * band), in = local % (mt * band);
      const int w = min(band, ncol - b * band);
      t.n_tile = b * band + in % w;
      t.m0 = (in / w) * BM;
    } else {
      t.n_tile = local / mt;
      t.m0 = (local % mt) * BM;
    }
    t.mb = tile_mb(rows - t.m0);
    return t;
  }
  const int mf = mt - 1, per = 2 * mf + 1, paired = (ncol / 2) * per;
  if (local < paired) {
    const int q = local / per, r = local % per;
    if (r < 2 * mf) {
      t.n_tile = 2 * q + r / mf;
      t.m0 = (r % mf) * BM;
      t.mb = 4;
    } else {
      t.n_tile = 2 * q;
      t.m0 = mf * BM;
      t.mb = kWideMB;
    }
  } else {
    t.n_tile = ncol - 1;
    t.m0 = (local - paired) * BM;
    t.mb = tile_mb(rows - t.m0);
  }
  return t;
}

// fragments of sub-step ks (k = 16 ks .. 16 ks + 15 of the slice)
template <int W, int MB, bool WIDE>
MOE_DEV void load_frags(const Stage &st, int lane, int wm, int wn, int ks, bf16x8_t (&af)[MB],
                        bf16x8_t (&bfr)[Cfg<W>::NB]) {
  const int chunk = ks * 2 + (lane >> 5);
  const char *sb = stage_b(st, WIDE);
  // in the order the MFMAs (mb outer, nb inner) consume them: A0, every B, then A1 ..
  // so that the first MFMAs of the sub-step wait only for the reads issued first
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    af[mb] = *reinterpret_cast<const bf16x8_t *>(st.a + swz(wm * 32 * MB + mb * 32 + (lane & 31), chunk));
    if (mb == 0) {
#pragma unroll
      for (int nb = 0; nb < Cfg<W>::NB; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8_t *>(
            sb + swz(wn * Cfg<W>::WCOLS + nb * 32 + (lane & 31), chunk));
    }
  }
}

template <int W, int MB>
MOE_DEV void mfma_block(const bf16x8_t (&af)[MB], const bf16x8_t (&bfr)[Cfg<W>::NB],
                        f32x16_t (&acc)[MB][Cfg<W>::NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < Cfg<W>::NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
}

// silu(g) * u of the bf16 paths: the hardware reciprocal (about 1 ulp) instead of a
// correctly rounded division; h is rounded to bf16 (8 significant bits) right after
MOE_DEV float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// keep the instruction order written here (no scheduling across this point)
MOE_DEV void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt until at most VM vector-memory and LGKM LDS/scalar operations are outstanding.
// Issued through the builtin, not inline asm, so the compiler's own wait insertion knows
// which copies have landed: after an opaque wait it would still count the previous slice's
// global->LDS copies as in flight and stall the first LDS read behind the copies just issued.
template <int VM, int LGKM> MOE_DEV void wait_vm_lgkm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "gfx9 s_waitcnt fields");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// The wait above, then the workgroup barrier; the empty asm statements keep the compiler
// from moving LDS accesses across either (they emit no instruction).
template <int VM> MOE_DEV void wait_and_barrier() {
  wait_vm_lgkm<VM, 0>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Instruction order of one sub-step's N MFMAs: after MFMA I come I-th shares of the DMA
// global->LDS copies and of the RD LDS fragment reads (one read after each of the first RD
// MFMAs when RD <= N).
template <int N, int DMA, int RD, int I = 0>
MOE_DEV void sched_sub() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int c = (DMA * (I + 1)) / N - (DMA * I) / N;
    if constexpr (c > 0) __builtin_amdgcn_sched_group_barrier(0x020, c, 0);
    constexpr int r = RD <= N ? (I < RD ? 1 : 0) : (RD * (I + 1)) / N - (RD * I) / N;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    sched_sub<N, DMA, RD, I + 1>();
  }
}

// Offset of tile element (tr, tc) (tc a B-tile column) in a partial tile stored in
// accumulator register order: wave (tr/(32 MB))*WN + tc/WCOLS, then block (mb, nb) =
// (tr%(32 MB)/32, tc%WCOLS/32), register i = 4*(tr%32/8) + tr%4, lane = tc%32 + 32*(tr%8/4).
// The row and column parts add, and 4 adjacent columns (tc % 4 == 0) are 4 adjacent floats.
template <int W> MOE_DEV int part_index(int tr, int tc, int MB) {
  using C = Cfg<W>;
  const int rpw = 32 * MB;
  const int row_part = (tr / rpw) * C::WN * C::PART_WAVE + ((tr % rpw) >> 5) * C::NB * 16 * 64 +
                       (4 * ((tr >> 3) & 3) + (tr & 3)) * 64 + 32 * ((tr >> 2) & 1);
  const int col_part = (tc / C::WCOLS) * C::PART_WAVE + ((tc % C::WCOLS) >> 5) * 16 * 64 + (tc & 31);
  return row_part + col_part;
}

// A unit of work: a row tile of 64*mb rows x 256 B-columns of group d over K-steps
// [k_begin, k_begin + nk), stored whole (punit < 0) or as the float32 partial tile punit.
struct Unit {
  GroupDesc d;
  int n_tile, m0, nk, k_begin, punit, mb;
};

// The fields of a unit are the same in every lane; readfirstlane keeps them in scalar registers
// (the buffer resources built from its pointers must be scalar operands)
MOE_DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename P> MOE_DEV P *uni_ptr(P *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
MOE_DEV void make_uniform(Unit &x) {
  x.d.A = uni_ptr(x.d.A); x.d.amap = uni_ptr(x.d.amap); x.d.B0 = uni_ptr(x.d.B0);
  x.d.B1 = uni_ptr(x.d.B1); x.d.C = uni_ptr(x.d.C);
  x.d.rows = uni(x.d.rows); x.d.N = uni(x.d.N); x.d.K = uni(x.d.K); x.d.lda = uni(x.d.lda);
  x.d.ldc = uni(x.d.ldc);
  x.n_tile = uni(x.n_tile); x.m0 = uni(x.m0); x.nk = uni(x.nk); x.k_begin = uni(x.k_begin);
  x.punit = uni(x.punit); x.mb = uni(x.mb);
}

// Per-lane byte offsets of a unit's copies from the slice bases (A: A_DMA used, B: B_DMA
// used; a wide tile copies its second 256 B rows from the same offsets plus one panel).
struct Offs { uint32_t a[4], b[4]; };

// Loader: wave wv fills A rows wv*TBM/W .. and B rows wv*BN/W .. with copies of 1 KB (8 rows of
// 128 B); lane L fetches row r0 + L/8, physical chunk L%8, i.e. logical K-chunk
// (L%8) ^ ((row/2)%8). For gate/up the B tile holds, per wave column wn, WCOLS/2 gate rows then
// the matching WCOLS/2 up rows (h columns n_tile*128 + wn*WCOLS/2 + j), so the B rows a wave
// loads are all gate (wv even) or all up (wv odd).
template <bool GATE_UP, int W, int MB, bool WIDE>
MOE_DEV void unit_offsets(const Unit &x, Offs &o) {
  using C = Cfg<W>;
  constexpr int TBM = WIDE ? 64 : 64 * MB;          // tile rows
  constexpr int A_DMA = TBM * kRowBytes / 1024 / W;
  static_assert(A_DMA <= 4 && C::B_DMA <= 4, "Offs holds 4 + 4 offsets");
  static_assert(!WIDE || (W == 8 && MB == 2), "a wide tile is 64 rows of 8 waves of 64 x 64");
  const int lane = threadIdx.x & 63;
  const int wvu = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const int r = wvu * (TBM / W) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int arow = min(x.m0 + r, x.d.rows - 1);
    if (x.d.amap) arow = x.d.amap[arow];   // dispatch gather folded into the operand load
    o.a[i] = ((uint32_t)arow * (uint32_t)x.d.lda + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < C::B_DMA; ++i) {
    const int r = wvu * (BN / W) + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int n = GATE_UP ? x.n_tile * (BN / 2) + (wvu >> 1) * (C::WCOLS / 2) +
                                (r & (C::WCOLS / 2 - 1))
                          : x.n_tile * BN + r;
    o.b[i] = ((uint32_t)min(n, x.d.N - 1) * (uint32_t)x.d.K + c * 8) * 2u;
  }
}

// Copies of K-slice kt of unit x into stage s. The B rows a wave copies are all gate rows (even
// wave) or all up rows (odd wave). A wide tile copies B-tile rows 256 + r from weight rows one
// panel further (BN/2 rows for gate/up, BN for down) than those of row r, through the scalar
// offset (the pair never reaches past N, see group_wide).
template <bool GATE_UP, int W, int MB, bool WIDE>
MOE_DEV void unit_issue(const Unit &x, const Offs &o, Stage &s, int kt) {
  using C = Cfg<W>;
  constexpr int A_DMA = (WIDE ? 64 : 64 * MB) * kRowBytes / 1024 / W;
  const int wvu = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const char *Ab = (const char *)x.d.A;
  const char *Bb = (const char *)((GATE_UP && (wvu & 1)) ? x.d.B1 : x.d.B0);
  const __amdgpu_buffer_rsrc_t ra = operand_rsrc(Ab), rb = operand_rsrc(Bb);
  const int aofs = wvu * A_DMA * 1024, bofs = wvu * C::B_DMA * 1024;
  char *sb = stage_b(s, WIDE);
  const int so = (x.k_begin + kt) * kRowBytes;   // K offset of the slice, bytes
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) b2lds16(ra, o.a[i], so, s.a + aofs + i * 1024);
#pragma unroll
  for (int i = 0; i < C::B_DMA; ++i) b2lds16(rb, o.b[i], so, sb + bofs + i * 1024);
  if constexpr (WIDE) {
    const int so2 = so + (GATE_UP ? BN / 2 : BN) * x.d.K * 2;
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i) b2lds16(rb, o.b[i], so2, sb + BN * kRowBytes + bofs + i * 1024);
  }
}

// The offsets of unit x and the copies of its first slice into st0.
template <bool GATE_UP, int W>
MOE_DEV void unit_prefetch(const Unit &x, Offs &o, Stage &st0) {
  switch (x.mb) {
    case 4: unit_offsets<GATE_UP, W, 4, false>(x, o); unit_issue<GATE_UP, W, 4, false>(x, o, st0, 0); break;
    case 3: unit_offsets<GATE_UP, W, 3, false>(x, o); unit_issue<GATE_UP, W, 3, false>(x, o, st0, 0); break;
    case 2: unit_offsets<GATE_UP, W, 2, false>(x, o); unit_issue<GATE_UP, W, 2, false>(x, o, st0, 0); break;
    case kWideMB:
      if constexpr (W == 8) {
        unit_offsets<GATE_UP, W, 2, true>(x, o); unit_issue<GATE_UP, W, 2, true>(x, o, st0, 0);
      }
      break;
    default: unit_offsets<GATE_UP, W, 1, false>(x, o); unit_issue<GATE_UP, W, 1, false>(x, o, st0, 0); break;
  }
}

// One unit, its first slice already in flight into st0. When the previous unit's epilogue
// left stores in flight (stores_pending: at least 16 of this wave's, issued after this unit's
// first copies), the first wait lets up to 16 operations stay outstanding: vector-memory
// operations complete in issue order, so the copies have landed and only stores remain. After
// the K loop the next unit's first slice is issued before this unit's epilogue, so its copies
// travel while the outputs are stored. Returns whether this wave's epilogue left stores in
// flight. A wide tile (WIDE, MB = 2) is 64 rows x 512 B-columns: one wave row, wave wv owns
// all 64 rows of B-columns wv*64 .. +63, the same 2 x 2 blocks as a wave of a 128-row tile.
template <bool GATE_UP, int W, int MB, bool WIDE>
MOE_DEV __attribute__((always_inline)) bool gemm_tile(const GemmArgs &args, const Unit &x,
                                                      const Offs &o, Stage &st0, Stage &st1,
                                                      bool stores_pending, bool has_next,
                                                      const Unit &nx, Offs &no) {
  using C = Cfg<W>;
  constexpr int NB = C::NB;
  constexpr int TBM = WIDE ? 64 : 64 * MB;        // tile rows
  constexpr int A_DMA = TBM * kRowBytes / 1024 / W;   // A copies per wave per slice
  constexpr int DMA = A_DMA + (WIDE ? 2 : 1) * C::B_DMA;
  constexpr int BNOUT = GATE_UP ? BN / 2 : BN;
  const GroupDesc &d = x.d;
  const int n_tile = x.n_tile, m0 = x.m0, nk = x.nk, punit = x.punit;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = WIDE ? 0 : wv / C::WN, wn = WIDE ? __builtin_amdgcn_readfirstlane(wv) : wv % C::WN;
  auto issue = [&](Stage &s, int kt) { unit_issue<GATE_UP, W, MB, WIDE>(x, o, s, kt); };
  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Pipeline. Slice s lives in stage s % 2. Step kt waits until slice kt has landed,
  // passes the barrier (every wave has its last fragments of slice kt-1 in registers by
  // then, so that stage is free), issues the copy of slice kt+1 into it, and runs the
  // MFMAs: those of the last sub-step of slice kt-1, then sub-steps 0..2 of slice kt, each
  // with the LDS reads of the next sub-step (and, in the first, the copies) slotted
  // between them. The last sub-step of slice kt runs after the next barrier. Fragments
  // alternate between two register sets (even and odd sub-steps).
  bf16x8_t fa0[MB], fb0[NB], fa1[MB], fb1[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) fa1[i] = bf16x8_t{};   // "slice -1": contributes 0 * 0
#pragma unroll
  for (int i = 0; i < NB; ++i) fb1[i] = bf16x8_t{};
  // (slice 0 was issued into st0 by unit_prefetch)
  // MFMAs of (fa, fb) with the fragment reads of the next sub-step between them
  auto sub = [&](const bf16x8_t (&fa)[MB], const bf16x8_t (&fb)[NB], const Stage &cur, int ks,
                 bf16x8_t (&na)[MB], bf16x8_t (&nb)[NB]) {
    load_frags<W, MB, WIDE>(cur, lane, wm, wn, ks, na, nb);
    mfma_block<W, MB>(fa, fb, acc);
    sched_sub<MB * NB, 0, MB + NB>();
    sched_fence();
  };
  auto step = [&](Stage &cur, Stage &refill, int kt, auto vm) {
    sched_fence();
    wait_and_barrier<decltype(vm)::value>();   // slice kt has landed
    sched_fence();
    issue(refill, min(kt + 1, nk - 1));   // past the end: re-read the last slice
    load_frags<W, MB, WIDE>(cur, lane, wm, wn, 0, fa0, fb0);
    mfma_block<W, MB>(fa1, fb1, acc);      // last sub-step of slice kt-1
    sched_sub<MB * NB, DMA, MB + NB>();    // copies and reads between the MFMAs
    sched_fence();
    sub(fa0, fb0, cur, 1, fa1, fb1);
    sub(fa1, fb1, cur, 2, fa0, fb0);
    sub(fa0, fb0, cur, 3, fa1, fb1);
  };
  static_assert(kSub == 4 && NSTAGE == 2, "the step above runs four sub-steps, two stages");
  using V0 = std::integral_constant<int, 0>;
  using V16 = std::integral_constant<int, 16>;
  // The first step (stores of the previous unit may still be in flight), then two steps per
  // iteration alternating the stages. The loop body is one branch-free block, so the
  // compiler's wait counts stay exact inside it; an odd last step follows it.
  if (stores_pending) step(st0, st1, 0, V16{});
  else step(st0, st1, 0, V0{});
  int kt = 1;
  for (; kt + 2 <= nk; kt += 2) {
    step(st1, st0, kt, V0{});
    step(st0, st1, kt + 1, V0{});
  }
  if (kt < nk) step(st1, st0, kt, V0{});
  mfma_block<W, MB>(fa1, fb1, acc);   // last sub-step of the last slice
  wait_vm_lgkm<0, 15>();   // the surplus copy of the last step
  __syncthreads();   // every wave is done with every stage before the next tile's loads
  if (has_next) unit_prefetch<GATE_UP, W>(nx, no, st0);
  if (punit >= 0) {
    // K-part of a split tile: the raw accumulators in register order (wave, mb, nb, i,
    // lane), so each store is 256 contiguous bytes; the reduction maps them back
    float *Pt = args.partials + (size_t)punit * (BM * BN) + wv * C::PART_WAVE + lane;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) Pt[((mb * NB + nb) * 16 + i) * 64] = acc[mb][nb][i];
    return true;   // MB * NB * 16 >= 32 stores
  }
  // epilogue: h in bf16 (it feeds the next bf16 GEMM), o in float32. Lane (c, r4) holds
  // column c of rows r4*4 + {0..3} + 8j of each 32 x 32 block. Stores go through a buffer
  // resource spanning exactly the group's output rows, so the hardware drops the stores of
  // rows past the group's end (a partial last row tile needs no per-element branch). The
  // lane index is made opaque so the per-lane offset is rebuilt each tile rather than
  // hoisted with 256 others.
  int lo = lane;
  asm volatile("" : "+v"(lo));
  constexpr int CE = GATE_UP ? 2 : 4;   // bytes per output element
  constexpr int OB = GATE_UP ? NB / 2 : NB;   // output blocks per wave row
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      d.C, (short)0, (int)((uint32_t)d.rows * (uint32_t)d.ldc * CE), 0x00020000);
  const int cw = n_tile * BNOUT + wn * (OB * 32);   // first output column of this wave
  const int nbv = (d.N - cw) >= OB * 32 ? OB : (d.N - cw) / 32;   // live blocks
  const uint32_t rowb = (uint32_t)d.ldc * CE;
  // running byte offset of this lane's current row, advanced row by row (kept opaque so the
  // compiler does not expand it into one live offset per row)
  uint32_t roff = (uint32_t)(m0 + wm * 32 * MB + 4 * (lo >> 5)) * rowb + (uint32_t)(cw + (lo & 31)) * CE;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int nb = 0; nb < OB; ++nb) {
        if (nb < nbv) {
          if (GATE_UP) {
            const float gv = acc[mb][nb][i], uv = acc[mb][nb + OB][i];
            const float h = swiglu(gv, uv);
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(h), rs, (int)(roff + nb * 32 * CE),
                                                  0, 0);
          } else {
            float v = acc[mb][nb][i];
            asm volatile("" : "+v"(v));
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs,
                                                  (int)(roff + nb * 32 * CE), 0, 0);
          }
        }
      }
      // next row of this lane: +1 inside a group of 4, +5 after the 4th (rows 4..7 belong
      // to the other half-wave), the last i of a block steps to the next block the same way
      roff += ((i & 3) == 3 ? 5u : 1u) * rowb;
      asm volatile("" : "+v"(roff));
    }
  return nbv > 0;   // MB * 16 * nbv >= 16 stores
}

template <bool GATE_UP, int W>
__global__ __launch_bounds__(64 * W, 1) void gemm_bf16_kernel(GemmArgs args) {
  __shared__ Stage st0, st1;
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int sm[kMaxWaves + 1];
  constexpr int BNOUT = GATE_UP ? BN / 2 : BN;   // output columns per tile (h or o)
  const bool wide = W == 8 && args.wide;
  const int G = build_tile_table<BM, BNOUT>(args, tstart, sm, wide);
  const int total = tstart[G];

  const SplitPlan sp = split_plan(total, kMaxPersistent, args.K / BK, args.split_ok);
  const int units = sp.full + sp.L * sp.S;
  // unit u of the list: its tile (or K-part of a split tile), group, position and K range
  auto unit_at = [&](int u) {
    Unit x;
    int tile = u, part = 0, nparts = 1;
    if (u >= sp.full) {
      tile = sp.full + (u - sp.full) / sp.S;
      part = (u - sp.full) % sp.S;
      nparts = sp.S;
    }
    const int g = find_group(tstart, G, tile);
    x.d = group_desc(args, g);
    const TileLoc tl = group_tile(x.d.rows, x.d.N, BNOUT, wide, tile - tstart[g], args.band);
    x.n_tile = tl.n_tile;
    x.m0 = tl.m0;
    x.mb = tl.mb;
    const int nk_all = x.d.K / BK;
    x.k_begin = part * nk_all / nparts;                  // first K-step of this unit
    x.nk = (part + 1) * nk_all / nparts - x.k_begin;     // K-steps of this unit
    x.punit = nparts > 1 ? u - sp.full : -1;
    make_uniform(x);
    return x;
  };
  int u = xcd_virtual_block();
  if (u >= units) return;   // workgroup-uniform
  Unit cur = unit_at(u);
  Offs co;
  unit_prefetch<GATE_UP, W>(cur, co, st0);
  bool pending = false;
  for (; u < units; u += gridDim.x) {
    const bool has_next = u + (int)gridDim.x < units;
    const Unit nx = has_next ? unit_at(u + gridDim.x) : cur;
    Offs no = co;
    switch (cur.mb) {
      case 4: pending = gemm_tile<GATE_UP, W, 4, false>(args, cur, co, st0, st1, pending, has_next, nx, no); break;
      case 3: pending = gemm_tile<GATE_UP, W, 3, false>(args, cur, co, st0, st1, pending, has_next, nx, no); break;
      case 2: pending = gemm_tile<GATE_UP, W, 2, false>(args, cur, co, st0, st1, pending, has_next, nx, no); break;
      case kWideMB:
        if constexpr (W == 8)
          pending = gemm_tile<GATE_UP, W, 2, true>(args, cur, co, st0, st1, pending, has_next, nx, no);
        break;
      default: pending = gemm_tile<GATE_UP, W, 1, false>(args, cur, co, st0, st1, pending, has_next, nx, no); break;
    }
    cur = nx;
    make_uniform(cur);
    co = no;
  }
}

// Sum of the K-parts of split tiles, in part order, then the same epilogue as a whole tile.
// Work item: 32 rows of one split tile; each thread owns 4 adjacent output columns of a row
// (all S part loads issued before the sums). The plan is the GEMM's (same tile count, same P),
// so any grid of this kernel sees the same split.
constexpr int kReduceRows = 32;

template <bool GATE_UP, int W>
__global__ __launch_bounds__(256) void gemm_tail_reduce_kernel(GemmArgs args) {
  using C = Cfg<W>;
  constexpr int BNOUT = GATE_UP ? BN / 2 : BN;
  constexpr int TPR = BNOUT / 4;        // threads per row
  constexpr int RPP = 256 / TPR;        // rows per pass
  constexpr int PART = BM * BN;         // floats per partial tile
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int sm[kMaxWaves + 1];
  const bool wide = W == 8 && args.wide;
  const int G = build_tile_table<BM, BNOUT>(args, tstart, sm, wide);
  const SplitPlan sp = split_plan(tstart[G], kMaxPersistent, args.K / BK, args.split_ok);
  const int items = sp.L * (BM / kReduceRows);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int l = it / (BM / kReduceRows), ri = it % (BM / kReduceRows);
    const int tile = sp.full + l;
    const int g = find_group(tstart, G, tile);
    const GroupDesc d = group_desc(args, g);
    const TileLoc tl = group_tile(d.rows, d.N, BNOUT, wide, tile - tstart[g], args.band);
    // item ri: rows ri*32 .. of the tile; of a wide tile (64 rows, two column panels) rows
    // (ri % 2)*32 .. of panel ri / 2 (items 4..7 have nothing to do)
    const bool wt = tl.mb == kWideMB;
    if (wt && ri >= 4) continue;
    const int r0 = (wt ? ri & 1 : ri) * kReduceRows;
    const int ch = wt ? ri >> 1 : 0;                   // column panel within the tile
    const int MB = wt ? 2 : tl.mb;                     // rows per wave row / 32 in the layout
    const int c = ch * BNOUT + (threadIdx.x % TPR) * 4;   // first of 4 output columns in the tile
    const int col = tl.n_tile * BNOUT + c;
    if (col >= d.N) continue;                         // N is a multiple of 64: whole groups of 4
    for (int rr = threadIdx.x / TPR; rr < kReduceRows; rr += RPP) {
      const int tr = r0 + rr, row = tl.m0 + tr;
      if (row >= d.rows) break;
      const float *P0 = args.partials + (size_t)l * sp.S * PART + part_index<W>(tr, 0, MB);
      if (GATE_UP) {
        // h column c: gate sum at B-tile column (c / (WCOLS/2)) * WCOLS + c % (WCOLS/2), up
        // sum WCOLS/2 columns further
        const int tc = (c / (C::WCOLS / 2)) * C::WCOLS + c % (C::WCOLS / 2);
        const int og = part_index<W>(0, tc, MB), ou = part_index<W>(0, tc + C::WCOLS / 2, MB);
        float4 gp[8], up[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          if (p < sp.S) {
            gp[p] = *(const float4 *)(P0 + (size_t)p * PART + og);
            up[p] = *(const float4 *)(P0 + (size_t)p * PART + ou);
          }
        float4 gs = gp[0], us = up[0];
#pragma unroll
        for (int p = 1; p < 8; ++p)
          if (p < sp.S) {
            gs.x += gp[p].x; gs.y += gp[p].y; gs.z += gp[p].z; gs.w += gp[p].w;
            us.x += up[p].x; us.y += up[p].y; us.z += up[p].z; us.w += up[p].w;
          }
        const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
        uint32_t pk[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float h0 = swiglu(gv[2 * j], uv[2 * j]);
          const float h1 = swiglu(gv[2 * j + 1], uv[2 * j + 1]);
          pk[j] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
        }
        *(uint2 *)((bf16_t *)d.C + (size_t)row * d.ldc + col) = make_uint2(pk[0], pk[1]);
      } else {
        float4 pp[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          if (p < sp.S) pp[p] = *(const float4 *)(P0 + (size_t)p * PART + part_index<W>(0, c, MB));
        float4 v = pp[0];
#pragma unroll
        for (int p = 1; p < 8; ++p)
          if (p < sp.S) { v.x += pp[p].x; v.y += pp[p].y; v.z += pp[p].z; v.w += pp[p].w; }
        *(float4 *)((float *)d.C + (size_t)row * d.ldc + col) = v;
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Skinny path: groups of at most 64 rows (gate/up) or 768 rows (down; decode-shaped and small
// batches). The GEMM is bound by streaming the weights from HBM: a 256-row tile would spend its
// MFMAs on padding, and its two LDS stages cannot cover the HBM latency of the weight slices
// once no other tile shares them in L2. A unit is 32*MB rows (MB = 1, 2 or 4: stages of 40, 40
// or 48 KB; a group of more than 128 rows takes 128-row blocks, each streaming the weights)
// x 256 B-columns x one K part of a group;
// 4 waves own 64 B-columns each (for gate/up 32 gate and the matching 32 up columns), K in
// slices of 64 through three LDS stages. K is cut into S parts only as far as the rule in
// skinny_plan asks (about one or two units per CU: longer units keep the copy pipeline full,
// and a thousand short units measured slower); with S > 1 each unit writes float32 sums to
// the partial buffer and gemm_skinny_reduce_kernel adds the parts in order.
struct SkinnyPlan { int mb, S, nt, snt, pitch; };
constexpr int kSkinnyMaxParts = 16;

SkinnyPlan skinny_plan(const GemmArgs &a, bool gate_up) {
  SkinnyPlan sp{0, 1, 0, 0, 0};
  // Groups of 65-128 rows (Mixtral-shaped weights, T = 96 and 128, same box, old and new library
  // in turn): the down GEMM on 128-row units streamed its weights at 70-71% of HBM against 37%
  // with 128-row regular tiles (324 -> 166-170 us, layer -15%), while the gate/up GEMM, whose
  // regular tiles already reach 61-63%, fell to 58-60% (386 -> 400 us): it keeps the regular
  // tiles above 64 rows.
  if (a.elt != 2 || a.max_group_rows > (gate_up ? kSkinnyRowsGateUp : kSkinnyRows)) return sp;
  sp.mb = a.max_group_rows <= 32 ? 1 : (a.max_group_rows <= 64 ? 2 : 4);
  const int bno = gate_up ? BN / 2 : BN;   // output columns per unit
  sp.nt = (a.N + bno - 1) / bno;
  sp.snt = a.s_rows > 0 ? (a.sN + bno - 1) / bno : 0;
  const int used = a.E < a.rcap ? a.E : a.rcap;   // groups that can receive rows
  const int tiles = used * sp.nt + sp.snt;
  const int nk = a.K / BK, snk = a.s_rows > 0 ? a.sK / BK : nk;
  // K parts: about one unit per CU, two per CU when there are fewer than 128 weight tiles, and
  // at least two parts for a gate/up GEMM whose groups hold at most 4 rows (measured on the
  // Mixtral-shaped weights, one box: down GEMM at T=2 94 -> 76 us and T=1 60 -> 56 us with the
  // larger target, where 512 units of T=4 and T=8 measured slower than 256; gate/up at T=2
  // 142 -> 130 us and at T=4 196 -> 176 us with two parts, while T=8 measured 254 -> 264 us
  // and T=64 no better)
  const int target = tiles < 128 ? 512 : 256;
  auto can_split = [&](int s) {   // parts of at least two slices that divide both K ranges
    return s <= kSkinnyMaxParts && nk % s == 0 && snk % s == 0 && nk / s >= 2 && snk / s >= 2;
  };
  int S = 1;
  while (tiles * S < target && can_split(2 * S)) S *= 2;
  if (gate_up && a.max_group_rows <= 4 && S < 2 && can_split(2)) S = 2;
  sp.S = S;
  const int nmax = a.s_rows > 0 && a.sN > a.N ? a.sN : a.N;
  sp.pitch = (gate_up ? 2 : 1) * nmax;
  return sp;
}

size_t skinny_partial_bytes(const GemmArgs &a, bool gate_up) {
  const SkinnyPlan sp = skinny_plan(a, gate_up);
  if (sp.mb == 0 || sp.S == 1) return 0;
  return (size_t)sp.S * (size_t)(a.rcap + a.s_rows) * sp.pitch * 4;
}


template <int MB> struct SkStage { char a[32 * MB * kRowBytes]; char b[BN * kRowBytes]; };

template <bool GATE_UP, int MB>
__global__ __launch_bounds__(256, 1) void gemm_skinny_kernel(GemmArgs args) {
  constexpr int SBM = 32 * MB;
  constexpr int DMA = MB + 8;   // 1 KB copies per wave per slice: A MB, B 8
  constexpr int BNOUT = GATE_UP ? BN / 2 : BN;
  constexpr int NS = 3;   // stages (a fourth measured no faster)
  __shared__ SkStage<MB> st0, st1, st2;
  __shared__ int ustart[kMaxGroups + 1];
  __shared__ int usm[kMaxWaves + 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int G = args.E + (args.s_rows > 0 ? 1 : 0);
  const int S = args.sk_S;
  // Units from the device-side row counts: group g has nb = ceil(rows / SBM) row blocks x its
  // column panels x S K-parts (ustart: prefix over groups). Groups of more than SBM rows (down
  // GEMM) stream their weights once per block; a group's blocks of one weight range are
  // consecutive units, which run at about the same time on workgroups of one XCD (when blocks
  // can exist), so the later reads of a weight slice mostly find it in its L2 or the
  // last-level cache.
  {
    int run = 0;
    for (int c0 = 0; c0 < G; c0 += blockDim.x) {
      const int g = c0 + threadIdx.x;
      int nu = 0;
      if (g < G) {
        const GroupDesc d = group_desc(args, g);
        nu = ((d.rows + SBM - 1) / SBM) * ((d.N + BNOUT - 1) / BNOUT) * S;
      }
      int tot;
      const int ex = block_excl_scan(nu, usm, &tot);
      if (g < G) ustart[g] = run + ex;
      run += tot;
    }
    if (threadIdx.x == 0) ustart[G] = run;
    __syncthreads();
  }
  const int units = ustart[G];
  for (int u = args.max_group_rows > SBM ? xcd_virtual_block() : (int)blockIdx.x; u < units;
       u += gridDim.x) {
    const int g = find_group(ustart, G, u);
    const GroupDesc d = group_desc(args, g);
    const int nb = (d.rows + SBM - 1) / SBM, lu = u - ustart[g];
    const int rb = lu % nb, part = (lu / nb) % S, n_tile = lu / (nb * S), m0 = rb * SBM;
    const int nk = (d.K / BK) / S, k_begin = part * nk;
    const char *Ab = (const char *)d.A;
    uint32_t aoff[MB], boff[8];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = (wvu * MB + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      int arow = min(m0 + r, d.rows - 1);
      if (d.amap) arow = d.amap[arow];
      aoff[i] = ((uint32_t)arow * (uint32_t)d.lda + c * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wvu * 64 + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int n = GATE_UP ? n_tile * BNOUT + wvu * 32 + (i & 3) * 8 + (lane >> 3)
                            : n_tile * BN + r;
      boff[i] = ((uint32_t)min(n, d.N - 1) * (uint32_t)d.K + c * 8) * 2u;
    }
    const char *Bg = (const char *)d.B0;
    const char *Bu = (const char *)(GATE_UP ? d.B1 : d.B0);
    auto issue = [&](SkStage<MB> &s, int kt) {
      const size_t ko = (size_t)(k_begin + kt) * kRowBytes;
#pragma unroll
      for (int i = 0; i < MB; ++i) g2lds16(Ab + ko + aoff[i], s.a + (wvu * MB + i) * 1024);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        g2lds16((GATE_UP && i >= 4 ? Bu : Bg) + ko + boff[i], s.b + (wvu * 8 + i) * 1024);
    };
    f32x16_t acc[MB][2];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][j][v] = 0.f;
    issue(st0, 0);
    sched_fence();
    issue(st1, min(1, nk - 1));
    auto step = [&](const SkStage<MB> &cur, SkStage<MB> &refill, int kt) {
      sched_fence();
      wait_and_barrier<(NS - 2) * DMA>();          // slice kt has landed (later ones may not)
      sched_fence();
      issue(refill, min(kt + NS - 1, nk - 1));      // past the end: re-read the last slice
#pragma unroll
      for (int ks = 0; ks < kSub; ++ks) {
        const int chunk = ks * 2 + (lane >> 5);
        bf16x8_t fa[MB], fb[2];
#pragma unroll
        for (int m = 0; m < MB; ++m)
          fa[m] = *reinterpret_cast<const bf16x8_t *>(cur.a + swz(m * 32 + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[j] = *reinterpret_cast<const bf16x8_t *>(cur.b + swz(wv * 64 + j * 32 + (lane & 31), chunk));
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[j], acc[m][j], 0, 0, 0);
      }
      sched_fence();
    };
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
      step(st0, st2, kt);
      step(st1, st0, kt + 1);
      step(st2, st1, kt + 2);
    }
    if (kt < nk) {
      step(st0, st2, kt);
      if (kt + 1 < nk) step(st1, st0, kt + 1);
    }
    wait_vm_lgkm<0, 15>();
    __syncthreads();   // every wave is done with every stage before the next unit's copies
    // lane (c, r4) of block (m, j) holds column c of rows m*32 + r4*4 + {0..3} + 8q
    if (S == 1) {
      constexpr int CE = GATE_UP ? 2 : 4;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          d.C, (short)0, (int)((uint32_t)d.rows * (uint32_t)d.ldc * CE), 0x00020000);
#pragma unroll
      for (int j = 0; j < (GATE_UP ? 1 : 2); ++j) {
        const int col = GATE_UP ? n_tile * BNOUT + wv * 32 + (lane & 31)
                                : n_tile * BN + wv * 64 + j * 32 + (lane & 31);
        if (col - (lane & 31) >= d.N) continue;   // whole 32-column block past N
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = m0 + m * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            const uint32_t off = ((uint32_t)row * d.ldc + col) * CE;
            if (GATE_UP) {
              const float gv = acc[m][0][i], uv = acc[m][1][i];
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(swiglu(gv, uv)),
                                                    rs, (int)off, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[m][j][i]), rs, (int)off,
                                                    0, 0);
            }
          }
      }
    } else {
      const int prow0 = g < args.E ? args.offsets[g] : args.rcap;
      float *P = args.partials + ((size_t)part * (args.rcap + args.s_rows) + prow0) * args.sk_pitch;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // gate/up: gate sums in columns [0, pitch/2), up sums in [pitch/2, pitch)
        const int col = GATE_UP ? (j ? args.sk_pitch / 2 : 0) + n_tile * BNOUT + wv * 32 + (lane & 31)
                                : n_tile * BN + wv * 64 + j * 32 + (lane & 31);
        const int ncol = GATE_UP ? n_tile * BNOUT + wv * 32 : n_tile * BN + wv * 64 + j * 32;
        if (ncol >= d.N) continue;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = m0 + m * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (row < d.rows) P[(size_t)row * args.sk_pitch + col] = acc[m][j][i];
          }
      }
    }
  }
}

// Sum of the skinny path's K parts, in part order, then the same epilogue. One item = 4
// adjacent output columns of one row (routed rows below rcap, shared rows from rcap on).
template <bool GATE_UP>
__global__ __launch_bounds__(256) void gemm_skinny_reduce_kernel(GemmArgs args) {
  const int S = args.sk_S, pitch = args.sk_pitch;
  const int rows_total = args.rcap + args.s_rows;
  const int q = GATE_UP ? pitch / 2 / 4 : pitch / 4;   // column quads per row
  const int routed = args.offsets[args.E];
  const size_t part = (size_t)rows_total * pitch;
  for (int it = blockIdx.x * blockDim.x + threadIdx.x; it < rows_total * q;
       it += gridDim.x * blockDim.x) {
    const int prow = it / q, c = (it % q) * 4;
    char *C;
    int ldc, N;
    if (prow < args.rcap) {
      if (prow >= routed) continue;
      C = (char *)args.C + (size_t)prow * args.ldc * args.c_elt; ldc = args.ldc; N = args.N;
    } else {
      C = (char *)args.sC + (size_t)(prow - args.rcap) * args.s_ldc * args.c_elt;
      ldc = args.s_ldc; N = args.sN;
    }
    (void)ldc;
    if (c >= N) continue;
    const float *P = args.partials + (size_t)prow * pitch + c;
    // every part's loads go out before the sums, which run in part order from 0
    if (GATE_UP) {
      float4 gp[kSkinnyMaxParts], up[kSkinnyMaxParts];
#pragma unroll
      for (int p = 0; p < kSkinnyMaxParts; ++p)
        if (p < S) {
          gp[p] = *(const float4 *)(P + p * part);
          up[p] = *(const float4 *)(P + p * part + pitch / 2);
        }
      float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
#pragma unroll
      for (int p = 0; p < kSkinnyMaxParts; ++p)
        if (p < S) {
          gs.x += gp[p].x; gs.y += gp[p].y; gs.z += gp[p].z; gs.w += gp[p].w;
          us.x += up[p].x; us.y += up[p].y; us.z += up[p].z; us.w += up[p].w;
        }
      const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
      uint32_t pk[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float h0 = swiglu(gv[2 * j], uv[2 * j]);
        const float h1 = swiglu(gv[2 * j + 1], uv[2 * j + 1]);
        pk[j] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
      }
      *(uint2 *)((bf16_t *)C + c) = make_uint2(pk[0], pk[1]);
    } else {
      float4 pp[kSkinnyMaxParts];
#pragma unroll
      for (int p = 0; p < kSkinnyMaxParts; ++p)
        if (p < S) pp[p] = *(const float4 *)(P + p * part);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int p = 0; p < kSkinnyMaxParts; ++p)
        if (p < S) { v.x += pp[p].x; v.y += pp[p].y; v.z += pp[p].z; v.w += pp[p].w; }
      *(float4 *)((float *)C + c) = v;
    }
  }
}

// Decode-shaped layer: the skinny down GEMM's K parts summed (as gemm_skinny_reduce_kernel
// does) straight into the weighted combine (as combine_kernel does), one launch instead of
// two. Thread (t, c) takes 4 output columns of token t: it forms each o row of the token from
// its parts in part order, adds it into the token's sum in CSR order with the pair's gate
// (rows in pairs, the second of an odd count with gate 0, as the combine does), then the
// shared expert's row likewise, and writes y once: the operations and their order are the two
// kernels', so y is bit for bit theirs.
template <typename TY>
__global__ __launch_bounds__(256) void skinny_down_combine_kernel(GemmArgs args,
                                                                  const int32_t *__restrict__ tok_ptr,
                                                                  const int32_t *__restrict__ tok_pos,
                                                                  const float *__restrict__ perm_w,
                                                                  TY *__restrict__ y, int T, int d) {
  const int S = args.sk_S, pitch = args.sk_pitch;
  const size_t part = (size_t)(args.rcap + args.s_rows) * pitch;
  const int q = d / 4;   // column quads per row
  auto row_sum = [&](int prow, int c) {   // o[prow][c .. c+3] from its K parts
    // every part's load goes out before the sums (S <= kSkinnyMaxParts)
    const float *P = args.partials + (size_t)prow * pitch + c;
    float4 u[kSkinnyMaxParts];
#pragma unroll
    for (int k = 0; k < kSkinnyMaxParts; ++k)
      if (k < S) u[k] = *(const float4 *)(P + k * part);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);   // from 0, as the reduction kernel sums
#pragma unroll
    for (int k = 0; k < kSkinnyMaxParts; ++k)
      if (k < S) { v.x += u[k].x; v.y += u[k].y; v.z += u[k].z; v.w += u[k].w; }
    return v;
  };
  for (int it = blockIdx.x * blockDim.x + threadIdx.x; it < T * q; it += gridDim.x * blockDim.x) {
    const int t = it / q, c = (it % q) * 4;
    const int b = tok_ptr[t], n = tok_ptr[t + 1] - b;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n; j += 2) {
      const int p0 = tok_pos[b + j];
      const bool two = j + 1 < n;
      const int p1 = two ? tok_pos[b + j + 1] : p0;
      const float w0 = perm_w[p0], w1 = two ? perm_w[p1] : 0.f;
      const float4 v0 = row_sum(p0, c), v1 = row_sum(p1, c);
      acc.x = fmaf(w0, v0.x, acc.x); acc.y = fmaf(w0, v0.y, acc.y);
      acc.z = fmaf(w0, v0.z, acc.z); acc.w = fmaf(w0, v0.w, acc.w);
      acc.x = fmaf(w1, v1.x, acc.x); acc.y = fmaf(w1, v1.y, acc.y);
      acc.z = fmaf(w1, v1.z, acc.z); acc.w = fmaf(w1, v1.w, acc.w);
    }
    if (args.s_rows > 0) {
      const float4 v = row_sum(args.rcap + t, c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    TY *yp = y + (size_t)t * d + c;
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

// ----------------------------------------------------------------------------------------
// float32 SIMT kernel: 64 x 64 output tile, K steps of 32, 256 threads with 4 x 4 outputs each
// (gate/up keeps a gate and an up accumulator per output). Each thread holds 8 elements of every
// operand tile; the next K step's elements are loaded into registers while the current step's
// FMAs run, so a K step waits for memory only when the loads take longer than the FMAs. Every
// output sums over k in ascending order.
template <bool GATE_UP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs args) {
  constexpr int TM = 64, TN = 64, TK = 32;
  constexpr int LPT = TM * TK / 256;   // elements of one operand tile per thread
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[2][TK][TN + 4];
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int sm[kMaxWaves + 1];
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
    float ra[LPT], rb0[LPT], rb1[LPT];
    // element q of this thread: row (tid + 256 q) / TK, column (tid + 256 q) % TK of the tile
    auto load = [&](int k0) {
#pragma unroll
      for (int q = 0; q < LPT; ++q) {
        const int idx = (int)threadIdx.x + 256 * q, r = idx / TK, c = idx % TK;
        const int m = m0 + r, k = k0 + c, n = n0 + r;
        ra[q] = (m < d.rows && k < d.K) ? A[(size_t)(d.amap ? d.amap[m] : m) * d.lda + k] : 0.f;
        const bool ok = n < d.N && k < d.K;
        rb0[q] = ok ? B0[(size_t)n * d.K + k] : 0.f;
        rb1[q] = (GATE_UP && ok) ? B1[(size_t)n * d.K + k] : 0.f;
      }
    };
    float acc[2][4][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][i][j] = 0.f;
    load(0);
    for (int k0 = 0; k0 < d.K; k0 += TK) {
      __syncthreads();   // every thread is done with the previous step's tiles
#pragma unroll
      for (int q = 0; q < LPT; ++q) {
        const int idx = (int)threadIdx.x + 256 * q, r = idx / TK, c = idx % TK;
        As[c][r] = ra[q];
        Bs[0][c][r] = rb0[q];
        if (GATE_UP) Bs[1][c][r] = rb1[q];
      }
      __syncthreads();
      if (k0 + TK < d.K) load(k0 + TK);   // in flight during the FMAs below
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

#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif

template <int W>
hipError_t launch_bf16(const GemmArgs &a0, bool gate_up, int max_rows, int num_cu, hipStream_t st) {
  GemmArgs a = a0;
  const int bn_out = gate_up ? BN / 2 : BN;
  int grid = gemm_tiles_upper(a, BM, bn_out, max_rows);
  int cap = num_cu;   // one workgroup per CU (the two 64 KB LDS stages)
  if (cap > kMaxPersistent) cap = kMaxPersistent;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  a.grid = grid;
  // Wide last row tiles (group_tile) for the down GEMM. Measured on one box, same-run A/B: the
  // down GEMM's 64-row tiles (K = d_ff, 224 slices on the Mixtral-shaped layer) wait on their
  // copies most of the time, and pairing them took that GEMM from 875 to 848 us (fine-grained
  // 362 -> 357 us); the gate/up GEMM, whose L2 misses already stream near the fabric's rate,
  // gained nothing (1619 -> 1626 us; capacity drop -2%, fine-grained +3%). MOE_GEMM_WIDE (read
  // at every call) = 0 turns them off, = all uses them in both GEMMs. The output is the same bit
  // for bit in every case: each output element sums its K products in the same MFMA order
  // whatever tile holds it.
  const char *wenv = std::getenv("MOE_GEMM_WIDE");
  const bool w_off = wenv && wenv[0] == '0', w_all = wenv && wenv[0] == 'a';
  a.wide = (W == 8 && !w_off && (!gate_up || w_all)) ? 1 : 0;
  // a wide tile's second-half copies add one panel (at most 256 rows of K elements) to the
  // slice's scalar byte offset, which must stay below 2^31
  const long long kmax = a.s_rows > 0 && a.sK > a.K ? a.sK : a.K;
  if (kmax * (2LL * BN + 2) * 2 >= (1LL << 31)) a.wide = 0;
  // Tile order inside a group: column panels in bands of 4, row tile by row tile within a band
  // (group_tile), so the 32 workgroups of an XCD, which take 32 consecutive tiles, share about 4
  // weight panels and 8 row tiles instead of 2-3 panels and up to 13 row tiles. Same-run A/B on
  // the Mixtral-shaped layer: gate/up 1643 -> 1618 us with bands of 4 (2: 1620, 6: 1632, 8: 1623);
  // fine-grained 492 -> 489 us, capacity drop unchanged, the down GEMM unchanged.
  // MOE_GEMM_BAND (read at every call) sets another band width (1: panel by panel). The order
  // changes no sum.
  const char *benv = std::getenv("MOE_GEMM_BAND");
  a.band = benv && *benv ? std::atoi(benv) : 4;
  if (!a.partials) a.split_ok = 0;
  // at most kMaxPersistent/2 split tiles, BM/kReduceRows reduction items each
  int rgrid = kMaxPersistent * (BM / kReduceRows) / 2 + 1;
  if (rgrid > 4 * num_cu) rgrid = 4 * num_cu;
  if (gate_up) {
    hipLaunchKernelGGL((gemm_bf16_kernel<true, W>), dim3(grid), dim3(64 * W), 0, st, a);
    if (a.split_ok)
      hipLaunchKernelGGL((gemm_tail_reduce_kernel<true, W>), dim3(rgrid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<false, W>), dim3(grid), dim3(64 * W), 0, st, a);
    if (a.split_ok)
      hipLaunchKernelGGL((gemm_tail_reduce_kernel<false, W>), dim3(rgrid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const GemmArgs &a0, bool gate_up, const SkinnyPlan &sp, int num_cu,
                         hipStream_t st, bool defer_reduce = false) {
  GemmArgs a = a0;
  a.sk_S = sp.S;
  a.sk_pitch = sp.pitch;
  if (sp.S > 1 && !a.partials) return hipErrorInvalidValue;
  const int G = a.E + (a.s_rows > 0 ? 1 : 0);
  const int ntmax = sp.snt > sp.nt ? sp.snt : sp.nt;
  int grid = G * ntmax * sp.S * ((a.max_group_rows + 32 * sp.mb - 1) / (32 * sp.mb));
  if (grid > num_cu) grid = num_cu;
  if (grid < 1) grid = 1;
  if (gate_up) {
    if (sp.mb == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, 1>), dim3(grid), dim3(256), 0, st, a);
    else if (sp.mb == 2)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, 2>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<true, 4>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (sp.mb == 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<false, 1>), dim3(grid), dim3(256), 0, st, a);
    else if (sp.mb == 2)
      hipLaunchKernelGGL((gemm_skinny_kernel<false, 2>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, 4>), dim3(grid), dim3(256), 0, st, a);
  }
  if (sp.S > 1 && !defer_reduce) {
    const long items = (long)(a.rcap + a.s_rows) * (gate_up ? sp.pitch / 2 : sp.pitch) / 4;
    long rg = (items + 255) / 256;
    if (rg > 4 * num_cu) rg = 4 * num_cu;
    if (rg < 1) rg = 1;
    if (gate_up)
      hipLaunchKernelGGL(gemm_skinny_reduce_kernel<true>, dim3(rg), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(gemm_skinny_reduce_kernel<false>, dim3(rg), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

bool skinny_split_down(const GemmArgs &a) {
  if (a.elt != 2 || !a.partials) return false;
  const SkinnyPlan sp = skinny_plan(a, false);
  return sp.mb != 0 && sp.S > 1;
}

hipError_t launch_skinny_down_combine(const GemmArgs &a0, int y_elt, const int32_t *tok_ptr,
                                      const int32_t *tok_pos, const float *perm_w, void *y,
                                      int T, int d, int num_cu, hipStream_t st) {
  const SkinnyPlan sp = skinny_plan(a0, false);
  if (!sp.mb || sp.S < 2 || !a0.partials) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.sk_S = sp.S;
  a.sk_pitch = sp.pitch;
  const long items = (long)T * d / 4;
  long rg = (items + 255) / 256;
  if (rg > 4 * num_cu) rg = 4 * num_cu;
  if (rg < 1) rg = 1;
  if (y_elt == 2)
    hipLaunchKernelGGL(skinny_down_combine_kernel<bf16_t>, dim3(rg), dim3(256), 0, st, a, tok_ptr,
                       tok_pos, perm_w, (bf16_t *)y, T, d);
  else
    hipLaunchKernelGGL(skinny_down_combine_kernel<float>, dim3(rg), dim3(256), 0, st, a, tok_ptr,
                       tok_pos, perm_w, (float *)y, T, d);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, bool gate_up, int max_rows, int num_cu,
                       hipStream_t st, bool defer_skinny_reduce) {
  if (a.elt == 2) {
    const SkinnyPlan sp = skinny_plan(a, gate_up);
    if (sp.mb) return launch_skinny(a, gate_up, sp, num_cu, st, defer_skinny_reduce);
    return launch_bf16<MOE_GEMM_WAVES>(a, gate_up, max_rows, num_cu, st);
  }
  int grid = gemm_tiles_upper(a, 64, 64, max_rows);
  if (grid > 4 * num_cu) grid = 4 * num_cu;
  if (grid < 1) grid = 1;
  if (gate_up)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t gemm_setup_attributes() { return hipSuccess; }

}  // namespace moe
