// Host layer of the C ABI: argument validation, workspace layout and launch sequencing.
// Everything here runs on the host; every check happens before the first enqueue.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <initializer_list>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  // route scratch
  size_t keys, blk_cnt, blk_base, cnt_pre, off_pre, cand_token, cand_slot, cand_key, cand_w,
      slot_pos,
      colkeys, tok_blk, tok_blk_off, stats_part, w3, partials;
  // routing arrays used when the caller passes no routing struct
  size_t logits, ids, topk_w, kept, counts, offsets, perm_token, perm_w, tok_ptr, tok_pos;
  // activations
  size_t h, h_shared, o_perm, o_shared;
  size_t total;
};

int elt_of(const moe_problem &p) { return p.dtype == MOE_BF16 ? 2 : 4; }
int64_t rows_cap(const moe_problem &p) { return (int64_t)p.T * p.k; }
int slot_width(const moe_problem &p) {
  return p.routing == MOE_EXPERT_CHOICE ? p.E : p.k + p.expand_m;
}

// sizes of one grouped GEMM of the problem (no pointers)
GemmArgs gemm_shape(const moe_problem &p, bool gate_up) {
  GemmArgs a{};
  a.E = p.E;
  a.elt = elt_of(p);
  a.c_elt = gate_up ? a.elt : 4;
  if (gate_up) {
    a.N = p.d_ff; a.K = p.d_model; a.lda = p.d_model; a.ldc = p.d_ff;
  } else {
    a.N = p.d_model; a.K = p.d_ff; a.lda = p.d_ff; a.ldc = p.d_model;
  }
  if (p.d_ff_shared > 0) {
    a.s_rows = p.T;
    if (gate_up) {
      a.sN = p.d_ff_shared; a.sK = p.d_model; a.s_lda = p.d_model; a.s_ldc = p.d_ff_shared;
    } else {
      a.sN = p.d_model; a.sK = p.d_ff_shared; a.s_lda = p.d_ff_shared; a.s_ldc = p.d_model;
    }
  }
  // rows one group can hold: a token picks an expert at most once (token choice), an
  // expert takes c <= T tokens (expert choice), the shared expert takes all T
  a.max_group_rows = p.T;
  a.rcap = (int)rows_cap(p);
  return a;
}

// float32 partial sums of the bf16 GEMMs: the last-round tail split, or the skinny path's
// K-parts, whichever needs more
size_t partial_bytes(const moe_problem &p) {
  size_t b = kPartialBytes;
  for (int gu = 0; gu < 2; ++gu) {
    const size_t s = skinny_partial_bytes(gemm_shape(p, gu == 1), gu == 1);
    if (s > b) b = s;
  }
  return b;
}

Layout make_layout(const moe_problem &p) {
  Layout L{};
  const size_t T = p.T, E = p.E, k = p.k, R = rows_cap(p), d = p.d_model, dff = p.d_ff,
               dfs = p.d_ff_shared, elt = elt_of(p), S = slot_width(p);
  const size_t nblk = (T + 255) / 256;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  L.keys = take(T * S * 4);
  L.blk_cnt = take(((T + 15) / 16) * E * 4);   // per 256-token block, or per top-k workgroup
  L.blk_base = take(nblk * E * 4);
  L.cnt_pre = take(E * 4);
  L.off_pre = take((E + 1) * 4);
  L.cand_token = take(T * S * 4);
  L.cand_slot = take(T * S * 4);
  L.cand_key = take(T * S * 4);
  L.cand_w = take(T * S * 4);
  L.slot_pos = take(T * S * 4);
  L.colkeys = take(p.routing == MOE_EXPERT_CHOICE ? E * T * 4 : 0);
  L.tok_blk = take(nblk * 4);
  L.tok_blk_off = take(nblk * 4);
  L.stats_part = take(nblk * E * 4);
  L.w3 = take(router_w3_bytes(p.dtype == MOE_BF16 ? 1 : 0, (int)d, (int)E));
  L.partials = take(p.dtype == MOE_BF16 ? partial_bytes(p) : 0);
  L.logits = take(T * E * 4);
  L.ids = take(T * S * 4);
  L.topk_w = take(T * S * 4);
  L.kept = take(T * S);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm_token = take(R * 4);
  L.perm_w = take(R * 4);
  L.tok_ptr = take((T + 1) * 4);
  L.tok_pos = take(R * 4);
  L.h = take(R * dff * elt);
  L.h_shared = take(T * dfs * elt);
  L.o_perm = take(R * d * 4);
  L.o_shared = take(dfs > 0 ? T * d * 4 : 0);
  L.total = o;
  return L;
}

bool aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool ptr_ok(const void *p) { return p != nullptr && aligned(p); }
bool opt_ptr_ok(const void *p) { return p == nullptr || aligned(p); }

moe_status check_problem(const moe_problem *pp) {
  if (!pp) return MOE_ERR_INVALID_ARG;
  const moe_problem &p = *pp;
  if (p.T < 1 || p.d_model < 1 || p.E < 1 || p.k < 1 || p.d_ff < 1 || p.d_ff_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (p.k > p.E) return MOE_ERR_INVALID_ARG;
  if (p.routing != MOE_TOKEN_CHOICE && p.routing != MOE_EXPERT_CHOICE) return MOE_ERR_INVALID_ARG;
  if (p.dtype != MOE_F32 && p.dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p.y_dtype != MOE_F32 && p.y_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p.dtype == MOE_F32 && p.y_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (p.renorm_topk != 0 && p.renorm_topk != 1) return MOE_ERR_INVALID_ARG;
  if (std::isnan(p.gamma) || std::isinf(p.gamma)) return MOE_ERR_INVALID_ARG;
  if (p.expand_m < 0 || p.cap_groups < 0) return MOE_ERR_INVALID_ARG;
  if (p.expand_m > 0 || p.cap_groups > 0) {
    if (p.routing != MOE_TOKEN_CHOICE || !(p.gamma > 0.f) || (p.expand_m > 0 && p.cap_groups > 0))
      return MOE_ERR_INVALID_ARG;
    if ((int64_t)p.k + p.expand_m > p.E) return MOE_ERR_INVALID_ARG;
    if (p.cap_groups > 0 && p.E % p.cap_groups != 0) return MOE_ERR_INVALID_ARG;
  }
  if (p.routing == MOE_EXPERT_CHOICE && ((int64_t)p.k * p.T < p.E || p.gamma > 0.f))
    return MOE_ERR_INVALID_ARG;
  const int64_t R = rows_cap(p);
  if (R > INT32_MAX || (int64_t)p.T * p.E > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (p.E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (p.cap_groups > 0 && p.k > 16) return MOE_ERR_UNSUPPORTED;   // picks per token in a group
  if (p.dtype == MOE_BF16) {
    if (p.d_model % 64 || p.d_ff % 64 || p.d_ff_shared % 64) return MOE_ERR_UNSUPPORTED;
  } else {
    if (p.d_model % 4) return MOE_ERR_UNSUPPORTED;
  }
  // 32-bit byte offsets inside one operand panel (elements < 2^31, bf16 or fp32 panels
  // of the sizes below stay under 4 GiB)
  const int64_t big = (int64_t)1 << (p.dtype == MOE_BF16 ? 31 : 30);
  const int64_t wmax = (int64_t)p.d_ff * p.d_model;
  const int64_t amax = R * (int64_t)(p.d_model > p.d_ff ? p.d_model : p.d_ff);
  const int64_t smax = (int64_t)p.T * (p.d_model > p.d_ff_shared ? p.d_model : p.d_ff_shared);
  if (wmax >= big || amax >= big || smax >= big) return MOE_ERR_UNSUPPORTED;
  // the bf16 GEMM stores one group's output rows (at most T of them) through a buffer
  // resource with a 32-bit byte range, at byte offsets computed in 32 bits for every row of
  // the group's last row tile, including up to 255 padding rows past its end: an offset
  // that wrapped past 2^32 would land back inside the range. So (T + 256) rows of every
  // output panel (o and o_shared: d_model float32; h and h_shared: d_ff or d_ff_shared bf16)
  // must stay under 4 GiB.
  if (p.dtype == MOE_BF16) {
    int64_t row_bytes = (int64_t)p.d_model * 4;
    if ((int64_t)p.d_ff * 2 > row_bytes) row_bytes = (int64_t)p.d_ff * 2;
    if ((int64_t)p.d_ff_shared * 2 > row_bytes) row_bytes = (int64_t)p.d_ff_shared * 2;
    if (((int64_t)p.T + 256) * row_bytes >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status check_ws(const moe_problem &p, const void *ws, size_t ws_bytes) {
  if (!ptr_ok(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < make_layout(p).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status check_routing_out(const moe_problem &p, const moe_routing *r) {
  if (!r) return MOE_ERR_INVALID_ARG;
  if (!ptr_ok(r->logits) || !ptr_ok(r->counts) || !ptr_ok(r->offsets) ||
      !ptr_ok(r->perm_token) || !ptr_ok(r->perm_w) || !ptr_ok(r->tok_ptr) || !ptr_ok(r->tok_pos))
    return MOE_ERR_INVALID_ARG;
  if (p.routing == MOE_TOKEN_CHOICE && (!ptr_ok(r->topk_ids) || !ptr_ok(r->topk_w)))
    return MOE_ERR_INVALID_ARG;
  if (!opt_ptr_ok(r->kept)) return MOE_ERR_INVALID_ARG;
  // the capacity variants keep their intermediate decisions in `kept`
  if ((p.expand_m > 0 || p.cap_groups > 0) && !r->kept) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Compute units the persistent grids may fill: the device's count, or fewer when the
// environment variable MOE_GRID_CUS (read at every call) asks for fewer. No result depends on
// it (the GEMMs' K-split plan is fixed independently of the grid); the determinism tests use it
// to run the same problem under different launch shapes.
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) n = 256;
  else if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
           n < 1)
    n = 256;
  const char *cap = std::getenv("MOE_GRID_CUS");
  if (cap && *cap) {
    const int v = std::atoi(cap);
    if (v >= 1 && v < n) n = v;
  }
  return n;
}

std::once_flag g_attr_once;
hipError_t g_attr_err = hipSuccess;
hipError_t ensure_attributes() {
  std::call_once(g_attr_once, [] { g_attr_err = gemm_setup_attributes(); });
  return g_attr_err;
}

#define MOE_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;       \
  } while (0)

RouteScratch scratch_of(const Layout &L, char *ws) {
  RouteScratch s;
  s.keys = (float *)(ws + L.keys);
  s.blk_cnt = (int32_t *)(ws + L.blk_cnt);
  s.blk_base = (int32_t *)(ws + L.blk_base);
  s.cnt_pre = (int32_t *)(ws + L.cnt_pre);
  s.off_pre = (int32_t *)(ws + L.off_pre);
  s.cand_token = (int32_t *)(ws + L.cand_token);
  s.cand_slot = (int32_t *)(ws + L.cand_slot);
  s.cand_key = (float *)(ws + L.cand_key);
  s.cand_w = (float *)(ws + L.cand_w);
  s.slot_pos = (int32_t *)(ws + L.slot_pos);
  s.colkeys = (uint32_t *)(ws + L.colkeys);
  s.tok_blk = (int32_t *)(ws + L.tok_blk);
  s.tok_blk_off = (int32_t *)(ws + L.tok_blk_off);
  s.stats_part = (float *)(ws + L.stats_part);
  s.w3 = (uint16_t *)(ws + L.w3);
  return s;
}

moe_routing internal_routing(const Layout &L, char *ws) {
  moe_routing r;
  r.logits = (float *)(ws + L.logits);
  r.topk_ids = (int32_t *)(ws + L.ids);
  r.topk_w = (float *)(ws + L.topk_w);
  r.kept = (uint8_t *)(ws + L.kept);
  r.counts = (int32_t *)(ws + L.counts);
  r.offsets = (int32_t *)(ws + L.offsets);
  r.perm_token = (int32_t *)(ws + L.perm_token);
  r.perm_w = (float *)(ws + L.perm_w);
  r.tok_ptr = (int32_t *)(ws + L.tok_ptr);
  r.tok_pos = (int32_t *)(ws + L.tok_pos);
  return r;
}

// floor(gamma * mean), computed in double and clamped to T*k before the conversion to int: no
// expert or group can have more candidates than T*k, so a larger capacity keeps everything,
// and a huge gamma (1e12 meant as "no limit") must not overflow the int
int clamped_capacity(const moe_problem &p, double mean) {
  const double c = std::floor((double)p.gamma * mean);
  const double all = (double)p.T * (double)p.k;
  return (int)(c < all ? c : all);
}

// C = floor(gamma * N-bar), N-bar = T*k/E; -1 = no capacity limit
int capacity_of(const moe_problem &p) {
  if (!(p.gamma > 0.f)) return -1;
  return clamped_capacity(p, (double)p.T * (double)p.k / (double)p.E);
}

// C_D = floor(gamma * T*k/D): the token-drop capacity of a device that holds E/D experts
int group_capacity_of(const moe_problem &p) {
  return clamped_capacity(p, (double)p.T * (double)p.k / (double)p.cap_groups);
}

// ---- the four steps, without validation --------------------------------------------------

hipError_t do_route(const moe_problem &p, const void *x, const float *w_router,
                    const float *bias, int flags, const moe_routing &r, char *ws,
                    hipStream_t st) {
  const Layout L = make_layout(p);
  const RouteScratch s = scratch_of(L, ws);
  hipError_t e;
  const int C = capacity_of(p);
  // token choice with at most 16 experts (plain, or with the per-expert token drop): the top-k
  // counts its picks per workgroup and one launch does the dispatch from those counts (with a
  // capacity: the candidate lists the selection reads)
  const bool blk_dispatch = p.routing == MOE_TOKEN_CHOICE && p.expand_m == 0 &&
                            p.cap_groups == 0 && p.E <= kBlkCountMaxE;
  const TopkOut tk{p.k + p.expand_m, p.k, p.renorm_topk, C >= 0 ? 1 : 0, r.topk_ids, r.topk_w,
                   s.keys, blk_dispatch ? s.blk_cnt : nullptr};
  bool topk_done = false, ex_done = false, disp_done = false;
  int cnt_block = 0;
  // token choice without a capacity limit: the dispatch outputs (final mode), which the router
  // writes itself when one workgroup holds every token
  BlkDispatchOut fin{};
  if (blk_dispatch && C < 0) {
    fin.counts = r.counts; fin.offsets = r.offsets; fin.perm_token = r.perm_token;
    fin.perm_w = r.perm_w; fin.kept = r.kept; fin.tok_ptr = r.tok_ptr; fin.tok_pos = r.tok_pos;
  }
  // expert choice with the register-held selection (at most 16384 tokens): the router may also
  // write the logits transposed (the selection's column reads)
  const RouterExtra ex{(float *)s.colkeys};
  const bool want_ex = p.routing == MOE_EXPERT_CHOICE && p.T <= 16384;
  if (!(flags & MOE_ROUTE_LOGITS_IN)) {
    e = launch_router(p.dtype == MOE_BF16 ? 1 : 0, x, w_router, bias, r.logits, p.T, p.d_model,
                      p.E, s.w3, st, p.routing == MOE_TOKEN_CHOICE ? &tk : nullptr, &topk_done,
                      &cnt_block, want_ex ? &ex : nullptr, &ex_done,
                      blk_dispatch && C < 0 ? &fin : nullptr, &disp_done);
    if (e != hipSuccess) return e;
  }
  if (p.routing == MOE_TOKEN_CHOICE) {
    if (!topk_done)
      e = launch_topk(r.logits, p.T, p.E, tk.k, tk.kden, tk.renorm, tk.want_key, r.topk_ids,
                      r.topk_w, s.keys, st, tk.blk_cnt, &cnt_block);
    if (e != hipSuccess) return e;
    if (blk_dispatch && cnt_block > 0) {
      BlkDispatchOut o{};
      if (C < 0) {   // every pair kept: the dispatch writes the token CSR as well
        if (disp_done) return hipSuccess;   // the router did it
        return launch_dispatch_blocks(r.topk_ids, r.topk_w, p.T, p.k, p.E, s.blk_cnt, cnt_block,
                                      fin, st);
      }
      o.counts = s.cnt_pre; o.offsets = s.off_pre; o.perm_token = s.cand_token;
      o.perm_w = s.cand_w; o.keys = s.keys; o.cand_slot = s.cand_slot; o.cand_key = s.cand_key;
      o.cnt_fin = r.counts; o.off_fin = r.offsets; o.C = C;
      e = launch_dispatch_blocks(r.topk_ids, r.topk_w, p.T, p.k, p.E, s.blk_cnt, cnt_block, o,
                                 st);
      if (e != hipSuccess) return e;
      e = launch_cap_select_final(s, p.E, C, p.k, r.perm_token, r.perm_w, r.kept, r.offsets, st);
      if (e != hipSuccess) return e;
      return launch_token_csr(s, p.T, slot_width(p), r.tok_ptr, r.tok_pos, st);
    }
    if (p.cap_groups > 0)
      e = launch_group_capacity(s, r.topk_ids, r.topk_w, p.T, p.k, p.E, p.cap_groups,
                                group_capacity_of(p), r.perm_token, r.perm_w, r.kept, r.counts,
                                r.offsets, st);
    else if (p.expand_m > 0)
      e = launch_expanded_drop(s, r.topk_ids, r.topk_w, p.T, p.k, p.expand_m, p.E, C,
                               r.perm_token, r.perm_w, r.kept, r.counts, r.offsets, st);
    else if (C < 0)   // every pair kept: the scatter writes the CSR as well
      return launch_token_dispatch(s, r.topk_ids, r.topk_w, p.T, p.k, p.E, C, r.perm_token,
                                   r.perm_w, r.kept, r.counts, r.offsets, r.tok_ptr, r.tok_pos,
                                   st);
    else
      e = launch_token_dispatch(s, r.topk_ids, r.topk_w, p.T, p.k, p.E, C, r.perm_token,
                                r.perm_w, r.kept, r.counts, r.offsets, nullptr, nullptr, st);
    if (e != hipSuccess) return e;
  } else {
    const int c = (int)(((int64_t)p.k * p.T) / p.E);
    e = launch_expert_choice(s, r.logits, p.T, p.E, c, r.perm_token, r.perm_w, r.counts,
                             r.offsets, st, ex_done ? ex.logits_t : nullptr);
    if (e != hipSuccess) return e;
  }
  return launch_token_csr(s, p.T, slot_width(p), r.tok_ptr, r.tok_pos, st);
}

hipError_t do_dispatch(const moe_problem &p, const void *x, const moe_routing &r, void *x_perm,
                       hipStream_t st) {
  return launch_gather(elt_of(p), x, r.perm_token, r.offsets + p.E, x_perm, p.d_model,
                       (int)rows_cap(p), num_cus(), st);
}

GemmArgs gemm_args(const moe_problem &p, const moe_routing &r, bool gate_up, const void *a_rows,
                   const void *w0, const void *w1, void *c_rows, const void *s_a,
                   const void *s_w0, const void *s_w1, void *s_c,
                   const int32_t *row_map = nullptr) {
  GemmArgs a = gemm_shape(p, gate_up);
  a.a_rows = row_map;
  a.counts = r.counts;
  a.offsets = r.offsets;
  a.A = a_rows; a.B0 = w0; a.B1 = w1; a.C = c_rows;
  if (p.d_ff_shared > 0) { a.sA = s_a; a.sB0 = s_w0; a.sB1 = s_w1; a.sC = s_c; }
  return a;
}

// x_perm given: routed rows are x_perm rows. x_perm null: routed row p is read as
// x[perm_token[p]] (the dispatch gather folded into the GEMM's operand loads).
hipError_t do_gate_up(const moe_problem &p, const void *x_perm, const moe_routing &r,
                      const void *w_gate, const void *w_up, const void *x, const void *ws_gate,
                      const void *ws_up, char *ws, hipStream_t st) {
  const Layout L = make_layout(p);
  GemmArgs a = gemm_args(p, r, true, x_perm ? x_perm : x, w_gate, w_up, ws + L.h, x, ws_gate,
                         ws_up, ws + L.h_shared, x_perm ? nullptr : r.perm_token);
  a.partials = p.dtype == MOE_BF16 ? (float *)(ws + L.partials) : nullptr;
  a.split_ok = 1;   // every group has K = d_model
  return launch_gemm(a, true, (int)rows_cap(p), num_cus(), st);
}

GemmArgs down_args(const moe_problem &p, const moe_routing &r, const void *w_down,
                   const void *ws_down, void *o_perm, void *o_shared, char *ws) {
  const Layout L = make_layout(p);
  GemmArgs a = gemm_args(p, r, false, ws + L.h, w_down, nullptr, o_perm, ws + L.h_shared,
                         ws_down, nullptr, o_shared);
  a.partials = p.dtype == MOE_BF16 ? (float *)(ws + L.partials) : nullptr;
  a.split_ok = (p.d_ff_shared == 0 || p.d_ff_shared == p.d_ff) ? 1 : 0;   // one K for all groups
  return a;
}

hipError_t do_down(const moe_problem &p, const moe_routing &r, const void *w_down,
                   const void *ws_down, void *o_perm, void *o_shared, char *ws, hipStream_t st,
                   bool defer_skinny_reduce = false) {
  const GemmArgs a = down_args(p, r, w_down, ws_down, o_perm, o_shared, ws);
  return launch_gemm(a, false, (int)rows_cap(p), num_cus(), st, defer_skinny_reduce);
}

hipError_t do_combine(const moe_problem &p, const void *o_perm, const void *o_shared,
                      const moe_routing &r, void *y, hipStream_t st) {
  return launch_combine(p.y_dtype == MOE_BF16 ? 2 : 4, (const float *)o_perm,
                        p.d_ff_shared > 0 ? (const float *)o_shared : nullptr, r.tok_ptr,
                        r.tok_pos, r.perm_w, y, p.T, p.d_model, (int)rows_cap(p), st);
}

// Debug mode (MOE_DEBUG): scan the floating-point inputs for NaN/Inf before anything else
// is enqueued; a non-finite value is an invalid argument.
moe_status debug_check(std::initializer_list<DebugSpan> spans, hipStream_t st) {
  if (!debug_checks_enabled()) return MOE_OK;
  bool bad = false;
  if (debug_any_nonfinite(spans.begin(), (int)spans.size(), st, &bad) != hipSuccess)
    return MOE_ERR_HIP;
  return bad ? MOE_ERR_INVALID_ARG : MOE_OK;
}

size_t nz(size_t a, size_t b, size_t c = 1) { return a * b * c; }

moe_status debug_check_weights(const moe_problem &p, const void *w_gate, const void *w_up,
                               const void *w_down, const void *x, const void *ws_gate,
                               const void *ws_up, const void *ws_down, hipStream_t st) {
  const int elt = elt_of(p);
  const size_t dff = p.d_ff, d = p.d_model, dfs = p.d_ff_shared;
  return debug_check({{w_gate, nz(p.E, dff, d), elt, nullptr, 0},
                      {w_up, nz(p.E, dff, d), elt, nullptr, 0},
                      {w_down, nz(p.E, d, dff), elt, nullptr, 0},
                      {dfs ? x : nullptr, nz(p.T, d), elt, nullptr, 0},
                      {dfs ? ws_gate : nullptr, nz(dfs, d), elt, nullptr, 0},
                      {dfs ? ws_up : nullptr, nz(dfs, d), elt, nullptr, 0},
                      {dfs ? ws_down : nullptr, nz(d, dfs), elt, nullptr, 0}},
                     st);
}

moe_status layer_forward(const moe_problem *pp, const void *x, const float *w_router,
                         const float *bias, const void *w_gate, const void *w_up,
                         const void *w_down, const void *ws_gate, const void *ws_up,
                         const void *ws_down, void *y, moe_routing *routing, void *ws,
                         size_t ws_bytes, hipStream_t st, hipEvent_t *ev) {
  moe_status s = check_problem(pp);
  if (s != MOE_OK) return s;
  const moe_problem &p = *pp;
  if (!ptr_ok(x) || !ptr_ok(w_router) || !opt_ptr_ok(bias) || !ptr_ok(w_gate) || !ptr_ok(w_up) ||
      !ptr_ok(w_down) || !ptr_ok(y))
    return MOE_ERR_INVALID_ARG;
  if (p.d_ff_shared > 0 && (!ptr_ok(ws_gate) || !ptr_ok(ws_up) || !ptr_ok(ws_down)))
    return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(p, ws, ws_bytes)) != MOE_OK) return s;
  char *w = (char *)ws;
  const Layout L = make_layout(p);
  moe_routing r = routing ? *routing : internal_routing(L, w);
  if (routing && (s = check_routing_out(p, routing)) != MOE_OK) return s;
  if ((s = debug_check({{x, nz(p.T, p.d_model), elt_of(p), nullptr, 0},
                        {w_router, nz(p.d_model, p.E), 4, nullptr, 0},
                        {bias, (size_t)p.E, 4, nullptr, 0}},
                       st)) != MOE_OK)
    return s;
  if ((s = debug_check_weights(p, w_gate, w_up, w_down, x, ws_gate, ws_up, ws_down, st)) != MOE_OK)
    return s;
  if (ensure_attributes() != hipSuccess) return MOE_ERR_HIP;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
  MOE_TRY(mark(MOE_STAGE_ROUTE));
  MOE_TRY(do_route(p, x, w_router, bias, 0, r, w, st));
  MOE_TRY(mark(MOE_STAGE_DISPATCH));   // the row gather runs inside the gate/up GEMM
  MOE_TRY(mark(MOE_STAGE_GATE_UP));
  MOE_TRY(do_gate_up(p, nullptr, r, w_gate, w_up, x, ws_gate, ws_up, w, st));
  MOE_TRY(mark(MOE_STAGE_DOWN));
  // decode-shaped batches whose down GEMM cuts K into parts: the parts' sum goes straight
  // into the combine (one launch fewer; o is never written)
  const GemmArgs da = down_args(p, r, w_down, ws_down, w + L.o_perm, w + L.o_shared, w);
  const bool fuse = skinny_split_down(da);
  MOE_TRY(do_down(p, r, w_down, ws_down, w + L.o_perm, w + L.o_shared, w, st, fuse));
  MOE_TRY(mark(MOE_STAGE_COMBINE));
  if (fuse)
    MOE_TRY(launch_skinny_down_combine(da, p.y_dtype == MOE_BF16 ? 2 : 4, r.tok_ptr, r.tok_pos,
                                       r.perm_w, y, p.T, p.d_model, num_cus(), st));
  else
    MOE_TRY(do_combine(p, w + L.o_perm, w + L.o_shared, r, y, st));
  MOE_TRY(mark(MOE_STAGE_COUNT));
  return MOE_OK;
}

// ---- allocation-free routing (moe_route_noalloc) -------------------------------------------
// The routing scratch of moe_route_noalloc lives in this library-held array instead of a
// caller's workspace: one copy per GPU the library runs on, held until the process ends. Its
// routing kernels write every scratch word they later read, so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`: looked up with hipGetSymbolAddress on
// the first call on that device (with that device current), then cached. Host code passes this
// address, never the array's name, to the kernels.
hipError_t scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Bytes of the workspace's routing regions: the layout puts them first, so the routing kernels
// touch only [0, partials) of a workspace.
size_t route_scratch_bytes(const moe_problem &p) { return make_layout(p).partials; }

moe_status route_checked(const moe_problem *problem, const void *x, const float *w_router,
                         const float *bias, int flags, moe_routing *routing, char *ws,
                         hipStream_t stream) {
  const moe_problem &p = *problem;
  moe_status s;
  if (flags & MOE_ROUTE_LOGITS_IN)
    s = debug_check({{routing->logits, nz(p.T, p.E), 4, nullptr, 0}}, stream);
  else
    s = debug_check({{x, nz(p.T, p.d_model), elt_of(p), nullptr, 0},
                     {w_router, nz(p.d_model, p.E), 4, nullptr, 0},
                     {bias, (size_t)p.E, 4, nullptr, 0}},
                    stream);
  if (s != MOE_OK) return s;
  if (do_route(p, x, w_router, bias, flags, *routing, ws, stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status check_route_args(const moe_problem *problem, const void *x, const float *w_router,
                            const float *bias, int flags, const moe_routing *routing) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  if (flags & ~MOE_ROUTE_LOGITS_IN) return MOE_ERR_INVALID_ARG;
  if (!(flags & MOE_ROUTE_LOGITS_IN) && (!ptr_ok(x) || !ptr_ok(w_router) || !opt_ptr_ok(bias)))
    return MOE_ERR_INVALID_ARG;
  return check_routing_out(*problem, routing);
}

}  // namespace

extern "C" {

moe_status moe_workspace_bytes(const moe_problem *problem, size_t *bytes) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = make_layout(*problem).total;
  return MOE_OK;
}

moe_status moe_route(const moe_problem *problem, const void *x, const float *w_router,
                     const float *bias, int flags, moe_routing *routing, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_route_args(problem, x, w_router, bias, flags, routing);
  if (s != MOE_OK) return s;
  if ((s = check_ws(*problem, ws, ws_bytes)) != MOE_OK) return s;
  return route_checked(problem, x, w_router, bias, flags, routing, (char *)ws, stream);
}

moe_status moe_route_noalloc(const moe_problem *problem, const void *x, const float *w_router,
                             const float *bias, int flags, moe_routing *routing,
                             hipStream_t stream) {
  moe_status s = check_route_args(problem, x, w_router, bias, flags, routing);
  if (s != MOE_OK) return s;
  if (route_scratch_bytes(*problem) > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return MOE_ERR_HIP;
  return route_checked(problem, x, w_router, bias, flags, routing, (char *)ws, stream);
}

moe_status moe_dispatch(const moe_problem *problem, const void *x, const moe_routing *routing,
                        void *x_perm, hipStream_t stream) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  if (!ptr_ok(x) || !ptr_ok(x_perm) || !routing || !ptr_ok(routing->perm_token) ||
      !ptr_ok(routing->offsets))
    return MOE_ERR_INVALID_ARG;
  if ((s = debug_check({{x, nz(problem->T, problem->d_model), elt_of(*problem), nullptr, 0}},
                       stream)) != MOE_OK)
    return s;
  if (do_dispatch(*problem, x, *routing, x_perm, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_problem *problem, const void *x_perm,
                          const moe_routing *routing, const void *w_gate, const void *w_up,
                          const void *w_down, const void *x, const void *ws_gate,
                          const void *ws_up, const void *ws_down, void *o_perm, void *o_shared,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  const moe_problem &p = *problem;
  if (!ptr_ok(x_perm) || !routing || !ptr_ok(routing->counts) || !ptr_ok(routing->offsets) ||
      !ptr_ok(w_gate) || !ptr_ok(w_up) || !ptr_ok(w_down) || !ptr_ok(o_perm))
    return MOE_ERR_INVALID_ARG;
  if (p.d_ff_shared > 0 && (!ptr_ok(x) || !ptr_ok(ws_gate) || !ptr_ok(ws_up) ||
                            !ptr_ok(ws_down) || !ptr_ok(o_shared)))
    return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(p, ws, ws_bytes)) != MOE_OK) return s;
  if ((s = debug_check({{x_perm, 0, elt_of(p), routing->offsets + p.E, p.d_model}}, stream)) !=
      MOE_OK)
    return s;
  if ((s = debug_check_weights(p, w_gate, w_up, w_down, x, ws_gate, ws_up, ws_down, stream)) !=
      MOE_OK)
    return s;
  if (ensure_attributes() != hipSuccess) return MOE_ERR_HIP;
  char *w = (char *)ws;
  if (do_gate_up(p, x_perm, *routing, w_gate, w_up, x, ws_gate, ws_up, w, stream) != hipSuccess)
    return MOE_ERR_HIP;
  if (do_down(p, *routing, w_down, ws_down, o_perm, o_shared, w, stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_combine(const moe_problem *problem, const void *o_perm, const void *o_shared,
                       const moe_routing *routing, void *y, hipStream_t stream) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  const moe_problem &p = *problem;
  if (!ptr_ok(o_perm) || !ptr_ok(y) || !routing || !ptr_ok(routing->tok_ptr) ||
      !ptr_ok(routing->tok_pos) || !ptr_ok(routing->perm_w))
    return MOE_ERR_INVALID_ARG;
  if (p.d_ff_shared > 0 && !ptr_ok(o_shared)) return MOE_ERR_INVALID_ARG;
  if ((s = debug_check({{o_perm, 0, 4, routing->tok_ptr + p.T, p.d_model},
                        {routing->perm_w, 0, 4, routing->tok_ptr + p.T, 1},
                        {p.d_ff_shared > 0 ? o_shared : nullptr, nz(p.T, p.d_model), 4, nullptr, 0}},
                       stream)) != MOE_OK)
    return s;
  if (do_combine(p, o_perm, o_shared, *routing, y, stream) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_problem *problem, const void *x, const float *w_router,
                             const float *bias, const void *w_gate, const void *w_up,
                             const void *w_down, const void *ws_gate, const void *ws_up,
                             const void *ws_down, void *y, moe_routing *routing, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
  return layer_forward(problem, x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                       y, routing, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_forward_traced(const moe_problem *problem, const void *x,
                                    const float *w_router, const float *bias,
                                    const void *w_gate, const void *w_up, const void *w_down,
                                    const void *ws_gate, const void *ws_up, const void *ws_down,
                                    void *y, moe_routing *routing, void *ws, size_t ws_bytes,
                                    hipStream_t stream, hipEvent_t *events, int n_events) {
  if (!events || n_events != MOE_STAGE_COUNT + 1) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return layer_forward(problem, x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                       y, routing, ws, ws_bytes, stream, events);
}

moe_status moe_routing_stats(const moe_problem *problem, const moe_routing *routing, float *out,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_problem(problem);
  if (s != MOE_OK) return s;
  const moe_problem &p = *problem;
  if (!routing || !ptr_ok(routing->logits) || !ptr_ok(routing->counts) ||
      !ptr_ok(routing->offsets) || !ptr_ok(out))
    return MOE_ERR_INVALID_ARG;
  if ((s = check_ws(p, ws, ws_bytes)) != MOE_OK) return s;
  if ((s = debug_check({{routing->logits, nz(p.T, p.E), 4, nullptr, 0}}, stream)) != MOE_OK)
    return s;
  const Layout L = make_layout(p);
  if (launch_stats(routing->logits, routing->counts, routing->offsets, p.T, p.E, p.k,
                   p.routing == MOE_TOKEN_CHOICE ? 1 : 0,
                   (float *)((char *)ws + L.stats_part), out, stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

const char *moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid shape, pointer or enum";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid problem without a kernel";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_bytes";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed";
  }
  return "unknown moe_status";
}

}  // extern "C"
