// Internal launch interface between the host layer (moe_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxGroups = kMaxExperts + 1;   // routed experts + one shared expert

// Workspace regions used by the routing kernels.
struct RouteScratch {
  float *keys;          // [T*S] routing score of each pick (capacity drop)
  int32_t *blk_cnt;     // [nblk*E] per-block per-expert counts
  int32_t *blk_base;    // [nblk*E] exclusive scan over blocks
  int32_t *cnt_pre;     // [E] candidates per expert (before the capacity drop)
  int32_t *off_pre;     // [E+1]
  int32_t *cand_token;  // [T*S] candidates grouped by expert (or expert group)
  int32_t *cand_slot;   // [T*S]
  float *cand_key;      // [T*S]
  float *cand_w;        // [T*S] gate of each candidate
  int32_t *slot_pos;    // [T*S] row of (token, slot) or -1; S = k + m (token choice) or E
  uint32_t *colkeys;    // [E*T] expert-choice column keys (or the transposed logits)
  int32_t *tok_blk;     // [nblk] per-block row counts of the token CSR
  int32_t *tok_blk_off; // [nblk]
  float *stats_part;    // [nblk*E]
  uint16_t *w3;         // [3][E_pad][d] bf16 parts of the router weight (bf16 x)
};

// Grouped GEMM: routed experts (rows from counts/offsets on the device) + optional shared.
struct GemmArgs {
  const void *A; int lda;          // routed rows, group e starts at row offsets[e]
  const int32_t *a_rows;           // optional row map: routed row p reads A row a_rows[p]
  const void *B0; const void *B1;  // [E, N, K] (B1: up weights for gate/up, else null)
  void *C; int ldc;
  const int32_t *counts, *offsets;
  int E, N, K, elt;                // elt: bytes per A/B element
  int c_elt;                       // bytes per C element (h: elt; o: 4)
  const void *sA; const void *sB0; const void *sB1; void *sC;   // shared group
  int s_rows, sN, sK, s_lda, s_ldc;
  // tail split: the tiles of the last, partial round of the persistent grid may run as S
  // K-parts whose float32 partial tiles go to `partials` (room for kMaxPersistent tiles)
  // and are summed by a second kernel; allowed when every group has the same K
  float *partials;
  int split_ok;
  int grid;                         // persistent grid size (set by the launcher)
  int wide;                         // bf16 tiles: a group's last row tile of at most 64 rows
                                    // spans two column panels (set by the launcher)
  int band;                         // bf16 tile order: column panels in bands of `band`, row
                                    // tile by row tile inside a band (<= 1: panel by panel)
  // few rows per group (decode-shaped batches): every group holds at most max_group_rows
  // rows; when that is <= kSkinnyRows (kSkinnyRowsGateUp for gate/up), 32/64/128-row units
  // stream the weights (once per 128-row block of a group), their K range cut into sk_S parts
  // whose float32 sums (rows of sk_pitch floats, routed rows first, then the shared rows at
  // row rcap) go to `partials`
  int max_group_rows;
  int rcap;                         // routed row capacity (T*k)
  int sk_S, sk_pitch;               // set by the launcher
};

constexpr int kMaxPersistent = 256;   // persistent GEMM workgroups (one per CU on MI355X)
constexpr size_t kPartialBytes = (size_t)kMaxPersistent * 256 * 256 * 4;
constexpr int kSkinnyRows = 768;      // groups of at most this many rows take the skinny path
constexpr int kSkinnyRowsGateUp = 64; // (the gate/up GEMM: only up to this many)
// float32 partial-sum bytes the skinny path needs for a GEMM (0 if it does not apply)
size_t skinny_partial_bytes(const GemmArgs &a, bool gate_up);

// Debug-mode input checks (environment MOE_DEBUG set and not "0").
struct DebugSpan {
  const void *p;               // device data (null: skipped)
  size_t n;                    // elements, unless n_rows_dev is given
  int elt;                     // 2: bf16, 4: float32
  const int32_t *n_rows_dev;   // optional device row count; elements = rows * row_elems
  int row_elems;
};
bool debug_checks_enabled();
// enqueue the checks on st, synchronise st; found = some element is NaN or infinite
hipError_t debug_any_nonfinite(const DebugSpan *spans, int n_spans, hipStream_t st, bool *found);

int router_epad(int E);   // experts padded for the matrix-core router (bf16 x)
size_t router_w3_bytes(int dtype, int d, int E);   // bf16 W_r parts the router needs
// token-choice top-k outputs a router may produce alongside the logits (launch_topk's
// arguments: k picks, renormalisation over the first kden, routing keys when want_key)
struct TopkOut {
  int k, kden, renorm, want_key;
  int32_t *ids;
  float *gates, *keys;
  int32_t *blk_cnt;   // optional: picks per expert of each workgroup's tokens (E <= 16)
};
constexpr int kBlkCountMaxE = 16;   // experts the per-block counts and their dispatch handle
// Optional extra output of the router for expert choice: the logits transposed ([E][T]).
struct RouterExtra {
  float *logits_t;
};
// logits = x W_r + b; with topk non-null, the router may also run the top-k of every token
// (same results as launch_topk) and then sets *topk_done; when it also wrote topk->blk_cnt,
// *cnt_block is the number of tokens per count block (else 0). With ex non-null, the
// matrix-core router for at most 10 experts also writes ex's outputs and sets *ex_done
// (other routers leave them and set it false). With disp non-null (final mode, the
// BlkDispatchOut of launch_dispatch_blocks) and at most 16 tokens, that router also writes
// the dispatch itself and sets *disp_done.
struct BlkDispatchOut;
hipError_t launch_router(int dtype, const void *x, const float *w, const float *bias,
                         float *logits, int T, int d, int E, uint16_t *w3, hipStream_t st,
                         const TopkOut *topk = nullptr, bool *topk_done = nullptr,
                         int *cnt_block = nullptr, const RouterExtra *ex = nullptr,
                         bool *ex_done = nullptr, const BlkDispatchOut *disp = nullptr,
                         bool *disp_done = nullptr);
// with blk_cnt non-null (E <= 16) the picks per expert of each workgroup's tokens go there and
// *cnt_block gets the tokens per workgroup
hipError_t launch_topk(const float *logits, int T, int E, int k, int kden, int renorm,
                       int want_key, int32_t *ids, float *gates, float *keys, hipStream_t st,
                       int32_t *blk_cnt = nullptr, int *cnt_block = nullptr);
// Outputs of the one-launch dispatch from per-block top-k counts (E <= 16). Final mode (token
// choice without a capacity limit): counts, offsets, perm_token, perm_w, the token CSR and
// kept (optional). Candidate mode (cand_slot non-null, before a capacity selection): counts /
// offsets are the candidates per expert, perm_token / perm_w / cand_slot / cand_key the
// candidate lists (routing keys read from keys), cnt_fin / off_fin the counts and offsets
// capped at C.
struct BlkDispatchOut {
  int32_t *counts, *offsets, *perm_token;
  float *perm_w;
  uint8_t *kept;
  int32_t *tok_ptr, *tok_pos;
  const float *keys;
  int32_t *cand_slot;
  float *cand_key;
  int32_t *cnt_fin, *off_fin;
  int C;
};
// one launch from the per-block counts of the top-k (blocks of bt tokens, bt in {16, 32})
hipError_t launch_dispatch_blocks(const int32_t *ids, const float *gates, int T, int k, int E,
                                  const int32_t *blk_cnt, int bt, const BlkDispatchOut &o,
                                  hipStream_t st);
// capacity selection of candidate lists already grouped per expert (cnt_pre / off_pre), final
// mode: the kept rows to perm_token / perm_w at off_fin, slot_pos and kept per (token, slot)
hipError_t launch_cap_select_final(const RouteScratch &s, int E, int C, int S, int32_t *perm_token,
                                   float *perm_w, uint8_t *kept, const int32_t *off_fin,
                                   hipStream_t st);
// with C < 0 (no capacity) and tok_ptr/tok_pos non-null the token -> rows CSR is written too
hipError_t launch_token_dispatch(const RouteScratch &s, const int32_t *ids, const float *gates,
                                 int T, int k, int E, int C, int32_t *perm_token, float *perm_w,
                                 uint8_t *kept, int32_t *counts, int32_t *offsets,
                                 int32_t *tok_ptr, int32_t *tok_pos, hipStream_t st);
hipError_t launch_group_capacity(const RouteScratch &s, const int32_t *ids, const float *gates,
                                 int T, int k, int E, int D, int C_D, int32_t *perm_token,
                                 float *perm_w, uint8_t *kept, int32_t *counts, int32_t *offsets,
                                 hipStream_t st);
hipError_t launch_expanded_drop(const RouteScratch &s, const int32_t *ids, const float *gates,
                                int T, int k, int m, int E, int C, int32_t *perm_token,
                                float *perm_w, uint8_t *kept, int32_t *counts, int32_t *offsets,
                                hipStream_t st);
// Expert choice. With logits_t (the logits transposed, [E][T]) the selection reads each
// expert's column as one contiguous row.
hipError_t launch_expert_choice(const RouteScratch &s, const float *logits, int T, int E, int c,
                                int32_t *perm_token, float *perm_w, int32_t *counts,
                                int32_t *offsets, hipStream_t st, const float *logits_t = nullptr);
hipError_t launch_token_csr(const RouteScratch &s, int T, int S, int32_t *tok_ptr,
                            int32_t *tok_pos, hipStream_t st);
hipError_t launch_stats(const float *logits, const int32_t *counts, const int32_t *offsets, int T,
                        int E, int k, int token_choice, float *part, float *out, hipStream_t st);
hipError_t launch_gather(int elt, const void *x, const int32_t *perm_token,
                         const int32_t *n_rows_dev, void *x_perm, int d, int max_rows,
                         int num_cu, hipStream_t st);
hipError_t launch_combine(int y_elt, const float *o, const float *o_shared,
                          const int32_t *tok_ptr, const int32_t *tok_pos, const float *perm_w,
                          void *y, int T, int d, int max_rows, hipStream_t st);
// defer_skinny_reduce: on the skinny path with K parts, leave the parts unsummed for
// launch_skinny_down_combine (down GEMM only)
hipError_t launch_gemm(const GemmArgs &a, bool gate_up, int max_rows, int num_cu,
                       hipStream_t st, bool defer_skinny_reduce = false);
// whether the down GEMM a takes the skinny path with its K range cut into parts
bool skinny_split_down(const GemmArgs &a);
// after launch_gemm(a, false, ..., defer_skinny_reduce = true): the parts' sum and the
// weighted combine into y (y_elt 2: bf16, 4: float32) in one launch
hipError_t launch_skinny_down_combine(const GemmArgs &a, int y_elt, const int32_t *tok_ptr,
                                      const int32_t *tok_pos, const float *perm_w, void *y,
                                      int T, int d, int num_cu, hipStream_t st);
hipError_t gemm_setup_attributes();

}  // namespace moe
