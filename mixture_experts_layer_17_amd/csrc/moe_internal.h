// Host-side launchers shared between libmoe's translation units.  Every
// launcher enqueues on `s` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct GemmTileCfg {
  int BM;        // rows per tile
  int BN;        // B columns per tile (SwiGLU: gate half + up half)
  int id;        // which compiled instance
  int wnt = 0;   // LDS configs: weight copies with the non-temporal hint
};

// Router: logits, top-k ids/weights, optional counts (counts must be zeroed
// first; launch_fill_i32 does that).
// Router variant (MindSpore moe.py, TokenChoiceTopKRouter.forward): scores
// are sigmoid (or softmax) of the logits times `scale`; with groups > 0 only
// the `limited` groups with the largest maximum score stay selectable;
// selection ranks score + ebias[e]; weights are the unbiased scores.  tpe,
// when set, accumulates the selections per expert.
struct RouterVariant {
  int sigmoid;
  float scale;
  const float* ebias;
  int groups;
  int limited;
  float* tpe;
};

// The permutation's first pass folded into the router's selection kernel
// (large batches on the split-K path): each 16-token block writes its
// slots' ranks among equal experts (`rank`, [N]) and its expert histogram
// (`sub`, [ceil(T / 16)][E]) and adds that histogram into the 1024-slot
// chunk histograms (`hist`, [ceil(N / 1024)][E], cleared by the router's
// first kernel).
struct PermuteFold {
  int32_t* hist;
  int32_t* sub;
  int32_t* rank;
};

// `parts` (optional, route_ws_bytes of it): float32 partial logits, which
// let large batches take the split-K router.  `fold` (only where
// route_can_fold holds): also run the permutation's first pass.
hipError_t launch_route(bool bf16, const void* x, const void* wr, const float* bias,
                        int T, int H, int E, int k, int norm, float* logits,
                        int32_t* ids, float* w, int32_t* counts, hipStream_t s,
                        const RouterVariant* var = nullptr, float* parts = nullptr,
                        size_t parts_bytes = 0, const PermuteFold* fold = nullptr);
size_t route_ws_bytes(int T, int H, int E, bool bf16);
bool route_can_fold(int T, int H, int E, int k, bool bf16);
hipError_t launch_update_expert_bias(float* bias, float* tpe, int E, float lr, int nrec,
                                     hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

// Token-choice permutation.  ws layout is given by permute_ws_bytes().
size_t permute_ws_bytes(int N, int E, int R);
// The folded first pass's scratch: the two-pass permutation's histogram and
// ranks (same place in a permute workspace), then the block histograms.
size_t permute_fold_ws_bytes(int T, int k, int E);
PermuteFold permute_fold_scratch(void* ws, int T, int k, int E);
// Optionally also writes the GEMMs' tile lists (tile_ws_a / tile_ws_b for
// row-tile heights BM_a / BM_b; NULL to skip).  With `fold` the first pass
// already ran inside the router (launch_route with the same fold).
hipError_t launch_permute_topk(const int32_t* ids, int T, int k, int E,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                               int32_t* sorted_slot, int32_t* slot_pos, void* ws,
                               hipStream_t s, void* tile_ws_a = nullptr, int BM_a = 0,
                               void* tile_ws_b = nullptr, int BM_b = 0,
                               const PermuteFold* fold = nullptr);
hipError_t launch_permute_rank_major(const int32_t* counts_rm, int R, int N, int E,
                                     int32_t* counts, int32_t* offsets,
                                     int32_t* sorted_token, int32_t* sorted_slot,
                                     int32_t* slot_pos, void* ws, hipStream_t s);

hipError_t launch_gather_rows(bool bf16, const void* x, int x_rows, const int32_t* idx, int N,
                              int H, void* out, hipStream_t s);

// out[t] = sum_j w[t, j] * y[slot(t, j)] (+ add[t] when add is set), summed in
// float32 and rounded once.
hipError_t launch_combine(bool bf16, const void* y, const int32_t* slot_pos,
                          const float* w, int T, int k, int H, const void* add, void* out,
                          hipStream_t s);

// A dense second problem run in the same LDS grouped-GEMM launch (the shared
// expert): `rows` rows of X read in order against one weight matrix, outputs
// stored in row order.  Its jobs (ceil(rows / BM) * n_ntiles) come before the
// grouped ones; jobs == 0 means there is none.
struct DenseAux {
  const void* X;
  const void* W;
  void* C;
  int ldx, ldw, K, up_off, ldc, rows, n_ntiles, jobs;
  void* g_save;   // training forward: the dense problem's pre-activations, or NULL
};
DenseAux dense_aux(const GemmTileCfg& c, bool swiglu, const void* X, int ldx, const void* W,
                   int ldw, int K, int up_off, void* C, int ldc, int rows, int cols);

// Grouped GEMMs.  Configs with id >= 10 run the LDS-ring kernel
// (moe_gemm_lds.hip); the others the register-transpose kernel.
bool lds_cfg_id(int id);
GemmTileCfg pick_lds_cfg(int N, int E, int cols, bool swiglu);
hipError_t launch_lds_gemm(bool swiglu, const GemmTileCfg& c, const void* X, int ldx,
                           const int32_t* x_index, int x_rows, const void* W,
                           long long w_estride, int ldw, int K, int up_off, void* C, int ldc,
                           const int32_t* c_index, int c_rows, const int32_t* offsets, int N,
                           int E, int n_ntiles, void* tile_ws, bool tiles_ready, hipStream_t s,
                           const DenseAux* aux = nullptr, void* g_save = nullptr);
// Builds the tile list of row-tile height BM into tile_ws (one block).
hipError_t launch_build_tiles(const int32_t* offsets, int E, int N, int BM, void* tile_ws,
                              hipStream_t s);
// One dense group of `rows` rows (a shared expert): with offsets == NULL the
// tile builders take the single group [0, N).
GemmTileCfg pick_lds_dense_cfg(int rows, int cols, bool swiglu);
GemmTileCfg pick_dense_cfg(bool bf16, int rows, int cols, bool swiglu);
GemmTileCfg pick_gate_up_cfg(bool bf16, int N, int H, int I, int E);
GemmTileCfg pick_down_cfg(bool bf16, int N, int H, int I, int E);
size_t tile_list_bytes(int N, int E, int BM);
// `aux` (LDS configs only) adds a dense problem to the same launch;
// `g_save` (LDS configs only) also stores the pre-activations [N, 2I].
hipError_t launch_gate_up(bool bf16, const GemmTileCfg& c, const void* x, int x_rows,
                          const int32_t* row_index, const int32_t* offsets, int N, int H,
                          int I, int E, const void* gate_up, void* h, void* tile_ws,
                          bool tiles_ready, hipStream_t s, const DenseAux* aux = nullptr,
                          void* g_save = nullptr);
hipError_t launch_down(bool bf16, const GemmTileCfg& c, const void* h,
                       const int32_t* offsets, const int32_t* out_index, int N, int H,
                       int I, int E, const void* down, void* y, void* tile_ws,
                       bool tiles_ready, hipStream_t s, const DenseAux* aux = nullptr);

// Backward (moe_gemm_bwd.hip, moe_backward.hip).  bf16 only; I % 128 == 0,
// H % 128 == 0.  The dgrad GEMMs use the row-tile list of height
// dgrad_bm(id).
int pick_dgrad_cfg(int N, int E);
int pick_dgrad1_cfg(int N, int E);
int dgrad_bm(int id);
// The shared expert's dgrads, folded into the routed dgrad launches as a
// dense problem of `rows` token rows (weight 1): dout . down^T with the
// SwiGLU backward into dG [rows, 2 Is] and hw [rows, Is], then
// dG . gate_up^T into dx [rows, H].
struct DgradShared {
  const void* gate_up;
  const void* down;
  const void* G;
  void* dG;
  void* hw;
  void* dx;
  int rows, Is;
};
// The first dgrad's config must use 128-column tiles (pick_dgrad1_cfg)
// so that any Is multiple of 128 fits.
// w == NULL: every row's weight is 1 (a shared expert); sorted_slot NULL:
// row p's weight is w[p].
// dw_parts (optional, [N, dgrad1_weight_parts(I)] float): for each
// expert-major row p the inner products <dout . down^T, h> over the
// epilogue's column slices, which launch_weight_grad adds up.
int dgrad1_weight_parts(int I);
hipError_t launch_dgrad_down_swiglu(int id, const void* dout, int T, const int32_t* sorted_token,
                                    const void* down, int N, int H, int I, int E,
                                    const void* G, const float* w, const int32_t* sorted_slot,
                                    void* dG, void* hw, const void* tile_ws, hipStream_t s,
                                    const DgradShared* sh = nullptr, float* dw_parts = nullptr);
hipError_t launch_dgrad_gate_up(int id, const void* dG, const void* gate_up, int N, int H, int I,
                                int E, const int32_t* out_index, void* dX, const void* tile_ws,
                                hipStream_t s, const DgradShared* sh = nullptr);
// A dense problem folded into a wgrad launch (the shared expert): C [M, N]
// = A^T B over `rows` rows; its jobs run first.
struct WgradAux {
  const void* A;
  int lda;
  const void* B;
  int ldb;
  int rows, M, N;
  void* C;
  int jobs;   // set by the launcher
};
bool wgrad_can_fold(int M, int N, int Ma, int Na);
// C[e] = A_e^T B_e over the expert-major rows [offsets[e], offsets[e + 1]);
// `aux` (when wgrad_can_fold) adds a dense problem to the same launch.
// job_counters (optional): kWgradCounters unsigned zeros, used up by the
// launch; with them the 256 x 256 tiles run the persistent kernel.
constexpr int kWgradCounters = 8;
hipError_t launch_wgrad(const void* A, int lda, const void* B, int ldb, const void* zero_row,
                        const int32_t* offsets, int E, int M, int N, void* C, hipStream_t s,
                        const WgradAux* aux = nullptr, unsigned* job_counters = nullptr);
// d_weights [N] (flat slot order) from the first dgrad's P partial inner
// products per expert-major row (dgrad1_weight_parts).
hipError_t launch_weight_grad(const float* parts, int P, const int32_t* slot_pos, int N,
                              float* dw, hipStream_t s);
// dL [T, E] for softmax or sigmoid scores times `scale`; when dL is zero
// off the selection (renormalised or sigmoid) also dl_perm [N] (dL of each
// selected entry, in the permutation's expert-major order).
hipError_t launch_router_grad(const float* logits, const int32_t* ids, const float* w,
                              const float* dw, const int32_t* slot_pos, int T, int E, int k,
                              int norm, int sigmoid, float scale, float* dL, float* dl_perm,
                              hipStream_t s);
// With ids (renormalised weights: dL is zero off the selection) only the
// selected experts' router rows are read; ids == NULL reads all E.
// add (optional, [T, H]) joins the sum (the shared expert's input gradient).
hipError_t launch_input_grad(bool bf16, const void* dX, const float* dL, const int32_t* ids,
                             const void* wr, int T, int k, int E, int H, const void* add,
                             void* dx, hipStream_t s);
// Router weight and bias gradients; ws holds router_weight_grad_ws(E, H)
// bytes of partial sums.  sparse: the expert-major rows x[sorted_token[p]]
// with dl_perm[p].
size_t router_weight_grad_ws(int E, int H);
hipError_t launch_router_weight_grad(bool bf16, const void* x, const int32_t* sorted_token,
                                     const float* dL, const float* dl_perm,
                                     const int32_t* offsets, int T, int E, int H, int sparse,
                                     float* dwr, float* dbias, void* ws, hipStream_t s);
hipError_t launch_fill_u32(void* p, long long n, uint32_t v, hipStream_t s);

}  // namespace moe
