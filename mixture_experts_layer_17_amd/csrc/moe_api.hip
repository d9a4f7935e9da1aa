// libmoe C ABI: argument validation, workspace carve-up and launch sequencing.
// Every entry point validates everything before it enqueues anything.
#include <stdint.h>

#include "../../include/libmoe.h"
#include <cmath>
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxE = 256;
constexpr int kMaxRankMajorBlocks = 4096;
constexpr int kVersion = 2;

size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

bool dtype_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }

int check_dims(int H, int I, int E, int k) {
  if (E < 1 || E > kMaxE) return MOE_ERR_SHAPE;
  if (k < 1 || k > E) return MOE_ERR_SHAPE;
  if (H <= 0 || H % 128 != 0) return MOE_ERR_SHAPE;
  if (I < 0 || I % 64 != 0) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Row counts are int32 on the device; keep N * max(H, 2I) element offsets
// inside 64-bit math and every row index inside int32.
bool rows_ok(long long rows) { return rows >= 0 && rows <= (1ll << 30); }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

struct LayerWs {
  int32_t *ids, *counts, *offsets, *sorted_token, *sorted_slot, *slot_pos;
  float *weights, *logits;
  void *perm, *h, *y, *tiles_up, *tiles_down;
  float* route_parts;                           // the router's partial logits
  size_t route_parts_bytes;
  void *h_s, *y_s, *tiles_s_up, *tiles_s_down;  // shared expert (Is > 0)
  // byte offsets of the pieces moe_layer_workspace_offset reports
  size_t at_offsets, at_sorted_token, at_sorted_slot, at_slot_pos, at_y;
  size_t total;
};

// The shared expert's region: h_s [T, Is], y_s [T, H] when with_y, and the
// two dense tile lists.
struct SharedWs {
  void *h, *y, *tiles_up, *tiles_down;
  size_t total;
};

SharedWs shared_ws(char* base, int T, int H, int Is, moe_dtype dt, bool with_y) {
  SharedWs w{};
  const bool bf16 = dt == MOE_BF16;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  };
  w.h = take((size_t)T * Is * esize(dt));
  if (with_y) w.y = take((size_t)T * H * esize(dt));
  w.tiles_up = take(tile_list_bytes(T, 1, pick_dense_cfg(bf16, T, Is, true).BM));
  w.tiles_down = take(tile_list_bytes(T, 1, pick_dense_cfg(bf16, T, H, false).BM));
  w.total = off;
  return w;
}

// FeedForward on every token: gate/up GEMM with SwiGLU into h, down GEMM into
// y.  No offsets: the tile builders take one group of T rows.
hipError_t run_shared(bool bf16, const void* x, const void* gate_up, const void* down, int T,
                      int H, int Is, const SharedWs& w, void* y, hipStream_t s) {
  const GemmTileCfg cu = pick_dense_cfg(bf16, T, Is, true);
  const GemmTileCfg cd = pick_dense_cfg(bf16, T, H, false);
  hipError_t e = launch_gate_up(bf16, cu, x, T, nullptr, nullptr, T, H, Is, 1, gate_up, w.h,
                                w.tiles_up, false, s);
  if (e != hipSuccess) return e;
  return launch_down(bf16, cd, w.h, nullptr, nullptr, T, H, Is, 1, down, y, w.tiles_down, false,
                     s);
}

LayerWs layer_ws(char* base, int T, int H, int I, int E, int k, moe_dtype dt, int Is = 0) {
  LayerWs w{};
  const size_t N = (size_t)T * k;
  const bool bf16 = dt == MOE_BF16;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  };
  w.ids = (int32_t*)take(N * 4);
  w.weights = (float*)take(N * 4);
  w.logits = (float*)take((size_t)T * E * 4);
  w.counts = (int32_t*)take((size_t)E * 4);
  w.at_offsets = off;
  w.offsets = (int32_t*)take((size_t)(E + 1) * 4);
  w.at_sorted_token = off;
  w.sorted_token = (int32_t*)take(N * 4);
  w.at_sorted_slot = off;
  w.sorted_slot = (int32_t*)take(N * 4);
  w.at_slot_pos = off;
  w.slot_pos = (int32_t*)take(N * 4);
  w.perm = take(permute_fold_ws_bytes(T, k, E));   // with the router-folded first pass
  w.h = take(N * (size_t)I * esize(dt));
  w.at_y = off;
  w.y = take(N * (size_t)H * esize(dt));
  const GemmTileCfg cu = pick_gate_up_cfg(bf16, (int)N, H, I, E);
  const GemmTileCfg cd = pick_down_cfg(bf16, (int)N, H, I, E);
  w.tiles_up = take(tile_list_bytes((int)N, E, cu.BM));
  w.tiles_down = take(tile_list_bytes((int)N, E, cd.BM));
  w.route_parts_bytes = route_ws_bytes(T, H, E, bf16);
  w.route_parts = (float*)take(w.route_parts_bytes);
  if (Is > 0) {
    const SharedWs sw = shared_ws(nullptr, T, H, Is, dt, true);
    const SharedWs sp = shared_ws(base ? base + off : nullptr, T, H, Is, dt, true);
    w.h_s = sp.h;
    w.y_s = sp.y;
    w.tiles_s_up = sp.tiles_up;
    w.tiles_s_down = sp.tiles_down;
    off += sw.total;
  }
  w.total = off;
  return w;
}

size_t swiglu_ws(int N, int H, int I, int E, moe_dtype dt, size_t* h_bytes,
                 size_t* up_bytes) {
  const bool bf16 = dt == MOE_BF16;
  const GemmTileCfg cu = pick_gate_up_cfg(bf16, N, H, I, E);
  const GemmTileCfg cd = pick_down_cfg(bf16, N, H, I, E);
  *h_bytes = al((size_t)N * I * esize(dt));
  *up_bytes = tile_list_bytes(N, E, cu.BM);
  return *h_bytes + *up_bytes + tile_list_bytes(N, E, cd.BM);
}

// Router variant from the public config (validated), or NULL for the
// default softmax router.
int router_variant(const moe_router_config* c, int E, int k, RouterVariant* out,
                   const RouterVariant** use) {
  *use = nullptr;
  if (!c) return MOE_OK;
  if (c->score_func != MOE_SCORE_SOFTMAX && c->score_func != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  if (!std::isfinite(c->route_scale)) return MOE_ERR_SHAPE;
  const int G = c->num_expert_groups;
  if (G < 0) return MOE_ERR_SHAPE;
  if (G > 0) {
    if (E % G != 0 || c->num_limited_groups < 1 || c->num_limited_groups > G ||
        (long long)k > (long long)c->num_limited_groups * (E / G))
      return MOE_ERR_SHAPE;
  }
  *out = RouterVariant{c->score_func == MOE_SCORE_SIGMOID ? 1 : 0, c->route_scale,
                       c->expert_bias, G, G > 0 ? c->num_limited_groups : 0,
                       c->tokens_per_expert};
  *use = out;
  return MOE_OK;
}

// Backward workspace: permutation of the forward's ids, the dgrad tile list,
// d_weights, dL, dG [N, 2I], w h [N, I], dX [N, H] and a zero row.
struct BwdWs {
  int32_t *counts, *offsets, *sorted_token, *sorted_slot, *slot_pos;
  void *perm, *tiles, *tiles1;
  float *dw, *dw_parts, *dL, *dl_perm;
  void *dG, *hw, *dX, *x_perm, *dout_perm, *zero, *rw_part;
  void *dG_s, *hw_s, *dx_s;   // shared expert (Is > 0)
  int32_t* offs_s;
  unsigned* counters;         // 2 x kWgradCounters, zeroed with the zero row
  size_t zero_bytes, total;
};

BwdWs bwd_ws(char* base, int T, int H, int I, int E, int k, moe_dtype dt, int Is = 0) {
  BwdWs w{};
  const size_t N = (size_t)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  };
  w.counts = (int32_t*)take((size_t)E * 4);
  w.offsets = (int32_t*)take((size_t)(E + 1) * 4);
  w.sorted_token = (int32_t*)take(N * 4);
  w.sorted_slot = (int32_t*)take(N * 4);
  w.slot_pos = (int32_t*)take(N * 4);
  w.perm = take(permute_ws_bytes((int)N, E, 0));
  w.tiles = take(tile_list_bytes((int)N, E, dgrad_bm(pick_dgrad_cfg((int)N, E))));
  w.tiles1 = take(tile_list_bytes((int)N, E, dgrad_bm(pick_dgrad1_cfg((int)N, E))));
  w.dw = (float*)take(N * 4);
  w.dw_parts = (float*)take(N * (size_t)std::max(1, dgrad1_weight_parts(I)) * 4);
  w.dL = (float*)take((size_t)T * E * 4);
  w.dl_perm = (float*)take(N * 4);
  w.rw_part = take(router_weight_grad_ws(E, H));
  w.dG = take(N * 2 * (size_t)I * esize(dt));
  w.hw = take(N * (size_t)I * esize(dt));
  w.dX = take(N * (size_t)H * esize(dt));
  w.x_perm = take(N * (size_t)H * esize(dt));
  w.dout_perm = take(N * (size_t)H * esize(dt));
  if (Is > 0) {
    w.dG_s = take((size_t)T * 2 * Is * esize(dt));
    w.hw_s = take((size_t)T * Is * esize(dt));
    w.dx_s = take((size_t)T * H * esize(dt));
    w.offs_s = (int32_t*)take(2 * sizeof(int32_t));
  }
  // one zero row, then the two wgrad launches' job counters (zeroed with it)
  const size_t row_bytes = al((size_t)std::max(std::max(H, 2 * I), 2 * Is) * esize(dt));
  w.zero_bytes = row_bytes + al(2 * kWgradCounters * sizeof(unsigned));
  w.zero = take(w.zero_bytes);
  w.counters = base ? (unsigned*)((char*)w.zero + row_bytes) : nullptr;
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int moe_version(void) { return kVersion; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported request";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_SCRATCH:
      return "request needs more than the library's static scratch buffer "
             "(MOE_STATIC_SCRATCH_BYTES); use the workspace entry point";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(int op, int T, int H, int I, int E, int top_k, int R, int N,
                          moe_dtype dt) {
  const size_t bad = (size_t)-1;
  if (!dtype_ok(dt)) return bad;
  switch (op) {
    case MOE_OP_ROUTE: return 0;
    case MOE_OP_PERMUTE:
      if (E < 1 || E > kMaxE) return bad;
      if (R > 0) {
        if ((long long)R * E > kMaxRankMajorBlocks || !rows_ok(N)) return bad;
        return permute_ws_bytes(N, E, R);
      }
      if (T < 0 || top_k < 1 || top_k > E || !rows_ok((long long)T * top_k)) return bad;
      return permute_ws_bytes(T * top_k, E, 0);
    case MOE_OP_GATE_UP:
    case MOE_OP_DOWN:
    case MOE_OP_GROUPED_SWIGLU: {
      if (check_dims(H, I, E, 1) != MOE_OK || !rows_ok(N)) return bad;
      const bool bf16 = dt == MOE_BF16;
      if (op == MOE_OP_GATE_UP) return tile_list_bytes(N, E, pick_gate_up_cfg(bf16, N, H, I, E).BM);
      if (op == MOE_OP_DOWN) return tile_list_bytes(N, E, pick_down_cfg(bf16, N, H, I, E).BM);
      size_t hb, ub;
      return swiglu_ws(N, H, I, E, dt, &hb, &ub);
    }
    case MOE_OP_LAYER:
      // R: the shared expert's intermediate size (0: no shared expert)
      if (check_dims(H, I, E, top_k) != MOE_OK || T < 0 || !rows_ok((long long)T * top_k) ||
          R < 0 || R % 64 != 0)
        return bad;
      return layer_ws(nullptr, T, H, I, E, top_k, dt, R).total;
    case MOE_OP_LAYER_BACKWARD:
      // R: the shared expert's intermediate size (0: none)
      if (check_dims(H, I, E, top_k) != MOE_OK || I == 0 || T < 0 ||
          !rows_ok((long long)T * top_k) || R < 0 || R % 64 != 0)
        return bad;
      return bwd_ws(nullptr, T, H, I, E, top_k, dt, R).total;
    case MOE_OP_SHARED:
      if (check_dims(H, I, 1, 1) != MOE_OK || I == 0 || T < 0 || !rows_ok(T)) return bad;
      return shared_ws(nullptr, T, H, I, dt, false).total;
    default: return bad;
  }
}

size_t moe_layer_workspace_offset(int piece, int T, int H, int I, int E, int top_k,
                                  int shared_I, moe_dtype dt) {
  const size_t bad = (size_t)-1;
  if (!dtype_ok(dt) || check_dims(H, I, E, top_k) != MOE_OK || I == 0 || T < 0 ||
      !rows_ok((long long)T * top_k) || shared_I < 0 || shared_I % 64 != 0)
    return bad;
  const LayerWs w = layer_ws(nullptr, T, H, I, E, top_k, dt, shared_I);
  switch (piece) {
    case MOE_LAYER_WS_OFFSETS: return w.at_offsets;
    case MOE_LAYER_WS_SORTED_TOKEN: return w.at_sorted_token;
    case MOE_LAYER_WS_SORTED_SLOT: return w.at_sorted_slot;
    case MOE_LAYER_WS_SLOT_POS: return w.at_slot_pos;
    case MOE_LAYER_WS_EXPERT_OUT: return w.at_y;
    default: return bad;
  }
}

int moe_route_cfg(const void* x, const void* wr, const float* bias, int T, int H, int E, int k,
                  int norm, moe_dtype dt, const moe_router_config* cfg, float* logits,
                  int32_t* ids, float* w, int32_t* counts, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (T < 0 || !rows_ok(T) || E < 1 || E > kMaxE || k < 1 || k > E || H <= 0 || H % 64 != 0)
    return MOE_ERR_SHAPE;
  RouterVariant rv;
  const RouterVariant* var = nullptr;
  const int st = router_variant(cfg, E, k, &rv, &var);
  if (st != MOE_OK) return st;
  if (T > 0 && (!x || !wr || !ids || !w)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(wr)) return MOE_ERR_ALIGN;
  return hip_status(launch_route(dt == MOE_BF16, x, wr, bias, T, H, E, k, norm, logits, ids, w,
                                 counts, s, var));
}

int moe_route(const void* x, const void* wr, const float* bias, int T, int H, int E, int k,
              int norm, moe_dtype dt, float* logits, int32_t* ids, float* w, int32_t* counts,
              hipStream_t s) {
  return moe_route_cfg(x, wr, bias, T, H, E, k, norm, dt, nullptr, logits, ids, w, counts, s);
}

int moe_update_expert_bias(float* bias, float* tpe, int E, float lr, int nrec, hipStream_t s) {
  if (E < 1 || E > kMaxE || nrec < 1 || !std::isfinite(lr)) return MOE_ERR_SHAPE;
  if (!bias || !tpe) return MOE_ERR_NULL;
  return hip_status(launch_update_expert_bias(bias, tpe, E, lr, nrec, s));
}

int moe_permute(const int32_t* ids, int T, int k, const int32_t* C, int R, int N, int E,
                int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* sorted_slot,
                int32_t* slot_pos, void* ws, size_t ws_bytes, hipStream_t s) {
  if (E < 1 || E > kMaxE) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if ((ids == nullptr) == (C == nullptr)) return MOE_ERR_NULL;
  if (ids) {
    if (T < 0 || k < 1 || k > E || !rows_ok((long long)T * k)) return MOE_ERR_SHAPE;
    const int n = T * k;
    if (n > 0 && (!sorted_token || !slot_pos)) return MOE_ERR_NULL;
    const size_t need = permute_ws_bytes(n, E, 0);
    if (n > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_permute_topk(ids, T, k, E, counts, offsets, sorted_token,
                                          sorted_slot, slot_pos, ws, s));
  }
  if (R < 1 || (long long)R * E > kMaxRankMajorBlocks || !rows_ok(N)) return MOE_ERR_SHAPE;
  if (N > 0 && (!sorted_token || !slot_pos)) return MOE_ERR_NULL;
  if (!ws || ws_bytes < permute_ws_bytes(N, E, R)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute_rank_major(C, R, N, E, counts, offsets, sorted_token,
                                              sorted_slot, slot_pos, ws, s));
}

int moe_gather_rows(const void* x, int x_rows, const int32_t* idx, int N, int H, moe_dtype dt,
                    void* out, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (N < 0 || !rows_ok(N) || x_rows < 0 || H <= 0 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (N > 0 && (!x || !idx || !out)) return MOE_ERR_NULL;
  if (N > 0 && x_rows < 1) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_ALIGN;
  return hip_status(launch_gather_rows(dt == MOE_BF16, x, x_rows, idx, N, H, out, s));
}

int moe_grouped_gate_up_swiglu(const void* x, int x_rows, const int32_t* row_index,
                               const int32_t* offsets, int N, int H, int I, int E,
                               const void* gate_up, moe_dtype dt, void* h, void* ws,
                               size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, I, E, 1) != MOE_OK || I == 0 || !rows_ok(N) || x_rows < 0)
    return MOE_ERR_SHAPE;
  if (N == 0) return MOE_OK;
  if (x_rows < 1) return MOE_ERR_SHAPE;
  if (!x || !offsets || !gate_up || !h) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(gate_up) || !aligned16(h)) return MOE_ERR_ALIGN;
  const bool bf16 = dt == MOE_BF16;
  const GemmTileCfg c = pick_gate_up_cfg(bf16, N, H, I, E);
  if (!ws || ws_bytes < tile_list_bytes(N, E, c.BM)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_gate_up(bf16, c, x, x_rows, row_index, offsets, N, H, I, E, gate_up,
                                   h, ws, false, s));
}

int moe_grouped_down(const void* h, const int32_t* offsets, const int32_t* out_index, int N,
                     int H, int I, int E, const void* down, moe_dtype dt, void* y, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, I, E, 1) != MOE_OK || I == 0 || !rows_ok(N)) return MOE_ERR_SHAPE;
  if (N == 0) return MOE_OK;
  if (!h || !offsets || !down || !y) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(down) || !aligned16(y)) return MOE_ERR_ALIGN;
  const bool bf16 = dt == MOE_BF16;
  const GemmTileCfg c = pick_down_cfg(bf16, N, H, I, E);
  if (!ws || ws_bytes < tile_list_bytes(N, E, c.BM)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_down(bf16, c, h, offsets, out_index, N, H, I, E, down, y, ws, false, s));
}

int moe_grouped_swiglu(const void* x, int x_rows, const int32_t* row_index,
                       const int32_t* out_index, const int32_t* offsets, int N, int H, int I,
                       int E, const void* gate_up, const void* down, moe_dtype dt, void* y,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, I, E, 1) != MOE_OK || I == 0 || !rows_ok(N) || x_rows < 0)
    return MOE_ERR_SHAPE;
  if (N == 0) return MOE_OK;
  if (x_rows < 1) return MOE_ERR_SHAPE;
  if (!x || !offsets || !gate_up || !down || !y) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(gate_up) || !aligned16(down) || !aligned16(y))
    return MOE_ERR_ALIGN;
  size_t hb, ub;
  const size_t need = swiglu_ws(N, H, I, E, dt, &hb, &ub);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const bool bf16 = dt == MOE_BF16;
  char* base = (char*)ws;
  void* h = base;
  const GemmTileCfg cu = pick_gate_up_cfg(bf16, N, H, I, E);
  const GemmTileCfg cd = pick_down_cfg(bf16, N, H, I, E);
  hipError_t e = launch_gate_up(bf16, cu, x, x_rows, row_index, offsets, N, H, I, E, gate_up, h,
                                base + hb, false, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_down(bf16, cd, h, offsets, out_index, N, H, I, E, down, y,
                                base + hb + ub, false, s));
}

int moe_combine(const void* y, const int32_t* slot_pos, const float* w, int T, int k, int H,
                moe_dtype dt, void* out, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (T < 0 || k < 1 || !rows_ok((long long)T * k) || H <= 0 || H % 8 != 0)
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !out) return MOE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out)) return MOE_ERR_ALIGN;
  return hip_status(launch_combine(dt == MOE_BF16, y, slot_pos, w, T, k, H, nullptr, out, s));
}

int moe_shared_expert_forward(const void* x, const void* gate_up, const void* down, int T,
                              int H, int Is, moe_dtype dt, void* out, void* ws, size_t ws_bytes,
                              hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, Is, 1, 1) != MOE_OK || Is == 0 || T < 0 || !rows_ok(T)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !gate_up || !down || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(gate_up) || !aligned16(down) || !aligned16(out))
    return MOE_ERR_ALIGN;
  if (!ws || ws_bytes < shared_ws(nullptr, T, H, Is, dt, false).total) return MOE_ERR_WORKSPACE;
  const SharedWs w = shared_ws((char*)ws, T, H, Is, dt, false);
  return hip_status(run_shared(dt == MOE_BF16, x, gate_up, down, T, H, Is, w, out, s));
}

}  // extern "C"

namespace {

// The layer forward.  g_save / y_out (training forward): also keep the
// gate/up pre-activations [N, 2I] in expert-major order and write the expert
// outputs [N, H] (flat slot order) to the caller's buffer.
int layer_forward_impl(const void* x, const void* wr, const float* bias, const void* gate_up,
                       const void* down, int T, int H, int I, int E, int k, int norm,
                       moe_dtype dt, const moe_router_config* cfg,
                       const moe_shared_expert* shared, void* out, float* logits, int32_t* ids,
                       float* weights, int32_t* counts, void* g_save, void* y_out,
                       void* g_save_shared, void* ws, size_t ws_bytes,
                       hipEvent_t* stage_events, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, I, E, k) != MOE_OK || I == 0 || T < 0 || !rows_ok((long long)T * k))
    return MOE_ERR_SHAPE;
  RouterVariant rv;
  const RouterVariant* var = nullptr;
  const int st = router_variant(cfg, E, k, &rv, &var);
  if (st != MOE_OK) return st;
  const int Is = shared ? shared->intermediate_size : 0;
  if (shared && (Is <= 0 || Is % 64 != 0)) return MOE_ERR_SHAPE;
  if (T > 0 && (!x || !wr || !gate_up || !down || !out)) return MOE_ERR_NULL;
  if (T > 0 && shared && (!shared->gate_up || !shared->down)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(wr) || !aligned16(gate_up) || !aligned16(down) ||
      !aligned16(out))
    return MOE_ERR_ALIGN;
  if (shared && (!aligned16(shared->gate_up) || !aligned16(shared->down))) return MOE_ERR_ALIGN;
  const size_t need = layer_ws(nullptr, T, H, I, E, k, dt, Is).total;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const bool bf16 = dt == MOE_BF16;
  const int N = T * k;
  const GemmTileCfg cu = pick_gate_up_cfg(bf16, N, H, I, E);
  const GemmTileCfg cd = pick_down_cfg(bf16, N, H, I, E);
  // the shared expert runs inside the grouped launches when both are LDS
  // configs and its widths fit their tiles
  const bool fusable = shared && T > 0 && lds_cfg_id(cu.id) && lds_cfg_id(cd.id) &&
                       Is % (cu.BN / 2) == 0 && H % cd.BN == 0;
  if (g_save_shared && shared && T > 0 && !fusable) return MOE_ERR_UNSUPPORTED;
  LayerWs w = layer_ws((char*)ws, T, H, I, E, k, dt, Is);
  if (!ids) ids = w.ids;
  if (!weights) weights = w.weights;
  if (!counts) counts = w.counts;
  if (!logits) logits = w.logits;
  auto mark = [&](int i) {
    if (stage_events && stage_events[i]) (void)hipEventRecord(stage_events[i], s);
  };
  mark(0);
  // the histogram comes from the permutation pass, so the router skips it.
  // On the split-K router path its selection kernel also runs the
  // permutation's first pass (ranks and block histograms).
  const bool fold_on = route_can_fold(T, H, E, k, bf16) && w.route_parts_bytes > 0;
  const PermuteFold fold = fold_on ? permute_fold_scratch(w.perm, T, k, E) : PermuteFold{};
  hipError_t e = launch_route(bf16, x, wr, bias, T, H, E, k, norm, logits, ids, weights, nullptr,
                              s, var, w.route_parts, w.route_parts_bytes,
                              fold_on ? &fold : nullptr);
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(1);
  // the permutation's scan pass also writes both GEMMs' tile lists (one
  // list when their row tiles have the same height)
  const bool one_list = cu.BM == cd.BM;
  void* const tiles_down = one_list ? w.tiles_up : w.tiles_down;
  e = launch_permute_topk(ids, T, k, E, counts, w.offsets, w.sorted_token, w.sorted_slot,
                          w.slot_pos, w.perm, s, w.tiles_up, cu.BM,
                          one_list ? nullptr : w.tiles_down, cd.BM, fold_on ? &fold : nullptr);
  if (e != hipSuccess) return MOE_ERR_HIP;
  mark(2);
  // The shared expert (MindSpore moe.py, MoE.forward) sees every token and
  // its output joins the combine's float32 sum.  On the LDS kernels it runs
  // as a dense second problem inside the two grouped launches, so its tiles
  // share the machine with the experts' instead of running on their own.
  DenseAux aux_up{}, aux_down{};
  bool fused = false;
  if (fusable) {
    aux_up = dense_aux(cu, true, x, H, shared->gate_up, 2 * Is, H, Is, w.h_s, Is, T, Is);
    aux_up.g_save = g_save_shared;
    aux_down = dense_aux(cd, false, w.h_s, Is, shared->down, H, Is, 0, w.y_s, H, T, H);
    fused = aux_up.jobs > 0 && aux_down.jobs > 0;
  }
  void* y = y_out ? y_out : w.y;
  if (N > 0) {
    e = launch_gate_up(bf16, cu, x, T, w.sorted_token, w.offsets, N, H, I, E, gate_up, w.h,
                       w.tiles_up, true, s, fused ? &aux_up : nullptr, g_save);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  mark(3);
  // outputs land in flat-slot order (row t * k + j), so the combine reads each
  // token's k rows contiguously.
  if (N > 0) {
    e = launch_down(bf16, cd, w.h, w.offsets, w.sorted_slot, N, H, I, E, down, y,
                    tiles_down, true, s, fused ? &aux_down : nullptr);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  mark(4);
  if (shared && T > 0 && !fused) {
    const SharedWs sw{w.h_s, w.y_s, w.tiles_s_up, w.tiles_s_down, 0};
    e = run_shared(bf16, x, shared->gate_up, shared->down, T, H, Is, sw, w.y_s, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  e = launch_combine(bf16, y, nullptr, weights, T, k, H, shared ? w.y_s : nullptr, out, s);
  mark(5);
  return hip_status(e);
}

}  // namespace

extern "C" {

int moe_layer_forward_ex(const void* x, const void* wr, const float* bias, const void* gate_up,
                         const void* down, int T, int H, int I, int E, int k, int norm,
                         moe_dtype dt, const moe_router_config* cfg,
                         const moe_shared_expert* shared, void* out, float* logits, int32_t* ids,
                         float* weights, int32_t* counts, void* ws, size_t ws_bytes,
                         hipEvent_t* stage_events, hipStream_t s) {
  return layer_forward_impl(x, wr, bias, gate_up, down, T, H, I, E, k, norm, dt, cfg, shared, out,
                            logits, ids, weights, counts, nullptr, nullptr, nullptr, ws, ws_bytes,
                            stage_events, s);
}

int moe_layer_forward_train(const void* x, const void* wr, const float* bias,
                            const void* gate_up, const void* down, int T, int H, int I, int E,
                            int k, int norm, moe_dtype dt, const moe_router_config* cfg,
                            const moe_shared_expert* shared, void* out, float* logits,
                            int32_t* ids, float* weights, int32_t* counts,
                            const moe_train_saved* saved, void* ws, size_t ws_bytes,
                            hipEvent_t* stage_events, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (dt != MOE_BF16 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (shared && shared->intermediate_size % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!saved) return MOE_ERR_NULL;
  if (T > 0 && (!saved->gate_up_out || !saved->expert_out || !logits || !ids || !weights))
    return MOE_ERR_NULL;
  if (T > 0 && shared && !saved->shared_gate_up_out) return MOE_ERR_NULL;
  if (!aligned16(saved->gate_up_out) || !aligned16(saved->expert_out) ||
      !aligned16(saved->shared_gate_up_out))
    return MOE_ERR_ALIGN;
  return layer_forward_impl(x, wr, bias, gate_up, down, T, H, I, E, k, norm, dt, cfg, shared,
                            out, logits, ids, weights, counts, saved->gate_up_out,
                            saved->expert_out, shared ? saved->shared_gate_up_out : nullptr, ws,
                            ws_bytes, stage_events, s);
}

int moe_layer_backward(const void* x, const void* wr, const void* gate_up, const void* down,
                       int T, int H, int I, int E, int k, int norm, moe_dtype dt,
                       const moe_router_config* cfg, const moe_shared_expert* shared,
                       const float* logits, const int32_t* ids, const float* weights,
                       const moe_train_saved* saved, const void* dout,
                       const moe_layer_grads* grads, void* ws, size_t ws_bytes,
                       hipEvent_t* stage_events, hipStream_t s) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (check_dims(H, I, E, k) != MOE_OK || I == 0 || T < 0 || !rows_ok((long long)T * k))
    return MOE_ERR_SHAPE;
  if (dt != MOE_BF16 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int Is = shared ? shared->intermediate_size : 0;
  if (shared && (Is <= 0 || Is % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  RouterVariant rv;
  const RouterVariant* var = nullptr;
  const int vst = router_variant(cfg, E, k, &rv, &var);
  if (vst != MOE_OK) return vst;
  const int sigmoid = var ? var->sigmoid : 0;
  const float scale = var ? var->scale : 1.0f;
  // dL is zero off the selection for renormalised or sigmoid scores
  const int sparse = (norm || sigmoid) ? 1 : 0;
  if (!saved || !grads) return MOE_ERR_NULL;
  const moe_layer_grads& g = *grads;
  if (T > 0 && (!x || !wr || !gate_up || !down || !logits || !ids || !weights ||
                !saved->gate_up_out || !dout || !g.dx || !g.d_router_weight || !g.d_gate_up ||
                !g.d_down))
    return MOE_ERR_NULL;
  if (T > 0 && shared && (!shared->gate_up || !shared->down || !saved->shared_gate_up_out ||
                          !g.d_shared_gate_up || !g.d_shared_down))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(wr) || !aligned16(gate_up) || !aligned16(down) ||
      !aligned16(saved->gate_up_out) || !aligned16(dout) ||
      !aligned16(g.dx) || !aligned16(g.d_router_weight) || !aligned16(g.d_gate_up) ||
      !aligned16(g.d_down))
    return MOE_ERR_ALIGN;
  if (shared && (!aligned16(shared->gate_up) || !aligned16(shared->down) ||
                 !aligned16(saved->shared_gate_up_out) || !aligned16(g.d_shared_gate_up) ||
                 !aligned16(g.d_shared_down)))
    return MOE_ERR_ALIGN;
  const size_t need = bwd_ws(nullptr, T, H, I, E, k, dt, Is).total;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const BwdWs w = bwd_ws((char*)ws, T, H, I, E, k, dt, Is);
  const bool bf16 = true;
  const int N = T * k;
  float* dw = g.d_topk_weights ? g.d_topk_weights : w.dw;
  const int id = pick_dgrad_cfg(N, E);
  const int id1 = pick_dgrad1_cfg(N, E);
  auto mark = [&](int i) {
    if (stage_events && stage_events[i]) (void)hipEventRecord(stage_events[i], s);
  };
  mark(0);
  hipError_t e = launch_permute_topk(ids, T, k, E, w.counts, w.offsets, w.sorted_token,
                                     w.sorted_slot, w.slot_pos, w.perm, s, w.tiles, dgrad_bm(id),
                                     w.tiles1, dgrad_bm(id1));
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (T == 0) {
    // no tokens: every weight gradient is zero
    e = launch_fill_u32(g.d_router_weight, (long long)E * H, 0u, s);
    if (e == hipSuccess && g.d_router_bias) e = launch_fill_u32(g.d_router_bias, E, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(g.d_gate_up, (long long)E * H * I, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(g.d_down, (long long)E * I * H / 2, 0u, s);
    if (e == hipSuccess && shared)
      e = launch_fill_u32(g.d_shared_gate_up, (long long)H * Is, 0u, s);
    if (e == hipSuccess && shared)
      e = launch_fill_u32(g.d_shared_down, (long long)Is * H / 2, 0u, s);
    return hip_status(e);
  }
  e = launch_fill_u32(w.zero, (long long)(w.zero_bytes / 4), 0u, s);
  if (e == hipSuccess && shared) {
    // offsets {0, T}: the shared expert as one group, for its wgrads when
    // they run on their own
    e = launch_fill_u32(w.offs_s, 1, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32(w.offs_s + 1, 1, (uint32_t)T, s);
  }
  mark(1);
  // dgrad: SwiGLU backward in the first GEMM's epilogue, then dX in slot
  // order.  The shared expert (weight 1 on every token) runs inside the same
  // launches (the first one's 128-column tiles fit any Is multiple of 128).
  // The first epilogue also leaves d_weights = <dout, y> = <dout . down^T, h>
  // in column-slice partials, which are added up before the softmax /
  // router gradient.
  const bool dfold = shared != nullptr;
  const DgradShared dsh{shared ? shared->gate_up : nullptr, shared ? shared->down : nullptr,
                        saved->shared_gate_up_out, w.dG_s, w.hw_s, w.dx_s, T, Is};
  if (e == hipSuccess)
    e = launch_dgrad_down_swiglu(id1, dout, T, w.sorted_token, down, N, H, I, E,
                                 saved->gate_up_out, weights, w.sorted_slot, w.dG, w.hw, w.tiles1,
                                 s, dfold ? &dsh : nullptr, w.dw_parts);
  if (e == hipSuccess)
    e = launch_weight_grad(w.dw_parts, dgrad1_weight_parts(I), w.slot_pos, N, dw, s);
  if (e == hipSuccess)
    e = launch_router_grad(logits, ids, weights, dw, w.slot_pos, T, E, k, norm, sigmoid, scale,
                           w.dL, w.dl_perm, s);
  mark(2);
  if (e == hipSuccess)
    e = launch_dgrad_gate_up(id, w.dG, gate_up, N, H, I, E, w.sorted_slot, w.dX, w.tiles, s,
                             dfold ? &dsh : nullptr);
  if (e == hipSuccess)
    e = launch_input_grad(bf16, w.dX, w.dL, sparse ? ids : nullptr, wr, T, k, E, H,
                          shared ? w.dx_s : nullptr, g.dx, s);
  mark(3);
  // wgrad: d down[e] = (w h)_e^T dout_e, d gate_up[e] = X_e^T dG_e, with
  // the gathered rows laid out expert-major first
  if (e == hipSuccess) e = launch_gather_rows(bf16, dout, T, w.sorted_token, N, H, w.dout_perm, s);
  if (e == hipSuccess) e = launch_gather_rows(bf16, x, T, w.sorted_token, N, H, w.x_perm, s);
  // the shared expert's weight gradients (h_s^T dout and x^T dG_s) run
  // inside these launches when their tiles fit, else on their own below
  const bool fold = shared && wgrad_can_fold(I, H, Is, H) && wgrad_can_fold(H, 2 * I, H, 2 * Is);
  const WgradAux aux_dn{w.hw_s, Is, dout, H, T, Is, H, g.d_shared_down, 0};
  const WgradAux aux_gu{x, H, w.dG_s, 2 * Is, T, H, 2 * Is, g.d_shared_gate_up, 0};
  if (e == hipSuccess)
    e = launch_wgrad(w.hw, I, w.dout_perm, H, w.zero, w.offsets, E, I, H, g.d_down, s,
                     fold ? &aux_dn : nullptr, w.counters);
  mark(4);
  if (e == hipSuccess)
    e = launch_wgrad(w.x_perm, H, w.dG, 2 * I, w.zero, w.offsets, E, H, 2 * I, g.d_gate_up, s,
                     fold ? &aux_gu : nullptr, w.counters + kWgradCounters);
  mark(5);
  if (e == hipSuccess)
    e = launch_router_weight_grad(bf16, x, w.sorted_token, w.dL, w.dl_perm, w.offsets, T, E, H,
                                  sparse, g.d_router_weight, g.d_router_bias, w.rw_part, s);
  if (e == hipSuccess && shared && !fold)
    e = launch_wgrad(w.hw_s, Is, dout, H, w.zero, w.offs_s, 1, Is, H, g.d_shared_down, s);
  if (e == hipSuccess && shared && !fold)
    e = launch_wgrad(x, H, w.dG_s, 2 * Is, w.zero, w.offs_s, 1, H, 2 * Is, g.d_shared_gate_up, s);
  mark(6);
  return hip_status(e);
}

int moe_layer_forward_cfg(const void* x, const void* wr, const float* bias,
                          const void* gate_up, const void* down, int T, int H, int I, int E,
                          int k, int norm, moe_dtype dt, const moe_router_config* cfg, void* out,
                          float* logits, int32_t* ids, float* weights, int32_t* counts, void* ws,
                          size_t ws_bytes, hipEvent_t* stage_events, hipStream_t s) {
  return moe_layer_forward_ex(x, wr, bias, gate_up, down, T, H, I, E, k, norm, dt, cfg, nullptr,
                              out, logits, ids, weights, counts, ws, ws_bytes, stage_events, s);
}

int moe_layer_forward(const void* x, const void* wr, const float* bias, const void* gate_up,
                      const void* down, int T, int H, int I, int E, int k, int norm,
                      moe_dtype dt, void* out, float* logits, int32_t* ids, float* weights,
                      int32_t* counts, void* ws, size_t ws_bytes, hipEvent_t* stage_events,
                      hipStream_t s) {
  return moe_layer_forward_cfg(x, wr, bias, gate_up, down, T, H, I, E, k, norm, dt, nullptr, out,
                               logits, ids, weights, counts, ws, ws_bytes, stage_events, s);
}

}  // extern "C"

// ---- the entry point that allocates nothing --------------------------------
//
// Its workspace is one file-scope device array of MOE_STATIC_SCRATCH_BYTES.
// Each GPU the library runs on holds its own copy (at its own address) until
// the process ends.  Host code never uses the array's name as a device
// address: the address is looked up once per device, with that device
// current, and kept in scratch_ptr[].
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const void* x, const void* wr, const float* bias,
                              const void* gate_up, const void* down, int T, int H, int I, int E,
                              int k, int norm, moe_dtype dt, const moe_router_config* cfg,
                              const moe_shared_expert* shared, void* out, float* logits,
                              int32_t* ids, float* weights, int32_t* counts,
                              hipEvent_t* stage_events, hipStream_t s) {
  // sizes first: invalid ones fall through to the full validation below,
  // valid ones that do not fit the array are refused before anything runs
  const int Is = shared ? shared->intermediate_size : 0;
  const long long N = (long long)T * k;
  const size_t need = (N >= 0 && N <= (1ll << 30))
                          ? moe_workspace_size(MOE_OP_LAYER, T, H, I, E, k, Is, (int)N, dt)
                          : (size_t)-1;
  if (need != (size_t)-1 && need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = current_scratch(&ws);
  if (st != MOE_OK) return st;
  return layer_forward_impl(x, wr, bias, gate_up, down, T, H, I, E, k, norm, dt, cfg, shared,
                            out, logits, ids, weights, counts, nullptr, nullptr, nullptr, ws,
                            (size_t)MOE_STATIC_SCRATCH_BYTES, stage_events, s);
}

}  // extern "C"
