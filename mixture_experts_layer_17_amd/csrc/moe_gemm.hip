// Grouped GEMMs of the expert FFN on MFMA (bf16 in, float32 accumulate).
//
// Semantics: Qwen3-Omni issue #115, SpeedupMoeExperts.forward
//   gate_up = x_e @ gate_up_proj[e]        ([n_e, H] x [H, 2I])
//   h       = up * silu(gate)               (gate = first I columns)
//   y_e     = h @ down_proj[e]              ([n_e, I] x [I, H])
// over the rows of each expert in expert-major order (MindSpore moe.py,
// _run_experts_for_loop: groups split by the per-expert counts, empty
// groups skipped).
//
// Design (gfx950):
//   * A device-side tile list maps each M-tile (BM rows of one expert) to
//     (expert, first row, rows); it is built from the expert offsets on the
//     device, so no count ever travels to the host.  The grid is sized from
//     the host-known bound floor(N / BM) + E tiles; surplus workgroups exit.
//   * Workgroup -> tile mapping is XCD-aware: hardware deals workgroups to the
//     8 XCDs round-robin, so workgroup b runs on XCD b % 8.  Jobs are cut into
//     8 contiguous ranges, one per XCD, so the N-tiles of one M-tile and the
//     M-tiles of one expert share an L2.
//   * A rows are gathered on load through the row index (the token
//     permutation is never materialised).  Both operands are staged in LDS,
//     double-buffered, in a [row][k] layout with 16-byte slots XOR-swizzled
//     by (row ^ row >> 3) & 7, which keeps the MFMA operand reads free of
//     bank conflicts.
//   * The weights are stored [K, N] (N contiguous) but the MFMA B operand
//     wants 8 consecutive k per lane, so each thread loads an 8(k) x 8(n)
//     block with eight 16-byte row loads and transposes it in registers on
//     its way into LDS.
//   * SwiGLU: a workgroup's B tile holds gate columns [n0, n0 + BN/2) and the
//     matching up columns [I + n0, ...); a wave's gate and up accumulators
//     have the same lane layout, so silu(g) * u is formed in registers.
#include "moe_common.h"
#include "moe_internal.h"
#include "moe_tiles.h"

namespace moe {
namespace {

constexpr int NUM_XCD = 8;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// One block builds the M-tile list from the expert offsets.
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int N, int BM,
                                                          int4* __restrict__ tiles,
                                                          int32_t* __restrict__ tiles_count) {
  __shared__ int s_nt[256];
  __shared__ int s_start[257];
  const int e = threadIdx.x;
  int lo = 0, hi = 0;
  if (e < E && offsets) {
    lo = min(max(offsets[e], 0), N);
    hi = min(max(offsets[e + 1], lo), N);
  } else if (e == 0) {
    hi = N;  // no offsets: one group of all N rows
  }
  build_tile_list(E, lo, hi, BM, tiles, tiles_count, s_nt, s_start);
}

// Bytes of 16-byte slots per LDS row: BK elements.
template <typename T, int BK> struct lds_geom {
  static constexpr int SLOTS = BK * (int)sizeof(T) / 16;  // 16-byte slots per row
  static constexpr int SPC = (int)sizeof(T) / 2;          // slots per 8-element chunk
  static_assert(SLOTS == 8, "rows are 128 bytes");
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWIGLU>
struct gemm_cfg {
  static constexpr int THREADS = 256;
  static constexpr int SLOTS = lds_geom<T, BK>::SLOTS;
  static constexpr int SPC = lds_geom<T, BK>::SPC;
  static constexpr int WROWS = BM / WM;                  // rows per wave
  static constexpr int TM = WROWS / 16;                  // 16-row MFMA tiles per wave
  static constexpr int WCOLS = SWIGLU ? (BN / 2) / WN : BN / WN;  // out cols per wave
  static constexpr int TNO = WCOLS / 16;                 // output 16-col tiles per wave
  static constexpr int TN = SWIGLU ? 2 * TNO : TNO;      // B 16-col tiles per wave
  static constexpr int A_SLOTS = BM * SLOTS;             // 16-byte slots per A stage
  static constexpr int A_PER_THREAD = (A_SLOTS + THREADS - 1) / THREADS;
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);   // 8x8 blocks per B stage
  static constexpr int B_PER_THREAD = (B_BLOCKS + THREADS - 1) / THREADS;
  static constexpr int KSUB = BK / 32;                   // MFMA k-steps per stage
  static constexpr int LDS_A = BM * SLOTS * 16;          // bytes per stage
  static constexpr int LDS_B = BN * SLOTS * 16;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM >= 1 && TNO >= 1, "wave tile at least 16 x 16");
  static_assert(WROWS % 16 == 0 && WCOLS % 16 == 0, "wave tile multiple of 16");
};

// Reads the 8-element chunk `chunk` of LDS row `row` (one or two 16-byte slots).
template <typename T, int SLOTS>
__device__ __forceinline__ chunk8<T> lds_chunk(const u32x4* base, int row, int chunk) {
  chunk8<T> c;
  if constexpr (sizeof(T) == 2) {
    c.v = base[row * SLOTS + (chunk ^ swz(row))];
  } else {
    c.lo = base[row * SLOTS + ((2 * chunk) ^ swz(row))];
    c.hi = base[row * SLOTS + ((2 * chunk + 1) ^ swz(row))];
  }
  return c;
}

// Writes one 8(k) x 8(n) block of B, held as 8 rows of 8 elements, into LDS
// transposed: LDS row n = 8 nb + c receives the 8 k values of column c.
template <typename T, int SLOTS>
__device__ __forceinline__ void store_b_block(u32x4* sb, const u32x4* rows, int kb, int nb) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int n = 8 * nb + c;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = reinterpret_cast<const uint32_t*>(&rows[2 * i])[c >> 1];
        const uint32_t hi = reinterpret_cast<const uint32_t*>(&rows[2 * i + 1])[c >> 1];
        o[i] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      sb[n * SLOTS + (kb ^ swz(n))] = u32x4{o[0], o[1], o[2], o[3]};
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int n = 8 * nb + c;
      uint32_t o[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        o[r] = reinterpret_cast<const uint32_t*>(&rows[r * 2 + (c >> 2)])[c & 3];
      sb[n * SLOTS + ((2 * kb) ^ swz(n))] = u32x4{o[0], o[1], o[2], o[3]};
      sb[n * SLOTS + ((2 * kb + 1) ^ swz(n))] = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const T* __restrict__ A, int lda, const int32_t* __restrict__ a_index, int a_rows,
    const T* __restrict__ B, long long b_estride, int ldb, int K, int up_off,
    T* __restrict__ C, int ldc, const int32_t* __restrict__ c_index, int c_rows,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tiles_count, int n_ntiles) {
  using G = gemm_cfg<T, BM, BN, BK, WM, WN, SWIGLU>;
  constexpr int SLOTS = G::SLOTS;
  constexpr int SPC = G::SPC;
  constexpr int EPS = 16 / (int)sizeof(T);  // elements per 16-byte slot

  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* sA = reinterpret_cast<u32x4*>(smem);                     // [2][BM][SLOTS]
  u32x4* sB = reinterpret_cast<u32x4*>(smem + 2 * G::LDS_A);      // [2][BN][SLOTS]

  // ---- job (M-tile, N-tile) for this workgroup, XCD-aware
  const int jobs = tiles_count[0] * n_ntiles;
  const int per_xcd = (jobs + NUM_XCD - 1) / NUM_XCD;
  const int xcd = blockIdx.x % NUM_XCD;
  const int local = blockIdx.x / NUM_XCD;
  if (local >= per_xcd) return;
  const int job = xcd * per_xcd + local;
  if (job >= jobs) return;
  const int mt = job / n_ntiles;
  const int nt = job - mt * n_ntiles;
  const int4 tile = tiles[mt];
  const int e = tile.x, row0 = tile.y, rows = tile.z;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, r16 = lane & 15;

  const T* Be = B + (long long)e * b_estride;
  const int n0 = SWIGLU ? nt * (BN / 2) : nt * BN;

  // ---- per-thread load assignments (fixed over K)
  // A: 16-byte slot q = tid + u * THREADS of the BM x BK tile (row q / SLOTS)
  constexpr bool A_PARTIAL = (G::A_SLOTS % G::THREADS) != 0;
  constexpr bool B_PARTIAL = (G::B_BLOCKS % G::THREADS) != 0;
  const bool a_active = !A_PARTIAL || tid < G::A_SLOTS;
  const bool b_active = !B_PARTIAL || tid < G::B_BLOCKS;
  long long a_off[G::A_PER_THREAD];
  int a_lds[G::A_PER_THREAD];
#pragma unroll
  for (int u = 0; u < G::A_PER_THREAD; ++u) {
    const int q = tid + u * G::THREADS;
    const int row = q / SLOTS, sl = q % SLOTS;
    int src = row0 + min(row, rows - 1);
    if (a_index) src = a_index[src];
    src = min(max(src, 0), a_rows - 1);
    a_off[u] = (long long)src * lda + sl * EPS;
    a_lds[u] = row * SLOTS + (sl ^ swz(row));
  }
  // B: 8x8 block (kb, nb) = tid + u * THREADS of the BK x BN tile
  long long b_off[G::B_PER_THREAD];
  int b_kb[G::B_PER_THREAD], b_nb[G::B_PER_THREAD];
#pragma unroll
  for (int u = 0; u < G::B_PER_THREAD; ++u) {
    const int q = tid + u * G::THREADS;
    const int kb = q / (BN / 8), nb = q % (BN / 8);
    int col;
    if constexpr (SWIGLU)
      col = (8 * nb < BN / 2) ? n0 + 8 * nb : up_off + n0 + (8 * nb - BN / 2);
    else
      col = n0 + 8 * nb;
    b_kb[u] = kb;
    b_nb[u] = nb;
    b_off[u] = (long long)(8 * kb) * ldb + col;
  }

  u32x4 ra[G::A_PER_THREAD];
  u32x4 rb[G::B_PER_THREAD][8 * SPC];

  f32x4_v acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int wrow0 = wm * G::WROWS;
  const bool wave_has_rows = wrow0 < rows;

  // LDS row (B-tile column n) and A row of each MFMA operand, fixed over K
  int b_row[G::TN];
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    if constexpr (SWIGLU)
      b_row[j] = j < G::TNO ? wn * G::WCOLS + 16 * j + r16
                            : BN / 2 + wn * G::WCOLS + 16 * (j - G::TNO) + r16;
    else
      b_row[j] = wn * G::WCOLS + 16 * j + r16;
  }

#define MOE_LOAD_REGS(K0)                                                              \
  do {                                                                                \
    if (a_active) {                                                                   \
      _Pragma("unroll") for (int u = 0; u < G::A_PER_THREAD; ++u)                     \
        ra[u] = *reinterpret_cast<const u32x4*>(A + a_off[u] + (K0));                 \
    }                                                                                 \
    if (b_active) {                                                                   \
      _Pragma("unroll") for (int u = 0; u < G::B_PER_THREAD; ++u)                     \
        _Pragma("unroll") for (int r = 0; r < 8; ++r)                                 \
          _Pragma("unroll") for (int h = 0; h < SPC; ++h)                             \
            rb[u][r * SPC + h] = reinterpret_cast<const u32x4*>(                       \
                Be + b_off[u] + (long long)((K0) + r) * ldb)[h];                       \
    }                                                                                 \
  } while (0)

#define MOE_STORE_LDS(STAGE)                                                           \
  do {                                                                                \
    u32x4* sa_ = sA + (STAGE) * (BM * SLOTS);                                         \
    u32x4* sb_ = sB + (STAGE) * (BN * SLOTS);                                         \
    if (a_active) {                                                                   \
      _Pragma("unroll") for (int u = 0; u < G::A_PER_THREAD; ++u) sa_[a_lds[u]] = ra[u]; \
    }                                                                                 \
    if (b_active) {                                                                   \
      _Pragma("unroll") for (int u = 0; u < G::B_PER_THREAD; ++u)                     \
        store_b_block<T, SLOTS>(sb_, rb[u], b_kb[u], b_nb[u]);                        \
    }                                                                                 \
  } while (0)

  const int KT = K / BK;
  MOE_LOAD_REGS(0);
  MOE_STORE_LDS(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) MOE_LOAD_REGS((kt + 1) * BK);
    if (wave_has_rows) {
      const u32x4* sa = sA + cur * (BM * SLOTS);
      const u32x4* sb = sB + cur * (BN * SLOTS);
#pragma unroll
      for (int ks = 0; ks < G::KSUB; ++ks) {
        chunk8<T> fa[G::TM], fb[G::TN];
        const int chunk = ks * 4 + g;
#pragma unroll
        for (int i = 0; i < G::TM; ++i) fa[i] = lds_chunk<T, SLOTS>(sa, wrow0 + 16 * i + r16, chunk);
#pragma unroll
        for (int j = 0; j < G::TN; ++j) fb[j] = lds_chunk<T, SLOTS>(sb, b_row[j], chunk);
#pragma unroll
        for (int i = 0; i < G::TM; ++i)
#pragma unroll
          for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma_16x16x32(fa[i], fb[j], acc[i][j]);
      }
    }
    if (kt + 1 < KT) MOE_STORE_LDS(cur ^ 1);
    __syncthreads();
  }
#undef MOE_LOAD_REGS
#undef MOE_STORE_LDS

  // ---- epilogue
  if (!wave_has_rows) return;
  const int ocol0 = n0 + wn * G::WCOLS;
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wrow0 + 16 * i + 4 * g + q;
      if (row >= rows) continue;
      const int p = row0 + row;
      int dst = p;
      if (!SWIGLU && c_index) dst = c_index[p];
      if (dst < 0 || dst >= c_rows) continue;
      T* crow = C + (long long)dst * ldc + ocol0 + r16;
#pragma unroll
      for (int j = 0; j < G::TNO; ++j) {
        float v;
        if constexpr (SWIGLU) v = silu_f32(acc[i][j][q]) * acc[i][G::TNO + j][q];
        else v = acc[i][j][q];
        crow[16 * j] = elem<T>::from_f32(v);
      }
    }
  }
}

// ---------------------------------------------------------------- configs
// id -> (T, BM, BN, BK, WM, WN)
//   0: bf16 128 x 256, 2 x 2 waves (prefill)
//   1: bf16  64 x 256, 1 x 4 waves
//   2: bf16  16 x 256, 1 x 4 waves (decode)
//   3: bf16  64 x 128, 2 x 2 waves (narrow fallback)
//   4: f32   32 x 128, 2 x 2 waves, BK 32
struct CfgDesc { int BM, BN; };
constexpr CfgDesc kCfg[] = {{128, 256}, {64, 256}, {16, 256}, {64, 128}, {32, 128}};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWIGLU>
hipError_t launch_one(const void* A, int lda, const int32_t* a_index, int a_rows, const void* B,
                      long long b_estride, int ldb, int K, int up_off, void* C, int ldc,
                      const int32_t* c_index, int c_rows, const int4* tiles,
                      const int32_t* tiles_count, int n_ntiles, int grid, hipStream_t s) {
  using G = gemm_cfg<T, BM, BN, BK, WM, WN, SWIGLU>;
  constexpr int lds = 2 * (G::LDS_A + G::LDS_B);
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)grouped_gemm_kernel<T, BM, BN, BK, WM, WN, SWIGLU>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((grouped_gemm_kernel<T, BM, BN, BK, WM, WN, SWIGLU>), dim3(grid), dim3(256),
                     lds, s, (const T*)A, lda, a_index, a_rows, (const T*)B, b_estride, ldb, K,
                     up_off, (T*)C, ldc, c_index, c_rows, tiles, tiles_count, n_ntiles);
  return hipGetLastError();
}

hipError_t launch_cfg(bool swiglu, int id, const void* A, int lda, const int32_t* a_index,
                      int a_rows, const void* B, long long b_estride, int ldb, int K, int up_off,
                      void* C, int ldc, const int32_t* c_index, int c_rows, const int4* tiles,
                      const int32_t* tiles_count, int n_ntiles, int grid, hipStream_t s) {
#define MOE_ARGS A, lda, a_index, a_rows, B, b_estride, ldb, K, up_off, C, ldc, c_index, c_rows, \
                 tiles, tiles_count, n_ntiles, grid, s
#define MOE_CASE(ID, T, BM, BN, BK, WM, WN)                                            \
  case ID:                                                                           \
    return swiglu ? launch_one<T, BM, BN, BK, WM, WN, true>(MOE_ARGS)                \
                  : launch_one<T, BM, BN, BK, WM, WN, false>(MOE_ARGS);
  switch (id) {
    MOE_CASE(0, bf16_t, 128, 256, 64, 2, 2)
    MOE_CASE(1, bf16_t, 64, 256, 64, 1, 4)
    MOE_CASE(2, bf16_t, 16, 256, 64, 1, 4)
    MOE_CASE(3, bf16_t, 64, 128, 64, 2, 2)
    MOE_CASE(4, float, 32, 128, 32, 2, 2)
    default: return hipErrorInvalidValue;
  }
#undef MOE_CASE
#undef MOE_ARGS
}

GemmTileCfg make_cfg(int id) { return GemmTileCfg{kCfg[id].BM, kCfg[id].BN, id}; }

GemmTileCfg pick_cfg(bool bf16, int N, int E, int ncols_half_or_full, bool swiglu) {
  if (!bf16) return make_cfg(4);
  const int need = swiglu ? 128 : 256;  // columns per tile for the wide configs
  const bool wide = ncols_half_or_full % need == 0;
  if (!wide) return make_cfg(3);
  const double mean_rows = E > 0 ? (double)N / E : 0.0;
  if (mean_rows >= 96.0) return make_cfg(0);
  if (mean_rows >= 24.0) return make_cfg(1);
  return make_cfg(2);
}

int grid_for(int N, int E, int BM, int n_ntiles) {
  const long long max_tiles = (long long)N / BM + std::min(E, N);
  long long jobs = max_tiles * n_ntiles;
  jobs = (jobs + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
  return (int)std::max<long long>(jobs, NUM_XCD);
}

}  // namespace

hipError_t launch_build_tiles(const int32_t* offsets, int E, int N, int BM, void* tile_ws,
                              hipStream_t s) {
  build_tiles_kernel<<<1, 256, 0, s>>>(offsets, E, N, BM, (int4*)((char*)tile_ws + 256),
                                       (int32_t*)tile_ws);
  return hipGetLastError();
}

size_t tile_list_bytes(int N, int E, int BM) {
  const size_t max_tiles = (size_t)N / BM + (size_t)E + 1;
  return 256 + ((max_tiles * sizeof(int4) + 255) & ~(size_t)255);
}

GemmTileCfg pick_gate_up_cfg(bool bf16, int N, int H, int I, int E) {
  (void)H;
  if (bf16) {
    const GemmTileCfg c = pick_lds_cfg(N, E, I, true);
    if (c.id >= 0) return c;
  }
  return pick_cfg(bf16, N, E, I, true);
}

GemmTileCfg pick_dense_cfg(bool bf16, int rows, int cols, bool swiglu) {
  if (bf16) {
    const GemmTileCfg c = pick_lds_dense_cfg(rows, cols, swiglu);
    if (c.id >= 0) return c;
  }
  return pick_cfg(bf16, rows, 1, cols, swiglu);
}

GemmTileCfg pick_down_cfg(bool bf16, int N, int H, int I, int E) {
  (void)I;
  if (bf16) {
    const GemmTileCfg c = pick_lds_cfg(N, E, H, false);
    if (c.id >= 0) return c;
  }
  return pick_cfg(bf16, N, E, H, false);
}

hipError_t launch_gate_up(bool bf16, const GemmTileCfg& c, const void* x, int x_rows,
                          const int32_t* row_index, const int32_t* offsets, int N, int H, int I,
                          int E, const void* gate_up, void* h, void* tile_ws, bool tiles_ready,
                          hipStream_t s, const DenseAux* aux, void* g_save) {
  if (lds_cfg_id(c.id)) {
    if (N <= 0 && !(aux && aux->jobs > 0)) return hipSuccess;
    return launch_lds_gemm(true, c, x, H, row_index, x_rows, gate_up, (long long)H * 2 * I, 2 * I,
                           H, I, h, I, nullptr, N, offsets, N, E, I / (c.BN / 2), tile_ws,
                           tiles_ready, s, aux, g_save);
  }
  if ((aux && aux->jobs > 0) || g_save) return hipErrorInvalidValue;
  if (N <= 0) return hipSuccess;
  int32_t* count = (int32_t*)tile_ws;
  int4* tiles = (int4*)((char*)tile_ws + 256);
  if (!tiles_ready) build_tiles_kernel<<<1, 256, 0, s>>>(offsets, E, N, c.BM, tiles, count);
  const int n_ntiles = I / (c.BN / 2);
  const int grid = grid_for(N, E, c.BM, n_ntiles);
  (void)bf16;
  return launch_cfg(true, c.id, x, H, row_index, x_rows, gate_up, (long long)H * 2 * I, 2 * I,
                          H, I, h, I, nullptr, N, tiles, count, n_ntiles, grid, s);
}

hipError_t launch_down(bool bf16, const GemmTileCfg& c, const void* h, const int32_t* offsets,
                       const int32_t* out_index, int N, int H, int I, int E, const void* down,
                       void* y, void* tile_ws, bool tiles_ready, hipStream_t s,
                       const DenseAux* aux) {
  if (lds_cfg_id(c.id)) {
    if (N <= 0 && !(aux && aux->jobs > 0)) return hipSuccess;
    return launch_lds_gemm(false, c, h, I, nullptr, N, down, (long long)I * H, H, I, 0, y, H,
                           out_index, N, offsets, N, E, H / c.BN, tile_ws, tiles_ready, s, aux);
  }
  if (aux && aux->jobs > 0) return hipErrorInvalidValue;
  if (N <= 0) return hipSuccess;
  int32_t* count = (int32_t*)tile_ws;
  int4* tiles = (int4*)((char*)tile_ws + 256);
  if (!tiles_ready) build_tiles_kernel<<<1, 256, 0, s>>>(offsets, E, N, c.BM, tiles, count);
  const int n_ntiles = H / c.BN;
  const int grid = grid_for(N, E, c.BM, n_ntiles);
  (void)bf16;
  return launch_cfg(false, c.id, h, I, nullptr, N, down, (long long)I * H, H, I, 0, y, H,
                           out_index, N, tiles, count, n_ntiles, grid, s);
}

}  // namespace moe
