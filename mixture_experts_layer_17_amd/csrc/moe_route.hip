// Router: logits = x @ Wr^T (+ b) on MFMA with float32 accumulation, then a
// fused epilogue per token: float32 softmax, top-k with the lower-id tie
// rule, optional renormalisation, expert histogram.
//
// Semantics: Qwen3-Omni issue #115, SpeedupMoeSparseMoeBlock.forward (gate,
// softmax in float32, topk, divide by the top-k sum when norm_topk_prob);
// MindSpore moe.py, TokenChoiceTopKRouter.forward (gate in float32,
// bincount of the selected experts).  The top-k ranks the float32 logits;
// softmax is monotone so the selected set equals the set ranked by
// probability, and the selection depends on the logits alone.
//
// Layout: one workgroup of 8 waves per 16 tokens, each reading all of Wr.
//   * Logits: K streams through an LDS ring in blocks of 128-byte rows (the
//     16 x rows, then the E Wr rows).  Every copy instruction moves 8 whole
//     rows of 128 bytes, which the load path serves at about twice the rate
//     of MFMA-shaped loads (16 rows x 64 bytes per instruction).  Wave w
//     owns expert tiles w, w + 8 over all of K, so no partial sums are
//     combined across waves.
//   * Epilogue: each wave takes 2 tokens, 32 lanes per token, each lane
//     holding its experts as 64-bit keys (order-preserving float bits of the
//     logit, then the complemented expert id, so a larger key is a larger
//     logit or, on a tie, a lower id).  k rounds of a DPP max over the keys
//     select the top-k in order; sums for the softmax use the same fixed
//     DPP pattern, so every result is deterministic.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT_TOK = 16;     // tokens per workgroup
constexpr int RT_WAVES = 8;
constexpr int RT_SPLIT_MAX_TILES = 32;   // up to 512 tokens take the split path

// Order-preserving key: larger key <=> larger logit, or equal logits
// (IEEE equality, so -0 == +0) and a lower expert id.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                      // -0 ranks as +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t k) {
  return (int)(0xffffffffu - (uint32_t)k);
}

// DPP lane exchange within 16-lane rows.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
constexpr int DPP_QUAD_1032 = 0xb1;   // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_2301 = 0x4e;   // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROR4 = 0x124;       // row_ror:4
constexpr int DPP_ROR8 = 0x128;       // row_ror:8

// Every lane of a 16-lane row gets the row's largest key.
__device__ __forceinline__ uint64_t row_max(uint64_t k) {
  uint64_t o = dpp64<DPP_QUAD_1032>(k); k = o > k ? o : k;
  o = dpp64<DPP_QUAD_2301>(k); k = o > k ? o : k;
  o = dpp64<DPP_ROR4>(k); k = o > k ? o : k;
  o = dpp64<DPP_ROR8>(k); k = o > k ? o : k;
  return k;
}
// Row sums in a fixed pattern; lane 0 of each row holds a deterministic sum.
__device__ __forceinline__ float row_sum(float v) {
  v += __uint_as_float(dpp32<DPP_QUAD_1032>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_QUAD_2301>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_ROR4>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_ROR8>(__float_as_uint(v)));
  return v;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  return ((uint64_t)hi << 32) | lo;
}
// Sum over the 32 lanes of this lane's half-wave (rows 0-1 or 2-3).
__device__ __forceinline__ float half_sum(float v, int half) {
  v = row_sum(v);
  const float a = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float b = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 16));
  const float c = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
  const float d = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 48));
  return half ? c + d : a + b;
}

// One global->LDS copy of 16 bytes per lane: lane i's bytes land at
// lds + 16 i (lds is wave-uniform, passed in M0).  Issued from asm, with
// explicit vmcnt waits below, so the compiler does not drain every copy in
// flight before each LDS read.  It writes no registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void rt_copy16(const void* g, const unsigned char* lds) {
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_u8*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(a)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void rt_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Rows of a K block in LDS are 128 bytes (8 chunks of 16 bytes); chunk c of
// row r sits at physical chunk c ^ f(r & 15).  f was chosen by timing the
// MFMA operand reads (16 rows, lane group g reading chunks 2 g and 2 g + 1)
// against the conflict-free rate; it depends on the row within its 16-row
// group only, so x rows and every Wr tile share the same offsets.
__device__ __forceinline__ int rt_swz(int row) { return (row ^ ((row & 15) >> 3)) & 7; }

// Top-k selection, softmax and renormalisation for the 16 tokens of a
// workgroup of 8 waves, whose float32 logits are in LDS (row stride lde).
// Wave w takes rows 2 w (lanes 0-31) and 2 w + 1 (lanes 32-63); each lane
// holds the keys of experts hl, hl + 32, ... (CPL of them).  sel is LDS
// scratch of 16 * k keys.
// Largest float over the 32 lanes of this lane's half-wave.
__device__ __forceinline__ float half_max(float v, int half) {
  v = fmaxf(v, __uint_as_float(dpp32<DPP_QUAD_1032>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp32<DPP_QUAD_2301>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp32<DPP_ROR4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp32<DPP_ROR8>(__float_as_uint(v))));
  const float a = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float b = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 16));
  const float c = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
  const float d = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 48));
  return half ? fmaxf(c, d) : fmaxf(a, b);
}

// The k largest of the half-wave's keys, in descending order, into sel[0..k):
// each lane sorts its CPL keys, then k rounds take the half-wave's largest
// head key (DPP row max, then the two rows), and the one lane holding it
// advances to its next key (keys are unique).
template <int CPL>
__device__ __forceinline__ void select_keys(uint64_t (&cand)[CPL], uint64_t* sel, int k, int half,
                                            int hl) {
#pragma unroll
  for (int p = 1; p < CPL; ++p)
#pragma unroll
    for (int q = p; q > 0; --q) {
      const uint64_t lo = cand[q - 1], hi = cand[q];
      cand[q - 1] = hi > lo ? hi : lo;
      cand[q] = hi > lo ? lo : hi;
    }
  // k rounds: the half-wave's largest head key is the next selection; the one
  // lane holding it advances to its next key (keys are unique)
  for (int j = 0; j < k; ++j) {
    const uint64_t rm = row_max(cand[0]);
    const uint64_t r0 = readlane64(rm, 0), r1 = readlane64(rm, 16);
    const uint64_t r2 = readlane64(rm, 32), r3 = readlane64(rm, 48);
    const uint64_t wa = r0 > r1 ? r0 : r1, wb = r2 > r3 ? r2 : r3;
    const uint64_t win = half ? wb : wa;
    const bool pop = cand[0] == win;
#pragma unroll
    for (int c = 0; c + 1 < CPL; ++c) cand[c] = pop ? cand[c + 1] : cand[c];
    if (pop) cand[CPL - 1] = 0ull;
    if (hl == 0) sel[j] = win;
  }
}

template <int CPL>
__device__ __forceinline__ void select_tokens(const float* s_log, int lde, uint64_t* sel_base,
                                              int t0, int wave, int lane, int T_, int E, int k,
                                              int norm, int32_t* __restrict__ ids_out,
                                              float* __restrict__ w_out,
                                              int32_t* __restrict__ counts) {
  const int half = lane >> 5, hl = lane & 31;
  const int trow = 2 * wave + half;
  const int t = t0 + trow;
  const float* L = s_log + trow * lde;
  uint64_t* sel = sel_base + (size_t)trow * k;

  uint64_t cand[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = hl + 32 * c;
    cand[c] = e < E ? rank_key(L[e], e) : 0ull;
  }
  select_keys<CPL>(cand, sel, k, half, hl);
  // LDS accesses of one wave complete in order, so the keys written above
  // are visible to the reads below
  const float m = key_value(sel[0]);          // the largest logit
  float part = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = hl + 32 * c;
    if (e < E) part += expf(L[e] - m);
  }
  const float den = half_sum(part, half);
  float sp = 0.f;
  for (int jb = 0; jb < k; jb += 32) {
    const int j = jb + hl;
    if (j < k) sp += expf(key_value(sel[j]) - m);
  }
  const float selsum = half_sum(sp, half);
  if (t < T_) {
    for (int jb = 0; jb < k; jb += 32) {
      const int j = jb + hl;
      if (j < k) {
        const uint64_t key = sel[j];
        const int e = key_expert(key);
        const float num = expf(key_value(key) - m);
        ids_out[(size_t)t * k + j] = e;
        w_out[(size_t)t * k + j] = norm ? num / selsum : num / den;
        if (counts) atomicAdd(&counts[e], 1);
      }
    }
  }
}

// The router variant's epilogue (MindSpore moe.py, TokenChoiceTopKRouter:
// score function, route_scale, node-limited groups, selection-only expert
// bias).  Same lane layout as select_tokens; the token's logits row in LDS
// is overwritten with its scores; gscr holds 16 rows of E floats for the
// group maxima.
template <int CPL>
__device__ __forceinline__ void select_tokens_var(float* s_log, int lde, uint64_t* sel_base,
                                                  float* gscr, int t0, int wave, int lane,
                                                  int T_, int E, int k, int norm,
                                                  const RouterVariant& v,
                                                  int32_t* __restrict__ ids_out,
                                                  float* __restrict__ w_out,
                                                  int32_t* __restrict__ counts) {
  const int half = lane >> 5, hl = lane & 31;
  const int trow = 2 * wave + half;
  const int t = t0 + trow;
  float* L = s_log + trow * lde;
  uint64_t* sel = sel_base + (size_t)trow * k;

  // scores: sigmoid, or softmax over the experts, then times the scale
  float sc[CPL];
  if (v.sigmoid) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = hl + 32 * c;
      sc[c] = e < E ? (1.0f / (1.0f + expf(-L[e]))) * v.scale : 0.f;
    }
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = hl + 32 * c;
      if (e < E) mx = fmaxf(mx, L[e]);
    }
    mx = half_max(mx, half);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = hl + 32 * c;
      sc[c] = e < E ? expf(L[e] - mx) : 0.f;
      part += sc[c];
    }
    const float den = half_sum(part, half);
#pragma unroll
    for (int c = 0; c < CPL; ++c) sc[c] = (sc[c] / den) * v.scale;
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = hl + 32 * c;
    if (e < E) L[e] = sc[c];
  }
  // node-limited routing: group maxima, then each expert's group rank
  bool keep[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) keep[c] = true;
  if (v.groups > 0) {
    const int epg = E / v.groups;
    float* gm = gscr + trow * E;
    for (int gi = hl; gi < v.groups; gi += 32) {
      float m = -INFINITY;
      for (int q = 0; q < epg; ++q) m = fmaxf(m, L[gi * epg + q]);
      gm[gi] = m;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = hl + 32 * c;
      if (e < E) {
        const int gi = e / epg;
        const float mine = gm[gi];
        int rank = 0;
        for (int gj = 0; gj < v.groups; ++gj) {
          const float o = gm[gj];
          rank += (o > mine || (o == mine && gj < gi)) ? 1 : 0;
        }
        keep[c] = rank < v.limited;
      }
    }
  }
  uint64_t cand[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = hl + 32 * c;
    const float key = sc[c] + (v.ebias ? v.ebias[min(e, E - 1)] : 0.f);
    cand[c] = (e < E && keep[c]) ? rank_key(key, e) : 0ull;
  }
  select_keys<CPL>(cand, sel, k, half, hl);
  // weights: the unbiased scores of the selected experts
  float sp = 0.f;
  for (int jb = 0; jb < k; jb += 32) {
    const int j = jb + hl;
    if (j < k) sp += L[key_expert(sel[j])];
  }
  const float selsum = half_sum(sp, half);
  if (t < T_) {
    for (int jb = 0; jb < k; jb += 32) {
      const int j = jb + hl;
      if (j < k) {
        const int e = key_expert(sel[j]);
        const float s = L[e];
        ids_out[(size_t)t * k + j] = e;
        w_out[(size_t)t * k + j] = norm ? s / selsum : s;
        if (counts) atomicAdd(&counts[e], 1);
        if (v.tpe) atomicAdd(&v.tpe[e], 1.0f);
      }
    }
  }
}

template <typename T, int NT>
struct rcfg {
  static constexpr int KB = 128 / (int)sizeof(T);   // K elements per block (128-byte rows)
  static constexpr int ROWS = RT_TOK + NT * 16;      // x rows, then Wr rows
  static constexpr int STAGE = ROWS * 128;
  static constexpr int Q = ROWS / 8;                 // copy instructions per block (8 rows each)
  static constexpr int LDE = NT * 16 + 4;            // logits row stride (floats)
  static constexpr int LOG_BYTES = RT_TOK * LDE * 4;
  static constexpr int NS0 = (160 * 1024 - LOG_BYTES) / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;       // ring stages
  static constexpr int LDS = NS * STAGE + LOG_BYTES;
  static constexpr int CPL = (NT * 16 + 31) / 32;    // experts per lane in the epilogue
  static_assert(NS >= 2, "ring");
  static_assert(ROWS % 8 == 0, "whole copy instructions");
};

template <typename T, int NT, bool VAR>
__global__ __launch_bounds__(RT_WAVES * 64) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias,
    int T_, int H, int E, int k, int norm, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts, RouterVariant var) {
  using C = rcfg<T, NT>;
  constexpr int NS = C::NS;
  // NS ring stages of [x rows | Wr rows] x 128 bytes, then the logits
  extern __shared__ __align__(16) unsigned char smem[];
  float* s_log = reinterpret_cast<float*>(smem + NS * C::STAGE);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * RT_TOK;
  const int g = lane >> 4;      // k group of the MFMA operands
  const int r = lane & 15;      // token row / expert column within a tile

  // ---- copies: instruction q of a block covers LDS rows 8q .. 8q + 7, one
  // 16-byte chunk per lane; waves take q = wave, wave + 8, ...
  constexpr int CPW = (C::Q + RT_WAVES - 1) / RT_WAVES;   // copies per wave (upper bound)
  const int cnt = (C::Q - wave + RT_WAVES - 1) / RT_WAVES; // this wave's copies per block
  constexpr int EL = 16 / (int)sizeof(T);                   // elements per chunk
  const T* src[CPW];
  int dst[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int q = min(wave + RT_WAVES * u, C::Q - 1);
    const int row = 8 * q + (lane >> 3);
    const int chunk = (lane & 7) ^ rt_swz(row);
    const T* rowp = row < RT_TOK ? x + (size_t)min(t0 + row, T_ - 1) * H
                                 : wr + (size_t)min(row - RT_TOK, E - 1) * H;
    src[u] = rowp + EL * chunk;
    dst[u] = q * 1024;
  }
  const int nblk = H / C::KB;
  auto issue = [&](int blk) {
    unsigned char* base = smem + (blk % NS) * C::STAGE;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
      if (u < cnt) rt_copy16(src[u] + (size_t)blk * C::KB, base + dst[u]);
  };
  // Wait until block b has landed: the blocks this wave issued after it may
  // stay in flight.  Steady state has NS - 2 of them; near the end, drain.
  auto wait_block = [&](int b) {
    const int after = min(b == 0 ? NS - 1 : NS - 2, nblk - 1 - b);
    if (after == NS - 1) {
      if (cnt == CPW) rt_wait_vmcnt<(NS - 1) * CPW>();
      else rt_wait_vmcnt<(NS - 1) * (CPW - 1)>();
    } else if (after == NS - 2) {
      if (cnt == CPW) rt_wait_vmcnt<(NS - 2) * CPW>();
      else rt_wait_vmcnt<(NS - 2) * (CPW - 1)>();
    } else {
      rt_wait_vmcnt<0>();
    }
  };

  // ---- MFMA operands: lane (g, r) takes chunks 2 g and 2 g + 1 of row r of
  // the x block and of row r of each of its expert tiles (tiles wave,
  // wave + 8); the swizzle of a row depends on r only.  bf16: one MFMA per
  // chunk (k = 16 g .. + 7 and 16 g + 8 .. + 15 of the block); float: the two
  // chunks form one chunk8 (k = 8 g .. + 7).  x and Wr use the same k
  // assignment, which is all the contraction needs.
  constexpr int TPW = (NT + RT_WAVES - 1) / RT_WAVES;   // expert tiles per wave
  const int c0 = 16 * ((2 * g) ^ rt_swz(r));
  const int c1 = 16 * ((2 * g + 1) ^ rt_swz(r));
  f32x4_v acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  auto rd = [&](const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p); };
  auto compute = [&](const unsigned char* base) {
    const unsigned char* xr = base + r * 128;
    const u32x4 xa = rd(xr + c0), xb = rd(xr + c1);
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
      const int j = wave + RT_WAVES * jj;
      if (j < NT) {
        const unsigned char* wrw = base + (RT_TOK + 16 * j + r) * 128;
        const u32x4 wa = rd(wrw + c0), wb = rd(wrw + c1);
        if constexpr (sizeof(T) == 2) {
          acc[jj] = mfma_16x16x32(chunk8<bf16_t>{xa}, chunk8<bf16_t>{wa}, acc[jj]);
          acc[jj] = mfma_16x16x32(chunk8<bf16_t>{xb}, chunk8<bf16_t>{wb}, acc[jj]);
        } else {
          acc[jj] = mfma_16x16x32(chunk8<float>{xa, xb}, chunk8<float>{wa, wb}, acc[jj]);
        }
      }
    }
  };

  // ---- K loop: one barrier per block publishes it and retires the slot
  // every wave finished reading in the previous iteration, which is then
  // refilled right away
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nblk) issue(p);
  for (int b = 0; b < nblk; ++b) {
    wait_block(b);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (b >= 1 && b - 1 + NS < nblk) issue(b - 1 + NS);
    compute(smem + (b % NS) * C::STAGE);
  }

  // ---- logits tile to LDS (+ bias): acc[jj][q] = L[token 4g + q][expert 16 j + r]
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int j = wave + RT_WAVES * jj;
    const int e = 16 * j + r;
    if (j < NT && e < E) {
      const float bv = bias ? bias[e] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) s_log[(4 * g + q) * C::LDE + e] = acc[jj][q] + bv;
    }
  }
  __syncthreads();
  if (logits_out) {
    for (int idx = threadIdx.x; idx < RT_TOK * E; idx += RT_WAVES * 64) {
      const int tr = idx / E, e = idx - tr * E;
      if (t0 + tr < T_) logits_out[(size_t)(t0 + tr) * E + e] = s_log[tr * C::LDE + e];
    }
  }

  // ---- top-k epilogue; the ring is free for the selected keys (every wave
  // passed the barrier above after its last LDS read of the ring)
  if constexpr (VAR)
    select_tokens_var<C::CPL>(s_log, C::LDE, reinterpret_cast<uint64_t*>(smem),
                              reinterpret_cast<float*>(smem + RT_TOK * k * 8), t0, wave, lane, T_,
                              E, k, norm, var, ids_out, w_out, counts);
  else
    select_tokens<C::CPL>(s_log, C::LDE, reinterpret_cast<uint64_t*>(smem), t0, wave, lane, T_,
                          E, k, norm, ids_out, w_out, counts);
}

// ---- Large-batch path with a workspace.  The kernel above streams all of
// Wr through LDS once per 16 tokens (at 4096 tokens about 150 MB of copies
// for 2 MB of logits).  Here a work-group takes 64 tokens and every expert
// over one slice of K, so Wr is streamed once per 64 tokens, and the slices
// keep enough work-groups for every CU; each writes float32 partial logits
// parts[slice][t][e], and route_select_kernel adds the slices in order.
constexpr int RP_TOK = 64;
constexpr int RP_NS = 4;          // ring stages (3 or 2 with 512 work-groups: slower)
constexpr int RP_TARGET = 256;    // work-groups the slices aim for

template <typename T, int NT>
struct rpcfg {
  static constexpr int KB = 128 / (int)sizeof(T);   // K elements per block (128-byte rows)
  static constexpr int ROWS = RP_TOK + NT * 16;      // x rows, then Wr rows
  static constexpr int STAGE = ROWS * 128;
  static constexpr int Q = ROWS / 8;                 // copy instructions per block (8 rows each)
  static constexpr int NS0 = (160 * 1024) / STAGE;
  static constexpr int NS = NS0 > RP_NS ? RP_NS : NS0;
  static constexpr int LDS = NS * STAGE;
  static_assert(NS >= 2, "ring");
  static_assert(ROWS % 8 == 0, "whole copy instructions");
};

template <typename T, int NT>
__global__ __launch_bounds__(RT_WAVES * 64) void route_part_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, int T_, int H, int E, int kslice,
    float* __restrict__ parts, int32_t* __restrict__ clear, int clear_n) {
  using C = rpcfg<T, NT>;
  constexpr int NS = C::NS;
  extern __shared__ __align__(16) unsigned char smem[];
  // the folded permutation's chunk histograms start from zero
  if (clear) {
    const int nthr = gridDim.x * gridDim.y * blockDim.x;
    for (int i = (blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < clear_n;
         i += nthr)
      clear[i] = 0;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * RP_TOK;
  const int sl = blockIdx.y;
  const int g = lane >> 4, r = lane & 15;

  // copies: instruction q of a block covers LDS rows 8q .. 8q + 7, one
  // 16-byte chunk per lane; waves take q = wave, wave + 8, ...
  constexpr int CPW = (C::Q + RT_WAVES - 1) / RT_WAVES;
  const int cnt = (C::Q - wave + RT_WAVES - 1) / RT_WAVES;
  constexpr int EL = 16 / (int)sizeof(T);
  const T* src[CPW];
  int dst[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int q = min(wave + RT_WAVES * u, C::Q - 1);
    const int row = 8 * q + (lane >> 3);
    const int chunk = (lane & 7) ^ rt_swz(row);
    const T* rowp = row < RP_TOK ? x + (size_t)min(t0 + row, T_ - 1) * H
                                 : wr + (size_t)min(row - RP_TOK, E - 1) * H;
    src[u] = rowp + (size_t)sl * kslice + EL * chunk;
    dst[u] = q * 1024;
  }
  const int nblk = kslice / C::KB;
  auto issue = [&](int blk) {
    unsigned char* base = smem + (blk % NS) * C::STAGE;
#pragma unroll
    for (int u = 0; u < CPW; ++u)
      if (u < cnt) rt_copy16(src[u] + (size_t)blk * C::KB, base + dst[u]);
  };
  auto wait_block = [&](int b) {
    const int after = min(b == 0 ? NS - 1 : NS - 2, nblk - 1 - b);
    if (after == NS - 1) {
      if (cnt == CPW) rt_wait_vmcnt<(NS - 1) * CPW>();
      else rt_wait_vmcnt<(NS - 1) * (CPW - 1)>();
    } else if (after == NS - 2) {
      if (cnt == CPW) rt_wait_vmcnt<(NS - 2) * CPW>();
      else rt_wait_vmcnt<(NS - 2) * (CPW - 1)>();
    } else {
      rt_wait_vmcnt<0>();
    }
  };

  // operands as in route_kernel: lane (g, r) takes chunks 2 g and 2 g + 1 of
  // row r of each 16-token group and of each of its expert tiles (tiles
  // wave, wave + 8, ...)
  constexpr int TPW = (NT + RT_WAVES - 1) / RT_WAVES;
  constexpr int TG = RP_TOK / 16;
  const int c0 = 16 * ((2 * g) ^ rt_swz(r));
  const int c1 = 16 * ((2 * g + 1) ^ rt_swz(r));
  f32x4_v acc[TPW][TG];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[j][tg] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  auto rd = [&](const unsigned char* p) { return *reinterpret_cast<const u32x4*>(p); };
  auto compute = [&](const unsigned char* base) {
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
      const int j = wave + RT_WAVES * jj;
      if (j < NT) {
        const unsigned char* wrw = base + (RP_TOK + 16 * j + r) * 128;
        const u32x4 wa = rd(wrw + c0), wb = rd(wrw + c1);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          const unsigned char* xr = base + (16 * tg + r) * 128;
          const u32x4 xa = rd(xr + c0), xb = rd(xr + c1);
          if constexpr (sizeof(T) == 2) {
            acc[jj][tg] = mfma_16x16x32(chunk8<bf16_t>{xa}, chunk8<bf16_t>{wa}, acc[jj][tg]);
            acc[jj][tg] = mfma_16x16x32(chunk8<bf16_t>{xb}, chunk8<bf16_t>{wb}, acc[jj][tg]);
          } else {
            acc[jj][tg] =
                mfma_16x16x32(chunk8<float>{xa, xb}, chunk8<float>{wa, wb}, acc[jj][tg]);
          }
        }
      }
    }
  };

#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nblk) issue(p);
  for (int b = 0; b < nblk; ++b) {
    wait_block(b);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (b >= 1 && b - 1 + NS < nblk) issue(b - 1 + NS);
    compute(smem + (b % NS) * C::STAGE);
  }

  // acc[jj][tg][q] = partial L[token 16 tg + 4 g + q][expert 16 j + r]
  float* const out = parts + (size_t)sl * T_ * E;
#pragma unroll
  for (int jj = 0; jj < TPW; ++jj) {
    const int j = wave + RT_WAVES * jj;
    const int e = 16 * j + r;
    if (j < NT && e < E) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + 16 * tg + 4 * g + q;
          if (t < T_) out[(size_t)t * E + e] = acc[jj][tg][q];
        }
    }
  }
}

// Slices of K for the partial-logits path: the fewest (1, 2, 4 or 8, each
// a whole number of 128-byte blocks) that give 256 work-groups.
int route_slices(int T, int H, bool bf16) {
  const int kb = bf16 ? 64 : 32;
  const int blocks = H / kb;
  const int tiles = (T + RP_TOK - 1) / RP_TOK;
  int S = 1;
  while (S < 8 && tiles * S < RP_TARGET && blocks % (2 * S) == 0) S *= 2;
  return S;
}

template <typename V, int NT>
hipError_t launch_route_part(const void* x, const void* wr, int T, int H, int E, int S,
                             float* parts, int32_t* clear, int clear_n, hipStream_t s) {
  using C = rpcfg<V, NT>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)route_part_kernel<V, NT>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (attr != hipSuccess) return attr;
  const dim3 grid((T + RP_TOK - 1) / RP_TOK, S);
  route_part_kernel<V, NT><<<grid, RT_WAVES * 64, C::LDS, s>>>((const V*)x, (const V*)wr, T, H, E,
                                                               H / S, parts, clear, clear_n);
  return hipGetLastError();
}

// ---- Small-batch path.  With few tokens the kernel above runs on few CUs,
// each streaming all of Wr; here the logits are spread over (16-token tile,
// 16-expert tile) workgroups first, then one workgroup per 16 tokens selects.

// Logits of one 16 x 16 tile: 4 waves split K in 64-wide blocks (wave w
// takes blocks w, w + 4, ...), loading MFMA operands straight from global
// memory D blocks ahead; the 4 partial tiles are added in wave order in LDS.
template <typename T>
__global__ __launch_bounds__(256) void route_logits_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias, int T_,
    int H, int E, float* __restrict__ logits) {
  constexpr int NWV = 4, D = 4, P = 2, KB = 32 * P;
  __shared__ float s_acc[NWV][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int g = lane >> 4, r = lane & 15;
  const T* xrow = x + (size_t)min(t0 + r, T_ - 1) * H + 8 * P * g;
  const T* wrow = wr + (size_t)min(e0 + r, E - 1) * H + 8 * P * g;
  const int nblk = H / KB;
  const int iters = (nblk + NWV - 1) / NWV;
  f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
  chunk8<T> a[D][P], b[D][P];
  auto load = [&](int s, int i) {
    const int c = KB * min(wave + NWV * i, nblk - 1);
#pragma unroll
    for (int h = 0; h < P; ++h) {
      a[s][h] = load_chunk<T>(xrow + c + 8 * h);
      b[s][h] = load_chunk<T>(wrow + c + 8 * h);
    }
  };
  auto mma = [&](int s, int i) {
    const bool on = wave + NWV * i < nblk;
#pragma unroll
    for (int h = 0; h < P; ++h) acc = mfma_16x16x32(on ? a[s][h] : zero_chunk<T>(), b[s][h], acc);
  };
  const int groups = (iters + D - 1) / D;
#pragma unroll
  for (int s = 0; s < D; ++s) load(s, s);
  for (int gi = 0; gi + 1 < groups; ++gi) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      mma(s, gi * D + s);
      load(s, (gi + 1) * D + s);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s) mma(s, (groups - 1) * D + s);
  // acc[q] = partial L[token 4 g + q][expert r]
#pragma unroll
  for (int q = 0; q < 4; ++q) s_acc[wave][4 * g + q][r] = acc[q];
  __syncthreads();
  const int tr = threadIdx.x >> 4, ec = threadIdx.x & 15;   // 16 x 16 outputs, one per thread
  const int t = t0 + tr, e = e0 + ec;
  if (t < T_ && e < E) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) v += s_acc[w][tr][ec];
    if (bias) v += bias[e];
    logits[(size_t)t * E + e] = v;
  }
}

// The permutation's first pass for the block's RT_TOK * k slots (MindSpore
// moe.py, MoE.permutation: a stable sort of the flat slots by expert): each
// 64-slot wave segment ranks its slots among equal experts with ballots on
// the id bits, the segments' histograms are scanned per expert, and the
// block writes each slot's rank within the block, its histogram, and adds
// the histogram into its 1024-slot chunk's (integer adds: any order gives
// the same sums).  k is 8, 16 or 32 (route_can_fold), so the block is 2, 4
// or 8 whole segments and lies inside one chunk.
__device__ __forceinline__ void fold_block(const uint64_t* keys, int t0, int wave, int lane,
                                           int T_, int E, int k, const PermuteFold& f) {
  __shared__ int s_seg[RT_WAVES][256];
  for (int i = threadIdx.x; i < RT_WAVES * 256; i += RT_WAVES * 64) (&s_seg[0][0])[i] = 0;
  __syncthreads();   // also: every token's keys are in LDS
  const int nseg = RT_TOK * k / 64;
  const int sl = wave * 64 + lane;
  int e = -1;
  if (wave < nseg && t0 + sl / k < T_) e = key_expert(keys[sl]);
  const bool valid = e >= 0 && e < E;
  int my_rank = 0;
  if (wave < nseg) {   // uniform over the wave
    unsigned long long match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    my_rank = valid ? __popcll(match & below) : 0;
    // the lowest lane of each equal-expert group records its size
    if (valid && (match & below) == 0ull) s_seg[wave][e] = __popcll(match);
  }
  __syncthreads();
  if (threadIdx.x < E) {
    const int x = threadIdx.x;
    int run = 0;
    for (int w = 0; w < nseg; ++w) {
      const int v = s_seg[w][x];
      s_seg[w][x] = run;
      run += v;
    }
    f.sub[(size_t)blockIdx.x * E + x] = run;
    if (run > 0) atomicAdd(&f.hist[(size_t)(t0 * k / 1024) * E + x], run);
  }
  __syncthreads();
  if (valid) f.rank[(size_t)t0 * k + sl] = s_seg[wave][e] + my_rank;
}

// Selection for 16 tokens from logits in global memory: the sum of S
// partial slices parts[s][t][e] (s = 0 .. S - 1, added in that order), plus
// the bias when there is one; written to logits_out when it is not null.
template <int NT, bool VAR>
__global__ __launch_bounds__(RT_WAVES * 64) void route_select_kernel(
    const float* __restrict__ parts, int S, const float* __restrict__ bias,
    float* __restrict__ logits_out, int T_, int E, int k, int norm,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ counts,
    RouterVariant var, PermuteFold fold) {
  constexpr int LDE = NT * 16 + 4;
  constexpr int CPL = (NT * 16 + 31) / 32;
  __shared__ float s_log[RT_TOK * LDE];
  extern __shared__ __align__(16) unsigned char s_sel[];   // 16 * k keys (+ 16 * E floats)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * RT_TOK;
  // every load of a thread is issued before the first sum (a runtime loop
  // over the slices would wait for each load in turn)
  const size_t slice = (size_t)T_ * E;
  constexpr int PER = (RT_TOK * NT * 16 + RT_WAVES * 64 - 1) / (RT_WAVES * 64);
  constexpr int SMAX = 8;
  float pv[PER][SMAX];
  size_t at[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + RT_WAVES * 64 * i;
    const int tr = min(idx / E, RT_TOK - 1), e = idx - (idx / E) * E;
    at[i] = (size_t)min(t0 + tr, T_ - 1) * E + min(e, E - 1);
#pragma unroll
    for (int sl = 0; sl < SMAX; ++sl) pv[i][sl] = sl < S ? parts[sl * slice + at[i]] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + RT_WAVES * 64 * i;
    if (idx < RT_TOK * E) {
      const int tr = idx / E, e = idx - tr * E;
      float v = pv[i][0];
#pragma unroll
      for (int sl = 1; sl < SMAX; ++sl)
        if (sl < S) v += pv[i][sl];
      if (bias) v += bias[e];
      s_log[tr * LDE + e] = v;
      if (logits_out && t0 + tr < T_) logits_out[at[i]] = v;
    }
  }
  __syncthreads();
  if constexpr (VAR)
    select_tokens_var<CPL>(s_log, LDE, reinterpret_cast<uint64_t*>(s_sel),
                           reinterpret_cast<float*>(s_sel + RT_TOK * k * 8), t0, wave, lane, T_, E,
                           k, norm, var, ids_out, w_out, counts);
  else
    select_tokens<CPL>(s_log, LDE, reinterpret_cast<uint64_t*>(s_sel), t0, wave, lane, T_, E, k,
                       norm, ids_out, w_out, counts);
  if (fold.hist) fold_block(reinterpret_cast<const uint64_t*>(s_sel), t0, wave, lane, T_, E, k,
                            fold);
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename V, int NT, bool VAR>
hipError_t launch_route_t(const void* x, const void* wr, const float* bias, int T, int H, int E,
                          int k, int norm, float* logits, int32_t* ids, float* w,
                          int32_t* counts, hipStream_t s, const RouterVariant& var) {
  using C = rcfg<V, NT>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)route_kernel<V, NT, VAR>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (attr != hipSuccess) return attr;
  const dim3 grid((T + RT_TOK - 1) / RT_TOK);
  route_kernel<V, NT, VAR><<<grid, RT_WAVES * 64, C::LDS, s>>>(
      (const V*)x, (const V*)wr, bias, T, H, E, k, norm, logits, ids, w, counts, var);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

bool route_can_fold(int T, int H, int E, int k, bool bf16) {
  return route_ws_bytes(T, H, E, bf16) > 0 && (k == 8 || k == 16 || k == 32) && E <= 256;
}

size_t route_ws_bytes(int T, int H, int E, bool bf16) {
  const int tiles = (T + RT_TOK - 1) / RT_TOK;
  if (T <= 0 || tiles <= RT_SPLIT_MAX_TILES || H % 64 != 0) return 0;
  return (size_t)route_slices(T, H, bf16) * T * E * sizeof(float);
}

hipError_t launch_route(bool bf16, const void* x, const void* wr, const float* bias,
                        int T, int H, int E, int k, int norm, float* logits,
                        int32_t* ids, float* w, int32_t* counts, hipStream_t s,
                        const RouterVariant* var, float* parts, size_t parts_bytes,
                        const PermuteFold* fold) {
  // the fold rides on the partial-logits path only
  if (fold && (!parts || parts_bytes < route_ws_bytes(T, H, E, bf16) ||
               !route_can_fold(T, H, E, k, bf16) || !fold->hist || !fold->sub || !fold->rank))
    return hipErrorInvalidValue;
  if (counts) {
    hipError_t e = launch_fill_i32(counts, E, 0, s);
    if (e != hipSuccess) return e;
  }
  if (T <= 0) return hipSuccess;
  const RouterVariant v = var ? *var : RouterVariant{0, 1.0f, nullptr, 0, 0, nullptr};
  const bool isvar = var != nullptr;
  const int nt = (E + 15) / 16;
  const int tiles = (T + RT_TOK - 1) / RT_TOK;
  // Small batches (and a logits buffer to pass through) take the split path;
  // large ones with a workspace the partial-logits path; both then select
  // with route_select_kernel.
  const float* sel_src = nullptr;
  const float* sel_bias = nullptr;
  float* sel_out = nullptr;
  int sel_S = 1;
  if (logits && tiles <= RT_SPLIT_MAX_TILES && H % 64 == 0) {
    const dim3 g1(tiles, nt);
    if (bf16)
      route_logits_kernel<bf16_t><<<g1, 256, 0, s>>>((const bf16_t*)x, (const bf16_t*)wr, bias, T,
                                                     H, E, logits);
    else
      route_logits_kernel<float><<<g1, 256, 0, s>>>((const float*)x, (const float*)wr, bias, T, H,
                                                    E, logits);
    sel_src = logits;   // bias already added
  } else if (parts && parts_bytes >= route_ws_bytes(T, H, E, bf16) &&
             route_ws_bytes(T, H, E, bf16) > 0) {
    sel_S = route_slices(T, H, bf16);
    hipError_t e;
    int32_t* const clear = fold ? fold->hist : nullptr;
    const int clear_n = fold ? (T * k + 1023) / 1024 * E : 0;
#define MOE_PART(NT)                                                                          \
  e = bf16 ? launch_route_part<bf16_t, NT>(x, wr, T, H, E, sel_S, parts, clear, clear_n, s)   \
           : launch_route_part<float, NT>(x, wr, T, H, E, sel_S, parts, clear, clear_n, s)
    if (nt <= 1) MOE_PART(1);
    else if (nt <= 2) MOE_PART(2);
    else if (nt <= 4) MOE_PART(4);
    else if (nt <= 8) MOE_PART(8);
    else MOE_PART(16);
#undef MOE_PART
    if (e != hipSuccess) return e;
    sel_src = parts;
    sel_bias = bias;
    sel_out = logits;
  }
  const PermuteFold pf = fold ? *fold : PermuteFold{nullptr, nullptr, nullptr};
  if (sel_src) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t sel_bytes = (size_t)RT_TOK * k * sizeof(uint64_t) +
                             (isvar ? (size_t)RT_TOK * E * sizeof(float) : 0);
#define MOE_SELECT(NT)                                                                          \
  do {                                                                                          \
    if (isvar)                                                                                  \
      route_select_kernel<NT, true><<<tiles, RT_WAVES * 64, sel_bytes, s>>>(                  \
          sel_src, sel_S, sel_bias, sel_out, T, E, k, norm, ids, w, counts, v, pf);             \
    else                                                                                        \
      route_select_kernel<NT, false><<<tiles, RT_WAVES * 64, sel_bytes, s>>>(                 \
          sel_src, sel_S, sel_bias, sel_out, T, E, k, norm, ids, w, counts, v, pf);             \
  } while (0)
    if (nt <= 1) MOE_SELECT(1);
    else if (nt <= 2) MOE_SELECT(2);
    else if (nt <= 4) MOE_SELECT(4);
    else if (nt <= 8) MOE_SELECT(8);
    else MOE_SELECT(16);
#undef MOE_SELECT
    return hipGetLastError();
  }
#define MOE_ROUTE(NT)                                                                         \
  return bf16 ? (isvar ? launch_route_t<bf16_t, NT, true>(x, wr, bias, T, H, E, k, norm,     \
                                                          logits, ids, w, counts, s, v)      \
                       : launch_route_t<bf16_t, NT, false>(x, wr, bias, T, H, E, k, norm,    \
                                                           logits, ids, w, counts, s, v))    \
              : (isvar ? launch_route_t<float, NT, true>(x, wr, bias, T, H, E, k, norm,      \
                                                         logits, ids, w, counts, s, v)       \
                       : launch_route_t<float, NT, false>(x, wr, bias, T, H, E, k, norm,     \
                                                          logits, ids, w, counts, s, v))
  if (nt <= 1) MOE_ROUTE(1);
  if (nt <= 2) MOE_ROUTE(2);
  if (nt <= 4) MOE_ROUTE(4);
  if (nt <= 8) MOE_ROUTE(8);
  MOE_ROUTE(16);
#undef MOE_ROUTE
}

// Expert-bias step (MindSpore moe.py, MoE.update_expert_bias): one
// workgroup; sums in a fixed tree.
__global__ __launch_bounds__(256) void update_expert_bias_kernel(float* __restrict__ bias,
                                                                 float* __restrict__ tpe, int E,
                                                                 float lr, int nrec) {
  __shared__ float s_v[256];
  const int t = threadIdx.x;
  float c = t < E ? tpe[t] : 0.f;
  if (nrec > 1) c = c / (float)nrec;
  s_v[t] = c;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) s_v[t] += s_v[t + off];
    __syncthreads();
  }
  const float avg = s_v[0] / (float)E;
  __syncthreads();
  float d = 0.f;
  if (t < E) {
    const float diff = avg - c;
    d = lr * (diff > 0.f ? 1.f : (diff < 0.f ? -1.f : 0.f));
  }
  s_v[t] = d;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) s_v[t] += s_v[t + off];
    __syncthreads();
  }
  const float dm = s_v[0] / (float)E;
  if (t < E) {
    bias[t] += d - dm;
    tpe[t] = 0.f;
  }
}

hipError_t launch_update_expert_bias(float* bias, float* tpe, int E, float lr, int nrec,
                                     hipStream_t s) {
  update_expert_bias_kernel<<<1, 256, 0, s>>>(bias, tpe, E, lr, nrec);
  return hipGetLastError();
}

}  // namespace moe
