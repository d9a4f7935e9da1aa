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
// Layout: one workgroup of 8 waves per 16 tokens.  Both operands are
// K-contiguous (x is [T, H], Wr is [E, H]), so each lane loads its MFMA
// operand chunk straight from global memory.  The waves split K: wave w
// takes the 32-wide k-chunks w, w + 8, ... for all E experts, so every wave
// has many independent loads in flight.  The 8 partial logit tiles are then
// added in a fixed tree through LDS (deterministic), and each wave runs the
// softmax / top-k epilogue for 2 tokens.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT_TOK = 16;     // tokens per workgroup
constexpr int RT_MAXE = 256;   // max experts
constexpr int RT_NT = RT_MAXE / 16;
constexpr int RT_WAVES = 8;
constexpr int RT_LD = RT_MAXE + 4;   // LDS row stride (floats)

// Larger logit first; equal logits (IEEE equality, so -0 == +0) go to the
// lower expert id.
__device__ __forceinline__ bool ranks_before(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

template <typename T, int NT>
__global__ __launch_bounds__(RT_WAVES * 64) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias,
    int T_, int H, int E, int k, int norm, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts) {
  // partial-sum buffers for the reduction tree; buffer 0 finally holds the
  // logits of the 16 tokens
  __shared__ float s_red[RT_WAVES / 2][RT_TOK][RT_LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RT_TOK;
  const int g = lane >> 4;      // k-chunk group
  const int r = lane & 15;      // row (token) / column (expert) within a tile

  f32x4_v acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  const int tok = min(t0 + r, T_ - 1);
  const T* xrow = x + (size_t)tok * H + 8 * g;
  // experts beyond E read row E - 1 (valid memory); their columns are never
  // stored as logits, so no branch is needed around the loads
  const T* wrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wrow[j] = wr + (size_t)min(j * 16 + r, E - 1) * H + 8 * g;

  // wave w takes blocks of CPB consecutive 32-wide k-chunks: w, w + 8, ...;
  // all loads of a block are issued before its MFMAs
  constexpr int CPB = 4;
  const int nchunk = H / 32;
  const int nfull = nchunk / CPB;           // full blocks
  for (int blk = wave; blk < nfull; blk += RT_WAVES) {
    chunk8<T> a[CPB];
    chunk8<T> b[CPB][NT];
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int k0 = 32 * (blk * CPB + u);
      a[u] = load_chunk<T>(xrow + k0);
#pragma unroll
      for (int j = 0; j < NT; ++j) b[u][j] = load_chunk<T>(wrow[j] + k0);
    }
#pragma unroll
    for (int u = 0; u < CPB; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mfma_16x16x32(a[u], b[u][j], acc[j]);
  }
  // leftover chunks (H / 32 not a multiple of CPB)
  for (int c = nfull * CPB + wave; c < nchunk; c += RT_WAVES) {
    const int k0 = 32 * c;
    const chunk8<T> a = load_chunk<T>(xrow + k0);
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = mfma_16x16x32(a, load_chunk<T>(wrow[j] + k0), acc[j]);
  }

  // ---- fixed-order tree: 8 -> 4 -> 2 -> 1 partial tiles
#pragma unroll
  for (int half = RT_WAVES / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[wave - half][4 * g + i][16 * j + r] = acc[j][i];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] += s_red[wave][4 * g + i][16 * j + r];
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int e = 16 * j + r;
      if (e < E) {
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[0][4 * g + i][e] = acc[j][i] + b;
      }
    }
  }
  __syncthreads();

  // ---- Epilogue: wave w handles tokens 2w, 2w + 1 of this workgroup.
  for (int q = 0; q < RT_TOK / RT_WAVES; ++q) {
    const int row = (RT_TOK / RT_WAVES) * wave + q;
    const int t = t0 + row;
    if (t >= T_) break;
    // lane owns experts lane, lane + 64, lane + 128, lane + 192
    float v[4];
    unsigned avail = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      if (e < E) {
        v[c] = s_red[0][row][e];
        avail |= 1u << c;
        if (logits_out) logits_out[(size_t)t * E + e] = v[c];
      } else {
        v[c] = -INFINITY;
      }
    }
    // top-k by repeated wave arg-max under the (value desc, id asc) order
    float sel_v[4] = {0.f, 0.f, 0.f, 0.f};
    int sel_e[4] = {0, 0, 0, 0};
    float m = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (avail & (1u << c)) {
          const int e = lane + 64 * c;
          if (be == 0x7fffffff || ranks_before(v[c], e, bv, be)) { bv = v[c]; be = e; }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (oe != 0x7fffffff && (be == 0x7fffffff || ranks_before(ov, oe, bv, be))) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
      if (j == 0) m = bv;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((j >> 6) == c && (j & 63) == lane) { sel_v[c] = bv; sel_e[c] = be; }
    }
    // softmax denominator over all experts (max-subtracted), and the sum of
    // the selected probabilities' numerators
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c < E) part += expf(v[c] - m);
    const float denom = wave_sum(part);
    float selpart = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c < k) selpart += expf(sel_v[c] - m);
    const float selsum = wave_sum(selpart);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      if (j < k) {
        const float num = expf(sel_v[c] - m);
        const float w = norm ? num / selsum : num / denom;
        ids_out[(size_t)t * k + j] = sel_e[c];
        w_out[(size_t)t * k + j] = w;
        if (counts) atomicAdd(&counts[sel_e[c]], 1);
      }
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_route(bool bf16, const void* x, const void* wr, const float* bias,
                        int T, int H, int E, int k, int norm, float* logits,
                        int32_t* ids, float* w, int32_t* counts, hipStream_t s) {
  if (counts) {
    hipError_t e = launch_fill_i32(counts, E, 0, s);
    if (e != hipSuccess) return e;
  }
  if (T <= 0) return hipSuccess;
  const dim3 grid((T + RT_TOK - 1) / RT_TOK);
  const dim3 block(RT_WAVES * 64);
  const int nt = (E + 15) / 16;
#define MOE_ROUTE(NT)                                                                          \
  do {                                                                                         \
    if (bf16)                                                                                  \
      route_kernel<bf16_t, NT><<<grid, block, 0, s>>>((const bf16_t*)x, (const bf16_t*)wr,     \
                                                      bias, T, H, E, k, norm, logits, ids, w, \
                                                      counts);                                 \
    else                                                                                       \
      route_kernel<float, NT><<<grid, block, 0, s>>>((const float*)x, (const float*)wr, bias,  \
                                                     T, H, E, k, norm, logits, ids, w, counts);\
  } while (0)
  if (nt <= 1) MOE_ROUTE(1);
  else if (nt <= 2) MOE_ROUTE(2);
  else if (nt <= 4) MOE_ROUTE(4);
  else if (nt <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
