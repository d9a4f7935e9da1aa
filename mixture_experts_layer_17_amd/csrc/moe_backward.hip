// Backward of the MoE layer outside the grouped GEMMs: the routing-weight
// gradient, the softmax/router gradient, the token reduction of dX and the
// router's weight gradient.  All sums run in a fixed order in float32, so
// results are deterministic.
//
// The pages train the layer through autograd (Qwen3-Omni issue #115,
// SpeedupMoeSparseMoeBlock: softmax routing weights, optionally renormalised;
// MindSpore moe.py, MoE.forward and MoE.unpermutation).  With dout the
// output gradient:
//   d_weights[t, j] = <dout[t], y[t, j]>
//   softmax scores (s = route_scale * p):
//     renormalised:  dL[t, ids] = w (d_weights - <d_weights, w>), 0 elsewhere
//     plain:         dL[t, e]   = p_e (route_scale g_e - <d_weights, w>),
//                    g = d_weights scattered to the ids
//   sigmoid scores (MindSpore moe.py, TokenChoiceTopKRouter: s = scale sg(L)):
//     renormalised:  dL[t, ids] = w (1 - sg) (d_weights - <d_weights, w>)
//     plain:         dL[t, ids] = d_weights w (1 - sg)
//   (bias and group limits steer the selection only: no gradient)
//   dx[t]  = sum_j dX[t k + j] + sum_e dL[t, e] Wr[e]
//   dWr[e] = sum_t dL[t, e] x[t],   d_bias[e] = sum_t dL[t, e]
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8], bool stream = false) {
  const chunk8<T> c = stream ? load_chunk_stream<T>(p) : load_chunk<T>(p);
  if constexpr (sizeof(T) == 2) {
    const uint32_t* d = reinterpret_cast<const uint32_t*>(&c.v);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      f[2 * x] = bf16_bits_to_f32(d[x] & 0xffffu);
      f[2 * x + 1] = bf16_bits_to_f32(d[x] >> 16);
    }
  } else {
    const float* a = reinterpret_cast<const float*>(&c.lo);
    const float* b = reinterpret_cast<const float*>(&c.hi);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      f[x] = a[x];
      f[4 + x] = b[x];
    }
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&f)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t d[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
      d[x] = (uint32_t)f32_to_bf16_bits(f[2 * x]) | ((uint32_t)f32_to_bf16_bits(f[2 * x + 1]) << 16);
    *reinterpret_cast<u32x4*>(p) = u32x4{d[0], d[1], d[2], d[3]};
  } else {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

// p[0] + p[stride] + ... + p[(n - 1) stride], added in that order, with the
// loads issued 8 at a time (a plain loop waited for each load in turn).
__device__ __forceinline__ float sum_in_order(const float* __restrict__ p, long long stride,
                                              int n) {
  constexpr int U = 8;
  float s = 0.f;
  for (int b = 0; b < n; b += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = b + u < n ? p[(long long)(b + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (b + u < n) s += v[u];
  }
  return s;
}

// d_weights[i] = <dout[i / k], y[i]> = <dout[i / k] . down[e]^T, h[i]>: the
// first dgrad's epilogue leaves the inner products of its column slices of
// that second form (P per expert-major row); one thread per flat slot adds
// them in slice order.
__global__ __launch_bounds__(256) void weight_grad_kernel(const float* __restrict__ parts, int P,
                                                          const int32_t* __restrict__ slot_pos,
                                                          int N, float* __restrict__ dw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const float* p = parts + (size_t)min(max(slot_pos[i], 0), N - 1) * P;
  dw[i] = sum_in_order(p, 1, P);
}

// dL[t, :] from the routing-weight gradient: one wave per token.
// With renormalised weights it also writes the selected entries in the
// permutation's expert-major order: dl_perm[slot_pos[t k + j]] = dL[t, ids].
__global__ __launch_bounds__(256) void router_grad_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ dw,
                                                          const int32_t* __restrict__ slot_pos,
                                                          int T, int E, int k, int norm,
                                                          int sigmoid, float scale,
                                                          float* __restrict__ dL,
                                                          float* __restrict__ dl_perm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* L = logits + (size_t)t * E;
  float* out = dL + (size_t)t * E;
  // <d_weights, w> in slot order (w are the softmax probabilities of the
  // selected experts, renormalised or not)
  float inner = 0.f;
  for (int j = 0; j < k; ++j) inner = fmaf(dw[(size_t)t * k + j], w[(size_t)t * k + j], inner);
  if (norm || sigmoid) {
    // nonzero only on the selection
    for (int e = lane; e < E; e += 64) {
      float g = 0.f;
      for (int j = 0; j < k; ++j)
        if (ids[(size_t)t * k + j] == e) {
          const float wj = w[(size_t)t * k + j], dj = dw[(size_t)t * k + j];
          const float one_m_sg = sigmoid ? __builtin_amdgcn_rcpf(1.0f + __expf(L[e])) : 1.0f;
          g = norm ? wj * one_m_sg * (dj - inner) : dj * wj * one_m_sg;
          dl_perm[slot_pos[(size_t)t * k + j]] = g;
        }
      out[e] = g;
    }
    return;
  }
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
  m = wave_max(m);
  float z = 0.f;
  for (int e = lane; e < E; e += 64) z += __expf(L[e] - m);
  z = wave_sum(z);
  const float rz = 1.0f / z;
  for (int e = lane; e < E; e += 64) {
    float g = 0.f;
    for (int j = 0; j < k; ++j)
      if (ids[(size_t)t * k + j] == e) g = dw[(size_t)t * k + j];
    const float p = __expf(L[e] - m) * rz;
    out[e] = p * (scale * g - inner);
  }
}

// dx[t] = sum_j dX[t k + j] + sum_e dL[t, e] Wr[e]; one thread per 8 columns.
template <typename T>
__global__ __launch_bounds__(256) void input_grad_kernel(const T* __restrict__ dX,
                                                         const float* __restrict__ dL,
                                                         const int32_t* __restrict__ ids,
                                                         const T* __restrict__ wr, int T_, int k,
                                                         int E, int H, const T* __restrict__ add,
                                                         T* __restrict__ dx) {
  const int per_row = H / 8;
  const long long total = (long long)T_ * per_row;
  for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (long long)gridDim.x * 256) {
    const int t = (int)(q / per_row);
    const int c = 8 * (int)(q - (long long)t * per_row);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // one row at a time: the latency hides behind the other resident waves
    // (holding 8 rows per thread in flight lowered the occupancy and
    // measured 15 % slower)
    for (int j = 0; j < k; ++j) {
      float v[8];
      load8(dX + ((size_t)t * k + j) * H + c, v, true);   // read once
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] += v[x];
    }
    const float* l = dL + (size_t)t * E;
    if (ids) {
      // dL is zero off the token's selection: its k router rows, slot order
      for (int j = 0; j < k; ++j) {
        const int e = min(max(ids[(size_t)t * k + j], 0), E - 1);
        const float g = l[e];
        float v[8];
        load8(wr + (size_t)e * H + c, v);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = fmaf(g, v[x], acc[x]);
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const float g = l[e];
        float v[8];
        load8(wr + (size_t)e * H + c, v);
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = fmaf(g, v[x], acc[x]);
      }
    }
    if (add) {
      float v[8];
      load8(add + (size_t)t * H + c, v);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] += v[x];
    }
    store8(dx + (size_t)t * H + c, acc);
  }
}

// dWr[e, :] = sum_t dL[t, e] x[t, :] and d_bias[e] = sum_t dL[t, e], in two
// passes: `splits` work-groups per expert each sum one contiguous share of
// its rows into a partial, then the partials are added in order.  With
// renormalised weights dL[t, e] is nonzero only where token t chose e, so
// the rows are the expert's rows of the permutation (dl_perm expert-major,
// x read through the permutation's row index, so the 16.8 MB of x serve all
// k selections from the caches instead of an expert-major copy k times its
// size); otherwise every token's x row with dL[t, e].
template <typename T>
__global__ __launch_bounds__(256) void router_weight_grad_part_kernel(
    const T* __restrict__ rows_x, const int32_t* __restrict__ row_index,
    const float* __restrict__ g, const int32_t* __restrict__ offsets, int T_, int E, int H,
    int sparse, int splits, float* __restrict__ part, float* __restrict__ part_b) {
  const int e = blockIdx.x / splits, r = blockIdx.x - (blockIdx.x / splits) * splits;
  const int lo0 = sparse ? offsets[e] : 0;
  const int hi0 = sparse ? max(offsets[e + 1], lo0) : T_;
  const int chunk = (hi0 - lo0 + splits - 1) / splits;
  const int lo = lo0 + r * chunk;
  const int hi = min(hi0, lo + chunk);
  for (int c = 8 * threadIdx.x; c < H; c += 8 * 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;
    constexpr int U = 8;   // rows in flight; sums stay in row order
    for (int p0 = lo; p0 < hi; p0 += U) {
      float gv[U], v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = min(p0 + u, hi - 1);
        gv[u] = p0 + u < hi ? (sparse ? g[p] : g[(size_t)p * E + e]) : 0.f;
        const int row = row_index ? min(max(row_index[p], 0), T_ - 1) : p;
        load8(rows_x + (size_t)row * H + c, v[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bsum += gv[u];
#pragma unroll
        for (int xx = 0; xx < 8; ++xx) acc[xx] = fmaf(gv[u], v[u][xx], acc[xx]);
      }
    }
    float* o = part + ((size_t)r * E + e) * H + c;
    reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (c == 0) part_b[(size_t)r * E + e] = bsum;
  }
}

__global__ __launch_bounds__(256) void router_weight_grad_sum_kernel(
    const float* __restrict__ part, const float* __restrict__ part_b, int E, int H, int splits,
    float* __restrict__ dwr, float* __restrict__ dbias) {
  const long long total = (long long)E * H;
  for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (long long)gridDim.x * 256) {
    dwr[q] = sum_in_order(part + q, total, splits);
  }
  if (dbias && blockIdx.x == 0)
    for (int e = threadIdx.x; e < E; e += 256) {
      float b = 0.f;
      for (int r = 0; r < splits; ++r) b += part_b[(size_t)r * E + e];
      dbias[e] = b;
    }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, long long n, uint32_t v) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (long long)gridDim.x * 256)
    p[i] = v;
}

constexpr int kRouterSplits = 8;   // row shares per expert in the router's weight gradient

int grid_for_total(long long total) {
  return (int)std::max<long long>(1, std::min<long long>((total + 255) / 256, 16384));
}

}  // namespace

hipError_t launch_weight_grad(const float* parts, int P, const int32_t* slot_pos, int N,
                              float* dw, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  weight_grad_kernel<<<(N + 255) / 256, 256, 0, s>>>(parts, P, slot_pos, N, dw);
  return hipGetLastError();
}

hipError_t launch_router_grad(const float* logits, const int32_t* ids, const float* w,
                              const float* dw, const int32_t* slot_pos, int T, int E, int k,
                              int norm, int sigmoid, float scale, float* dL, float* dl_perm,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  router_grad_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, ids, w, dw, slot_pos, T, E, k, norm,
                                                 sigmoid, scale, dL, dl_perm);
  return hipGetLastError();
}

hipError_t launch_input_grad(bool bf16, const void* dX, const float* dL, const int32_t* ids,
                             const void* wr, int T, int k, int E, int H, const void* add,
                             void* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int grid = grid_for_total((long long)T * (H / 8));
  if (bf16)
    input_grad_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)dX, dL, ids, (const bf16_t*)wr,
                                                   T, k, E, H, (const bf16_t*)add, (bf16_t*)dx);
  else
    input_grad_kernel<float><<<grid, 256, 0, s>>>((const float*)dX, dL, ids, (const float*)wr, T,
                                                  k, E, H, (const float*)add, (float*)dx);
  return hipGetLastError();
}

size_t router_weight_grad_ws(int E, int H) {
  return (size_t)kRouterSplits * E * (H + 1) * sizeof(float);
}

hipError_t launch_router_weight_grad(bool bf16, const void* x, const int32_t* sorted_token,
                                     const float* dL, const float* dl_perm,
                                     const int32_t* offsets, int T, int E, int H, int sparse,
                                     float* dwr, float* dbias, void* ws, hipStream_t s) {
  float* part = (float*)ws;
  float* part_b = part + (size_t)kRouterSplits * E * H;
  const int32_t* idx = sparse ? sorted_token : nullptr;
  const float* g = sparse ? dl_perm : dL;
  const int grid = E * kRouterSplits;
  if (bf16)
    router_weight_grad_part_kernel<bf16_t><<<grid, 256, 0, s>>>(
        (const bf16_t*)x, idx, g, offsets, T, E, H, sparse, kRouterSplits, part, part_b);
  else
    router_weight_grad_part_kernel<float><<<grid, 256, 0, s>>>(
        (const float*)x, idx, g, offsets, T, E, H, sparse, kRouterSplits, part, part_b);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  router_weight_grad_sum_kernel<<<grid_for_total((long long)E * H), 256, 0, s>>>(
      part, part_b, E, H, kRouterSplits, dwr, dbias);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, long long n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_u32_kernel<<<grid_for_total(n), 256, 0, s>>>((uint32_t*)p, n, v);
  return hipGetLastError();
}

}  // namespace moe
