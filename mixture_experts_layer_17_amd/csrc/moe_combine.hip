// Weighted un-permute / combine: out[t] = sum_j w[t, j] * y[src(t, j)],
// plus the shared expert's row when there is one.
//
// Semantics: Qwen3-Omni issue #115, SpeedupMoeExperts.forward (expert output
// times routing weight, index_add_ into the token rows); MindSpore moe.py,
// MoE.unpermutation (scatter_add back to token order).  Here each token's k
// rows are gathered and summed in float32 in ascending j, then rounded once:
// no atomics, so the result is bitwise deterministic.  The shared expert's
// output (MindSpore moe.py, MoE.forward: added after the unpermutation) joins
// the same float32 sum last, before that single rounding.
//
// Each thread owns 8 consecutive columns (one 16-byte bf16 load per row), so
// a wave reads 1 KB contiguous per source row: HBM-bound streaming.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ w, int T_, int k,
                                                      int H, const T* __restrict__ add,
                                                      T* __restrict__ out) {
  const int per_row = H / 8;
  const int N = T_ * k;
  const long long total = (long long)T_ * per_row;
  for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (long long)gridDim.x * 256) {
    const int t = (int)(q / per_row);
    const int c = (int)(q - (long long)t * per_row);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // slots in batches of U: their positions and weights, then their rows,
    // are loaded together (a plain loop waited for each load in turn); the
    // products are added in slot order as before
    constexpr int U = 8;
    for (int jb = 0; jb < k; jb += U) {
      int src[U];
      float wt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = t * k + jb + u;
        const bool on = jb + u < k;
        const int sp = on ? (slot_pos ? slot_pos[i] : i) : -1;
        src[u] = (sp >= 0 && sp < N) ? sp : -1;
        wt[u] = (on && w) ? w[i] : 1.0f;
      }
      chunk8<T> v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = src[u] >= 0 ? load_chunk_stream<T>(y + (size_t)src[u] * H + 8 * c) : zero_chunk<T>();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (src[u] < 0) continue;
        if constexpr (sizeof(T) == 2) {
          const uint32_t* d = reinterpret_cast<const uint32_t*>(&v[u].v);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            acc[2 * x] = fmaf(wt[u], bf16_bits_to_f32(d[x] & 0xffffu), acc[2 * x]);
            acc[2 * x + 1] = fmaf(wt[u], bf16_bits_to_f32(d[x] >> 16), acc[2 * x + 1]);
          }
        } else {
          const float* f0 = reinterpret_cast<const float*>(&v[u].lo);
          const float* f1 = reinterpret_cast<const float*>(&v[u].hi);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            acc[x] = fmaf(wt[u], f0[x], acc[x]);
            acc[4 + x] = fmaf(wt[u], f1[x], acc[4 + x]);
          }
        }
      }
    }
    if (add) {
      const chunk8<T> v = load_chunk<T>(add + (size_t)t * H + 8 * c);
      if constexpr (sizeof(T) == 2) {
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&v.v);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc[2 * x] += bf16_bits_to_f32(d[x] & 0xffffu);
          acc[2 * x + 1] += bf16_bits_to_f32(d[x] >> 16);
        }
      } else {
        const float* f0 = reinterpret_cast<const float*>(&v.lo);
        const float* f1 = reinterpret_cast<const float*>(&v.hi);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc[x] += f0[x];
          acc[4 + x] += f1[x];
        }
      }
    }
    T* o = out + (size_t)t * H + 8 * c;
    if constexpr (sizeof(T) == 2) {
      uint32_t d[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        d[x] = (uint32_t)f32_to_bf16_bits(acc[2 * x]) |
               ((uint32_t)f32_to_bf16_bits(acc[2 * x + 1]) << 16);
      *reinterpret_cast<u32x4*>(o) = u32x4{d[0], d[1], d[2], d[3]};
    } else {
      reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, const void* y, const int32_t* slot_pos, const float* w,
                          int T, int k, int H, const void* add, void* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const long long total = (long long)T * (H / 8);
  const int grid = (int)std::min<long long>((total + 255) / 256, 16384);
  if (bf16)
    combine_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)y, slot_pos, w, T, k, H,
                                                (const bf16_t*)add, (bf16_t*)out);
  else
    combine_kernel<float><<<grid, 256, 0, s>>>((const float*)y, slot_pos, w, T, k, H,
                                               (const float*)add, (float*)out);
  return hipGetLastError();
}

}  // namespace moe
