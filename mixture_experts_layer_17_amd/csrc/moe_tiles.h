// Device-side M-tile list for the grouped GEMMs, built by one 256-thread
// block from the per-expert row ranges.  An expert with c rows gets
// nt = ceil(c / BM) tiles of ceil(c / nt) rows rounded up to 16 (the last
// one shorter), so ragged groups are split evenly.  tiles[t] =
// {expert, first row, rows, 0}; *count = number of tiles.  The bound
// sum_e ceil(c_e / BM) <= floor(N / BM) + E sizes the list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Exclusive scan of v[0..255] (LDS) into out[0..256] by wave 0; out[256] is
// the total.  Every thread of the block must call it (it ends with a
// barrier); blocks of any size >= 64 threads work.
__device__ __forceinline__ void block_scan256(const int* v, int* out) {
  const int t = threadIdx.x;
  if (t < 64) {
    int a[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { a[q] = v[4 * t + q]; sum += a[q]; }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (t >= off) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) { out[4 * t + q] = run; run += a[q]; }
    if (t == 63) out[256] = incl;
  }
  __syncthreads();
}

// Thread e (< E) holds its expert's row range [lo, hi).  s_nt, s_start are
// LDS scratch of 256 and 257 ints.  Every thread of the block (256 or more
// threads) must call it; threads from 256 on only take part in the barriers.
__device__ __forceinline__ void build_tile_list(int E, int lo, int hi, int BM,
                                                int4* __restrict__ tiles,
                                                int32_t* __restrict__ count, int* s_nt,
                                                int* s_start) {
  const int e = threadIdx.x;
  const bool own = e < 256;
  const int c = (own && e < E) ? max(0, hi - lo) : 0;
  const int nt = (c + BM - 1) / BM;
  if (own) s_nt[e] = nt;
  __syncthreads();
  block_scan256(s_nt, s_start);
  if (e == 0) count[0] = s_start[256];
  if (own && nt > 0) {
    const int per = ((c + nt - 1) / nt + 15) & ~15;
    const int t0 = s_start[e];
    for (int t = 0; t < nt; ++t) {
      const int r0 = lo + t * per;
      tiles[t0 + t] = make_int4(e, r0, max(0, min(per, hi - r0)), 0);
    }
  }
  __syncthreads();
}

}  // namespace moe
