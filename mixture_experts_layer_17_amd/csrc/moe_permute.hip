// Expert histogram, offsets and the stable expert-major permutation.
//
// Semantics: MindSpore moe.py, MoE.permutation (argsort(stable=True) of the
// flattened expert ids; token index = flat index // top_k; bincount with
// minlength = num_experts).  Rank-major mode: transformers PR "Qwen3 moe",
// Ep2DpParallel._token_dispatch (received rows grouped by source rank, each
// group ordered by local expert, to be reshuffled to expert-major order).
//
// Token-choice mode, deterministic and atomic-free on the ordering:
//   1. chunk pass: the N flat slots are cut into chunks of 1024.  Each wave
//      takes 64 consecutive slots at a time and finds, with 8 ballots over
//      the expert id bits, the lanes holding the same expert; the lane's rank
//      among equal lanes below it is a popcount.  Per-expert counts of the 16
//      segments of a chunk are prefix-summed in LDS, giving each slot its
//      stable rank inside the chunk and the chunk's histogram.
//   (N <= 1024: both passes in one workgroup.)
//   2. place pass (one workgroup per chunk): every workgroup sums the chunk
//      histograms per expert (all chunks -> counts, earlier chunks -> the
//      chunk's base within the expert), scans the counts over experts into
//      offsets, and places its slots at offset + base + rank.
#include "moe_common.h"
#include "moe_internal.h"
#include "moe_tiles.h"

namespace moe {
namespace {

constexpr int PM_CHUNK = 1024;            // slots per chunk
constexpr int PM_SEG = 64;                // slots per wave step
constexpr int PM_NSEG = PM_CHUNK / PM_SEG;
constexpr int PM_MAXE = 256;
constexpr int PM_MAXSUB = 8;              // router blocks per chunk when folded
constexpr int PM_MAX_RE = 4096;           // rank-major: max R * E

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Pass 1: chunk histogram + stable rank of each slot inside its chunk.
__global__ __launch_bounds__(256) void permute_chunk_kernel(
    const int32_t* __restrict__ ids, int N, int E, int32_t* __restrict__ hist /*[nchunk][E]*/,
    int32_t* __restrict__ rank /*[N]*/) {
  __shared__ int s_cnt[PM_NSEG][PM_MAXE];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < PM_NSEG * PM_MAXE; i += 256) (&s_cnt[0][0])[i] = 0;
  __syncthreads();

  int my_e[4], my_rank[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int seg = q * 4 + wave;
    const int i = c * PM_CHUNK + seg * PM_SEG + lane;
    int e = (i < N) ? ids[i] : -1;
    const bool valid = (e >= 0 && e < E);
    if (!valid) e = -1;
    unsigned long long match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long bb = __ballot(bit);
      match &= bit ? bb : ~bb;
    }
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    my_e[q] = e;
    my_rank[q] = valid ? __popcll(match & below) : 0;
    // the lowest lane of each equal-expert group records the group size
    if (valid && (match & below) == 0ull) s_cnt[seg][e] = __popcll(match);
  }
  __syncthreads();
  // per-expert exclusive prefix over the 16 segments
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = 0;
#pragma unroll
    for (int sg = 0; sg < PM_NSEG; ++sg) {
      const int v = s_cnt[sg][e];
      s_cnt[sg][e] = run;
      run += v;
    }
    hist[(size_t)c * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int seg = q * 4 + wave;
    const int i = c * PM_CHUNK + seg * PM_SEG + lane;
    if (i < N) rank[i] = (my_e[q] >= 0) ? s_cnt[seg][my_e[q]] + my_rank[q] : -1;
  }
}

// Pass 2, one workgroup per chunk c (1024 threads, one slot each).  Thread
// (e, part) sums a quarter of the chunk histograms of expert e, both over
// all chunks (the expert's total) and over the chunks before c; the totals
// are scanned over experts into offsets; slot i of the chunk then goes to
// offsets[e] + (expert e's slots in earlier chunks) + its rank in the chunk.
// Every workgroup computes the same totals (integers, so identically), and
// workgroup 0 also writes counts, offsets and the grouped GEMMs' tile lists.
__global__ __launch_bounds__(1024) void permute_place_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ hist /*[nchunk][E]*/, int nchunk, int N, int E, int k,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int4* __restrict__ tiles_a, int32_t* __restrict__ count_a, int BM_a,
    int4* __restrict__ tiles_b, int32_t* __restrict__ count_b, int BM_b,
    const int32_t* __restrict__ sub /*[nsub][E] or NULL*/, int sub_slots) {
  __shared__ int s_tot_p[4][PM_MAXE];
  __shared__ int s_sub[PM_MAXSUB][PM_MAXE];
  __shared__ int s_bef_p[4][PM_MAXE];
  __shared__ int s_tot[PM_MAXE];
  __shared__ int s_off[PM_MAXE + 1];
  __shared__ int s_base[PM_MAXE];
  __shared__ int s_nt[PM_MAXE];
  __shared__ int s_start[PM_MAXE + 1];
  const int c = blockIdx.x;
  const int e = threadIdx.x & (PM_MAXE - 1);
  const int part = threadIdx.x >> 8;
  const int per = (nchunk + 3) / 4;
  const int c0 = part * per, c1 = min(nchunk, c0 + per);
  int tot = 0, bef = 0;
  // loads in batches of 8 in flight (a plain loop waited for each in turn)
  constexpr int U = 8;
  if (e < E)
    for (int cb = c0; cb < c1; cb += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = cb + u < c1 ? hist[(size_t)(cb + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot += v[u];
        bef += cb + u < c ? v[u] : 0;
      }
    }
  // Folded first pass: ranks count within the router's blocks of sub_slots
  // slots, so a slot's base also takes its expert's slots in the earlier
  // blocks of this chunk (an exclusive scan of their histograms).
  if (sub && part == 1 && e < E) {
    const int spc = PM_CHUNK / sub_slots;
    const int nsub = (N + sub_slots - 1) / sub_slots;
    int v[PM_MAXSUB];
#pragma unroll
    for (int q = 0; q < PM_MAXSUB; ++q) {
      const int b = c * spc + q;
      v[q] = (q < spc && b < nsub) ? sub[(size_t)b * E + e] : 0;
    }
    int run = 0;
#pragma unroll
    for (int q = 0; q < PM_MAXSUB; ++q) {
      s_sub[q][e] = run;
      run += v[q];
    }
  }
  s_tot_p[part][e] = tot;
  s_bef_p[part][e] = bef;
  __syncthreads();
  if (part == 0) s_tot[e] = s_tot_p[0][e] + s_tot_p[1][e] + s_tot_p[2][e] + s_tot_p[3][e];
  __syncthreads();
  block_scan256(s_tot, s_off);
  if (part == 0)
    s_base[e] = s_off[e] + s_bef_p[0][e] + s_bef_p[1][e] + s_bef_p[2][e] + s_bef_p[3][e];
  __syncthreads();

  const int i = c * PM_CHUNK + threadIdx.x;
  if (i < N) {
    const int ei = ids[i];
    const int rk = rank[i];
    int pos = -1;
    if (ei >= 0 && ei < E && rk >= 0) {
      pos = s_base[ei] + rk;
      if (sub) pos += s_sub[threadIdx.x / sub_slots][ei];
      if (pos >= N) pos = -1;
    }
    if (pos >= 0) {
      sorted_token[pos] = i / k;
      if (sorted_slot) sorted_slot[pos] = i;
    }
    slot_pos[i] = pos;
  }

  if (c != 0) return;   // uniform over the block
  if (part == 0 && e < E) {
    counts[e] = s_tot[e];
    offsets[e] = s_off[e];
  }
  if (threadIdx.x == 0) offsets[E] = s_off[E];
  if (tiles_a == nullptr && tiles_b == nullptr) return;   // uniform over the block
  const int lo = min(s_off[e], N), hi = min(s_off[e] + s_tot[e], N);
  if (tiles_a) build_tile_list(E, lo, hi, BM_a, tiles_a, count_a, s_nt, s_start);
  if (tiles_b) build_tile_list(E, lo, hi, BM_b, tiles_b, count_b, s_nt, s_start);
}

// Single-launch variant for N <= 1024 (one chunk): 16 waves, one 64-slot
// segment each; ranks, counts, offsets, placement and tile lists in one
// workgroup.
__global__ __launch_bounds__(1024) void permute_single_kernel(
    const int32_t* __restrict__ ids, int N, int E, int k, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ tiles_a,
    int32_t* __restrict__ count_a, int BM_a, int4* __restrict__ tiles_b,
    int32_t* __restrict__ count_b, int BM_b) {
  __shared__ int s_cnt[PM_NSEG][PM_MAXE];
  __shared__ int s_tot[PM_MAXE];
  __shared__ int s_off[PM_MAXE + 1];
  __shared__ int s_nt[PM_MAXE];
  __shared__ int s_start[PM_MAXE + 1];
  const int lane = threadIdx.x & 63;
  const int seg = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < PM_NSEG * PM_MAXE; i += 1024) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const int i = threadIdx.x;
  int e = (i < N) ? ids[i] : -1;
  const bool valid = (e >= 0 && e < E);
  if (!valid) e = -1;
  unsigned long long match = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const unsigned long long bb = __ballot(bit);
    match &= bit ? bb : ~bb;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rk_seg = valid ? __popcll(match & below) : 0;
  if (valid && (match & below) == 0ull) s_cnt[seg][e] = __popcll(match);
  __syncthreads();
  // per-expert exclusive prefix over the 16 segments (threads 0..255)
  if (threadIdx.x < PM_MAXE) {
    const int ee = threadIdx.x;
    int run = 0;
#pragma unroll
    for (int sg = 0; sg < PM_NSEG; ++sg) {
      const int v = ee < E ? s_cnt[sg][ee] : 0;
      s_cnt[sg][ee] = run;
      run += v;
    }
    s_tot[ee] = run;
  }
  __syncthreads();
  block_scan256(s_tot, s_off);
  if (i < N) {
    int pos = -1;
    if (valid) {
      pos = s_off[e] + s_cnt[seg][e] + rk_seg;
      if (pos >= N) pos = -1;
    }
    if (pos >= 0) {
      sorted_token[pos] = i / k;
      if (sorted_slot) sorted_slot[pos] = i;
    }
    slot_pos[i] = pos;
  }
  const int ee = threadIdx.x & (PM_MAXE - 1);
  if (threadIdx.x < PM_MAXE && ee < E) {
    counts[ee] = s_tot[ee];
    offsets[ee] = s_off[ee];
  }
  if (threadIdx.x == 0) offsets[E] = s_off[E];
  if (tiles_a == nullptr && tiles_b == nullptr) return;   // uniform over the block
  const int lo = min(s_off[ee], N), hi = min(s_off[ee] + s_tot[ee], N);
  if (tiles_a) build_tile_list(E, lo, hi, BM_a, tiles_a, count_a, s_nt, s_start);
  if (tiles_b) build_tile_list(E, lo, hi, BM_b, tiles_b, count_b, s_nt, s_start);
}

// Rank-major mode, pass 1 (one workgroup of 256 threads): prefix tables of
// the count matrix.
//   rm_start[r * E + e]: first received row of block (r, e) (rank-major order)
//   em_start[r * E + e]: first expert-major position of block (r, e)
__global__ __launch_bounds__(256) void rank_major_scan_kernel(
    const int32_t* __restrict__ C, int R, int E, int N, int32_t* __restrict__ rm_start,
    int32_t* __restrict__ em_start, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int s_v[256];
  __shared__ int s_x[257];
  const int t = threadIdx.x;
  const int RE = R * E;
  // rank-major prefix: thread t owns blocks [t * per, (t + 1) * per)
  const int per = (RE + 255) / 256;
  int sum = 0;
  for (int i = t * per; i < min(RE, (t + 1) * per); ++i) sum += max(0, C[i]);
  s_v[t] = sum;
  __syncthreads();
  block_scan256(s_v, s_x);
  int run = s_x[t];
  for (int i = t * per; i < min(RE, (t + 1) * per); ++i) {
    rm_start[i] = run;
    run += max(0, C[i]);
  }
  // expert totals and expert-major starts
  int tot = 0;
  if (t < E)
    for (int r = 0; r < R; ++r) tot += max(0, C[r * E + t]);
  __syncthreads();
  s_v[t] = tot;
  __syncthreads();
  block_scan256(s_v, s_x);
  if (t < E) {
    int acc = s_x[t];
    for (int r = 0; r < R; ++r) {
      em_start[r * E + t] = acc;
      acc += max(0, C[r * E + t]);
    }
    counts[t] = tot;
    offsets[t] = min(s_x[t], N);
  }
  if (t == 0) offsets[E] = min(s_x[256], N);
}

// Rank-major mode, pass 2: each received row finds its block by binary search
// over the rank-major starts and moves to the block's expert-major start.
__global__ __launch_bounds__(256) void rank_major_scatter_kernel(
    const int32_t* __restrict__ C, const int32_t* __restrict__ rm_start,
    const int32_t* __restrict__ em_start, int RE, int N, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos) {
  __shared__ int s_rm[PM_MAX_RE];
  for (int i = threadIdx.x; i < RE; i += 256) s_rm[i] = rm_start[i];
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  // largest block index b with s_rm[b] <= i (that block is non-empty)
  int lo = 0, hi = RE - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_rm[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int within = i - s_rm[b];
  if (within >= max(0, C[b])) { slot_pos[i] = -1; return; }   // rows beyond sum(C)
  const int p = em_start[b] + within;
  if (p < 0 || p >= N) { slot_pos[i] = -1; return; }
  sorted_token[p] = i;
  if (sorted_slot) sorted_slot[p] = i;
  slot_pos[i] = p;
}

template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ x,
                                                          const int32_t* __restrict__ idx,
                                                          int N, int H, int nrows_x,
                                                          T* __restrict__ out) {
  const int per_row = H / 8;
  const long long total = (long long)N * per_row;
  for (long long q = (long long)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (long long)gridDim.x * 256) {
    const int p = (int)(q / per_row);
    const int c = (int)(q % per_row);
    const int src = clampi(idx[p], 0, nrows_x - 1);
    const chunk8<T> v = load_chunk<T>(x + (size_t)src * H + 8 * c);
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x4*>(out + (size_t)p * H + 8 * c) = v.v;
    } else {
      reinterpret_cast<u32x4*>(out + (size_t)p * H + 8 * c)[0] = v.lo;
      reinterpret_cast<u32x4*>(out + (size_t)p * H + 8 * c)[1] = v.hi;
    }
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t permute_ws_bytes(int N, int E, int R) {
  if (R > 0) return 2 * align256((size_t)R * E * sizeof(int32_t));
  const size_t nchunk = (size_t)(N + PM_CHUNK - 1) / PM_CHUNK;
  return align256(nchunk * E * sizeof(int32_t)) + align256((size_t)N * sizeof(int32_t));
}

size_t permute_fold_ws_bytes(int T, int k, int E) {
  const size_t nsub = (size_t)(T + 15) / 16;
  return permute_ws_bytes(T * k, E, 0) + align256(nsub * E * sizeof(int32_t));
}

PermuteFold permute_fold_scratch(void* ws, int T, int k, int E) {
  const int N = T * k;
  const size_t nchunk = (size_t)(N + PM_CHUNK - 1) / PM_CHUNK;
  char* const b = (char*)ws;
  PermuteFold f;
  f.hist = (int32_t*)b;
  f.rank = (int32_t*)(b + align256(nchunk * E * sizeof(int32_t)));
  f.sub = (int32_t*)(b + permute_ws_bytes(N, E, 0));
  return f;
}

hipError_t launch_permute_topk(const int32_t* ids, int T, int k, int E, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_token, int32_t* sorted_slot,
                               int32_t* slot_pos, void* ws, hipStream_t s, void* tile_ws_a,
                               int BM_a, void* tile_ws_b, int BM_b, const PermuteFold* fold) {
  const int N = T * k;
  if (N <= 0) {
    hipError_t e = launch_fill_i32(counts, E, 0, s);
    if (e != hipSuccess) return e;
    return launch_fill_i32(offsets, E + 1, 0, s);
  }
  const int nchunk = (N + PM_CHUNK - 1) / PM_CHUNK;
  auto tl = [](void* w) { return w ? (int4*)((char*)w + 256) : (int4*)nullptr; };
  // the router's blocks of 16 tokens must tile the chunks exactly
  if (fold && (nchunk == 1 || PM_CHUNK % (16 * k) != 0 || PM_CHUNK / (16 * k) > PM_MAXSUB ||
               E > PM_MAXE))
    return hipErrorInvalidValue;
  if (nchunk == 1) {
    permute_single_kernel<<<1, 1024, 0, s>>>(ids, N, E, k, sorted_token, sorted_slot, slot_pos,
                                             counts, offsets, tl(tile_ws_a), (int32_t*)tile_ws_a,
                                             BM_a, tl(tile_ws_b), (int32_t*)tile_ws_b, BM_b);
    return hipGetLastError();
  }
  int32_t* hist = fold ? fold->hist : (int32_t*)ws;
  int32_t* rank = fold ? fold->rank
                       : (int32_t*)((char*)ws + align256((size_t)nchunk * E * sizeof(int32_t)));
  if (!fold) permute_chunk_kernel<<<nchunk, 256, 0, s>>>(ids, N, E, hist, rank);
  permute_place_kernel<<<nchunk, 1024, 0, s>>>(ids, rank, hist, nchunk, N, E, k, sorted_token,
                                               sorted_slot, slot_pos, counts, offsets,
                                               tl(tile_ws_a), (int32_t*)tile_ws_a, BM_a,
                                               tl(tile_ws_b), (int32_t*)tile_ws_b, BM_b,
                                               fold ? fold->sub : nullptr, 16 * k);
  return hipGetLastError();
}

hipError_t launch_permute_rank_major(const int32_t* C, int R, int N, int E, int32_t* counts,
                                     int32_t* offsets, int32_t* sorted_token,
                                     int32_t* sorted_slot, int32_t* slot_pos, void* ws,
                                     hipStream_t s) {
  int32_t* rm = (int32_t*)ws;
  int32_t* em = (int32_t*)((char*)ws + align256((size_t)R * E * sizeof(int32_t)));
  rank_major_scan_kernel<<<1, 256, 0, s>>>(C, R, E, N, rm, em, counts, offsets);
  if (N > 0)
    rank_major_scatter_kernel<<<(N + 255) / 256, 256, 0, s>>>(C, rm, em, R * E, N, sorted_token,
                                                              sorted_slot, slot_pos);
  return hipGetLastError();
}

hipError_t launch_gather_rows(bool bf16, const void* x, int x_rows, const int32_t* idx, int N,
                              int H, void* out, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const long long total = (long long)N * (H / 8);
  const int grid = (int)std::min<long long>((total + 255) / 256, 8192);
  // source indices are clamped to [0, x_rows)
  if (bf16)
    gather_rows_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)x, idx, N, H, x_rows,
                                                    (bf16_t*)out);
  else
    gather_rows_kernel<float><<<grid, 256, 0, s>>>((const float*)x, idx, N, H, x_rows,
                                                   (float*)out);
  return hipGetLastError();
}

}  // namespace moe
