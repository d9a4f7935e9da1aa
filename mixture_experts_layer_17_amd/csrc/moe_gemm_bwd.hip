// Backward grouped GEMMs of the MoE layer on gfx950: bf16 operands, MFMA
// 32x32x16 with float32 accumulation.
//
// The layer is trained through autograd on the pages (Qwen3-Omni issue #115,
// SpeedupMoeExperts' per-expert training loop; MindSpore moe.py,
// _run_experts_for_loop and MoE.forward).  Per expert e over its rows in
// expert-major order, with dY = w * dout[token] and dG = [dg | du]:
//   dgrad   dH_e = dout_e . down[e]^T          rows x I,  K = H
//           dX_e = dG_e . gate_up[e]^T         rows x H,  K = 2I
//   wgrad   d down[e]    = (w h)_e^T . dout_e  I x H,     K = rows of e
//           d gate_up[e] = X_e^T . dG_e        H x 2I,    K = rows of e
//
// dgrad: the weight is used as stored ([n][k], k contiguous), so both
// operands are row tiles of KB k per block (KB = 64: every row copy is one
// whole 128-byte line), XOR-swizzled like the forward's activation tile and
// read with ds_read_b128; no transposed copy of any weight exists.  The
// first dgrad's epilogue is the SwiGLU backward.
//
// wgrad: K runs over the expert's rows, so both operands arrive as k-rows
// with their output dimension contiguous, the layout of the forward's weight
// tile: 32-byte segments XOR-swizzled per row and read with the transposing
// ds_read_b64_tr_b16.  Both operands are expert-major buffers (the gathered
// x and dout rows are laid out once, before), so a copy's source is plain
// address arithmetic.  Rows past the expert's end read a zero row.  Every
// output element is reduced by one work-group over all of K: deterministic,
// no atomics; experts without rows get exact zeros.
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"
#include "moe_lds.h"

namespace moe {
namespace {

using namespace lds;

// The K loop shared by both kernels: a ring of STAGES LDS slots filled by
// issue(slot, block); wait_blocks(n) leaves n blocks of this wave's copies
// in flight (PRE: the caller has issued the first blocks itself).  A block
// holds KS k-steps of 16.  The fragments of the next
// k-step are read while the MFMAs of the current one run (read_b for the
// whole step, then each m-tile's read_a right after its MFMAs are issued);
// sched_barrier keeps that interleave.  One barrier per block sits before
// its last k-step: it publishes the next block and retires the one just
// read, whose slot is refilled at once.
template <int TM, int TN, int STAGES, int KS, bool PRE = false, class Issue, class Wait,
          class ReadA, class ReadB>
__device__ __forceinline__ void pipelined_k_loop(int KT, unsigned char* smem, int stage_bytes,
                                                 Issue&& issue, Wait&& wait_blocks,
                                                 ReadA&& read_a, ReadB&& read_b,
                                                 f32x16_v (&acc)[TM][TN]) {
  static_assert(KS >= 2, "k-steps per block");
  if constexpr (!PRE) {
#pragma unroll
    for (int p = 0; p < STAGES; ++p)
      if (p < KT) issue(smem + p * stage_bytes, p);
  }
  if (KT <= 0) return;
  wait_blocks(min(STAGES, KT) - 1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  bf16x8_v bf[2][TN], af[TM];   // k-step s of a block multiplies bf[s & 1]
  auto mma_roll = [&](const bf16x8_v (&b)[TN], const unsigned char* nbase, int nkk) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], af[i], acc[i][j], 0, 0, 0);
      af[i] = read_a(nbase, nkk, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_bs = [&](const unsigned char* base, int kk, bf16x8_v (&b)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = read_b(base, kk, j);
  };
  read_bs(smem, 0, bf[0]);
#pragma unroll
  for (int i = 0; i < TM; ++i) af[i] = read_a(smem, 0, i);
  // k-steps 0 .. KS - 2 of block 0, each reading the next
#pragma unroll
  for (int st = 0; st + 1 < KS; ++st) {
    read_bs(smem, st + 1, bf[(st + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    mma_roll(bf[st & 1], smem, st + 1);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (KT > 1) wait_blocks(min(STAGES - 2, KT - 2));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int slot = 0;
  for (int kb = 0; kb + 1 < KT; ++kb) {
    unsigned char* cur = smem + slot * stage_bytes;
    slot = (slot + 1 == STAGES) ? 0 : slot + 1;
    unsigned char* nxt = smem + slot * stage_bytes;
    if (kb + STAGES < KT) issue(cur, kb + STAGES);
    // last k-step of block kb, reading block kb + 1's first
    read_bs(nxt, 0, bf[KS & 1]);
    __builtin_amdgcn_sched_barrier(0);
    mma_roll(bf[(KS - 1) & 1], nxt, 0);
    // k-steps 0 .. KS - 2 of block kb + 1, each reading the next
#pragma unroll
    for (int st = 0; st + 1 < KS; ++st) {
      read_bs(nxt, st + 1, bf[(KS + st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma_roll(bf[(KS + st) & 1], nxt, st + 1);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (kb + 2 < KT) wait_blocks(min(STAGES - 2, KT - 3 - kb));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[(KS - 1) & 1][j], af[i], acc[i][j], 0, 0, 0);
}

// ---------------------------------------------------------------- dgrad

enum { DG_PLAIN = 0, DG_SWIGLU_BWD = 1 };

// Row chunk swizzle of a dgrad stage: rows of KB k hold KB / 8 chunks of 16
// bytes.  Four chunks take the measured f(row); eight (whole 128-byte lines)
// take (row >> 1) & 7, so the 16 rows one 16-lane phase of a ds_read_b128
// reads fall on 16 distinct 16-byte bank groups.
template <int KB>
__device__ __forceinline__ int dswz(int row) {
  if constexpr (KB == 32) return fswz(row);
  else return (row >> 1) & 7;
}

template <int BM, int BN, int WM, int WN, int STAGES, int KB>
struct dcfg {
  static_assert(KB == 32 || KB == 64, "k per block");
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = NW * 64;
  static constexpr int TM = BM / 32 / WM;            // 32-row m-tiles per wave
  static constexpr int CW = BN / WN;                 // output columns per wave
  static constexpr int TN = CW / 32;                 // 32-column n-tiles per wave
  static constexpr int KS = KB / 16;                 // MFMA k-steps per block
  static constexpr int CH = KB / 8;                  // 16-byte chunks per row
  static constexpr int ROWB = KB * 2;                // bytes per stage row
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;   // A rows then B rows
  static constexpr int RING = STAGES * STAGE_BYTES;
  static constexpr int INST = STAGE_BYTES / 1024;    // wave copies per stage
  static constexpr int PER = INST / NW;
  static constexpr int A_INST = BM * ROWB / 1024;    // of which activation rows
  // activation copies come first in each wave's list (u < A_PER); the last
  // of them may be left out (below) when they split evenly over the waves
  static constexpr int A_PER = A_INST % NW == 0 ? A_INST / NW : 0;
  static constexpr int OBF = CW * 4 + 16;            // fp32 staging row stride
  static constexpr int OBP = CW * 2 + 8;             // bf16 staging row stride
  static constexpr int STG = 32 * OBF * NW;
  static constexpr int LDS = RING > STG ? RING : STG;
  static_assert(BM % (32 * WM) == 0 && TM >= 1 && TN >= 1, "wave tiles");
  static_assert(INST % NW == 0, "copies split evenly over the waves");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Epilogue operands of the SwiGLU backward (DG_SWIGLU_BWD).
struct SwigluBwd {
  const bf16_t* G;        // [N, 2I] pre-activations saved by the forward
  int ldg, up_off;        // 2I, I
  const float* w;         // routing weights, flat slot order
  const int32_t* slot;    // sorted_slot: flat slot of each expert-major row
  bf16_t* dG;             // [N, 2I]
  bf16_t* hw;             // [N, I]  w * silu(g) * u
  int ldh;
  float* dw_part;         // [N, I / 64] <z, silu(g) u> per 64-column slice, or NULL
  int dw_ld;              // I / 64
};

// Column slice of the first dgrad's epilogue (CW of its configs): one
// partial routing-weight gradient per expert-major row and slice.
constexpr int kDgrad1Slice = 64;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over each 16-lane row (pairs, quads, half-rows, rows): every lane of
// the row ends with the same value, in a fixed order.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  return v;
}

// A dense problem folded into a dgrad launch (the shared expert): `rows`
// rows of X read in order against one weight, outputs in row order, with its
// own epilogue operands.
struct DgradAux {
  const bf16_t* X;
  int ldx;
  const bf16_t* W;
  int ldw, K;
  bf16_t* C;
  int ldc, rows, n_ntiles, jobs;
  SwigluBwd sb;
};

template <int BM, int BN, int WM, int WN, int STAGES, int KB, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void dgrad_kernel(
    const bf16_t* __restrict__ gX, int g_ldx, const int32_t* __restrict__ g_x_index, int g_x_rows,
    const bf16_t* __restrict__ gW, long long g_w_estride, int g_ldw, int g_K,
    bf16_t* __restrict__ gC, int g_ldc, const int32_t* __restrict__ g_c_index, int g_c_rows,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tiles_count, int g_n_ntiles,
    SwigluBwd g_sb, DgradAux aux) {
  using G = dcfg<BM, BN, WM, WN, STAGES, KB>;
  extern __shared__ __align__(16) unsigned char smem[];

  // each XCD takes an equal share of the dense jobs first, then of the
  // grouped ones
  const int g_jobs = tiles_count[0] * g_n_ntiles;
  const int d_per = (aux.jobs + NUM_XCD - 1) / NUM_XCD;
  const int g_per = (g_jobs + NUM_XCD - 1) / NUM_XCD;
  const int xcd = blockIdx.x % NUM_XCD;
  const int local = blockIdx.x / NUM_XCD;
  const bool dense = local < d_per;   // uniform over the work-group
  int job;
  if (dense) {
    job = xcd * d_per + local;
    if (job >= aux.jobs) return;
  } else {
    if (local - d_per >= g_per) return;
    job = xcd * g_per + (local - d_per);
    if (job >= g_jobs) return;
  }
  const int n_ntiles = dense ? aux.n_ntiles : g_n_ntiles;
  const int mt = job / n_ntiles;
  const int nt = job - mt * n_ntiles;
  int e = 0, row0, rows;
  if (dense) {
    row0 = mt * BM;
    rows = min(BM, aux.rows - row0);
  } else {
    const int4 tile = tiles[mt];
    e = tile.x;
    row0 = tile.y;
    rows = tile.z;
  }
  const int n0 = nt * BN;
  const bf16_t* __restrict__ X = dense ? aux.X : gX;
  const int ldx = dense ? aux.ldx : g_ldx;
  const int32_t* __restrict__ x_index = dense ? nullptr : g_x_index;
  const int x_rows = dense ? aux.rows : g_x_rows;
  const bf16_t* __restrict__ W = dense ? aux.W : gW;
  const long long w_estride = dense ? 0 : g_w_estride;
  const int ldw = dense ? aux.ldw : g_ldw;
  const int K = dense ? aux.K : g_K;
  bf16_t* __restrict__ C = dense ? aux.C : gC;
  const int ldc = dense ? aux.ldc : g_ldc;
  const int32_t* __restrict__ c_index = dense ? nullptr : g_c_index;
  const int c_rows = dense ? aux.rows : g_c_rows;
  const SwigluBwd& sb = dense ? aux.sb : g_sb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bf16_t* We = W + (long long)e * w_estride;

  // copy assignments: stage row r < BM is activation row r of the tile, row
  // BM + c is weight row n0 + c; lane q of a copy moves chunk
  // (q % CH) ^ swizzle(r)
  const bf16_t* src[G::PER];
#pragma unroll
  for (int u = 0; u < G::PER; ++u) {
    const int inst = wave + u * G::NW;
    const int q = inst * 64 + lane;
    const int r = q / G::CH;
    const int c = (q % G::CH) ^ dswz<KB>(r);
    if (r < BM) {
      int s = row0 + min(r, rows - 1);
      if (x_index) s = x_index[s];
      s = min(max(s, 0), x_rows - 1);
      src[u] = X + (long long)s * ldx + 8 * c;
    } else {
      src[u] = We + (long long)(n0 + r - BM) * ldw + 8 * c;
    }
  }
  // A wave's last activation copy is left out when all its rows lie past
  // the tile's end: those rows feed only outputs that are never stored.
  // The choice is per wave, and so are the vmcnt counts it changes.  Only
  // where the accumulators take at most half of a wave's registers: with
  // both copy counts in one kernel the 320 x 256 tile spilled 10 registers
  // and its launch ran 8 % slower.
  constexpr int UA = G::A_PER - 1;
  constexpr bool SKIP_OK = G::A_PER > 0 && G::TM * G::TN * 16 <= 128;
  const int skl = __builtin_amdgcn_readfirstlane(
      (SKIP_OK && (wave + UA * G::NW) * (64 / G::CH) >= rows) ? 1 : 0);
  const int KT = K / KB;

  // fragment offsets: lane l reads row 32 t + l % 32, k chunk 2 kk + l / 32;
  // the swizzle depends on l % 32 only (tiles start at multiples of 32), so
  // m- and n-tiles are constant offsets from the wave's first
  const int l32 = lane & 31, hl = lane >> 5;
  int a_off[G::KS], b_off[G::KS];
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk) {
    const int ch = 16 * ((2 * kk + hl) ^ dswz<KB>(l32));
    a_off[kk] = (32 * wm + l32) * G::ROWB + ch;
    b_off[kk] = (BM + wn * G::CW + l32) * G::ROWB + ch;
  }

  f32x16_v acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  auto read_a = [&](const unsigned char* base, int kk, int i) {
    return __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4*>(
                                            base + a_off[kk] + 32 * WM * G::ROWB * i));
  };
  auto read_b = [&](const unsigned char* base, int kk, int j) {
    return __builtin_bit_cast(bf16x8_v,
                              *reinterpret_cast<const u32x4*>(base + b_off[kk] + 32 * G::ROWB * j));
  };
  auto run = [&](auto sk_c) {
    constexpr int SK = decltype(sk_c)::value;
    constexpr int PX = G::PER - SK;               // this wave's copies per block
    // called once per block, in block order
    auto issue = [&](unsigned char* base, int) {
#pragma unroll
      for (int u = 0; u < G::PER; ++u) {
        if (SK && u == UA) continue;
        copy16_to_lds(src[u], base + (wave + u * G::NW) * 1024);
        src[u] += KB;
      }
    };
    auto wait_blocks = [&](int nb) {
      static_assert(STAGES <= 4 && (STAGES - 1) * PX < 64, "wait table");
      switch (nb) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<PX>(); break;
        case 2: wait_vmcnt<2 * PX>(); break;
        default: wait_vmcnt<3 * PX>(); break;
      }
    };
    pipelined_k_loop<G::TM, G::TN, STAGES, G::KS>(KT, smem, G::STAGE_BYTES, issue, wait_blocks,
                                                  read_a, read_b, acc);
  };
  if constexpr (SKIP_OK) {
    if (skl) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }

  // ---- epilogue.  acc[i][j][q] = C[row 32 (wm + WM i) + l % 32]
  //                                 [col wn CW + 32 j + 8 (q / 4) + 4 hl + q % 4]
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (EPI == DG_PLAIN) {
    constexpr int LPR = G::CW * 2 / 16;        // lanes per staged row
    constexpr int RPI = 64 / LPR;
    unsigned char* stg = smem + wave * 32 * G::OBP;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16_v& v = acc[i][j];
          const uint2 d = make_uint2(
              (uint32_t)f32_to_bf16_bits(v[4 * a]) | ((uint32_t)f32_to_bf16_bits(v[4 * a + 1]) << 16),
              (uint32_t)f32_to_bf16_bits(v[4 * a + 2]) |
                  ((uint32_t)f32_to_bf16_bits(v[4 * a + 3]) << 16));
          *reinterpret_cast<uint2*>(stg + l32 * G::OBP + 2 * (32 * j + 8 * a + 4 * hl)) = d;
        }
#pragma unroll
      for (int rr = 0; rr < 32 / RPI; ++rr) {
        const int r = rr * RPI + lane / LPR;
        const int m = 32 * (wm + WM * i) + r;
        const uint2 lo = *reinterpret_cast<const uint2*>(stg + r * G::OBP + 16 * (lane % LPR));
        const uint2 hi = *reinterpret_cast<const uint2*>(stg + r * G::OBP + 16 * (lane % LPR) + 8);
        if (m < rows) {
          const int dst = c_index ? c_index[row0 + m] : row0 + m;
          if (dst >= 0 && dst < c_rows)   // read once, by the input gradient
            __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y},
                                        reinterpret_cast<u32x4*>(C + (long long)dst * ldc + n0 +
                                                                 wn * G::CW + 8 * (lane % LPR)));
        }
      }
    }
  } else {
    static_assert(G::CW == kDgrad1Slice, "one partial per slice of the first dgrad");
    // SwiGLU backward.  z = dout . down^T for row p, column n of I:
    //   h = silu(g) u,  dh = w z,  du = dh silu(g),  dg = dh u silu'(g),
    //   hw = w h   (the first operand of the down-projection's wgrad)
    constexpr int LPR = G::CW * 4 / 16;        // lanes per staged fp32 row
    constexpr int RPI = 64 / LPR;
    static_assert(LPR == 16, "a staged row is one 16-lane DPP row");
    unsigned char* stg = smem + wave * 32 * G::OBF;
    float hzs[G::TM][32 / RPI];   // this lane's part of <z, h> per staged row
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16_v& v = acc[i][j];
          *reinterpret_cast<float4*>(stg + l32 * G::OBF + 4 * (32 * j + 8 * a + 4 * hl)) =
              make_float4(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
        }
#pragma unroll
      for (int rr = 0; rr < 32 / RPI; ++rr) {
        const int r = rr * RPI + lane / LPR;
        const int m = 32 * (wm + WM * i) + r;
        const float4 z = *reinterpret_cast<const float4*>(stg + r * G::OBF + 16 * (lane % LPR));
        float hz = 0.f;   // <z, silu(g) u> over this lane's 4 columns
        if (m < rows) {
          const int p = row0 + m;
          const int n = n0 + wn * G::CW + 4 * (lane % LPR);
          const float wt = sb.w ? sb.w[sb.slot ? sb.slot[p] : p] : 1.0f;
          const uint2 g2 = *reinterpret_cast<const uint2*>(sb.G + (long long)p * sb.ldg + n);
          const uint2 u2 = *reinterpret_cast<const uint2*>(sb.G + (long long)p * sb.ldg + sb.up_off + n);
          const float zz[4] = {z.x, z.y, z.z, z.w};
          const uint32_t gw[2] = {g2.x, g2.y}, uw[2] = {u2.x, u2.y};
          uint32_t dg[2], du[2], hv[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            float o_dg[2], o_du[2], o_h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const float g = bf16_bits_to_f32(hh ? gw[c] >> 16 : gw[c] & 0xffffu);
              const float u = bf16_bits_to_f32(hh ? uw[c] >> 16 : uw[c] & 0xffffu);
              const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              const float a = g * s;
              const float dh = wt * zz[2 * c + hh];
              o_du[hh] = dh * a;
              o_dg[hh] = dh * u * (s * (1.0f + g * (1.0f - s)));
              o_h[hh] = wt * (a * u);
              hz = fmaf(zz[2 * c + hh], a * u, hz);
            }
            dg[c] = (uint32_t)f32_to_bf16_bits(o_dg[0]) | ((uint32_t)f32_to_bf16_bits(o_dg[1]) << 16);
            du[c] = (uint32_t)f32_to_bf16_bits(o_du[0]) | ((uint32_t)f32_to_bf16_bits(o_du[1]) << 16);
            hv[c] = (uint32_t)f32_to_bf16_bits(o_h[0]) | ((uint32_t)f32_to_bf16_bits(o_h[1]) << 16);
          }
          *reinterpret_cast<uint2*>(sb.dG + (long long)p * sb.ldg + n) = make_uint2(dg[0], dg[1]);
          *reinterpret_cast<uint2*>(sb.dG + (long long)p * sb.ldg + sb.up_off + n) =
              make_uint2(du[0], du[1]);
          *reinterpret_cast<uint2*>(sb.hw + (long long)p * sb.ldh + n) = make_uint2(hv[0], hv[1]);
        }
        hzs[i][rr] = hz;
      }
    }
    if (sb.dw_part) {
      // after every row is written (so the loop above keeps its loads in
      // flight): the 16 lanes of a staged row add their parts, the first
      // stores the slice's partial
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int rr = 0; rr < 32 / RPI; ++rr) {
          const float v = row16_sum(hzs[i][rr]);
          const int m = 32 * (wm + WM * i) + rr * RPI + lane / LPR;
          if (m < rows && lane % LPR == 0)
            sb.dw_part[(long long)(row0 + m) * sb.dw_ld + (n0 + wn * G::CW) / kDgrad1Slice] = v;
        }
    }
  }
}

// ---------------------------------------------------------------- wgrad

template <int BM, int BN, int WM, int WN, int STAGES>
struct wcfg {
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = NW * 64;
  static constexpr int TM = BM / 32 / WM;            // 32-row m-tiles per wave
  static constexpr int CW = BN / WN;                 // output columns per wave
  static constexpr int TN = CW / 32;
  static constexpr int A_ROWB = BM * 2;              // bytes per k-row
  static constexpr int B_ROWB = BN * 2;
  static constexpr int A_BYTES = BK * A_ROWB;
  static constexpr int B_BYTES = BK * B_ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int RING = STAGES * STAGE_BYTES;
  static constexpr int A_INST = A_BYTES / 1024;
  static constexpr int INST = STAGE_BYTES / 1024;
  static constexpr int PER = INST / NW;
  static constexpr int OBP = CW * 2 + 8;
  static constexpr int STG = 32 * OBP * NW;
  static constexpr int LDS = RING > STG ? RING : STG;
  static_assert(BM / 16 >= 8 && BN / 16 >= 8, "swizzle needs 8 segments per row");
  static_assert(INST % NW == 0 && A_BYTES % 1024 == 0, "copies split evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tiles");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int BM, int BN, int WM, int WN, int STAGES, bool PERSIST = false>
__global__ __launch_bounds__(WM * WN * 64) void wgrad_kernel(
    const bf16_t* __restrict__ gA, int g_lda, const bf16_t* __restrict__ gB, int g_ldb,
    const bf16_t* __restrict__ zero_row, const int32_t* __restrict__ offsets, int E, int M,
    int N, bf16_t* __restrict__ gC, long long g_c_estride, int g_ldc, WgradAux aux,
    unsigned* __restrict__ job_counters) {
  using G = wcfg<BM, BN, WM, WN, STAGES>;
  extern __shared__ __align__(16) unsigned char smem[];

  // ---- jobs (expert, m-tile, n-tile); consecutive jobs share an expert's
  // rows.  Each XCD takes an equal share of the dense problem's jobs (all of
  // its rows each: the long ones go first), then of the grouped jobs.
  // PERSIST: one work-group per CU takes the jobs of its XCD's share one at
  // a time from that XCD's counter in job_counters (zero at launch; one
  // vector atomic per job, issued a job ahead), so the CUs of an XCD stay
  // balanced even when a share mixes long dense jobs with short grouped
  // ones; the next job's first block is copied into slot 0 while the
  // current job's epilogue stages through the other slots, so the K loop of
  // every job but the first starts on a landed block (measured 9 % faster at
  // the prefill shape: the jobs are short, K being an expert's rows).
  const int m_tiles = M / BM, n_tiles = N / BN;
  const int g_jobs = E * m_tiles * n_tiles;
  const int d_per = (aux.jobs + NUM_XCD - 1) / NUM_XCD;
  const int g_per = (g_jobs + NUM_XCD - 1) / NUM_XCD;
  const int xcd = blockIdx.x % NUM_XCD;
  const int lstride = PERSIST ? max(1, (int)(gridDim.x / NUM_XCD)) : (1 << 30);
  // the first share index >= loc that holds a job, or -1 (uniform)
  auto next_job = [&](int loc) {
    while (loc < d_per + g_per) {
      if (loc < d_per) {
        if (xcd * d_per + loc < aux.jobs) return loc;
      } else {
        // grouped jobs of a share are contiguous: past the end, none follow
        return xcd * g_per + (loc - d_per) < g_jobs ? loc : -1;
      }
      loc += lstride;
    }
    return -1;
  };
  struct Job {
    int e, m0, n0, lo, hi, lda, ldb, ldc;   // rows [lo, hi) of expert e
    const bf16_t* A;
    const bf16_t* B;
    bf16_t* C;
    long long c_estride;
  };
  // PERSIST: the XCD's share without holes, dense jobs first
  const int d_lo = min(xcd * d_per, aux.jobs);
  const int d_cnt = max(0, min(d_per, aux.jobs - d_lo));
  const int g_lo = min(xcd * g_per, g_jobs);
  const int g_cnt = max(0, min(g_per, g_jobs - g_lo));
  const int share = d_cnt + g_cnt;
  auto make_job = [&](int loc) {
    Job J;
    const bool dense = PERSIST ? loc < d_cnt : loc < d_per;
    const int job = PERSIST ? (dense ? d_lo + loc : g_lo + (loc - d_cnt))
                            : (dense ? xcd * d_per + loc : xcd * g_per + (loc - d_per));
    const int nt_of = dense ? aux.N / BN : n_tiles;
    J.e = dense ? 0 : job / (m_tiles * n_tiles);
    const int rem = dense ? job : job - J.e * m_tiles * n_tiles;
    const int mt = rem / nt_of;
    const int nt = rem - mt * nt_of;
    J.m0 = mt * BM;
    J.n0 = nt * BN;
    J.lo = dense ? 0 : offsets[J.e];
    J.hi = dense ? aux.rows : max(offsets[J.e + 1], J.lo);
    J.A = dense ? (const bf16_t*)aux.A : gA;
    J.lda = dense ? aux.lda : g_lda;
    J.B = dense ? (const bf16_t*)aux.B : gB;
    J.ldb = dense ? aux.ldb : g_ldb;
    J.C = dense ? (bf16_t*)aux.C : gC;
    J.c_estride = dense ? 0 : g_c_estride;
    J.ldc = dense ? aux.N : g_ldc;
    return J;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bf16_t* zr = zero_row;

  // copy u of this wave moves 1 KB = 1024 / ROWB k-rows of the A or B tile;
  // lane q takes 16-byte piece p of k-row r, whose 32-byte segment is
  // swizzled by h(r)
  int c_col0[G::PER], c_row[G::PER], c_lds[G::PER];
  bool c_isa[G::PER];
#pragma unroll
  for (int u = 0; u < G::PER; ++u) {
    const int inst = wave + u * G::NW;
    const bool isa = inst < G::A_INST;
    const int rowb = isa ? G::A_ROWB : G::B_ROWB;
    const int local_inst = isa ? inst : inst - G::A_INST;
    const int q = local_inst * 64 + lane;
    const int r = q / (rowb / 16);
    const int p = q % (rowb / 16);
    const int seg = (p >> 1) ^ hswz(r);
    c_isa[u] = isa;
    c_row[u] = r;
    c_col0[u] = 16 * seg + 8 * (p & 1);
    c_lds[u] = (isa ? 0 : G::A_BYTES) + local_inst * 1024;
  }
  // source of copy u for K-block kb of job I (the job whose blocks are
  // being issued): expert-major row lo + 32 kb + r, or the zero row past
  // the expert's end
  Job I;
  auto issue = [&](unsigned char* base, int kb) {
#pragma unroll
    for (int u = 0; u < G::PER; ++u) {
      const int rg = I.lo + kb * BK + c_row[u];
      const bf16_t* g = rg < I.hi ? (c_isa[u] ? I.A + (long long)rg * I.lda + I.m0
                                              : I.B + (long long)rg * I.ldb + I.n0)
                                  : zr;
      copy16_to_lds(g + c_col0[u], base + c_lds[u]);
    }
  };
  auto wait_blocks = [&](int nb) {
    static_assert(STAGES <= 4 && (STAGES - 1) * G::PER < 64, "wait table");
    switch (nb) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<G::PER>(); break;
      case 2: wait_vmcnt<2 * G::PER>(); break;
      default: wait_vmcnt<3 * G::PER>(); break;
    }
  };

  // transposing fragment reads: 16-lane group q reads columns 16 (q & 1) ..
  // + 15 and k 8 (q >> 1) .. + 7 of a 32-column sub-tile
  const int gq = lane >> 4, s16 = lane & 15;
  const int wrow = 8 * (gq >> 1) + (s16 >> 2);
  const int wsw = ((s16 >> 2) << 1) | (gq >> 1);
  auto frag_off = [&](int rowb, int cb) {
    const int col = cb + 16 * (gq & 1) + 4 * (s16 & 3);
    return wrow * rowb + 32 * ((col >> 4) ^ wsw) + 2 * (col & 15);
  };
  int a_off[G::TM], b_off[G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i) a_off[i] = frag_off(G::A_ROWB, (BM / WM) * wm + 32 * i);
#pragma unroll
  for (int j = 0; j < G::TN; ++j) b_off[j] = G::A_BYTES + frag_off(G::B_ROWB, G::CW * wn + 32 * j);
  auto read_tr = [](const unsigned char* p, int rowb) {
    const i16x4_v x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4_v x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * rowb));
    return __builtin_bit_cast(bf16x8_v, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_a = [&](const unsigned char* base, int kk, int i) {
    return read_tr(base + a_off[i] + 16 * kk * G::A_ROWB, G::A_ROWB);
  };
  auto read_b = [&](const unsigned char* base, int kk, int j) {
    return read_tr(base + b_off[j] + 16 * kk * G::B_ROWB, G::B_ROWB);
  };
  const int l32 = lane & 31, hl = lane >> 5;
  constexpr int LPR = G::CW * 2 / 16;
  constexpr int RPI = 64 / LPR;
  // PERSIST stages the output through slots 1 .. STAGES - 1 (slot 0 holds
  // the next job's first block)
  static_assert(!PERSIST || 32 * G::OBP * G::NW <= (STAGES - 1) * G::STAGE_BYTES, "staging");

  // PERSIST: thread 0 takes share indices from the XCD's counter; the one
  // for the next job is taken while this one runs and published through
  // LDS at its epilogue.  Publications alternate between two LDS words: a
  // job without rows passes no barrier in its K loop, so the word read
  // after one publication's barrier is written again only after the next
  // publication's barrier, which every wave reaches after its read.
  unsigned* const ctr = PERSIST ? job_counters + xcd : nullptr;
  int* const s_loc = reinterpret_cast<int*>(smem + G::LDS);
  int pub = 0;   // LDS word of the next publication
  int pref = 0;
  int loc;
  if constexpr (PERSIST) {
    if (tid == 0) s_loc[0] = (int)atomicAdd(ctr, 1u);
    __syncthreads();
    loc = s_loc[0];
    pub = 1;
    if (loc >= share) return;
    if (tid == 0) pref = (int)atomicAdd(ctr, 1u);
  } else {
    loc = next_job((int)(blockIdx.x / NUM_XCD));
    if (loc < 0) return;
  }
  Job J = make_job(loc);   // the job being multiplied and stored
  I = J;
  int KT = (J.hi - J.lo + BK - 1) / BK;
#pragma unroll
  for (int p = 0; p < STAGES; ++p)
    if (p < KT) issue(smem + p * G::STAGE_BYTES, p);
  f32x16_v acc[G::TM][G::TN];
  for (;;) {
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    // the loop's first wait also covers anything issued before block 1,
    // such as the previous job's output stores
    pipelined_k_loop<G::TM, G::TN, STAGES, 2, true>(KT, smem, G::STAGE_BYTES, issue, wait_blocks,
                                                     read_a, read_b, acc);
    // ---- epilogue: acc[i][j][q] = C[m0 + (BM / WM) wm + 32 i + l % 32]
    //                                 [n0 + CW wn + 32 j + 8 (q / 4) + 4 hl + q % 4]
    int nloc = -1, nKT = 0;
    if constexpr (PERSIST) {
      if (tid == 0) s_loc[pub] = pref;
      __syncthreads();                            // the ring is free; the index is visible
      nloc = s_loc[pub];
      pub ^= 1;
      if (nloc >= share) nloc = -1;
      if (nloc >= 0) {
        if (tid == 0) pref = (int)atomicAdd(ctr, 1u);
        I = make_job(nloc);
        nKT = (I.hi - I.lo + BK - 1) / BK;
        if (nKT > 0) issue(smem, 0);
      }
    } else {
      __builtin_amdgcn_s_barrier();               // every wave is done with the ring
      asm volatile("" ::: "memory");
    }
    unsigned char* stg = smem + (PERSIST ? G::STAGE_BYTES : 0) + wave * 32 * G::OBP;
    bf16_t* Ce = J.C + (long long)J.e * J.c_estride;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16_v& v = acc[i][j];
          const uint2 d = make_uint2(
              (uint32_t)f32_to_bf16_bits(v[4 * a]) | ((uint32_t)f32_to_bf16_bits(v[4 * a + 1]) << 16),
              (uint32_t)f32_to_bf16_bits(v[4 * a + 2]) | ((uint32_t)f32_to_bf16_bits(v[4 * a + 3]) << 16));
          *reinterpret_cast<uint2*>(stg + l32 * G::OBP + 2 * (32 * j + 8 * a + 4 * hl)) = d;
        }
#pragma unroll
      for (int rr = 0; rr < 32 / RPI; ++rr) {
        const int r = rr * RPI + lane / LPR;
        const int m = J.m0 + (BM / WM) * wm + 32 * i + r;
        const uint2 x0 = *reinterpret_cast<const uint2*>(stg + r * G::OBP + 16 * (lane % LPR));
        const uint2 x1 = *reinterpret_cast<const uint2*>(stg + r * G::OBP + 16 * (lane % LPR) + 8);
        // the weight gradients are not read again here: non-temporal stores
        __builtin_nontemporal_store(
            u32x4{x0.x, x0.y, x1.x, x1.y},
            reinterpret_cast<u32x4*>(Ce + (long long)m * J.ldc + J.n0 + wn * G::CW + 8 * (lane % LPR)));
      }
    }
    if (nloc < 0) break;
    __builtin_amdgcn_s_barrier();                 // the staged rows are read
    asm volatile("" ::: "memory");
#pragma unroll
    for (int p = 1; p < STAGES; ++p)
      if (p < nKT) issue(smem + p * G::STAGE_BYTES, p);
    J = I;
    KT = nKT;
    loc = nloc;
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int KB, int EPI>
hipError_t launch_dgrad_t(const void* X, int ldx, const int32_t* x_index, int x_rows,
                          const void* W, long long w_estride, int ldw, int K, void* C, int ldc,
                          const int32_t* c_index, int c_rows, const void* tile_ws, int N, int E,
                          int n_ntiles, const SwigluBwd& sb, hipStream_t s,
                          const DgradAux& aux) {
  using G = dcfg<BM, BN, WM, WN, STAGES, KB>;
  if (K % KB != 0) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)dgrad_kernel<BM, BN, WM, WN, STAGES, KB, EPI>,
      hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  if (attr != hipSuccess) return attr;
  DgradAux a = aux;
  a.jobs = a.rows > 0 ? (a.rows + BM - 1) / BM * a.n_ntiles : 0;
  const long long max_tiles = (long long)N / BM + std::min(E, N);
  const long long g_per = (max_tiles * n_ntiles + NUM_XCD - 1) / NUM_XCD;
  const long long d_per = ((long long)a.jobs + NUM_XCD - 1) / NUM_XCD;
  const int grid = (int)std::max<long long>((g_per + d_per) * NUM_XCD, NUM_XCD);
  hipLaunchKernelGGL((dgrad_kernel<BM, BN, WM, WN, STAGES, KB, EPI>), dim3(grid), dim3(G::THREADS),
                     G::LDS, s, (const bf16_t*)X, ldx, x_index, x_rows, (const bf16_t*)W,
                     w_estride, ldw, K, (bf16_t*)C, ldc, c_index, c_rows,
                     (const int4*)((const char*)tile_ws + 256), (const int32_t*)tile_ws, n_ntiles,
                     sb, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_dgrad_cfg(int id, const void* X, int ldx, const int32_t* x_index, int x_rows,
                            const void* W, long long w_estride, int ldw, int K, void* C, int ldc,
                            const int32_t* c_index, int c_rows, const void* tile_ws, int N, int E,
                            int n_ntiles, const SwigluBwd& sb, hipStream_t s,
                            const DgradAux& aux) {
#define MOE_DG(ID, BM, BN, WM, WN, ST, KB)                                                  \
  case ID:                                                                               \
    return launch_dgrad_t<BM, BN, WM, WN, ST, KB, EPI>(X, ldx, x_index, x_rows, W, w_estride, \
                                                       ldw, K, C, ldc, c_index, c_rows, tile_ws, \
                                                       N, E, n_ntiles, sb, s, aux);
  switch (id) {
    MOE_DG(0, 128, 128, 2, 2, 4, 32)
    MOE_DG(1, 64, 128, 2, 2, 4, 32)
    MOE_DG(2, 32, 128, 1, 2, 4, 32)
    MOE_DG(3, 256, 256, 2, 4, 2, 64)
    MOE_DG(4, 256, 128, 4, 2, 3, 64)
    MOE_DG(5, 320, 256, 2, 4, 2, 64)
    MOE_DG(6, 320, 128, 2, 2, 2, 64)
    default: return hipErrorInvalidValue;
  }
#undef MOE_DG
}

// Row-tile classes (the tile list's height: 128, 64, 32, 256, 320 rows)
// and, within the 256- and 320-row classes, the 256-column config when the
// output width allows it.  The tall configs take 64 k per block, so every
// row copy of both operands is one whole 128-byte line: at the prefill shape
// that measured 323 against 356 us for the second dgrad and, as 256 x 128
// tiles on 4 x 2 waves, 253 against 270 us for the first.  With groups of
// 160 rows and more the second dgrad takes 320-row tiles, which hold a
// whole expert up to 320 rows (280 against 344 us with the 256-row tiles,
// which split the larger groups and read their weights twice); the first
// keeps 256 x 128 (equal to 320 x 256 there, and 128-column tiles fit any
// shared expert).  The shorter tiles measured slower with 64 k and keep 32.
constexpr int kDgradBM[] = {128, 64, 32, 256, 320};

int dgrad_id(int cls, int n_cols) {
  if (cls == 3) return n_cols % 256 == 0 ? 3 : 4;
  if (cls == 4) return n_cols % 256 == 0 ? 5 : 6;
  return cls;
}

// The config's output columns per tile.
int dgrad_bn(int cfg) { return (cfg == 3 || cfg == 5) ? 256 : 128; }

template <int BM, int BN, int WM, int WN, int STAGES, bool PERSIST = false>
hipError_t launch_wgrad_t(const void* A, int lda, const void* B, int ldb, const void* zero_row,
                          const int32_t* offsets, int E, int M, int N, void* C,
                          long long c_estride, int ldc, hipStream_t s, const WgradAux& aux,
                          unsigned* job_counters = nullptr) {
  using G = wcfg<BM, BN, WM, WN, STAGES>;
  // PERSIST: 16 more bytes publish the next job's share index
  constexpr int LDS = G::LDS + (PERSIST ? 16 : 0);
  static_assert(LDS <= 160 * 1024, "LDS");
  if (PERSIST && !job_counters) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)wgrad_kernel<BM, BN, WM, WN, STAGES, PERSIST>,
      hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (attr != hipSuccess) return attr;
  WgradAux a = aux;
  a.jobs = a.rows > 0 ? (a.M / BM) * (a.N / BN) : 0;
  const long long g_per = ((long long)E * (M / BM) * (N / BN) + NUM_XCD - 1) / NUM_XCD;
  const long long d_per = ((long long)a.jobs + NUM_XCD - 1) / NUM_XCD;
  const int grid = (int)std::max<long long>((g_per + d_per) * NUM_XCD, NUM_XCD);
  // PERSIST: one work-group per CU (the ring needs all of a CU's LDS); a
  // multiple of NUM_XCD so that every XCD's share has the same walkers
  const int g = PERSIST ? std::min(grid, NUM_CU) : grid;
  hipLaunchKernelGGL((wgrad_kernel<BM, BN, WM, WN, STAGES, PERSIST>), dim3(g), dim3(G::THREADS), LDS,
                     s, (const bf16_t*)A, lda, (const bf16_t*)B, ldb, (const bf16_t*)zero_row,
                     offsets, E, M, N, (bf16_t*)C, c_estride, ldc, a, job_counters);
  return hipGetLastError();
}

}  // namespace

int pick_dgrad_cfg(int N, int E) {
  const double mean_rows = E > 0 ? (double)N / E : 0.0;
  return mean_rows >= 160.0 ? 4 : mean_rows >= 96.0 ? 0 : mean_rows >= 40.0 ? 1 : 2;
}

int dgrad_bm(int id) { return kDgradBM[id]; }

// The first dgrad takes the 256-row class where the second takes 320 rows
// (see launch_dgrad_down_swiglu), else the same class.
int pick_dgrad1_cfg(int N, int E) {
  const int c = pick_dgrad_cfg(N, E);
  return c == 4 ? 3 : c;
}

int dgrad1_weight_parts(int I) { return I / kDgrad1Slice; }

hipError_t launch_dgrad_down_swiglu(int id, const void* dout, int T, const int32_t* sorted_token,
                                    const void* down, int N, int H, int I, int E,
                                    const void* G, const float* w, const int32_t* sorted_slot,
                                    void* dG, void* hw, const void* tile_ws, hipStream_t s,
                                    const DgradShared* sh, float* dw_parts) {
  if (N <= 0) return hipSuccess;
  const SwigluBwd sb{(const bf16_t*)G, 2 * I,       I,  w, sorted_slot, (bf16_t*)dG,
                     (bf16_t*)hw,      I,           dw_parts, dgrad1_weight_parts(I)};
  // the tall classes: always 128 columns wide
  const int cfg = id == 3 ? 4 : id == 4 ? 6 : id;
  const int bn = 128;
  DgradAux aux{};
  if (sh) {
    // dout rows in order against the shared down projection, weight 1
    if (sh->Is % bn != 0) return hipErrorInvalidValue;
    aux = DgradAux{(const bf16_t*)dout, H, (const bf16_t*)sh->down, H, H, nullptr, 0, sh->rows,
                   sh->Is / bn, 0,
                   SwigluBwd{(const bf16_t*)sh->G, 2 * sh->Is, sh->Is, nullptr, nullptr,
                             (bf16_t*)sh->dG, (bf16_t*)sh->hw, sh->Is, nullptr, 0}};
  }
  return launch_dgrad_cfg<DG_SWIGLU_BWD>(cfg, dout, H, sorted_token, T, down, (long long)I * H, H,
                                         H, nullptr, 0, nullptr, 0, tile_ws, N, E, I / bn, sb, s,
                                         aux);
}

hipError_t launch_dgrad_gate_up(int id, const void* dG, const void* gate_up, int N, int H, int I,
                                int E, const int32_t* out_index, void* dX, const void* tile_ws,
                                hipStream_t s, const DgradShared* sh) {
  if (N <= 0) return hipSuccess;
  const SwigluBwd none{};
  const int cfg = dgrad_id(id, H);
  const int bn = dgrad_bn(cfg);
  DgradAux aux{};
  if (sh)
    aux = DgradAux{(const bf16_t*)sh->dG, 2 * sh->Is, (const bf16_t*)sh->gate_up, 2 * sh->Is,
                   2 * sh->Is, (bf16_t*)sh->dx, H, sh->rows, H / bn, 0, none};
  return launch_dgrad_cfg<DG_PLAIN>(cfg, dG, 2 * I, nullptr, N, gate_up, (long long)H * 2 * I,
                                    2 * I, 2 * I, dX, H, out_index, N, tile_ws, N, E, H / bn,
                                    none, s, aux);
}

// Output tile of the wgrad config chosen for an M x N gradient.
static void wgrad_tile(int M, int N, int* bm, int* bn) {
  if (M % 256 == 0 && N % 256 == 0) {
    *bm = 256;
    *bn = 256;
  } else {
    *bm = 128;
    *bn = N % 256 == 0 ? 256 : 128;
  }
}

bool wgrad_can_fold(int M, int N, int Ma, int Na) {
  int bm, bn;
  wgrad_tile(M, N, &bm, &bn);
  return Ma % bm == 0 && Na % bn == 0;
}

hipError_t launch_wgrad(const void* A, int lda, const void* B, int ldb, const void* zero_row,
                        const int32_t* offsets, int E, int M, int N, void* C, hipStream_t s,
                        const WgradAux* aux, unsigned* job_counters) {
  const WgradAux none{nullptr, 0, nullptr, 0, 0, 0, 0, nullptr, 0};
  const WgradAux& a = aux ? *aux : none;
  if (a.rows > 0 && !wgrad_can_fold(M, N, a.M, a.N)) return hipErrorInvalidValue;
  int bm, bn;
  wgrad_tile(M, N, &bm, &bn);
  if (bm == 256 && job_counters)
    return launch_wgrad_t<256, 256, 2, 4, 3, true>(A, lda, B, ldb, zero_row, offsets, E, M, N, C,
                                                   (long long)M * N, N, s, a, job_counters);
  if (bm == 256)
    return launch_wgrad_t<256, 256, 2, 4, 3, false>(A, lda, B, ldb, zero_row, offsets, E, M, N,
                                                    C, (long long)M * N, N, s, a);
  if (bn == 256)
    return launch_wgrad_t<128, 256, 2, 2, 4>(A, lda, B, ldb, zero_row, offsets, E, M, N, C,
                                             (long long)M * N, N, s, a);
  return launch_wgrad_t<128, 128, 2, 2, 4>(A, lda, B, ldb, zero_row, offsets, E, M, N, C,
                                           (long long)M * N, N, s, a);
}

}  // namespace moe
