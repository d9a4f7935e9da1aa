// Grouped expert GEMMs for bf16 on gfx950: asynchronous global->LDS loads
// into a multi-stage ring, transposing LDS reads for the weights, MFMA
// 32x32x16 bf16 with float32 accumulation.
//
// Semantics as the float path (moe_gemm.hip): Qwen3-Omni issue #115,
// SpeedupMoeExperts.forward -- per expert e, gate_up = x_e @ gate_up_proj[e],
// h = up * silu(gate), y_e = h @ down_proj[e]; MindSpore moe.py,
// _run_experts_for_loop -- rows in expert-major order split by counts.
//
// Data path per K-block of KB = 32 (two MFMA k-steps of 16; KB = 64 gives
// four k-steps and 128-byte activation rows, see aswz):
//   * activations: BM gathered rows x 64 bytes, loaded with
//     global_load_lds_dwordx4 (lane i of a wave instruction lands at
//     base + 16 i); each lane picks the global 16-byte chunk that belongs at
//     its LDS slot, which realises an XOR swizzle of the 4 chunks of a row
//     by f(row) = (row ^ (row >> 2)) & 3.  Reads are ds_read_b128.
//   * weights: 32 rows (k) x BN columns in their natural [k][n] layout
//     (n contiguous), loaded the same way (WNT: with the non-temporal
//     hint, for launches whose experts mostly fit one row tile, so that no
//     other job re-reads a weight tile) with 32-byte segments of a row
//     XOR-swizzled by h(row) = ((row & 3) << 1) | ((row >> 3) & 1).  The MFMA
//     operand needs 8 consecutive k of one column per lane; two
//     ds_read_b64_tr_b16 deliver that: within each 16-lane group, lane s
//     reads 4 consecutive columns of row (kbase + s / 4) and lane j receives
//     column j of rows kbase .. kbase + 3.
//   * MFMA operands are (weights, activations), so the accumulator tile is
//     C^T: each lane holds 4 consecutive output columns of one row.
//   * Software pipeline: the LDS fragments of the next k-step are read while
//     the MFMAs of the current one run, so LDS traffic hides under the
//     matrix pipe.  One barrier per K-block, before its last k-step, both
//     publishes the next landed block and retires the block just read, whose
//     slot is refilled right away; STAGES - 2 further blocks stay in flight.
//   * 32-row m-tiles are dealt to the WM wave rows round-robin; m-tiles
//     beyond the tile's rows skip their MFMAs.
#include <type_traits>

#include "moe_common.h"
#include "moe_internal.h"
#include "moe_lds.h"


namespace moe {
namespace {

using namespace lds;

// Activation rows hold KB k-values (KB / 8 chunks of 16 bytes).  Four chunks
// take the measured swizzle; eight chunks (whole 128-byte lines per row)
// take (row >> 1) & 7, which gives the 16 rows one 16-lane phase of a
// ds_read_b128 reads 16 distinct 16-byte bank groups.
template <int KB>
__device__ __forceinline__ int aswz(int row) {
  if constexpr (KB == 32) return fswz(row);
  else return (row >> 1) & 7;
}

// f(integral_constant<int, i>) for i = I .. N - 1, unrolled at compile time.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// STAGES ring slots for the activation tiles, then STAGES for the weight
// tiles.
template <int BM, int BN, int WM, int WN, int STAGES, bool SWIGLU, int KB = BK>
struct lcfg {
  static_assert(KB == 32 || KB == 64, "k per block");
  static constexpr int KS = KB / 16;                 // MFMA k-steps per block
  static constexpr int CH = KB / 8;                  // 16-byte chunks per activation row
  static constexpr int ABR = KB * 2;                 // bytes per activation row
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = NW * 64;
  static constexpr int MT = BM / 32;                 // 32-row m-tiles per workgroup tile
  static constexpr int TM = MT / WM;                 // m-tiles per wave
  static constexpr int CW = SWIGLU ? (BN / 2) / WN : BN / WN;  // output cols per wave
  static constexpr int TNO = CW / 32;                // 32-col output tiles per wave
  static constexpr int TN = SWIGLU ? 2 * TNO : TNO;  // weight tiles per wave
  static constexpr int A_BYTES = BM * KB * 2;        // per stage
  static constexpr int B_BYTES = KB * BN * 2;
  static constexpr int B_RING = STAGES * A_BYTES;     // weight slots follow the activation slots
  static constexpr int RING = STAGES * (A_BYTES + B_BYTES);
  // 1 KB that absorbs the surplus activation copies of waves with a short
  // share, so every wave issues the same number of copies per block
  static constexpr int DUMP = (BM * KB * 2 / 1024) % NW ? 1024 : 0;
  static constexpr int LDS = RING + DUMP;
  static constexpr int A_INST = A_BYTES / 1024;      // wave instructions per stage
  static constexpr int B_INST = B_BYTES / 1024;
  static constexpr int A_PER = (A_INST + NW - 1) / NW;
  static constexpr int B_PER = B_INST / NW;
  static constexpr int ROWB = BN * 2;                // bytes per weight row in LDS
  static constexpr int SEGS = BN / 16;               // 32-byte segments per weight row
  static_assert(BM % 32 == 0 && MT % WM == 0 && TM >= 1, "m-tiles per wave");
  static_assert(CW % 32 == 0 && TNO >= 1, "n-tiles per wave");
  static_assert(B_INST % NW == 0, "weight loads split evenly");
  static_assert(SEGS >= 8, "swizzle needs 8 segments per row");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int BM, int BN, int WM, int WN, int STAGES, bool SWIGLU, int KB, bool WNT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_lds_kernel(
    const bf16_t* __restrict__ gX, int g_ldx, const int32_t* __restrict__ g_x_index,
    int g_x_rows, const bf16_t* __restrict__ gW, long long g_w_estride, int g_ldw, int g_K,
    int g_up_off, bf16_t* __restrict__ gC, int g_ldc, const int32_t* __restrict__ g_c_index,
    int g_c_rows, const int4* __restrict__ tiles, const int32_t* __restrict__ tiles_count,
    int g_n_ntiles, DenseAux aux, bf16_t* __restrict__ g_save) {
  using G = lcfg<BM, BN, WM, WN, STAGES, SWIGLU, KB>;
  static_assert(STAGES >= 2, "at least double buffering");
  // STAGES ring slots of STAGE_BYTES.  The copies are invisible to the
  // compiler (asm), so it inserts no waits for them; the explicit vmcnt
  // waits plus the barrier order each slot's fill before its reads, and the
  // asm memory clobbers keep the compiler from moving LDS reads across them.
  extern __shared__ __align__(16) unsigned char smem[];

  // ---- job (M-tile, N-tile), XCD-aware: consecutive jobs share an XCD.
  // Each XCD takes an equal contiguous share of the dense problem's jobs
  // first, then an equal contiguous share of the grouped tiles' jobs.
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
  const bf16_t* __restrict__ X = dense ? (const bf16_t*)aux.X : gX;
  const int ldx = dense ? aux.ldx : g_ldx;
  const int32_t* __restrict__ x_index = dense ? nullptr : g_x_index;
  const int x_rows = dense ? aux.rows : g_x_rows;
  const bf16_t* __restrict__ W = dense ? (const bf16_t*)aux.W : gW;
  const long long w_estride = dense ? 0 : g_w_estride;
  const int ldw = dense ? aux.ldw : g_ldw;
  const int K = dense ? aux.K : g_K;
  const int up_off = dense ? aux.up_off : g_up_off;
  bf16_t* __restrict__ C = dense ? (bf16_t*)aux.C : gC;
  const int ldc = dense ? aux.ldc : g_ldc;
  const int32_t* __restrict__ c_index = dense ? nullptr : g_c_index;
  const int c_rows = dense ? aux.rows : g_c_rows;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = SWIGLU ? nt * (BN / 2) : nt * BN;
  const bf16_t* We = W + (long long)e * w_estride;

  // ---- load assignments: global source of this lane's 16 bytes in each of
  // the wave's load instructions (advanced by one K-block per issue)
  const bf16_t* a_src[G::A_PER];
  int a_lds[G::A_PER];
  bool a_on[G::A_PER];
#pragma unroll
  for (int u = 0; u < G::A_PER; ++u) {
    const int inst = wave + u * G::NW;
    a_on[u] = inst < G::A_INST;
    const int q = (a_on[u] ? inst : 0) * 64 + lane;   // 16-byte slot in the A block
    const int row = q / G::CH;
    const int c = (q % G::CH) ^ aswz<KB>(row);
    int src = row0 + min(row, rows - 1);
    if (x_index) src = x_index[src];
    src = min(max(src, 0), x_rows - 1);
    a_src[u] = X + (long long)src * ldx + 8 * c;
    a_lds[u] = (a_on[u] ? inst : 0) * 1024;
  }
  const bf16_t* b_src[G::B_PER];
  int b_lds[G::B_PER];
#pragma unroll
  for (int u = 0; u < G::B_PER; ++u) {
    const int inst = wave + u * G::NW;
    const int q = inst * 64 + lane;                   // 16-byte slot in the B block
    const int row = q / (BN / 8);
    const int p = q % (BN / 8);
    const int seg = (p >> 1) ^ hswz(row);
    int col = 16 * seg + 8 * (p & 1);                  // logical B-tile column
    if constexpr (SWIGLU)
      col = col < BN / 2 ? n0 + col : up_off + n0 + (col - BN / 2);
    else
      col = n0 + col;
    b_src[u] = We + (long long)row * ldw + col;
    b_lds[u] = inst * 1024;
  }

  // A wave's last activation copy is left out when all its rows lie past
  // the tile's end (or it only fills the dump area): such rows feed only
  // outputs that are never stored, so their LDS rows may stay stale.  The
  // choice is per wave, and so are the vmcnt counts it changes.
  constexpr int AL = G::A_PER - 1;
  const int skl = __builtin_amdgcn_readfirstlane(
      (!a_on[AL] || (wave + AL * G::NW) * (64 / G::CH) >= rows) ? 1 : 0);

  // Copies of the next activation block into activation slot `as` and of
  // the next weight block into weight slot `bs`.
  auto issue_a = [&](int as) {
    unsigned char* const base = smem + as * G::A_BYTES;
#pragma unroll
    for (int u = 0; u < G::A_PER; ++u) {
      if (u == AL && skl) break;
      // a copy past the A block re-reads row chunk 0 into the dump area
      copy16_to_lds(a_src[u], a_on[u] ? base + a_lds[u] : smem + G::RING);
      a_src[u] += KB;
    }
  };
  auto issue_b = [&](int bs) {
    unsigned char* const base = smem + G::B_RING + bs * G::B_BYTES;
#pragma unroll
    for (int u = 0; u < G::B_PER; ++u) {
      if constexpr (WNT) copy16_to_lds_nt(b_src[u], base + b_lds[u]);
      else copy16_to_lds(b_src[u], base + b_lds[u]);
      b_src[u] += (long long)KB * ldw;
    }
  };
  // The same copies one at a time, for the main loop, which spreads them
  // between its MFMAs: copy c (compile-time) of a block into activation
  // slot `as` and weight slot `bs`.  The weight copies go first: they come
  // from HBM, the activation rows mostly from the caches.
  constexpr int PER = G::A_PER + G::B_PER;   // copies per block, every wave
  auto issue_one = [&](auto c_c, int as, int bs, bool on) {
    constexpr int c = decltype(c_c)::value;
    if (!on) return;
    if constexpr (c < G::B_PER) {
      unsigned char* const base = smem + G::B_RING + bs * G::B_BYTES;
      if constexpr (WNT) copy16_to_lds_nt(b_src[c], base + b_lds[c]);
      else copy16_to_lds(b_src[c], base + b_lds[c]);
      b_src[c] += (long long)KB * ldw;
    } else {
      constexpr int u = c - G::B_PER;
      unsigned char* const base = smem + as * G::A_BYTES;
      copy16_to_lds(a_src[u], a_on[u] ? base + a_lds[u] : smem + G::RING);
      a_src[u] += KB;
    }
  };

  // ---- per-lane LDS read offsets (bytes within a stage) for the 32x32x16
  // MFMA operands.  Activations ("B" operand): lane l needs row
  // 32 * mtile + l % 32, k = 8 (l / 32) .. + 7 of the k-step, i.e. chunk
  // 2 kk + l / 32 of the row; the row swizzle f depends only on l % 32
  // because m-tiles start at multiples of 32, so m-tiles differ by a
  // constant offset.  Weights ("A" operand): lane l needs column n = l % 32
  // of the tile and the same k values; 16-lane group q reads columns
  // 16 (q & 1) .. + 15 and k 8 (q >> 1) .. + 7 with two transposing reads of
  // 4 rows each.  Those rows are 16 kk + 8 (q >> 1) + 4 hf + s / 4, whose
  // swizzle h = (s / 4) << 1 | (q >> 1) does not depend on kk or hf, so kk
  // and hf are constant offsets too.
  const int l32 = lane & 31, hl = lane >> 5;
  constexpr int XI = 32 * WM * G::ABR;             // bytes between a wave's m-tiles
  int xa_off[G::KS];
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
    xa_off[kk] = (32 * wm + l32) * G::ABR + 16 * ((2 * kk + hl) ^ aswz<KB>(l32));
  // this wave's m-tiles wm, wm + WM, ... that hold rows (wave-uniform)
  const int tm_on = __builtin_amdgcn_readfirstlane(
      min(G::TM, max(0, ((rows + 31) / 32 - wm + WM - 1) / WM)));
  const int gq = lane >> 4, s16 = lane & 15;
  const int wrow = 8 * (gq >> 1) + (s16 >> 2);
  const int wsw = ((s16 >> 2) << 1) | (gq >> 1);
  int wb_off[G::TN];
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    int cb;  // logical column base of this 32-column tile
    if constexpr (SWIGLU)
      cb = j < G::TNO ? wn * G::CW + 32 * j : BN / 2 + wn * G::CW + 32 * (j - G::TNO);
    else
      cb = wn * G::CW + 32 * j;
    const int col = cb + 16 * (gq & 1) + 4 * (s16 & 3);
    wb_off[j] = wrow * G::ROWB + 32 * ((col >> 4) ^ wsw) + 2 * (col & 15);
  }

  f32x16_v acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Fragment reads of k-step kk of the block at `base` (rows past the
  // tile's end read in-bounds stale LDS and are never stored).
  auto read_w = [&](const unsigned char* base, int kk, bf16x8_v (&wf)[G::TN]) {
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      const unsigned char* p = base + wb_off[j] + 16 * kk * G::ROWB;
      const i16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * G::ROWB));
      wf[j] = __builtin_bit_cast(bf16x8_v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto read_x = [&](const unsigned char* base, int kk, int i) {
    return __builtin_bit_cast(bf16x8_v,
                              *reinterpret_cast<const u32x4*>(base + xa_off[kk] + XI * i));
  };
  const int KT = K / KB;
  // Wait until at most `nb` of this wave's most recent blocks are in flight.
  auto wait_blocks = [&](auto px_c, int nb) {
    constexpr int PB = decltype(px_c)::value;   // this wave's loads per block
    static_assert(STAGES <= 8 && (STAGES - 1) * PB < 64, "wait table");
    // nb never exceeds STAGES - 1; larger cases clamp to it
    constexpr int M = STAGES - 1;
    switch (nb) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<(M < 1 ? M : 1) * PB>(); break;
      case 2: wait_vmcnt<(M < 2 ? M : 2) * PB>(); break;
      case 3: wait_vmcnt<(M < 3 ? M : 3) * PB>(); break;
      case 4: wait_vmcnt<(M < 4 ? M : 4) * PB>(); break;
      case 5: wait_vmcnt<(M < 5 ? M : 5) * PB>(); break;
      case 6: wait_vmcnt<(M < 6 ? M : 6) * PB>(); break;
      default: wait_vmcnt<(M < 7 ? M : 7) * PB>(); break;
    }
  };
  // The copy stream, in issue order: the prologue gives block p its
  // activation copies then its weight copies, p = 0 .. STAGES - 1; the
  // loop's iteration kb then issues block kb + STAGES.  Blocks are waited
  // for whole, so the order inside a block does not matter.
  // prologue: every slot gets a block
#pragma unroll
  for (int p = 0; p < STAGES; ++p) {
    if (p < KT) {
      issue_a(p);
      issue_b(p);
    }
  }

  // block 0 landed (blocks 1 .. min(STAGES, KT) - 1 may stay in flight)
  if (skl) wait_blocks(std::integral_constant<int, PER - 1>{}, min(STAGES, KT) - 1);
  else wait_blocks(std::integral_constant<int, PER>{}, min(STAGES, KT) - 1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // The main loop, specialised on the number of this wave's m-tiles that
  // hold rows (TA), so it is straight-line code: m-tiles past TA are neither
  // read nor multiplied.
  auto main_loop = [&](auto ta_c, auto sk_c) {
    constexpr int TA = decltype(ta_c)::value;
    constexpr int KS = G::KS;
    constexpr int PX = PER - decltype(sk_c)::value;   // copies per block, this wave
    const auto px_c = std::integral_constant<int, PX>{};
    bf16x8_v wf[2][G::TN], xf[TA];   // k-step s of a block uses wf[s & 1]
    // MFMAs of one k-step, m-tile by m-tile; right after m-tile i's MFMAs
    // are issued its activation register is refilled with the fragment of
    // the next k-step (`nbase`, `nkk`), so the LDS read runs under the
    // remaining MFMAs and one register set serves both k-steps.
    //
    // Inside the loop, step STEP (0 .. KS - 1) of an iteration also issues
    // that iteration's copies of the next blocks, one per MFMA group over
    // its first groups (m-tile i of step STEP is group STEP * TA + i),
    // instead of all at the top: the load unit takes a CU's copies only as
    // fast as it drains them (about 16 clocks per 1 KB copy), so issuing a
    // block's copies together held the later waves of the work-group at
    // the top of each iteration (timestamps: 1,640 clocks per iteration for
    // waves 4-7 against 570 for waves 0-3) while their MFMAs waited.
    // Packing the copies into the first 2-5 groups, or spreading them over
    // the whole iteration, measured slower.  STEP < 0: none.
    constexpr int GROUPS = TA * KS;
    constexpr int GP = GROUPS < PX ? GROUPS : PX;     // groups that issue copies
    auto mma_roll = [&](auto step_c, const bf16x8_v (&wf)[G::TN], const unsigned char* nbase,
                        int nkk, int as, int bs, bool on) {
      constexpr int STEP = decltype(step_c)::value;
      static_for<0, TA>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
#pragma unroll
        for (int j = 0; j < G::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        xf[i] = read_x(nbase, nkk, i);
        if constexpr (STEP >= 0) {
          constexpr int g = STEP * TA + i;
          if constexpr (g < GP)
            static_for<g * PX / GP, (g + 1) * PX / GP>(
                [&](auto c_c) { issue_one(c_c, as, bs, on); });
        }
        // keep this order: the scheduler would otherwise gather the reads
        // next to their first use and expose their latency
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Block b's k-steps 0 .. KS - 2 are multiplied before the barrier that
    // publishes block b + 1, its last k-step after it.  Between the two,
    // every wave has finished reading slot b (LDS reads waited), so the
    // barrier also retires slot b, which is refilled with block b + STAGES
    // right after it.  The loop body starts after a barrier, where no LDS
    // read is pending, so the wait-count state at the loop head is exact.
    const unsigned char* const b0 = smem + G::B_RING;
    read_w(b0, 0, wf[0]);
#pragma unroll
    for (int i = 0; i < TA; ++i) xf[i] = read_x(smem, 0, i);
    static_for<0, KS - 1>([&](auto st_c) {
      constexpr int st = decltype(st_c)::value;
      read_w(b0, st + 1, wf[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma_roll(std::integral_constant<int, -1>{}, wf[st & 1], smem, st + 1, 0, 0, false);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (KT > 1) wait_blocks(px_c, min(STAGES - 2, KT - 2));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    int slot = 0;                                      // kb % STAGES
    for (int kb = 0; kb + 1 < KT; ++kb) {
      const int cur = slot;
      slot = (slot + 1 == STAGES) ? 0 : slot + 1;
      const unsigned char* const an = smem + slot * G::A_BYTES;
      const unsigned char* const bn = smem + G::B_RING + slot * G::B_BYTES;
      // block kb + STAGES goes into the slot of block kb, retired by the
      // barrier that ended the previous iteration
      const bool on = kb + STAGES < KT;
      // last k-step of block kb, reading block kb + 1's first
      read_w(bn, 0, wf[KS & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma_roll(std::integral_constant<int, 0>{}, wf[(KS - 1) & 1], an, 0, cur, cur, on);
      // k-steps 0 .. KS - 2 of block kb + 1, each reading the next
      static_for<0, KS - 1>([&](auto st_c) {
        constexpr int st = decltype(st_c)::value;
        read_w(bn, st + 1, wf[(KS + st + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mma_roll(std::integral_constant<int, st + 1>{}, wf[(KS + st) & 1], an, st + 1, cur, cur,
                 on);
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (kb + 2 < KT) wait_blocks(px_c, min(STAGES - 2, KT - 3 - kb));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // last k-step of the last block
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[(KS - 1) & 1][j], xf[i], acc[i][j], 0, 0, 0);
  };
  // Waves without rows issue the same copies and join the same barriers.
  auto empty_loop = [&](auto sk_c) {
    const auto px_c = std::integral_constant<int, PER - decltype(sk_c)::value>{};
    if (KT > 1) wait_blocks(px_c, min(STAGES - 2, KT - 2));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int kb = 0; kb + 1 < KT; ++kb) {
      if (kb + STAGES < KT) {
        issue_b(kb % STAGES);
        issue_a(kb % STAGES);
      }
      if (kb + 2 < KT) wait_blocks(px_c, min(STAGES - 2, KT - 3 - kb));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  };
  static_assert(G::TM <= 8, "m-tiles per wave");
  auto run = [&](auto sk_c) {
    switch (tm_on) {
      case 0: empty_loop(sk_c); break;
      case 1: main_loop(std::integral_constant<int, 1>{}, sk_c); break;
      case 2: if constexpr (G::TM >= 2) main_loop(std::integral_constant<int, 2>{}, sk_c); break;
      case 3: if constexpr (G::TM >= 3) main_loop(std::integral_constant<int, 3>{}, sk_c); break;
      case 4: if constexpr (G::TM >= 4) main_loop(std::integral_constant<int, 4>{}, sk_c); break;
      case 5: if constexpr (G::TM >= 5) main_loop(std::integral_constant<int, 5>{}, sk_c); break;
      case 6: if constexpr (G::TM >= 6) main_loop(std::integral_constant<int, 6>{}, sk_c); break;
      case 7: if constexpr (G::TM >= 7) main_loop(std::integral_constant<int, 7>{}, sk_c); break;
      default: if constexpr (G::TM >= 8) main_loop(std::integral_constant<int, 8>{}, sk_c); break;
    }
  };
  if (skl) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  // ---- epilogue.  acc[i][j][q] = C[row m][col cb_j + 8 (q / 4) + 4 hl + q % 4]
  // with m = 32 * mtile + l % 32.  Results go through LDS so that global
  // stores write whole row segments with 16-byte lanes.  Staged rows are
  // padded by 8 bytes: the 32 rows a wave writes at once then fall on
  // distinct banks.
  auto to_bf16x4 = [](const float (&v)[4]) {
    return make_uint2((uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                      (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16));
  };
  __builtin_amdgcn_s_barrier();              // every wave is done with the ring
  asm volatile("" ::: "memory");
  {
    // Each wave stages one 32-row m-tile of its CW columns at a time and
    // stores every row segment of 2 CW bytes (rows of the second GEMM are
    // scattered through c_index).  The destination rows are loaded up front,
    // all at once, rather than one m-tile at a time.
    constexpr int OB = G::CW * 2;              // bytes per staged output row
    constexpr int OBP = OB + 8;                // padded row stride
    constexpr int LPR = OB / 16;               // lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;              // rows per store instruction
    constexpr int NRI = 32 / RPI;              // store instructions per m-tile
    static_assert(32 * OBP * G::NW <= G::RING, "output staging fits in the ring");
    int dsts[G::TM][NRI];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int rr = 0; rr < NRI; ++rr) {
        const int m = 32 * (wm + WM * i) + rr * RPI + lane / LPR;
        int dst = -1;
        if (i < tm_on && m < rows) dst = (!SWIGLU && c_index) ? c_index[row0 + m] : row0 + m;
        dsts[i][rr] = dst;
      }
    unsigned char* stg = smem + wave * 32 * OBP;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      if (i >= tm_on) continue;
#pragma unroll
      for (int j = 0; j < G::TNO; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][j][4 * a + q];
            if constexpr (SWIGLU) {
              // silu(g) * u in float32; rounded to bf16 on store
              const float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              v[q] = sg * acc[i][G::TNO + j][4 * a + q];
            } else {
              v[q] = g;
            }
          }
          *reinterpret_cast<uint2*>(stg + l32 * OBP + 2 * (32 * j + 8 * a + 4 * hl)) = to_bf16x4(v);
        }
      // LDS writes above and reads below are this wave's own: program order
      // plus the compiler's lgkmcnt waits order them.
#pragma unroll
      for (int rr = 0; rr < NRI; ++rr) {
        const int r = rr * RPI + lane / LPR;
        const uint2 lo = *reinterpret_cast<const uint2*>(stg + r * OBP + 16 * (lane % LPR));
        const uint2 hi = *reinterpret_cast<const uint2*>(stg + r * OBP + 16 * (lane % LPR) + 8);
        const int dst = dsts[i][rr];
        // plain stores: h is re-read by every n-tile of the second GEMM and
        // the second GEMM's rows by the combine right after (non-temporal
        // stores here slowed the combine by 15 %)
        if (dst >= 0 && dst < c_rows)
          *reinterpret_cast<u32x4*>(C + (long long)dst * ldc + n0 + wn * G::CW + 8 * (lane % LPR)) =
              u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      if constexpr (SWIGLU) {
        // training forward: also keep the pre-activations, gate at column n
        // and up at column up_off + n of the [rows, 2 up_off] buffer
        bf16_t* const gs = dense ? (bf16_t*)aux.g_save : g_save;
        if (gs) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int j = 0; j < G::TNO; ++j)
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = acc[i][half * G::TNO + j][4 * a + q];
                *reinterpret_cast<uint2*>(stg + l32 * OBP + 2 * (32 * j + 8 * a + 4 * hl)) =
                    to_bf16x4(v);
              }
#pragma unroll
            for (int rr = 0; rr < NRI; ++rr) {
              const int r = rr * RPI + lane / LPR;
              const uint2 lo = *reinterpret_cast<const uint2*>(stg + r * OBP + 16 * (lane % LPR));
              const uint2 hi =
                  *reinterpret_cast<const uint2*>(stg + r * OBP + 16 * (lane % LPR) + 8);
              const int dst = dsts[i][rr];
              if (dst >= 0 && dst < c_rows)   // read by the backward only
                __builtin_nontemporal_store(
                    u32x4{lo.x, lo.y, hi.x, hi.y},
                    reinterpret_cast<u32x4*>(gs + (long long)dst * (2 * up_off) + half * up_off +
                                             n0 + wn * G::CW + 8 * (lane % LPR)));
            }
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, bool SWIGLU, int KB, bool WNT>
hipError_t launch_lds(const void* X, int ldx, const int32_t* x_index, int x_rows, const void* W,
                      long long w_estride, int ldw, int K, int up_off, void* C, int ldc,
                      const int32_t* c_index, int c_rows, const int4* tiles,
                      const int32_t* tiles_count, int n_ntiles, int grid, hipStream_t s,
                      const DenseAux& aux, void* g_save) {
  using G = lcfg<BM, BN, WM, WN, STAGES, SWIGLU, KB>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)gemm_lds_kernel<BM, BN, WM, WN, STAGES, SWIGLU, KB, WNT>,
      hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, WM, WN, STAGES, SWIGLU, KB, WNT>), dim3(grid),
                     dim3(G::THREADS), G::LDS, s, (const bf16_t*)X, ldx, x_index, x_rows,
                     (const bf16_t*)W, w_estride, ldw, K, up_off, (bf16_t*)C, ldc, c_index,
                     c_rows, tiles, tiles_count, n_ntiles, aux, (bf16_t*)g_save);
  return hipGetLastError();
}

struct LdsCfg { int BM, BN; };
// id: tile, waves (M x N), wave tile
// 10: 256 x 256, 2 x 2 waves, 128 x 128   (1 wave per SIMD)
// 11: 128 x 256, 2 x 2 waves,  64 x 128
// 12:  64 x 256, 1 x 4 waves,  64 x  64
// 13:  32 x 256, 1 x 4 waves,  32 x  64   (decode)
// 14: (retired) the 320 x 256 tile below with 32 k per block in four
//     stages, measured 2-4 % slower than 15 at the prefill shape
// 15: 320 x 256, 2 x 4 waves, 160 x  64   (2 waves per SIMD; one tile per
//     expert when groups hold up to 320 rows), 64 k per block in two
//     stages, so every activation row copy is one whole 128-byte line (for
//     the shorter tiles 64 k per block was slower)
// The configs the grouped picker returns (11, 12, 13, 15) also come with
// non-temporal weight copies (WNT), taken when the mean rows per expert fit
// one row tile.
// (a 256 x 256 tile with two activation slots and three weight slots,
// copying the weights two blocks ahead in exactly the 160 KB of LDS,
// measured 15-20 % slower than 15 at the prefill shape and 1-3 % at the
// skewed one: the copies' latency was not what held the loop back)
constexpr LdsCfg kLds[] = {{256, 256}, {128, 256}, {64, 256}, {32, 256}, {320, 256},
                           {320, 256}};

hipError_t launch_lds_cfg(bool swiglu, int id, bool wnt, const void* X, int ldx,
                          const int32_t* x_index, int x_rows, const void* W,
                          long long w_estride, int ldw, int K, int up_off, void* C, int ldc,
                          const int32_t* c_index, int c_rows,
                          const int4* tiles, const int32_t* tiles_count, int n_ntiles, int grid,
                          hipStream_t s, const DenseAux& aux, void* g_save) {
#define MOE_ARGS X, ldx, x_index, x_rows, W, w_estride, ldw, K, up_off, C, ldc, c_index, c_rows, \
                 tiles, tiles_count, n_ntiles, grid, s, aux, g_save
#define MOE_LAUNCH(BM, BN, WM, WN, ST, KB, NT)                                  \
  (swiglu ? launch_lds<BM, BN, WM, WN, ST, true, KB, NT>(MOE_ARGS)            \
          : launch_lds<BM, BN, WM, WN, ST, false, KB, NT>(MOE_ARGS))
// configs the grouped picker returns come in both cache-hint variants
#define MOE_CASE2(ID, BM, BN, WM, WN, ST, KB)                                   \
  case ID:                                                                    \
    return wnt ? MOE_LAUNCH(BM, BN, WM, WN, ST, KB, true)                     \
               : MOE_LAUNCH(BM, BN, WM, WN, ST, KB, false);
#define MOE_CASE1(ID, BM, BN, WM, WN, ST, KB)                                   \
  case ID:                                                                    \
    return MOE_LAUNCH(BM, BN, WM, WN, ST, KB, false);

  switch (id) {
    MOE_CASE1(10, 256, 256, 2, 2, 4, 32)
    MOE_CASE2(11, 128, 256, 2, 2, 4, 32)
    MOE_CASE2(12, 64, 256, 1, 4, 4, 32)
    MOE_CASE2(13, 32, 256, 1, 4, 4, 32)
    MOE_CASE2(15, 320, 256, 2, 4, 2, 64)
    default: return hipErrorInvalidValue;
  }
#undef MOE_CASE1
#undef MOE_CASE2
#undef MOE_LAUNCH
#undef MOE_ARGS
}

}  // namespace

bool lds_cfg_id(int id) { return id >= 10 && id <= 15 && id != 14; }

GemmTileCfg pick_lds_cfg(int N, int E, int cols, bool swiglu) {
  // weight columns per tile: 256 (SwiGLU: 128 gate + 128 up)
  const int need = swiglu ? 128 : 256;
  if (cols % need != 0) return GemmTileCfg{0, 0, -1};
  const double mean_rows = E > 0 ? (double)N / E : 0.0;
  // measured at the Qwen3-30B-A3B shapes: 64 k per block helps the tall
  // tiles (a few percent); the short ones stream weights and prefer more,
  // smaller stages
  int id;
  if (mean_rows >= 160.0) id = 15;
  else if (mean_rows >= 64.0) id = 11;
  else if (mean_rows >= 24.0) id = 12;
  else id = 13;
  // mean rows within one row tile: each weight tile is read by about one
  // job, so its copies take the non-temporal hint (copy16_to_lds_nt)
  const int wnt = mean_rows <= kLds[id - 10].BM ? 1 : 0;
  return GemmTileCfg{kLds[id - 10].BM, kLds[id - 10].BN, id, wnt};
}

GemmTileCfg pick_lds_dense_cfg(int rows, int cols, bool swiglu) {
  // One group of `rows` rows: the tallest row tile that still gives every
  // compute unit a job, else the shortest.
  const int need = swiglu ? 128 : 256;
  if (cols % need != 0) return GemmTileCfg{0, 0, -1};
  const long long n_ntiles = cols / need;
  constexpr int kOrder[] = {15, 10, 11, 12, 13};
  for (const int id : kOrder) {
    const LdsCfg& g = kLds[id - 10];
    if (((long long)rows + g.BM - 1) / g.BM * n_ntiles >= NUM_CU) return GemmTileCfg{g.BM, g.BN, id};
  }
  return GemmTileCfg{kLds[3].BM, kLds[3].BN, 13};
}

DenseAux dense_aux(const GemmTileCfg& c, bool swiglu, const void* X, int ldx, const void* W,
                   int ldw, int K, int up_off, void* C, int ldc, int rows, int cols) {
  DenseAux a{X, W, C, ldx, ldw, K, up_off, ldc, rows, 0, 0, nullptr};
  const int per_tile = swiglu ? c.BN / 2 : c.BN;   // output columns per job
  if (rows <= 0 || cols % per_tile != 0) return a;
  a.n_ntiles = cols / per_tile;
  a.jobs = (rows + c.BM - 1) / c.BM * a.n_ntiles;
  return a;
}

hipError_t launch_lds_gemm(bool swiglu, const GemmTileCfg& c, const void* X, int ldx,
                           const int32_t* x_index, int x_rows, const void* W,
                           long long w_estride, int ldw, int K, int up_off, void* C, int ldc,
                           const int32_t* c_index, int c_rows, const int32_t* offsets, int N,
                           int E, int n_ntiles, void* tile_ws, bool tiles_ready, hipStream_t s,
                           const DenseAux* aux, void* g_save) {
  int32_t* count = (int32_t*)tile_ws;
  int4* tiles = (int4*)((char*)tile_ws + 256);
  if (!tiles_ready) {
    const hipError_t err = launch_build_tiles(offsets, E, N, c.BM, tile_ws, s);
    if (err != hipSuccess) return err;
  }
  const DenseAux none{nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0, nullptr};
  const DenseAux& a = aux ? *aux : none;
  // one work-group slot per job of each XCD's two shares (the grouped tile
  // count on the device never exceeds max_tiles)
  const long long max_tiles = (long long)N / c.BM + std::min(E, N);
  const long long g_per = (max_tiles * n_ntiles + NUM_XCD - 1) / NUM_XCD;
  const long long d_per = ((long long)a.jobs + NUM_XCD - 1) / NUM_XCD;
  const int grid = (int)std::max<long long>((g_per + d_per) * NUM_XCD, NUM_XCD);
  return launch_lds_cfg(swiglu, c.id, c.wnt != 0, X, ldx, x_index, x_rows, W, w_estride, ldw, K, up_off, C,
                        ldc, c_index, c_rows, tiles, count, n_ntiles, grid, s, a, g_save);
}

}  // namespace moe
