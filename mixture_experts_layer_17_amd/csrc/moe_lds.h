// Device helpers shared by the LDS-staged GEMM kernels (forward and
// backward): chip constants, the measured LDS swizzles, the asynchronous
// global->LDS copy and its wait.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace moe {
namespace lds {

constexpr int NUM_XCD = 8;
constexpr int NUM_CU = 256;
constexpr int BK = 32;   // k per stage

typedef short i16x4_v __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_v;
typedef __attribute__((address_space(3))) i16x4_v lds_i16x4;

// Swizzles chosen by timing every lane pattern the kernel reads against the
// conflict-free rate (ds_read_b128: 4 clocks per wave instruction,
// ds_read_b64_tr_b16: 2 clocks).
__device__ __forceinline__ int fswz(int row) { return (row ^ (row >> 2)) & 3; }
__device__ __forceinline__ int hswz(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// One 16-byte-per-lane asynchronous copy global -> LDS: lane i's 16 bytes
// land at lds + 16 i (lds is wave-uniform, passed in M0).  Issued from asm
// so that the compiler's wait-count pass, which cannot tell the four stage
// buffers apart across loop iterations, does not drain every copy in flight
// before each LDS read; completion is tracked with explicit vmcnt waits
// below.  The instruction writes no registers, so nothing the compiler
// allocates can be overwritten while it is in flight.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* g, const unsigned char* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_u8*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(a)
               : "memory", "m0");
}

// The same copy with the non-temporal hint, for weight tiles that no other
// work-group reads (an expert whose rows fit one m-tile): keeping them in
// the caches only displaces the activation rows that every job re-reads.
// Measured at the Qwen3-30B-A3B shapes: the decode GEMMs, which stream
// every hit expert's weights once, 12-13 % faster (gate_up 136 -> 119 us,
// down 70 -> 62 us), the prefill ones 2-5 % faster.  Where several m-tiles
// share an expert's weights (the EP rank's 2000-row experts) the hint cost
// 5 %, and on the activation rows it was slower everywhere.
__device__ __forceinline__ void copy16_to_lds_nt(const void* g, const unsigned char* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_u8*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(a)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N of this wave's vector-memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}


}  // namespace lds
}  // namespace moe
