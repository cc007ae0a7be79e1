// Device helpers shared by the flash prefill kernels (head dimension 128 in
// prefill.hip, 256 in prefill_d256.hip).
#pragma once

#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {
namespace {

// Value of lane l ^ 32 combined with this lane's: sum / max.
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier that waits only for this wave's LDS operations: tile
// loads still in flight from global memory into LDS keep flying (a
// __syncthreads() would wait for every outstanding memory operation).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte global -> LDS load per lane (global_load_lds_dwordx4): lane L
// writes LDS bytes [lds_addr + 16 L, +16), lds_addr taken from M0.  Written
// as inline asm rather than the builtin so the compiler does not treat every
// later LDS read as dependent on it (it cannot tell the tile buffers apart
// and would wait for all loads in flight); the kernels order these loads
// themselves with explicit vmcnt waits before the barrier that publishes a
// tile.  M0 is declared clobbered (the compiler re-sets it if it needs it).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_addr)
      : "m0");
}
// The same with a wave-uniform base in SGPRs and a 32-bit per-lane byte
// offset: fewer per-lane address operands, no 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds_addr)
      : "m0");
}

// A zero K/V row (up to 256 dims): the source of tile rows whose key does
// not exist and of pad positions.
__device__ __attribute__((aligned(256))) uint16_t g_zero_row[256] = {0};

// floor(x / N) for a positive power-of-two N and any sign of x.
template <int N>
__device__ __forceinline__ int floor_div(int x) {
  return x >= 0 ? x / N : -((N - 1 - x) / N);
}

// Visible key range of query position i (inclusive), or lo > hi if none:
// causal, extended to the end of i's image span, clipped to the window on a
// local layer and to the first key that exists (kmin_avail).
struct RowRange {
  int lo, hi;
};
__device__ __forceinline__ RowRange row_range(int i, int b, int kmin_avail, const PrefillArgs& a,
                                              const SpanTable& spt) {
  int hi = i;
  for (int s = 0; s < spt.n; ++s) {
    const Span sp = spt.s[s];
    if (sp.batch == b && sp.start <= i && i < sp.end) hi = max(hi, sp.end - 1);
  }
  int lo = kmin_avail;
  if (a.local) {
    lo = max(lo, i - a.window + 1);
    hi = min(hi, i + a.window - 1);
  }
  return RowRange{lo, hi};
}

}  // namespace
}  // namespace g3
