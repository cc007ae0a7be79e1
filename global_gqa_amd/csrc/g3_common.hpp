// Shared device helpers for the g3attn HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g3 {

constexpr int kD = 128;          // head dimension of the 27B-shaped kernels
constexpr int kDMax = 256;       // largest head dimension (Gemma 3 1B)
constexpr int kMaxSpans = 64;    // image spans per call (kernel-argument table)
constexpr int kMaxBatchPos0 = 256;  // sequences per prefill call with explicit pos0

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// One image span [start, end) of sequence `batch`, absolute positions.
struct Span {
  int32_t batch, start, end;
};

// Spans of one call, passed by value in the kernel arguments.
struct SpanTable {
  int32_t n;
  Span s[kMaxSpans];
};

// Per-sequence first position of a prefill chunk (kernel arguments).
struct Pos0Table {
  int32_t uniform;   // 1: every sequence starts at pos0[0]
  int32_t v[kMaxBatchPos0];
};

__device__ __forceinline__ int pos0_of(const Pos0Table& t, int b) { return t.uniform ? t.v[0] : t.v[b]; }

// RoPE frequencies of the D/2 rotation pairs in revolutions per position,
// base^(-2k/D) / (2 pi) / interp_scale, computed once per call in fp64
// (entries past D/2 unused).
struct RopeTable {
  double rev[kDMax / 2];
};

// bf16 <-> f32 on packed 32-bit words (low half = element 0).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {  // round to nearest even
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sin/cos of 2*pi*(pos * rev): the product is reduced to [-1/2, 1/2]
// revolutions in fp64 before the fp32 hardware sin/cos (which take
// revolutions), so the angle stays accurate at positions near 2^17.
__device__ __forceinline__ void rope_sincos(int pos, double rev, float& s, float& c) {
  double r = (double)pos * rev;
  float f = (float)(r - __builtin_rint(r));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// Map a hardware workgroup index to a logical one so that consecutive
// logical indices land on the same XCD: the dispatcher hands workgroups to
// the 8 XCDs round-robin, and tiles that share K/V should share an L2.
__host__ __device__ inline int xcd_remap(int x, int n) {
  const int q = n / 8, r = n % 8;
  const int xcd = x % 8, slot = x / 8;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// The same dispatcher dealing rounds of 8 consecutive logical indices to
// the 8 XCDs in alternating directions (serpentine): XCD j takes index
// 8 r + j in even rounds r and 8 r + 7 - j in odd ones (a last, partial
// round in order).  With indices ordered heaviest first, every XCD gets an
// even mix of heavy and light items.
__host__ __device__ inline int xcd_serpentine(int x, int n) {
  const int r = x / 8, j = x % 8;
  return ((r & 1) == 0 || 8 * r + 8 > n) ? x : 8 * r + 7 - j;
}

// Prefill work items: one per (sequence, kv head) run bg < n_groups and
// query tile, nq tiles per run.  A logical item index li is either
// run-major (li = bg * nq + rank) or rank-major (li = rank * n_groups + bg);
// rank 0 is the run's heaviest item (the last query tile: under the causal
// mask it sees the most keys).
__host__ __device__ inline void prefill_item_coords(int li, int n_groups, int nq, bool rank_major, int& bg,
                                                    int& qt) {
  int rank;
  if (rank_major) {
    rank = li / n_groups;
    bg = li - rank * n_groups;
  } else {
    bg = li / nq;
    rank = li - bg * nq;
  }
  qt = nq - 1 - rank;
}

// Whether a one-item-per-workgroup prefill launch orders its items
// rank-major and deals them serpentine over the XCDs.  Run-major blocks per
// XCD keep a run's tiles in one L2, and with a multiple of 8 runs every XCD
// gets whole runs and equal work.  With fewer or other counts of runs, whole
// runs cannot be spread evenly and a run's tiles differ in weight (global
// layers: 1 to S/64 key tiles), so contiguous blocks would give one XCD the
// heaviest tiles of a run and another its lightest: the items go out
// rank-major (the heaviest tile of every run first) and serpentine.  Local
// layers' items all cost about the same (window plus query tile) and keep
// the run-major blocks for their L2 reuse.
__host__ __device__ inline bool prefill_rank_major(bool local, int n_groups) { return !local && n_groups % 8 != 0; }

// Local layers with K = items / workgroups > 1 (nq a multiple of K):
// workgroup slot s (an XCD's slots are consecutive) takes the K query tiles
// j, j + nq/K, ..., j + (K-1) nq/K of one (sequence, kv head) run, the last
// (latest rank: the lightest, near the start of the sequence) first.  The
// workgroups that hold one of a run's short first tiles then run out of step
// with the rest, so the item boundaries, where every workgroup loads its Q
// rows and first K/V tiles at once, are spread over time.  At each step an
// XCD's workgroups cover nq/K consecutive query tiles of each of its runs.
__host__ __device__ inline int prefill_spread_item(int s, int kk, int K, int nq) {
  const int per = nq / K;
  const int bg = s / per, j = s - bg * per;
  const int k = kk == 0 ? K - 1 : kk - 1;
  return bg * nq + j + per * k;
}

// Logical item of hardware workgroup x in a launch of n = n_groups * nq
// workgroups, one item each.
__host__ __device__ inline int prefill_item_of_workgroup(int x, int n, bool rank_major) {
  return rank_major ? xcd_serpentine(x, n) : xcd_remap(x, n);
}

}  // namespace g3
