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
__device__ __forceinline__ int xcd_remap(int x, int n) {
  const int q = n / 8, r = n % 8;
  const int xcd = x % 8, slot = x / 8;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

}  // namespace g3
