// QK-RMSNorm + RoPE prologue and the KV-cache append used by chunked prefill.
//
// Norm: x / sqrt(mean(x^2) + eps) * gamma over the head dimension (Gemma 3
// Technical Report, section 2: QK-norm replaces soft-capping; "Gemma
// explained" 27B module print: RMSNorm((128,), eps=1e-06)).  RoPE: pairs
// (x_k, x_{k+64}) rotated by (p / s) * base^(-2k/128) (Technical Report,
// section 2 "Long context": base 10k local / 1M global, linear position
// interpolation on the global layers).  Memory bound: one read and one write
// of each 256-byte head row.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

// 16 lanes per head row; lane j owns dims [4j, 4j+4) and [64+4j, 64+4j+4),
// so every rotation pair stays inside one lane.
template <bool NORM>
__global__ __launch_bounds__(256) void qknorm_rope_rows(RowsArgs a, Pos0Table p0t, RopeTable rt) {
  const int j = threadIdx.x & 15;
  double rev[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rev[i] = rt.rev[4 * j + i];
  float gam[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gam[i] = NORM ? a.gamma[4 * j + i] : 1.f;
    gam[4 + i] = NORM ? a.gamma[64 + 4 * j + i] : 1.f;
  }
  const long long n_rows = (long long)a.T * a.H;
  const long long stride = (long long)gridDim.x * 16;
  for (long long R = (long long)blockIdx.x * 16 + (threadIdx.x >> 4); R < n_rows; R += stride) {
    const long long t = R / a.H;
    const int h = (int)(R - t * a.H);
    const int bt = (int)(t / a.S);
    const int st = (int)(t - (long long)bt * a.S);
    const int pos = a.positions ? a.positions[t] : pos0_of(p0t, bt) + st;
    const uint16_t* src = a.in + R * kD;
    const u32x2 lo = *(const u32x2*)(src + 4 * j);
    const u32x2 hi = *(const u32x2*)(src + 64 + 4 * j);
    float x[8] = {bf_lo(lo[0]), bf_hi(lo[0]), bf_lo(lo[1]), bf_hi(lo[1]),
                  bf_lo(hi[0]), bf_hi(hi[0]), bf_lo(hi[1]), bf_hi(hi[1])};
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
      ss += __shfl_xor(ss, 8, 16);
      ss += __shfl_xor(ss, 4, 16);
      ss += __shfl_xor(ss, 2, 16);
      ss += __shfl_xor(ss, 1, 16);
      const float r = __frsqrt_rn(ss * (1.f / kD) + a.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = x[i] * r * gam[i];
    }
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sn, cs;
      rope_sincos(pos, rev[i], sn, cs);
      y[i] = x[i] * cs - x[4 + i] * sn;
      y[4 + i] = x[i] * sn + x[4 + i] * cs;
    }
    uint16_t* dst = a.out + (a.head_major ? (((long long)bt * a.H + h) * a.S + st) * kD : R * kD);
    *(u32x2*)(dst + 4 * j) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    *(u32x2*)(dst + 64 + 4 * j) = u32x2{pack2(y[4], y[5]), pack2(y[6], y[7])};
  }
}

// Copy a prefill chunk's normed+rotated keys (head-major workspace) and raw
// values into their cache slots.  A ring keeps only the last `cap` positions
// of the chunk, so earlier rows (which would land on the same slots) are
// skipped instead of racing.
__global__ __launch_bounds__(256) void append_chunk(AppendArgs a, Pos0Table p0t) {
  const long long n = (long long)a.B * a.Hkv * a.S * 16;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long long)gridDim.x * blockDim.x) {
    const int c16 = (int)(x & 15);
    const long long row = x >> 4;  // (b, g, r)
    const int r = (int)(row % a.S);
    const long long bg = row / a.S;
    const int g = (int)(bg % a.Hkv);
    const int b = (int)(bg / a.Hkv);
    if (a.is_ring && r < a.S - a.cap) continue;
    const int pos = pos0_of(p0t, b) + r;
    const long long slot = a.is_ring ? (pos % a.cap) : pos;
    const long long dst = ((bg)*a.cap + slot) * kD + c16 * 8;
    *(u32x4*)(a.ck + dst) = *(const u32x4*)(a.khat + row * kD + c16 * 8);
    *(u32x4*)(a.cv + dst) = *(const u32x4*)(a.v + (((long long)b * a.S + r) * a.Hkv + g) * kD + c16 * 8);
  }
}

static int grid_for(long long work_items, int per_block) {
  long long g = (work_items + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_qknorm_rope(const RowsArgs& a, const Pos0Table& p0t, const RopeTable& rt, hipStream_t st) {
  // a grid-stride loop over rows: at most 8 workgroups per CU
  long long grid = ((long long)a.T * a.H + 15) / 16;
  if (grid > 2048) grid = 2048;
  if (a.gamma)
    hipLaunchKernelGGL(qknorm_rope_rows<true>, dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
  else
    hipLaunchKernelGGL(qknorm_rope_rows<false>, dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
  return hipGetLastError();
}

hipError_t launch_append_chunk(const AppendArgs& a, const Pos0Table& p0t, hipStream_t st) {
  const int grid = grid_for((long long)a.B * a.Hkv * a.S * 16, 256);
  hipLaunchKernelGGL(append_chunk, dim3(grid), dim3(256), 0, st, a, p0t);
  return hipGetLastError();
}

}  // namespace g3
