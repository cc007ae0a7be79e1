// QK-RMSNorm + RoPE prologue and the KV-cache append used by chunked prefill.
//
// Norm: x / sqrt(mean(x^2) + eps) * gamma over the head dimension D (Gemma 3
// Technical Report, section 2: QK-norm replaces soft-capping; "Gemma
// explained" module prints: RMSNorm over the head dimension, eps=1e-06; D is
// 128 for the 27B model, 256 for the 1B one).  RoPE: pairs (x_k, x_{k+D/2})
// rotated by (p / s) * base^(-2k/D) (Technical Report, section 2 "Long
// context": base 10k local / 1M global, linear position interpolation on the
// global layers).  Memory bound: one read and one write
// of each head row (256 bytes at D = 128, 512 at D = 256).
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

// D/16 lanes per head row (8 at D = 128, 16 at D = 256); lane j owns dims
// [8 j, 8 j + 8) and [D/2 + 8 j, D/2 + 8 j + 8), one 16-byte load and store
// per half, so every rotation pair (k, k + D/2) stays inside one lane.  A lane
// group takes one token and HB of its heads: the rotation angles depend on
// the position only, so their sin/cos (fp64 reduction, two transcendentals
// per pair) are computed once for the HB heads, and the HB rows' loads are
// all in flight before the first is used.
template <int D, bool NORM>
__global__ __launch_bounds__(256) void qknorm_rope_rows(RowsArgs a, Pos0Table p0t, RopeTable rt) {
  constexpr int LPR = D / 16;     // lanes per row
  constexpr int RPB = 256 / LPR;  // lane groups per workgroup
  constexpr int HB = kRopeHeadsPerGroup;
  const int j = threadIdx.x % LPR;
  double rev[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rev[i] = rt.rev[8 * j + i];
  float gam[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gam[i] = NORM ? a.gamma[8 * j + i] : 1.f;
    gam[8 + i] = NORM ? a.gamma[D / 2 + 8 * j + i] : 1.f;
  }
  const int nhb = (a.H + HB - 1) / HB;  // head blocks per token
  const long long n_groups = (long long)a.T * nhb;
  const long long stride = (long long)gridDim.x * RPB;
  for (long long X = (long long)blockIdx.x * RPB + threadIdx.x / LPR; X < n_groups; X += stride) {
    const long long t = X / nhb;
    const int h0 = (int)(X - t * nhb) * HB;
    const int bt = (int)(t / a.S);
    const int st = (int)(t - (long long)bt * a.S);
    const int pos = a.positions ? a.positions[t] : pos0_of(p0t, bt) + st;
    // rows past the last head re-read the last one (in bounds, never stored)
    u32x4 lo[HB], hi[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const uint16_t* src = a.in + (t * a.H + min(h0 + u, a.H - 1)) * D;
      lo[u] = *(const u32x4*)(src + 8 * j);
      hi[u] = *(const u32x4*)(src + D / 2 + 8 * j);
    }
    float sn[8], cs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rope_sincos(pos, rev[i], sn[i], cs[i]);
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int h = h0 + u;
      if (h >= a.H) break;
      float x[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf_lo(lo[u][e]);
        x[2 * e + 1] = bf_hi(lo[u][e]);
        x[8 + 2 * e] = bf_lo(hi[u][e]);
        x[8 + 2 * e + 1] = bf_hi(hi[u][e]);
      }
      if (NORM) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += x[i] * x[i];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, LPR);
        const float r = __frsqrt_rn(ss * (1.f / D) + a.eps);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = x[i] * r * gam[i];
      }
      float y[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y[i] = x[i] * cs[i] - x[8 + i] * sn[i];
        y[8 + i] = x[i] * sn[i] + x[8 + i] * cs[i];
      }
      const long long R = t * a.H + h;
      uint16_t* dst = a.out + (a.head_major ? (((long long)bt * a.H + h) * a.S + st) * D : R * D);
      u32x4 wlo, whi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wlo[e] = pack2(y[2 * e], y[2 * e + 1]);
        whi[e] = pack2(y[8 + 2 * e], y[8 + 2 * e + 1]);
      }
      *(u32x4*)(dst + 8 * j) = wlo;
      *(u32x4*)(dst + D / 2 + 8 * j) = whi;
    }
  }
}

// Copy a prefill chunk's normed+rotated keys (head-major workspace) and raw
// values into their cache slots.  A ring keeps only the last `cap` positions
// of the chunk, so earlier rows (which would land on the same slots) are
// skipped instead of racing.
__global__ __launch_bounds__(256) void append_chunk(AppendArgs a, Pos0Table p0t) {
  const int cpr = a.D / 8;  // 16-byte chunks per row
  const long long n = (long long)a.B * a.Hkv * a.S * cpr;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long long)gridDim.x * blockDim.x) {
    const int c16 = (int)(x % cpr);
    const long long row = x / cpr;  // (b, g, r)
    const int r = (int)(row % a.S);
    const long long bg = row / a.S;
    const int g = (int)(bg % a.Hkv);
    const int b = (int)(bg / a.Hkv);
    if (a.is_ring && r < a.S - a.cap) continue;
    const int pos = pos0_of(p0t, b) + r;
    const long long slot = a.is_ring ? (pos % a.cap) : pos;
    const long long dst = ((bg)*a.cap + slot) * a.D + c16 * 8;
    *(u32x4*)(a.ck + dst) = *(const u32x4*)(a.khat + row * a.D + c16 * 8);
    *(u32x4*)(a.cv + dst) = *(const u32x4*)(a.v + (((long long)b * a.S + r) * a.Hkv + g) * a.D + c16 * 8);
  }
}

static int grid_for(long long work_items, int per_block) {
  long long g = (work_items + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_qknorm_rope(const RowsArgs& a, const Pos0Table& p0t, const RopeTable& rt, hipStream_t st) {
  // a grid-stride loop over (token, head block) groups: at most 8 workgroups per CU
  const int rpb = 256 / (a.D / 16);
  const long long groups = (long long)a.T * ((a.H + kRopeHeadsPerGroup - 1) / kRopeHeadsPerGroup);
  long long grid = (groups + rpb - 1) / rpb;
  if (grid > 2048) grid = 2048;
  if (a.D == 256) {
    if (a.gamma)
      hipLaunchKernelGGL((qknorm_rope_rows<256, true>), dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
    else
      hipLaunchKernelGGL((qknorm_rope_rows<256, false>), dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
  } else {
    if (a.gamma)
      hipLaunchKernelGGL((qknorm_rope_rows<128, true>), dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
    else
      hipLaunchKernelGGL((qknorm_rope_rows<128, false>), dim3((int)grid), dim3(256), 0, st, a, p0t, rt);
  }
  return hipGetLastError();
}

hipError_t launch_append_chunk(const AppendArgs& a, const Pos0Table& p0t, hipStream_t st) {
  const int grid = grid_for((long long)a.B * a.Hkv * a.S * (a.D / 8), 256);
  hipLaunchKernelGGL(append_chunk, dim3(grid), dim3(256), 0, st, a, p0t);
  return hipGetLastError();
}

}  // namespace g3
