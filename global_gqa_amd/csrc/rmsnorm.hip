// Row RMSNorm over the model width, with an optional residual add: the
// layer's input_layernorm before the attention and its
// post_attention_layernorm after o_proj ("Gemma explained: What's new in
// Gemma 3", 27B module print: Gemma3RMSNorm((5376,), eps=1e-06); Gemma 3
// Technical Report, section 2: pre-norm and post-norm with RMSNorm).
//
//   out[t] = residual[t] + x[t] / sqrt(mean(x[t]^2) + eps) * gamma   (residual optional)
//
// One workgroup of 256 threads per row; each thread keeps its (at most 4)
// 16-byte pieces of the row in registers between the sum of squares and the
// scaled store, so the row is read once.  HBM bound: 2 bytes read and 2
// written per element (plus 2 read for the residual).
//
// The input norm can also be folded into the q/k/v projection that follows
// it: (x / rms(x) * gamma) W^T = (1 / rms(x)) * x (W diag(gamma))^T.  For that
// path this file also holds the row scale alone (1 / rms(x) per row, no
// normed copy of x written) and the one-time fold of gamma into W.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormPieces = 4;  // 16-byte pieces per thread: width <= 8 * 4 * 256 = 8192

__global__ __launch_bounds__(kNormThreads) void rmsnorm_rows(NormArgs a) {
  __shared__ float s_part[kNormThreads / 64];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_pieces = a.W / 8;
  const uint16_t* src = a.x + row * a.W;
  u32x4 v[kNormPieces];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int pc = tid + kNormThreads * i;
    if (pc < n_pieces) {
      v[i] = *(const u32x4*)(src + 8 * pc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(v[i][e]), hi = bf_hi(v[i][e]);
        ss += lo * lo + hi * hi;
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += s_part[w];
  const float r = __frsqrt_rn(tot / (float)a.W + a.eps);
  uint16_t* dst = a.out + row * a.W;
  const uint16_t* res = a.residual ? a.residual + row * a.W : nullptr;
#pragma unroll
  for (int i = 0; i < kNormPieces; ++i) {
    const int pc = tid + kNormThreads * i;
    if (pc >= n_pieces) continue;
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = bf_lo(v[i][e]) * r;
      y[2 * e + 1] = bf_hi(v[i][e]) * r;
    }
    if (a.gamma) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= a.gamma[8 * pc + e];
    }
    if (res) {
      const u32x4 rv = *(const u32x4*)(res + 8 * pc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[2 * e] += bf_lo(rv[e]);
        y[2 * e + 1] += bf_hi(rv[e]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2(y[2 * e], y[2 * e + 1]);
    *(u32x4*)(dst + 8 * pc) = o;
  }
}

// Only the row scale 1 / sqrt(mean(x^2) + eps), fp32: the input norm of a
// layer whose gamma is folded into the projection weights.  One wave per row
// (16-byte pieces, four in flight per lane); 2 bytes read per element.
__global__ __launch_bounds__(256) void rms_scale_rows(NormArgs a, float* scale) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int n_pieces = a.W / 8;
  const uint16_t* src = a.x + row * a.W;
  float ss = 0.f;
  for (int p0 = 0; p0 < n_pieces; p0 += 4 * 64) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = p0 + lane + 64 * i;
      v[i] = pc < n_pieces ? *(const u32x4*)(src + 8 * pc) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(v[i][e]), hi = bf_hi(v[i][e]);
        ss += lo * lo + hi * hi;
      }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) scale[row] = __frsqrt_rn(ss / (float)a.W + a.eps);
}

// out[n][k] = w[n][k] * gamma[k] in fp32, rounded to bf16 once; width is a
// multiple of 8 (one 16-byte piece per thread and step).
__global__ __launch_bounds__(256) void fold_gamma_rows(const uint16_t* w, const float* gamma, uint16_t* out,
                                                       long long n_pieces, int width) {
  const int ppr = width / 8;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n_pieces; x += (long long)gridDim.x * 256) {
    const int k0 = 8 * (int)(x % ppr);
    const u32x4 v = *(const u32x4*)(w + 8 * x);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2(bf_lo(v[e]) * gamma[k0 + 2 * e], bf_hi(v[e]) * gamma[k0 + 2 * e + 1]);
    *(u32x4*)(out + 8 * x) = o;
  }
}

}  // namespace

int rmsnorm_max_width() { return 8 * kNormPieces * kNormThreads; }

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_rows, dim3(a.T), dim3(kNormThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_rms_scale(const NormArgs& a, float* scale, hipStream_t st) {
  hipLaunchKernelGGL(rms_scale_rows, dim3((int)(((long long)a.T + 3) / 4)), dim3(256), 0, st, a, scale);
  return hipGetLastError();
}

hipError_t launch_fold_gamma(const uint16_t* w, const float* gamma, uint16_t* out, long long rows, int width,
                             hipStream_t st) {
  const long long n_pieces = rows * (width / 8);
  long long grid = (n_pieces + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(fold_gamma_rows, dim3((int)grid), dim3(256), 0, st, w, gamma, out, n_pieces, width);
  return hipGetLastError();
}

}  // namespace g3
