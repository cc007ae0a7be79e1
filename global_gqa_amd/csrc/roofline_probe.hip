// Roofline probes for gfx950: the ceilings the kernels' "fraction of peak"
// figures are read against, measured on the card in use.
//
//  * MFMA: every wave of 256 x k workgroups issues independent chains of
//    v_mfma_f32_32x32x16_bf16 (32768 flop each) and nothing else, so the
//    rate is the dense bf16 matrix-core ceiling at the clock the card holds
//    under that load.  Each workgroup also reads the shader clock
//    (s_memtime) and the 100 MHz reference clock (s_memrealtime) at its start
//    and end, which gives that clock.
//  * Stream: a read of a buffer well past the 256 MB Infinity Cache with
//    16-byte non-temporal loads, every lane folding its words into one value
//    written once: the HBM read ceiling a KV-streaming kernel can approach.
//
// Built as its own library (libg3probe.so): measurement support, not part of
// the attention library's interface.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;  // independent accumulators per wave

// iters x 32 MFMAs per wave; out: one float per thread (keeps the chains
// live), clk: per workgroup {memtime start, memtime end, realtime start,
// realtime end}.
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out, unsigned long long* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 32; ++m)
      acc[m % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m % kChains], 0, 0, 0);
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[4 * blockIdx.x + 0] = t0;
    clk[4 * blockIdx.x + 1] = t1;
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = r1;
  }
}

// Read of n16 16-byte words, each workgroup streaming its own contiguous
// share (as a decode split does), eight loads in flight per lane.
__global__ __launch_bounds__(256) void stream_read_blocks(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t per = n16 / gridDim.x;  // the remainder past gridDim.x * per is not read
  const u32x4* p = src + (size_t)blockIdx.x * per;
  uint32_t x = 0;
  size_t j = threadIdx.x;
  for (; j + 7 * 256 < per; j += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + j + 256 * k);
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; j < per; j += 256) {
    const u32x4 v = __builtin_nontemporal_load(p + j);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Grid-stride read of n16 16-byte words.
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    x ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// Dense bf16 MFMA ceiling.  workgroups of 256 threads (4 waves), iters x 32
// MFMAs per wave; reps timed launches after one untimed.  On success
// *tflops is the best rep's rate, *clock_ghz the shader clock over that rep
// (median over workgroups).  Returns 0, or the HIP error code.
int g3probe_mfma(int workgroups, int iters, int reps, double* tflops, double* clock_ghz, double* ms_best) {
  if (workgroups <= 0 || iters <= 0 || reps <= 0 || !tflops || !clock_ghz || !ms_best) return -1;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&out, (size_t)workgroups * 256 * sizeof(float));
  if (err == hipSuccess) err = hipMalloc(&clk, (size_t)workgroups * 4 * sizeof(unsigned long long));
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  double best = 1e30;
  unsigned long long* host = nullptr;
  if (err == hipSuccess) {
    host = new unsigned long long[(size_t)workgroups * 4];
    for (int r = 0; r <= reps && err == hipSuccess; ++r) {
      if (r == 0) {  // untimed warm-up
        hipLaunchKernelGGL(mfma_loop, dim3(workgroups), dim3(256), 0, 0, iters, out, clk);
        err = hipGetLastError();
        if (err == hipSuccess) err = hipDeviceSynchronize();
        continue;
      }
      err = hipEventRecord(e0, 0);
      hipLaunchKernelGGL(mfma_loop, dim3(workgroups), dim3(256), 0, 0, iters, out, clk);
      if (err == hipSuccess) err = hipGetLastError();
      if (err == hipSuccess) err = hipEventRecord(e1, 0);
      if (err == hipSuccess) err = hipEventSynchronize(e1);
      float ms = 0.f;
      if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
      if (err == hipSuccess && ms < best) {
        best = ms;
        err = hipMemcpy(host, clk, (size_t)workgroups * 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
      }
    }
  }
  if (err == hipSuccess) {
    const double flop = (double)workgroups * 4 /*waves*/ * (double)iters * 32 * 32768.0;
    *tflops = flop / (best * 1e-3) / 1e12;
    *ms_best = best;
    // median over workgroups of shader cycles / reference ticks (100 MHz)
    double* ratio = new double[workgroups];
    int n = 0;
    for (int w = 0; w < workgroups; ++w) {
      const double dc = (double)(host[4 * w + 1] - host[4 * w + 0]);
      const double dr = (double)(host[4 * w + 3] - host[4 * w + 2]);
      if (dr > 0) ratio[n++] = dc / dr * 0.1;  // GHz
    }
    for (int i = 1; i < n; ++i)  // insertion sort: workgroup counts are small
      for (int j = i; j > 0 && ratio[j - 1] > ratio[j]; --j) {
        const double t = ratio[j];
        ratio[j] = ratio[j - 1];
        ratio[j - 1] = t;
      }
    *clock_ghz = n ? ratio[n / 2] : 0.0;
    delete[] ratio;
  }
  delete[] host;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (clk) (void)hipFree(clk);
  if (out) (void)hipFree(out);
  return err == hipSuccess ? 0 : (int)err;
}

// HBM read ceiling over `bytes` (rounded down to 16) of device memory at
// `buf` (the caller's, contents irrelevant); reps timed launches after one
// untimed.  blocks = 0: a grid-stride pattern; 1: each workgroup reads its
// own contiguous share (bytes counted are the ones read).  *gbps is the best
// rep's rate.  Returns 0, or the HIP error code.
int g3probe_stream(const void* buf, size_t bytes, int workgroups, int reps, int blocks, double* gbps,
                   double* ms_best) {
  if (!buf || bytes < 16 || workgroups <= 0 || reps <= 0 || !gbps || !ms_best) return -1;
  const size_t n16 = blocks ? (bytes / 16 / workgroups) * workgroups : bytes / 16;
  if (n16 == 0) return -1;
  uint32_t* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&out, (size_t)workgroups * 256 * sizeof(uint32_t));
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  double best = 1e30;
  for (int r = 0; r <= reps && err == hipSuccess; ++r) {
    if (r > 0) err = hipEventRecord(e0, 0);
    if (blocks)
      hipLaunchKernelGGL(stream_read_blocks, dim3(workgroups), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
    else
      hipLaunchKernelGGL(stream_read, dim3(workgroups), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
    if (err == hipSuccess) err = hipGetLastError();
    if (r == 0) {
      if (err == hipSuccess) err = hipDeviceSynchronize();
      continue;
    }
    if (err == hipSuccess) err = hipEventRecord(e1, 0);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess && ms < best) best = ms;
  }
  if (err == hipSuccess) {
    *gbps = (double)(n16 * 16) / (best * 1e-3) / 1e9;
    *ms_best = best;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  return err == hipSuccess ? 0 : (int)err;
}

}  // extern "C"
