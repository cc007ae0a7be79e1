// Split-K decode attention over a per-layer KV cache (gfx950).
//
// One new token per sequence at position p: QK-RMSNorm + RoPE of q and of
// the new key, the new key/value written to their cache slot (slot p of a
// linear cache for global layers; slot p mod capacity of the ring a local
// layer keeps, since local layers only look back 1024 tokens: Gemma 3
// Technical Report, abstract and section 1), then softmax attention over
// [0, p] (global) or (p - window, p] (local).  GQA: the G query heads of a kv
// group share every K/V byte read (Technical Report, section 2).
//
// Pure HBM streaming: each workgroup owns (sequence, kv head, chunk of 256
// cache slots), loads the chunk's K and V rows once with 16-byte coalesced
// loads (all issued up front), scores every slot for all G heads (two-pass:
// exact chunk max, then exp and PV, so no rescaling), and writes an
// unnormalised partial (o, m, l).  A second kernel merges the partials of a
// head in fixed chunk order, so results are bitwise reproducible.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {
constexpr int kL = kDecodeChunk;       // slots per workgroup
constexpr int kKeysPerWave = kL / 4;    // 64
constexpr int kSteps = kKeysPerWave / 4;  // 16 steps of 4 keys per wave

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// RMSNorm + RoPE of one raw 128-vector by one wave: lane owns (k, k + 64).
__device__ __forceinline__ void norm_rope_vec(const uint16_t* src, const float* gamma, float eps, int pos,
                                              float base, float inv_scale, int lane, float& y0, float& y1) {
  float x0 = __uint_as_float((uint32_t)src[lane] << 16);
  float x1 = __uint_as_float((uint32_t)src[lane + 64] << 16);
  if (gamma) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rn = rsqrtf(ss * (1.f / kD) + eps);
    x0 *= rn * gamma[lane];
    x1 *= rn * gamma[lane + 64];
  }
  float sn, cs;
  rope_sincos(pos, rope_rev_freq(lane, base, inv_scale), sn, cs);
  y0 = x0 * cs - x1 * sn;
  y1 = x0 * sn + x1 * cs;
}

__device__ __forceinline__ float round_bf16(float x) {
  const uint32_t w = pack2(x, 0.f);
  return bf_lo(w);
}
}  // namespace

template <int G>
__global__ __launch_bounds__(256) void decode_splitk(DecodeArgs a) {
  __shared__ float qh[G][kD];
  __shared__ float kn[kD];
  __shared__ float vn[kD];
  __shared__ float sc[G][kL];
  __shared__ float red[4][G][kD];
  __shared__ float stat[G][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  int p = a.positions[b];
  p = max(0, min(p, a.max_pos));
  const int s0 = c * kL;
  const int s_new = a.is_ring ? (p % a.cap) : p;
  const bool owner = s_new >= s0 && s_new < s0 + kL;
  const long long head_base = ((long long)b * a.Hkv + g) * (long long)a.cap;
  float* part = a.ws + (((long long)b * a.Hq + g * G) * a.n_chunks + c) * (kD + 2);
  const long long head_stride = (long long)a.n_chunks * (kD + 2);

  // Whole chunk invisible (linear cache past p, or before the window)?
  bool empty = false;
  if (!a.is_ring) {
    if (s0 > p) empty = true;
    if (a.local && s0 + kL - 1 < p - a.window + 1) empty = true;
  }
  if (empty) {
    for (int x = tid; x < G * (kD + 2); x += 256) {
      const int hg = x / (kD + 2), e = x - hg * (kD + 2);
      part[hg * head_stride + e] = (e == kD) ? -__builtin_huge_valf() : 0.f;
    }
    return;
  }

  // ---- issue all K and V loads of this wave's 64 slots (16 B per lane per slot)
  const int j16 = lane & 15;   // dims [8 j16, 8 j16 + 8)
  const int kg = lane >> 4;    // key within a step of 4
  u32x4 kr[kSteps], vr[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int slot = s0 + wave * kKeysPerWave + 4 * st + kg;
    u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (slot < a.n_slots && slot != s_new) {
      const long long off = (head_base + slot) * kD + 8 * j16;
      kk = __builtin_nontemporal_load((const u32x4*)(a.ck + off));
      vv = __builtin_nontemporal_load((const u32x4*)(a.cv + off));
    }
    kr[st] = kk;
    vr[st] = vv;
  }

  // ---- q_hat for the G heads (and k_hat/v of the new token in its owner)
  for (int hg = wave; hg < G; hg += 4) {
    float y0, y1;
    norm_rope_vec(a.q + ((long long)b * a.Hq + g * G + hg) * kD, a.q_gamma, a.eps, p, a.base, a.inv_scale,
                  lane, y0, y1);
    qh[hg][lane] = round_bf16(y0);
    qh[hg][lane + 64] = round_bf16(y1);
  }
  if (owner && wave == 3) {
    float y0, y1;
    const long long src = ((long long)b * a.Hkv + g) * kD;
    norm_rope_vec(a.k_new + src, a.k_gamma, a.eps, p, a.base, a.inv_scale, lane, y0, y1);
    const uint32_t w = pack2(y0, y1);
    kn[lane] = bf_lo(w);
    kn[lane + 64] = bf_hi(w);
    const uint16_t v0 = a.v_new[src + lane], v1 = a.v_new[src + lane + 64];
    vn[lane] = __uint_as_float((uint32_t)v0 << 16);
    vn[lane + 64] = __uint_as_float((uint32_t)v1 << 16);
    a.ck[(head_base + s_new) * kD + lane] = (uint16_t)(w & 0xffffu);
    a.ck[(head_base + s_new) * kD + lane + 64] = (uint16_t)(w >> 16);
    a.cv[(head_base + s_new) * kD + lane] = v0;
    a.cv[(head_base + s_new) * kD + lane + 64] = v1;
  }
  __syncthreads();

  // ---- pass 1: scores for every slot and head
  float qv[G][8];
#pragma unroll
  for (int hg = 0; hg < G; ++hg)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hg][e] = qh[hg][8 * j16 + e];
  const float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int slot = s0 + wave * kKeysPerWave + 4 * st + kg;
    float kf[8];
    if (slot == s_new) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = kn[8 * j16 + e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf_lo(kr[st][e]);
        kf[2 * e + 1] = bf_hi(kr[st][e]);
      }
    }
    // visibility of this slot
    bool vis = slot < a.n_slots;
    if (vis) {
      if (a.is_ring) {
        const int d = ((p - slot) % a.cap + a.cap) % a.cap;
        const int jpos = p - d;
        vis = jpos >= 0 && (!a.local || d < a.window);
      } else {
        vis = slot <= p && (!a.local || p - slot < a.window);
      }
    }
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += qv[hg][e] * kf[e];
      d += __shfl_xor(d, 8, 16);
      d += __shfl_xor(d, 4, 16);
      d += __shfl_xor(d, 2, 16);
      d += __shfl_xor(d, 1, 16);
      if (j16 == 0) sc[hg][wave * kKeysPerWave + 4 * st + kg] = vis ? d : NEG_INF;
    }
  }
  __syncthreads();

  // ---- chunk max, probabilities and their sum (wave hg handles head hg)
  for (int hg = wave; hg < G; hg += 4) {
    float m = NEG_INF;
    for (int x = lane; x < kL; x += 64) m = fmaxf(m, sc[hg][x]);
    m = wave_max(m);
    const float mu = (m == NEG_INF) ? 0.f : m;
    float l = 0.f;
    for (int x = lane; x < kL; x += 64) {
      const float pr = fast_exp2((sc[hg][x] - mu) * a.sl2);
      sc[hg][x] = pr;
      l += pr;
    }
    l = wave_sum(l);
    if (lane == 0) {
      stat[hg][0] = m;
      stat[hg][1] = l;
    }
  }
  __syncthreads();

  // ---- pass 2: acc[hg][dims] = sum_slots p * v
  float acc[G][8];
#pragma unroll
  for (int hg = 0; hg < G; ++hg)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hg][e] = 0.f;
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int sl = wave * kKeysPerWave + 4 * st + kg;
    float vf[8];
    if (s0 + sl == s_new) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = vn[8 * j16 + e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf_lo(vr[st][e]);
        vf[2 * e + 1] = bf_hi(vr[st][e]);
      }
    }
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      const float pr = sc[hg][sl];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hg][e] += pr * vf[e];
    }
  }
  // reduce over the 4 key groups of the wave (lanes j16 + 16 kg)
#pragma unroll
  for (int hg = 0; hg < G; ++hg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[hg][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[hg][e] = x;
    }
  if (kg == 0) {
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][hg][8 * j16 + e] = acc[hg][e];
  }
  __syncthreads();
  for (int x = tid; x < G * kD; x += 256) {
    const int hg = x / kD, d = x - hg * kD;
    part[hg * head_stride + d] = red[0][hg][d] + red[1][hg][d] + red[2][hg][d] + red[3][hg][d];
  }
  if (tid < G) {
    part[tid * head_stride + kD] = stat[tid][0];
    part[tid * head_stride + kD + 1] = stat[tid][1];
  }
}

// Merge the split-K partials of one head: o = sum_c w_c o_c / sum_c w_c l_c
// with w_c = exp2((m_c - M) * scale * log2 e), chunks in ascending order.
__global__ __launch_bounds__(128) void decode_combine(DecodeArgs a) {
  const int h = blockIdx.x;  // b * Hq + head
  const int d = threadIdx.x;
  const float* part = a.ws + (long long)h * a.n_chunks * (kD + 2);
  const float NEG_INF = -__builtin_huge_valf();
  float M = NEG_INF;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part[c * (kD + 2) + kD]);
  float num = 0.f, den = 0.f;
  if (M != NEG_INF) {
    for (int c = 0; c < a.n_chunks; ++c) {
      const float mc = part[c * (kD + 2) + kD];
      if (mc == NEG_INF) continue;
      const float w = fast_exp2((mc - M) * a.sl2);
      num += w * part[c * (kD + 2) + d];
      den += w * part[c * (kD + 2) + kD + 1];
    }
  }
  const float o = den > 0.f ? num / den : 0.f;
  a.o[(long long)h * kD + d] = (uint16_t)(pack2(o, 0.f) & 0xffffu);
}

hipError_t launch_decode(const DecodeArgs& a, int G, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(a.n_chunks, a.B * a.Hkv);
  if (ev_start) hipEventRecord(ev_start, st);
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_splitk<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_splitk<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_splitk<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_splitk<8>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) hipEventRecord(ev_stop, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine, dim3(a.B * a.Hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace g3
