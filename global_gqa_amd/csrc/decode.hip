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
// Pure HBM streaming: each workgroup owns (sequence, kv head, split of the
// cache slots) and streams the split's K and V rows once with 16-byte
// coalesced non-temporal loads, each wave keeping eight steps of loads in
// flight.  D/8 lanes share a key row (8 dims each: 16 lanes at D = 128, 32 at
// D = 256; DPP row reductions) and all G heads of the group use every row.  The partial (o, m, l) of the
// split goes to the workspace; a second kernel merges the partials of a head
// in a fixed order, so results are bitwise reproducible.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

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

// RMSNorm + RoPE of one raw D-vector by one wave: lane owns the rotation
// pairs (k, k + D/2) for k = lane + 64 i, i < D/128.
template <int D>
__device__ __forceinline__ void norm_rope_vec(const uint16_t* src, const float* gamma, float eps, int pos,
                                              const RopeTable& rt, int lane, float (&y0)[D / 128],
                                              float (&y1)[D / 128]) {
  constexpr int NP = D / 128;
  float x0[NP], x1[NP];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    x0[i] = __uint_as_float((uint32_t)src[lane + 64 * i] << 16);
    x1[i] = __uint_as_float((uint32_t)src[lane + 64 * i + D / 2] << 16);
    ss += x0[i] * x0[i] + x1[i] * x1[i];
  }
  if (gamma) {
    ss = wave_sum(ss);
    const float rn = rsqrtf(ss * (1.f / D) + eps);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      x0[i] *= rn * gamma[lane + 64 * i];
      x1[i] *= rn * gamma[lane + 64 * i + D / 2];
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float sn, cs;
    rope_sincos(pos, rt.rev[lane + 64 * i], sn, cs);
    y0[i] = x0[i] * cs - x1[i] * sn;
    y1[i] = x0[i] * sn + x1[i] * cs;
  }
}

__device__ __forceinline__ float round_bf16(float x) {
  const uint32_t w = pack2(x, 0.f);
  return bf_lo(w);
}
}  // namespace

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in all 16.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad xor 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad xor 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // half mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // row mirror
  return x;
}

// Sum over the D/8 lanes that share a key row.
template <int D>
__device__ __forceinline__ float row_sum(float x) {
  x = row16_sum(x);
  if (D == 256) x += __shfl_xor(x, 16);
  return x;
}

// Per-lane running state of one kv group's G heads over the keys this lane's
// row group sees (dims 8 jl .. 8 jl + 7 of the accumulator).
template <int G>
struct StreamState {
  float m[G], l[G], acc[G][8];
  int nvis;  // visible keys seen by this lane
};

// Stream the split's slots: step st covers 4 RW consecutive slots (RW = 64 /
// (D/8) per wave, one per row group); each step's K and V rows are loaded
// kDepth steps ahead so the memory pipe never drains.  ONLINE = false:
// p = exp2(s) directly (QK-RMSNorm bounds the logits); ONLINE = true:
// running maximum.
template <int G, int D, bool ONLINE>
__device__ __forceinline__ void stream_split(const DecodeArgs& a, const float (&qv)[G][8], const float* kn,
                                             const float* vn, long long head_base, int s0, int nsteps, int p,
                                             int p_mod, int s_new, int wave, int lane, StreamState<G>& st) {
  constexpr int kDepth = 8;
  constexpr int LPR = D / 8, RW = 64 / LPR;
  const int j16 = lane % LPR;
  const int kg = lane / LPR;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = ONLINE ? -__builtin_huge_valf() : 0.f;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
  }
  st.nvis = 0;
  u32x4 kb[kDepth], vb[kDepth];
  auto slot_of = [&](int step) { return s0 + 4 * RW * step + RW * wave + kg; };
  auto issue = [&](int step, int d) {
    int slot = slot_of(step);
    if (slot >= a.n_slots) slot = 0;  // stays in bounds; masked below
    const long long off = (head_base + slot) * D + 8 * j16;
    kb[d] = __builtin_nontemporal_load((const u32x4*)(a.ck + off));
    vb[d] = __builtin_nontemporal_load((const u32x4*)(a.cv + off));
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (d < nsteps) issue(d, d);
  for (int st0 = 0; st0 < nsteps; st0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int step = st0 + d;
      if (step < nsteps) {
        const int slot = slot_of(step);
        bool vis = slot < a.n_slots;
        if (a.is_ring) {
          int dist = p_mod - slot;
          if (dist < 0) dist += a.cap;
          vis = vis && (p - dist >= 0) && (!a.local || dist < a.window);
        } else {
          vis = vis && slot <= p && (!a.local || p - slot < a.window);
        }
        float kf[8], vf[8];
        if (slot == s_new) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kf[e] = kn[8 * j16 + e];
            vf[e] = vn[8 * j16 + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[2 * e] = bf_lo(kb[d][e]);
            kf[2 * e + 1] = bf_hi(kb[d][e]);
            vf[2 * e] = bf_lo(vb[d][e]);
            vf[2 * e + 1] = bf_hi(vb[d][e]);
          }
        }
        if (step + kDepth < nsteps) issue(step + kDepth, d);
        st.nvis += vis ? 1 : 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot += qv[h][e] * kf[e];
          const float sc = row_sum<D>(dot);
          float pr;
          if (ONLINE) {
            const float m_new = vis ? fmaxf(st.m[h], sc) : st.m[h];
            const float alpha = (m_new == st.m[h]) ? 1.f : fast_exp2(st.m[h] - m_new);
            pr = vis ? fast_exp2(sc - m_new) : 0.f;
            st.m[h] = m_new;
            st.l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
          } else {
            pr = vis ? fast_exp2(sc) : 0.f;
          }
          st.l[h] += pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) st.acc[h][e] += pr * vf[e];
        }
      }
    }
  }
}

template <int G, int D>
// Three workgroups per CU where the registers allow (G = 4: 168 VGPRs with a
// few spills instead of 174 at two per CU, 5% faster on the 1B 32 x 32K global
// layer, the same bits); G = 8 at D = 256 stays at two.
__global__ __launch_bounds__(256, (D == 256 && G == 8) ? 2 : 3) void decode_splitk(DecodeArgs a, RopeTable rt) {
  constexpr int LPR = D / 8, RW = 64 / LPR, NP = D / 128;
  __shared__ float kn[D];
  __shared__ float vn[D];
  __shared__ float part_m[4][RW][G];           // [wave][row group][head]
  __shared__ float part_l[4][RW][G];
  __shared__ float part_acc[4][RW][G][D];      // unnormalised, relative to part_m
  __shared__ int bad_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  int p = a.positions[b];
  p = max(0, min(p, a.max_pos));
  const int s0 = c * a.split;
  const int s_end = min(s0 + a.split, a.n_slots);
  const int nsteps = (s_end - s0 + 4 * RW - 1) / (4 * RW);
  const int s_new = a.is_ring ? (p % a.cap) : p;
  const int p_mod = a.is_ring ? (p % a.cap) : p;
  const bool owner = s_new >= s0 && s_new < s_end;
  const long long head_base = ((long long)b * a.Hkv + g) * (long long)a.cap;
  float* part = a.ws + (((long long)b * a.Hq + g * G) * a.n_chunks + c) * (D + 2);
  const long long head_stride = (long long)a.n_chunks * (D + 2);

  // Whole split invisible (linear cache past p, or before the window)?
  bool empty = false;
  if (!a.is_ring) {
    if (s0 > p) empty = true;
    if (a.local && s_end - 1 < p - a.window + 1) empty = true;
  }
  if (empty) {
    if (a.n_chunks == 1) {  // (unreachable: the token's own slot is visible)
      for (int x = tid; x < G * D; x += 256) a.o[((long long)b * a.Hq + g * G) * D + x] = 0;
      return;
    }
    for (int x = tid; x < G * (D + 2); x += 256) {
      const int hg = x / (D + 2), e = x - hg * (D + 2);
      part[hg * head_stride + e] = (e == D) ? -__builtin_huge_valf() : 0.f;
    }
    return;
  }

  // q_hat for the G heads, scaled by softmax_scale * log2(e) (scores in log2
  // units), and k_hat / v of the new token in the workgroup that owns its slot
  const int j16 = lane % LPR;
  float qv[G][8];
  {
    __shared__ float qh[G][D];
    for (int hg = wave; hg < G; hg += 4) {
      float y0[NP], y1[NP];
      norm_rope_vec<D>(a.q + ((long long)b * a.Hq + g * G + hg) * D, a.q_gamma, a.eps, p, rt, lane, y0, y1);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        qh[hg][lane + 64 * i] = round_bf16(y0[i] * a.sl2);
        qh[hg][lane + 64 * i + D / 2] = round_bf16(y1[i] * a.sl2);
      }
    }
    if (owner && wave == 3) {
      float y0[NP], y1[NP];
      const long long src = ((long long)b * a.Hkv + g) * D;
      norm_rope_vec<D>(a.k_new + src, a.k_gamma, a.eps, p, rt, lane, y0, y1);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d0 = lane + 64 * i, d1 = d0 + D / 2;
        const uint32_t w = pack2(y0[i], y1[i]);
        kn[d0] = bf_lo(w);
        kn[d1] = bf_hi(w);
        const uint16_t v0 = a.v_new[src + d0], v1 = a.v_new[src + d1];
        vn[d0] = __uint_as_float((uint32_t)v0 << 16);
        vn[d1] = __uint_as_float((uint32_t)v1 << 16);
        a.ck[(head_base + s_new) * D + d0] = (uint16_t)(w & 0xffffu);
        a.ck[(head_base + s_new) * D + d1] = (uint16_t)(w >> 16);
        a.cv[(head_base + s_new) * D + d0] = v0;
        a.cv[(head_base + s_new) * D + d1] = v1;
      }
    }
    if (tid == 0) bad_flag = 0;
    __syncthreads();
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hg][e] = qh[hg][8 * j16 + e];
  }

  StreamState<G> st;
  stream_split<G, D, false>(a, qv, kn, vn, head_base, s0, nsteps, p, p_mod, s_new, wave, lane, st);
  // The fast pass needs no running maximum because QK-RMSNorm bounds the
  // logits; if a sum leaves [2^-64, 2^64] (extreme gammas, no norm, foreign
  // cache contents) the split is streamed again with the running maximum.
  bool bad = false;
#pragma unroll
  for (int h = 0; h < G; ++h) bad = bad || !(st.l[h] <= 0x1p64f) || (st.nvis > 0 && !(st.l[h] >= 0x1p-64f));
  if (bad) bad_flag = 1;
  __syncthreads();
  if (bad_flag) stream_split<G, D, true>(a, qv, kn, vn, head_base, s0, nsteps, p, p_mod, s_new, wave, lane, st);

  // ---- merge the 4 RW partial states (4 waves x RW row groups) of each head
  const int kgrp = lane / LPR;
  if (j16 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      part_m[wave][kgrp][h] = st.m[h];
      part_l[wave][kgrp][h] = st.l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) part_acc[wave][kgrp][h][8 * j16 + e] = st.acc[h][e];
  __syncthreads();
  const float NEG_INF = -__builtin_huge_valf();
  for (int x = tid; x < G * D; x += 256) {
    const int h = x / D, d = x - h * D;
    float M = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4 * RW; ++i) M = fmaxf(M, part_m[i / RW][i % RW][h]);
    float num = 0.f, den = 0.f;
    if (M != NEG_INF) {
#pragma unroll
      for (int i = 0; i < 4 * RW; ++i) {
        const float mi = part_m[i / RW][i % RW][h];
        const float wgt = (mi == NEG_INF) ? 0.f : fast_exp2(mi - M);
        num += wgt * part_acc[i / RW][i % RW][h][d];
        den += wgt * part_l[i / RW][i % RW][h];
      }
    }
    if (a.n_chunks == 1) {
      // a single split is the whole answer (the merge below would weigh it by
      // exp2(0) = 1): normalise and store o here, no merge pass
      const float o = den > 0.f ? num / den : 0.f;
      a.o[((long long)b * a.Hq + g * G + h) * D + d] = (uint16_t)(pack2(o, 0.f) & 0xffffu);
      continue;
    }
    part[h * head_stride + d] = num;
    if (d == 0) {
      part[h * head_stride + D] = (den > 0.f) ? M : NEG_INF;
      part[h * head_stride + D + 1] = den;
    }
  }
}

// Merge the split-K partials of one head: o = sum_c w_c o_c / sum_c w_c l_c
// with w_c = exp2(m_c - M) (maxima are in log2 units).  1024 / D groups of D
// threads (one per dim) take the splits c = j, j + groups, ...
// with a running maximum, then thread group 0 merges the groups' (M, num,
// den) in group order: a fixed order, so the result is bitwise
// reproducible, and a long cache's hundreds of splits are read by many
// threads at once instead of one after another.
template <int D>
__global__ __launch_bounds__(1024) void decode_combine(DecodeArgs a) {
  constexpr int kCombineGroups = 1024 / D;
  __shared__ float gm[kCombineGroups], gnum[kCombineGroups][D], gden[kCombineGroups];
  const int h = blockIdx.x;  // b * Hq + head
  const int d = threadIdx.x % D;
  const int grp = threadIdx.x / D;
  const float* part = a.ws + (long long)h * a.n_chunks * (D + 2);
  const float NEG_INF = -__builtin_huge_valf();
  float M = NEG_INF, num = 0.f, den = 0.f;
  for (int c = grp; c < a.n_chunks; c += kCombineGroups) {
    const float* pc = part + (long long)c * (D + 2);
    const float mc = pc[D];
    if (mc == NEG_INF) continue;
    if (mc > M) {
      const float r = (M == NEG_INF) ? 0.f : fast_exp2(M - mc);
      num *= r;
      den *= r;
      M = mc;
    }
    const float w = fast_exp2(mc - M);
    num += w * pc[d];
    den += w * pc[D + 1];
  }
  gnum[grp][d] = num;
  if (d == 0) {
    gm[grp] = M;
    gden[grp] = den;
  }
  __syncthreads();
  if (grp != 0) return;
  float MM = NEG_INF;
#pragma unroll
  for (int g = 0; g < kCombineGroups; ++g) MM = fmaxf(MM, gm[g]);
  float n2 = 0.f, d2 = 0.f;
  if (MM != NEG_INF) {
#pragma unroll
    for (int g = 0; g < kCombineGroups; ++g) {
      if (gm[g] == NEG_INF) continue;
      const float w = fast_exp2(gm[g] - MM);
      n2 += w * gnum[g][d];
      d2 += w * gden[g];
    }
  }
  const float o = d2 > 0.f ? n2 / d2 : 0.f;
  a.o[(long long)h * D + d] = (uint16_t)(pack2(o, 0.f) & 0xffffu);
}

hipError_t launch_decode(const DecodeArgs& a, const RopeTable& rt, int G, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  const dim3 grid(a.n_chunks, a.B * a.Hkv);
  if (ev_start) hipEventRecord(ev_start, st);
  if (a.D == 256) {
    switch (G) {
      case 1: hipLaunchKernelGGL((decode_splitk<1, 256>), grid, dim3(256), 0, st, a, rt); break;
      case 2: hipLaunchKernelGGL((decode_splitk<2, 256>), grid, dim3(256), 0, st, a, rt); break;
      case 4: hipLaunchKernelGGL((decode_splitk<4, 256>), grid, dim3(256), 0, st, a, rt); break;
      case 8: hipLaunchKernelGGL((decode_splitk<8, 256>), grid, dim3(256), 0, st, a, rt); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (G) {
      case 1: hipLaunchKernelGGL((decode_splitk<1, 128>), grid, dim3(256), 0, st, a, rt); break;
      case 2: hipLaunchKernelGGL((decode_splitk<2, 128>), grid, dim3(256), 0, st, a, rt); break;
      case 4: hipLaunchKernelGGL((decode_splitk<4, 128>), grid, dim3(256), 0, st, a, rt); break;
      case 8: hipLaunchKernelGGL((decode_splitk<8, 128>), grid, dim3(256), 0, st, a, rt); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) hipEventRecord(ev_stop, st);
  if (e != hipSuccess || a.n_chunks == 1) return e;
  if (a.D == 256)
    hipLaunchKernelGGL(decode_combine<256>, dim3(a.B * a.Hq), dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(decode_combine<128>, dim3(a.B * a.Hq), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace g3
