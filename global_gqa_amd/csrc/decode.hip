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
// flight.  Sixteen lanes share a key row (8 dims each, DPP row reductions)
// and all G heads of the group use every row.  The partial (o, m, l) of the
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

// RMSNorm + RoPE of one raw 128-vector by one wave: lane owns (k, k + 64).
__device__ __forceinline__ void norm_rope_vec(const uint16_t* src, const float* gamma, float eps, int pos,
                                              double rev, int lane, float& y0, float& y1) {
  float x0 = __uint_as_float((uint32_t)src[lane] << 16);
  float x1 = __uint_as_float((uint32_t)src[lane + 64] << 16);
  if (gamma) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rn = rsqrtf(ss * (1.f / kD) + eps);
    x0 *= rn * gamma[lane];
    x1 *= rn * gamma[lane + 64];
  }
  float sn, cs;
  rope_sincos(pos, rev, sn, cs);
  y0 = x0 * cs - x1 * sn;
  y1 = x0 * sn + x1 * cs;
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

// Per-lane running state of one kv group's G heads over the keys this lane's
// 16-lane group sees (dims 8*j16 .. 8*j16+7 of the accumulator).
template <int G>
struct StreamState {
  float m[G], l[G], acc[G][8];
  int nvis;  // visible keys seen by this lane
};

// Stream the split's slots: step st covers 16 consecutive slots (4 per wave,
// one per 16-lane group); each step's K and V rows are loaded kDepth steps
// ahead so the memory pipe never drains.  ONLINE = false: p = exp2(s)
// directly (QK-RMSNorm bounds the logits); ONLINE = true: running maximum.
template <int G, bool ONLINE>
__device__ __forceinline__ void stream_split(const DecodeArgs& a, const float (&qv)[G][8], const float* kn,
                                             const float* vn, long long head_base, int s0, int nsteps, int p,
                                             int p_mod, int s_new, int wave, int lane, StreamState<G>& st) {
  constexpr int kDepth = 8;
  const int j16 = lane & 15;
  const int kg = lane >> 4;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = ONLINE ? -__builtin_huge_valf() : 0.f;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
  }
  st.nvis = 0;
  u32x4 kb[kDepth], vb[kDepth];
  auto slot_of = [&](int step) { return s0 + 16 * step + 4 * wave + kg; };
  auto issue = [&](int step, int d) {
    int slot = slot_of(step);
    if (slot >= a.n_slots) slot = 0;  // stays in bounds; masked below
    const long long off = (head_base + slot) * kD + 8 * j16;
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
          const float sc = row16_sum(dot);
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

template <int G>
__global__ __launch_bounds__(256) void decode_splitk(DecodeArgs a, RopeTable rt) {
  __shared__ float kn[kD];
  __shared__ float vn[kD];
  __shared__ float part_m[4][4][G];            // [wave][key group][head]
  __shared__ float part_l[4][4][G];
  __shared__ float part_acc[4][4][G][kD];      // unnormalised, relative to part_m
  __shared__ int bad_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  int p = a.positions[b];
  p = max(0, min(p, a.max_pos));
  const int s0 = c * a.split;
  const int s_end = min(s0 + a.split, a.n_slots);
  const int nsteps = (s_end - s0 + 15) / 16;
  const int s_new = a.is_ring ? (p % a.cap) : p;
  const int p_mod = a.is_ring ? (p % a.cap) : p;
  const bool owner = s_new >= s0 && s_new < s_end;
  const long long head_base = ((long long)b * a.Hkv + g) * (long long)a.cap;
  float* part = a.ws + (((long long)b * a.Hq + g * G) * a.n_chunks + c) * (kD + 2);
  const long long head_stride = (long long)a.n_chunks * (kD + 2);

  // Whole split invisible (linear cache past p, or before the window)?
  bool empty = false;
  if (!a.is_ring) {
    if (s0 > p) empty = true;
    if (a.local && s_end - 1 < p - a.window + 1) empty = true;
  }
  if (empty) {
    if (a.n_chunks == 1) {  // (unreachable: the token's own slot is visible)
      for (int x = tid; x < G * kD; x += 256) a.o[((long long)b * a.Hq + g * G) * kD + x] = 0;
      return;
    }
    for (int x = tid; x < G * (kD + 2); x += 256) {
      const int hg = x / (kD + 2), e = x - hg * (kD + 2);
      part[hg * head_stride + e] = (e == kD) ? -__builtin_huge_valf() : 0.f;
    }
    return;
  }

  // q_hat for the G heads, scaled by softmax_scale * log2(e) (scores in log2
  // units), and k_hat / v of the new token in the workgroup that owns its slot
  const int j16 = lane & 15;
  float qv[G][8];
  {
    __shared__ float qh[G][kD];
    for (int hg = wave; hg < G; hg += 4) {
      float y0, y1;
      norm_rope_vec(a.q + ((long long)b * a.Hq + g * G + hg) * kD, a.q_gamma, a.eps, p, rt.rev[lane], lane, y0, y1);
      qh[hg][lane] = round_bf16(y0 * a.sl2);
      qh[hg][lane + 64] = round_bf16(y1 * a.sl2);
    }
    if (owner && wave == 3) {
      float y0, y1;
      const long long src = ((long long)b * a.Hkv + g) * kD;
      norm_rope_vec(a.k_new + src, a.k_gamma, a.eps, p, rt.rev[lane], lane, y0, y1);
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
    if (tid == 0) bad_flag = 0;
    __syncthreads();
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hg][e] = qh[hg][8 * j16 + e];
  }

  StreamState<G> st;
  stream_split<G, false>(a, qv, kn, vn, head_base, s0, nsteps, p, p_mod, s_new, wave, lane, st);
  // The fast pass needs no running maximum because QK-RMSNorm bounds the
  // logits; if a sum leaves [2^-64, 2^64] (extreme gammas, no norm, foreign
  // cache contents) the split is streamed again with the running maximum.
  bool bad = false;
#pragma unroll
  for (int h = 0; h < G; ++h) bad = bad || !(st.l[h] <= 0x1p64f) || (st.nvis > 0 && !(st.l[h] >= 0x1p-64f));
  if (bad) bad_flag = 1;
  __syncthreads();
  if (bad_flag) stream_split<G, true>(a, qv, kn, vn, head_base, s0, nsteps, p, p_mod, s_new, wave, lane, st);

  // ---- merge the 16 partial states (4 waves x 4 key groups) of each head
  if (j16 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      part_m[wave][lane >> 4][h] = st.m[h];
      part_l[wave][lane >> 4][h] = st.l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) part_acc[wave][lane >> 4][h][8 * j16 + e] = st.acc[h][e];
  __syncthreads();
  const float NEG_INF = -__builtin_huge_valf();
  for (int x = tid; x < G * kD; x += 256) {
    const int h = x / kD, d = x - h * kD;
    float M = NEG_INF;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, part_m[i >> 2][i & 3][h]);
    float num = 0.f, den = 0.f;
    if (M != NEG_INF) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float mi = part_m[i >> 2][i & 3][h];
        const float wgt = (mi == NEG_INF) ? 0.f : fast_exp2(mi - M);
        num += wgt * part_acc[i >> 2][i & 3][h][d];
        den += wgt * part_l[i >> 2][i & 3][h];
      }
    }
    if (a.n_chunks == 1) {
      // a single split is the whole answer (the merge below would weigh it by
      // exp2(0) = 1): normalise and store o here, no merge pass
      const float o = den > 0.f ? num / den : 0.f;
      a.o[((long long)b * a.Hq + g * G + h) * kD + d] = (uint16_t)(pack2(o, 0.f) & 0xffffu);
      continue;
    }
    part[h * head_stride + d] = num;
    if (d == 0) {
      part[h * head_stride + kD] = (den > 0.f) ? M : NEG_INF;
      part[h * head_stride + kD + 1] = den;
    }
  }
}

// Merge the split-K partials of one head: o = sum_c w_c o_c / sum_c w_c l_c
// with w_c = exp2(m_c - M) (maxima are in log2 units).  kCombineGroups
// groups of 128 threads (one per dim) take the splits c = j, j + groups, ...
// with a running maximum, then thread group 0 merges the groups' (M, num,
// den) in group order: a fixed order, so the result is bitwise
// reproducible, and a long cache's hundreds of splits are read by many
// threads at once instead of one after another.
constexpr int kCombineGroups = 8;
__global__ __launch_bounds__(128 * kCombineGroups) void decode_combine(DecodeArgs a) {
  __shared__ float gm[kCombineGroups], gnum[kCombineGroups][kD], gden[kCombineGroups];
  const int h = blockIdx.x;  // b * Hq + head
  const int d = threadIdx.x & (kD - 1);
  const int grp = threadIdx.x >> 7;
  const float* part = a.ws + (long long)h * a.n_chunks * (kD + 2);
  const float NEG_INF = -__builtin_huge_valf();
  float M = NEG_INF, num = 0.f, den = 0.f;
  for (int c = grp; c < a.n_chunks; c += kCombineGroups) {
    const float* pc = part + (long long)c * (kD + 2);
    const float mc = pc[kD];
    if (mc == NEG_INF) continue;
    if (mc > M) {
      const float r = (M == NEG_INF) ? 0.f : fast_exp2(M - mc);
      num *= r;
      den *= r;
      M = mc;
    }
    const float w = fast_exp2(mc - M);
    num += w * pc[d];
    den += w * pc[kD + 1];
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
  a.o[(long long)h * kD + d] = (uint16_t)(pack2(o, 0.f) & 0xffffu);
}

hipError_t launch_decode(const DecodeArgs& a, const RopeTable& rt, int G, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
  const dim3 grid(a.n_chunks, a.B * a.Hkv);
  if (ev_start) hipEventRecord(ev_start, st);
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_splitk<1>, grid, dim3(256), 0, st, a, rt); break;
    case 2: hipLaunchKernelGGL(decode_splitk<2>, grid, dim3(256), 0, st, a, rt); break;
    case 4: hipLaunchKernelGGL(decode_splitk<4>, grid, dim3(256), 0, st, a, rt); break;
    case 8: hipLaunchKernelGGL(decode_splitk<8>, grid, dim3(256), 0, st, a, rt); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) hipEventRecord(ev_stop, st);
  if (e != hipSuccess || a.n_chunks == 1) return e;
  hipLaunchKernelGGL(decode_combine, dim3(a.B * a.Hq), dim3(128 * kCombineGroups), 0, st, a);
  return hipGetLastError();
}

}  // namespace g3
