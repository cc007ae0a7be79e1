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
// flight (the first eight go out before q is normalised, so their latency
// overlaps it).  D/8 lanes share a key row (8 dims each: 16 lanes at D = 128,
// 32 at D = 256; DPP row reductions, plus v_permlane16_swap across the two
// rows at D = 256) and all G heads of the group use every row.  Scores and
// P V run on packed bf16 with v_dot2_f32_bf16 (fp32 accumulation).  The
// partial (o, m, l) of the split goes to the workspace; a second kernel
// merges the partials of a head in a fixed order, so results are bitwise
// reproducible.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

#include <mutex>

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

// RMSNorm + RoPE of one raw D-vector by one wave, from inputs already in
// registers: lane owns the rotation pairs (k, k + D/2) for k = lane + 64 i,
// i < D/128; xr[2 i] / xr[2 i + 1] are elements k and k + D/2 (bf16 bits),
// gr the matching gamma entries, rev[i] the rotation rate of pair k.
template <int D>
__device__ __forceinline__ void norm_rope_regs(const uint32_t (&xr)[D / 64], bool norm, const float (&gr)[D / 64],
                                               float eps, int pos, const double (&rev)[D / 128], float (&y0)[D / 128],
                                               float (&y1)[D / 128]) {
  constexpr int NP = D / 128;
  float x0[NP], x1[NP];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    x0[i] = __uint_as_float(xr[2 * i] << 16);
    x1[i] = __uint_as_float(xr[2 * i + 1] << 16);
    ss += x0[i] * x0[i] + x1[i] * x1[i];
  }
  if (norm) {
    ss = wave_sum(ss);
    const float rn = rsqrtf(ss * (1.f / D) + eps);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      x0[i] *= rn * gr[2 * i];
      x1[i] *= rn * gr[2 * i + 1];
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float sn, cs;
    rope_sincos(pos, rev[i], sn, cs);
    y0[i] = x0[i] * cs - x1[i] * sn;
    y1[i] = x0[i] * sn + x1[i] * cs;
  }
}

template <int D>
__device__ __forceinline__ void load_pairs(const uint16_t* src, int lane, uint32_t (&xr)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 128; ++i) {
    xr[2 * i] = src[lane + 64 * i];
    xr[2 * i + 1] = src[lane + 64 * i + D / 2];
  }
}
template <int D>
__device__ __forceinline__ void load_pairs(const float* src, int lane, float (&xr)[D / 64]) {
#pragma unroll
  for (int i = 0; i < D / 128; ++i) {
    xr[2 * i] = src[lane + 64 * i];
    xr[2 * i + 1] = src[lane + 64 * i + D / 2];
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
  if (D == 256) {
    // rows 2i and 2i+1 trade values (v_permlane16_swap): the sum of the two
    // results is the 32-lane sum in both rows, without an LDS round trip
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Per-lane running state of one kv group's G heads over the keys this lane's
// row group sees (dims 8 jl .. 8 jl + 7 of the accumulator).
template <int G>
struct StreamState {
  float m[G], l[G], acc[G][8];
  int nvis;  // visible keys seen by this lane
};

// The careful pass over a split, for the rare split whose fast-pass sums left
// range: fp32 q and K, and a running maximum.  Step st covers 4 RW
// consecutive slots (RW = 64 / (D/8) per wave, one per row group); each
// step's K and V rows are loaded kDepth steps ahead.
template <int G, int D>
__device__ __forceinline__ void stream_split_online(const DecodeArgs& a, const float (&qv)[G][8], const float* kn,
                                             const float* vn, long long head_base, int s0, int nsteps, int p,
                                             int p_mod, int s_new, int wave, int lane, StreamState<G>& st) {
  constexpr int kDepth = 8;
  constexpr int LPR = D / 8, RW = 64 / LPR;
  const int j16 = lane % LPR;
  const int kg = lane / LPR;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -__builtin_huge_valf();
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
        if (!vis) {  // a never-written slot may hold NaN: keep 0 * NaN out of the sums
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = 0.f;
        }
        if (step + kDepth < nsteps) issue(step + kDepth, d);
        st.nvis += vis ? 1 : 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot += qv[h][e] * kf[e];
          const float sc = row_sum<D>(dot);
          const float m_new = vis ? fmaxf(st.m[h], sc) : st.m[h];
          const float alpha = (m_new == st.m[h]) ? 1.f : fast_exp2(st.m[h] - m_new);
          const float pr = vis ? fast_exp2(sc - m_new) : 0.f;
          st.m[h] = m_new;
          st.l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
          st.l[h] += pr;
#pragma unroll
          for (int e = 0; e < 8; ++e) st.acc[h][e] += pr * vf[e];
        }
      }
    }
  }
}

// The fast pass over a split (no running maximum) on packed bf16: each
// lane takes its rows two steps at a time, the scores come from
// v_dot2_f32_bf16 on the cache's bf16 K and the bf16-rounded q (fp32
// accumulation; 4 instructions per head and row for 8 dims, against 8
// conversions and 8 FMAs), and P V accumulates both rows at once: the two
// rows' values of a dim paired in one word (v_perm_b32) against the pair
// (p0, p1) rounded to bf16 (as P is in the prefill), one v_dot2 per dim and
// head for two rows.  The row sums l stay fp32.
constexpr int kDecodeDepth = 8;  // steps of K/V loads each wave keeps in flight

// K and V words of this lane at step `step` of the split starting at s0.
template <int D>
__device__ __forceinline__ void split_load(const DecodeArgs& a, long long head_base, int s0, int step, int wave,
                                           int lane, u32x4& k, u32x4& v) {
  constexpr int LPR = D / 8, RW = 64 / LPR;
  int slot = s0 + 4 * RW * step + RW * wave + lane / LPR;
  if (slot >= a.n_slots) slot = 0;  // stays in bounds; masked by the caller
  const long long off = (head_base + slot) * D + 8 * (lane % LPR);
  k = __builtin_nontemporal_load((const u32x4*)(a.ck + off));
  v = __builtin_nontemporal_load((const u32x4*)(a.cv + off));
}

// `prologue` (which fills qpk and the new token's LDS rows) runs once the
// first kDecodeDepth steps' loads are issued, so their latency overlaps it.
// The split is slots [s0, s_end); its step count is rounded up to a whole
// number of kDecodeDepth groups, rows past s_end masked like invisible ones.
template <int G, int D, class Prologue>
__device__ __forceinline__ void stream_split_fast(const DecodeArgs& a, const uint32_t (&qpk)[G][4],
                                                  const uint16_t* kn16, const uint16_t* vn16, long long head_base,
                                                  int s0, int s_end, int p, int p_mod, int s_new, int wave, int lane,
                                                  Prologue&& prologue, StreamState<G>& st) {
  constexpr int kDepth = kDecodeDepth;
  constexpr int LPR = D / 8, RW = 64 / LPR;
  const int nsteps = ((s_end - s0 + 4 * RW * kDepth - 1) / (4 * RW * kDepth)) * kDepth;
  const int j16 = lane % LPR;
  const int kg = lane / LPR;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = 0.f;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
  }
  st.nvis = 0;
  u32x4 kb[kDepth], vb[kDepth];
  auto slot_of = [&](int step) { return s0 + 4 * RW * step + RW * wave + kg; };
  auto issue = [&](int step, int d) { split_load<D>(a, head_base, s0, step, wave, lane, kb[d], vb[d]); };
  auto visible = [&](int slot) {
    bool vis = slot < s_end;
    if (a.is_ring) {
      int dist = p_mod - slot;
      if (dist < 0) dist += a.cap;
      vis = vis && (p - dist >= 0) && (!a.local || dist < a.window);
    } else {
      vis = vis && slot <= p && (!a.local || p - slot < a.window);
    }
    return vis;
  };
  // Every step issues its loads unconditionally (the last kDepth steps
  // repeat the split's last step: cache hits, never used).  Loads skipped on
  // some paths would leave the compiler unsure how many are younger than the
  // one a step needs, and it would wait for all of them (vmcnt(0)) each step.
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    issue(min(d, nsteps - 1), d);
  prologue();
  const u32x4 kn_w = *(const u32x4*)(kn16 + 8 * j16);
  const u32x4 vn_w = *(const u32x4*)(vn16 + 8 * j16);
  // Steps step0, step0 + 1 from buffers d, d + 1.
  auto pair = [&](int step0, int d) {
    const int step1 = step0 + 1;
    const int slot0 = slot_of(step0), slot1 = slot_of(step1);
    const bool vis0 = visible(slot0), vis1 = visible(slot1);
    const u32x4 k0 = slot0 == s_new ? kn_w : kb[d], k1 = slot1 == s_new ? kn_w : kb[d + 1];
    u32x4 v0 = slot0 == s_new ? vn_w : vb[d], v1 = slot1 == s_new ? vn_w : vb[d + 1];
    // a row the token cannot see gets p = 0, and its V words are zeroed
    // too: a slot never written (a fresh cache past p) may hold NaN, and
    // 0 * NaN would reach the sums
    if (!vis0) v0 = u32x4{0, 0, 0, 0};
    if (!vis1) v1 = u32x4{0, 0, 0, 0};
    st.nvis += (vis0 ? 1 : 0) + (vis1 ? 1 : 0);
    // dim e of the two rows in one word: row 0 low, row 1 high
    uint32_t vp[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      vp[2 * w] = __builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u);
      vp[2 * w + 1] = __builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // through plain words: a bit cast of a vector element reads element 0
        const uint32_t k0w = k0[w], k1w = k1[w];
        const bf16x2 qw = __builtin_bit_cast(bf16x2, qpk[h][w]);
        d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k0w), qw, d0, false);
        d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k1w), qw, d1, false);
      }
      const float sc0 = row_sum<D>(d0), sc1 = row_sum<D>(d1);
      const float p0 = vis0 ? fast_exp2(sc0) : 0.f;
      const float p1 = vis1 ? fast_exp2(sc1) : 0.f;
      st.l[h] += p0 + p1;
      const bf16x2 pp = __builtin_bit_cast(bf16x2, pack2(p0, p1));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        st.acc[h][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vp[e]), pp, st.acc[h][e], false);
    }
  };
  // nsteps is a multiple of kDepth, so the guard below always holds; it
  // stays because the compiler keeps far fewer registers live with it.  The
  // loads sit outside it, on every path, so the compiler's wait counts stay
  // exact, and after the pair, once the rows in their buffers are used up,
  // so they land in the same registers (a load into a spare register would
  // need a copy, and the copy a wait for that load).
  for (int st0 = 0; st0 < nsteps; st0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; d += 2) {
      if (st0 + d < nsteps) pair(st0 + d, d);
      issue(min(st0 + d + kDepth, nsteps - 1), d);
      issue(min(st0 + d + 1 + kDepth, nsteps - 1), d + 1);
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
  __shared__ __attribute__((aligned(16))) uint16_t kn16[D];  // the new key / value as bf16 (fast pass)
  __shared__ __attribute__((aligned(16))) uint16_t vn16[D];
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
  // units), and k_hat / v of the new token in the workgroup that owns its
  // slot.  Their raw inputs are loaded first; the split's first K/V loads go
  // out next, and the arithmetic runs while those are in flight (loads
  // return in order, so raw inputs loaded after the K/V rows would wait for
  // them).
  constexpr int HPW = (G + 3) / 4;  // q heads per wave
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // branches on it stay scalar
  const int j16 = lane % LPR;
  const bool kv_wave = owner && wave_u == 3;
  const long long kv_src = ((long long)b * a.Hkv + g) * D;
  uint32_t qr[HPW][2 * NP], kr[2 * NP], vr[2 * NP];  // bf16 bits, one per word (no packing waits)
  float gq[2 * NP], gk[2 * NP];
  double rev[NP];
  // (every wave loads: one without a head of its own reads the last head's
  // row, unused, so no branch around the loads costs a wait)
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    load_pairs<D>(a.q + ((long long)b * a.Hq + g * G + min(wave_u + 4 * j, G - 1)) * D, lane, qr[j]);
  if (a.q_gamma) load_pairs<D>(a.q_gamma, lane, gq);
#pragma unroll
  for (int i = 0; i < NP; ++i) rev[i] = rt.rev[lane + 64 * i];
  if (kv_wave) {
    load_pairs<D>(a.k_new + kv_src, lane, kr);
    load_pairs<D>(a.v_new + kv_src, lane, vr);
    if (a.k_gamma) load_pairs<D>(a.k_gamma, lane, gk);
  }
  __shared__ float qh[G][D];
  uint32_t qpk[G][4];
  auto prologue = [&]() {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hg = wave_u + 4 * j;
      if (hg < G) {
        float y0[NP], y1[NP];
        norm_rope_regs<D>(qr[j], a.q_gamma != nullptr, gq, a.eps, p, rev, y0, y1);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          qh[hg][lane + 64 * i] = round_bf16(y0[i] * a.sl2);
          qh[hg][lane + 64 * i + D / 2] = round_bf16(y1[i] * a.sl2);
        }
      }
    }
    if (kv_wave) {
      float y0[NP], y1[NP];
      norm_rope_regs<D>(kr, a.k_gamma != nullptr, gk, a.eps, p, rev, y0, y1);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d0 = lane + 64 * i, d1 = d0 + D / 2;
        const uint32_t w = pack2(y0[i], y1[i]);
        kn[d0] = bf_lo(w);
        kn[d1] = bf_hi(w);
        kn16[d0] = (uint16_t)(w & 0xffffu);
        kn16[d1] = (uint16_t)(w >> 16);
        const uint16_t v0 = (uint16_t)vr[2 * i], v1 = (uint16_t)vr[2 * i + 1];
        vn[d0] = __uint_as_float((uint32_t)v0 << 16);
        vn[d1] = __uint_as_float((uint32_t)v1 << 16);
        vn16[d0] = v0;
        vn16[d1] = v1;
        a.ck[(head_base + s_new) * D + d0] = (uint16_t)(w & 0xffffu);
        a.ck[(head_base + s_new) * D + d1] = (uint16_t)(w >> 16);
        a.cv[(head_base + s_new) * D + d0] = v0;
        a.cv[(head_base + s_new) * D + d1] = v1;
      }
    }
    if (tid == 0) bad_flag = 0;
    __syncthreads();
    // q as bf16 pairs for the fast pass (its values are bf16 already:
    // exact); the online pass reads its fp32 copy from LDS only when it runs
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int w = 0; w < 4; ++w) qpk[hg][w] = pack2(qh[hg][8 * j16 + 2 * w], qh[hg][8 * j16 + 2 * w + 1]);
  };

  StreamState<G> st;
  stream_split_fast<G, D>(a, qpk, kn16, vn16, head_base, s0, s_end, p, p_mod, s_new, wave, lane, prologue, st);
  // The fast pass needs no running maximum because QK-RMSNorm bounds the
  // logits; if a sum leaves [2^-64, 2^64] (extreme gammas, no norm, foreign
  // cache contents) the split is streamed again with the running maximum.
  bool bad = false;
#pragma unroll
  for (int h = 0; h < G; ++h) bad = bad || !(st.l[h] <= 0x1p64f) || (st.nvis > 0 && !(st.l[h] >= 0x1p-64f));
  if (bad) bad_flag = 1;
  __syncthreads();
  if (bad_flag) {
    float qv[G][8];
#pragma unroll
    for (int hg = 0; hg < G; ++hg)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hg][e] = qh[hg][8 * j16 + e];
    stream_split_online<G, D>(a, qv, kn, vn, head_base, s0, nsteps, p, p_mod, s_new, wave, lane, st);
  }

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
  // The thread's splits are read kCombineBatch at a time, all loads issued
  // before the first is used (one memory round trip per batch instead of
  // one per split: a 32K cache's 64 splits at D = 256 are 16 per thread),
  // then folded in the same order as one at a time.  Eight keep the kernel
  // within 64 VGPRs, two 1024-thread workgroups per CU.
  constexpr int kCombineBatch = 8;
  for (int c0 = grp; c0 < a.n_chunks; c0 += kCombineGroups * kCombineBatch) {
    float mv[kCombineBatch], xv[kCombineBatch], lv[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int c = c0 + i * kCombineGroups;
      mv[i] = NEG_INF;
      xv[i] = lv[i] = 0.f;
      if (c < a.n_chunks) {
        const float* pc = part + (long long)c * (D + 2);
        mv[i] = pc[D];
        xv[i] = pc[d];
        lv[i] = pc[D + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const float mc = mv[i];
      if (mc == NEG_INF) continue;
      if (mc > M) {
        const float r = (M == NEG_INF) ? 0.f : fast_exp2(M - mc);
        num *= r;
        den *= r;
        M = mc;
      }
      const float w = fast_exp2(mc - M);
      num += w * xv[i];
      den += w * lv[i];
    }
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

// Split-K partials of the decode entry point that allocates nothing: one
// fixed array per GPU the library runs on, held until the process ends and
// shared by every such call on that GPU.  On the host the name `scratch`
// is only a stand-in for the device array (passing it to a kernel would
// fault); decode_scratch() looks up each device's own address of it once,
// with that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] { err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
  if (err[dev] != hipSuccess) return err[dev];
  *ptr = addr[dev];
  return hipSuccess;
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
