// Flash-style prefill attention for the Gemma 3 local/global layers (gfx950).
//
// What it computes, per query position i and query head h (kv head h / G):
//   o_i = sum_j softmax_j(scale * <q_hat_i, k_hat_j>) v_j   over visible j,
// visible = causal j <= i, or i and j in one image span (bidirectional), and
// for local layers also |i - j| < window.  Sources: Gemma 3 Technical Report,
// section 1 (1024-token local span, global layers see the long context) and
// section 2 (GQA, QK-norm instead of soft-capping: logits are not capped);
// "Gemma explained: What's new in Gemma 3", vision section (bidirectional
// attention over image tokens).  For every row the visible keys form one
// contiguous range [lo(i), hi(i)], so tiles outside the union of the rows'
// ranges are never loaded ("window-aware tile skipping").
//
// Design (per workgroup = 4 waves, one (sequence, kv head, query tile)):
//   * GQA packing: each wave owns 64 query rows = (64/G positions) x (G heads
//     of one kv group), so one K/V tile in LDS feeds 64 rows per wave.
//   * Q is loaded once, QK-RMSNorm + RoPE are applied in registers (fp64
//     angle reduction), and Q stays in VGPRs as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  Computing
//     S transposed puts one query per lane, so row max / row sum are
//     in-lane plus one cross-half swap (v_permlane32_swap).
//   * P^T goes straight from the S^T accumulators to the B operand of
//     O^T = V^T P^T; V^T comes from a row-major V tile in LDS through the
//     transposing LDS read ds_read_b64_tr_b16, with the key order inside each
//     16-key step matched to the accumulator layout.
//   * K/V tiles of 64 keys are double-buffered in LDS; the next tile's
//     global loads are in flight while the current one is computed.
//   * Workgroups are mapped to XCDs so a kv head's query tiles share one L2,
//     heaviest (most keys) tiles first.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

constexpr int kBN = 64;           // keys per tile
constexpr int kLdsStride = 136;   // bf16 elements per LDS row (256 B + 16 B pad)
constexpr int kTileElems = kBN * kLdsStride;

__device__ __forceinline__ float wave_min_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Value of lane l ^ 32 combined with this lane's: max / sum.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int floor_div64(int x) { return x >= 0 ? x / 64 : -((63 - x) / 64); }

// Visible key range of query position i (inclusive), or lo > hi if none.
struct RowRange {
  int lo, hi;
};
__device__ __forceinline__ RowRange row_range(int i, int b, int kmin_avail, const PrefillArgs& a,
                                              const SpanTable& spt) {
  int hi = i;
  for (int s = 0; s < spt.n; ++s) {
    const Span sp = spt.s[s];
    if (sp.batch == b && sp.start <= i && i < sp.end) hi = max(hi, sp.end - 1);
  }
  int lo = kmin_avail;
  if (a.local) {
    lo = max(lo, i - a.window + 1);
    hi = min(hi, i + a.window - 1);
  }
  return RowRange{lo, hi};
}

}  // namespace

template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_fwd(PrefillArgs a, Pos0Table p0t, SpanTable spt) {
  constexpr int P = 64 / G;   // positions per wave
  constexpr int WP = 4 * P;   // positions per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kTileElems];
  __shared__ double theta_rev[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h2 = lane >> 5;
  const int ln = lane & 31;

  const int li = xcd_remap(blockIdx.x, gridDim.x);
  const int bg = li / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (li - bg * a.n_qtiles);  // heaviest tiles first
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int p0 = pos0_of(p0t, b);
  const int chunk_end = p0 + a.S;
  const int kmin_avail = a.has_cache ? (a.is_ring ? max(0, p0 - a.cap) : 0) : p0;
  const int qbase = p0 + qt * WP;  // first query position of the workgroup

  if (tid < 64) theta_rev[tid] = rope_rev_freq(tid, a.base, a.inv_scale);

  // ---- key ranges: whole workgroup (tiles to stream) and this wave
  int wg_lo = 0x7fffffff, wg_hi = -0x7fffffff;
#pragma unroll
  for (int k = 0; k < (WP + 63) / 64; ++k) {
    const int idx = lane + 64 * k;
    const int i = qbase + idx;
    if (idx < WP && i < chunk_end) {
      const RowRange r = row_range(i, b, kmin_avail, a, spt);
      wg_lo = min(wg_lo, r.lo);
      wg_hi = max(wg_hi, r.hi);
    }
  }
  wg_lo = wave_min_i(wg_lo);
  wg_hi = wave_max_i(wg_hi);

  int row_lo[2], row_hi[2], row_pos[2], row_head[2];
  bool row_ok[2];
  int w_lo_min = 0x7fffffff, w_hi_max = -0x7fffffff, w_lo_max = -0x7fffffff, w_hi_min = 0x7fffffff;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = ln + 32 * qb;
    const int hg = r / P;
    const int poff = r - hg * P;
    const int i = qbase + wave * P + poff;
    row_pos[qb] = i;
    row_head[qb] = g * G + hg;
    row_ok[qb] = i < chunk_end;
    if (row_ok[qb]) {
      const RowRange rr = row_range(i, b, kmin_avail, a, spt);
      row_lo[qb] = rr.lo;
      row_hi[qb] = rr.hi;
      w_lo_min = min(w_lo_min, rr.lo);
      w_hi_max = max(w_hi_max, rr.hi);
      w_lo_max = max(w_lo_max, rr.lo);
      w_hi_min = min(w_hi_min, rr.hi);
    } else {
      row_lo[qb] = 0x7fffffff;
      row_hi[qb] = -0x7fffffff;
    }
  }
  w_lo_min = wave_min_i(w_lo_min);
  w_hi_max = wave_max_i(w_hi_max);
  w_lo_max = wave_max_i(w_lo_max);
  w_hi_min = wave_min_i(w_hi_min);

  const int t_begin = floor_div64(wg_lo - p0);
  const int t_end = floor_div64(wg_hi - p0);  // inclusive

  // ---- tile loader: thread -> 4 rows (16 threads per 256-byte row)
  const int ld_col = (tid & 15) * 8;
  const int ld_row = tid >> 4;
  const long long kv_head_base_chunk = ((long long)b * a.Hkv + g) * a.S;  // khat rows
  const long long cache_head_base = ((long long)b * a.Hkv + g) * (long long)a.cap;
  u32x4 pk[4], pv[4];
  auto load_tile = [&](int t) {
    const int ts = p0 + t * kBN;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = ts + ld_row + 16 * u;
      u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (j >= p0 && j < chunk_end) {
        const int r = j - p0;
        kk = *(const u32x4*)(a.khat + (kv_head_base_chunk + r) * kD + ld_col);
        vv = *(const u32x4*)(a.v + (((long long)b * a.S + r) * a.Hkv + g) * kD + ld_col);
      } else if (a.has_cache && j < p0 && j >= kmin_avail) {
        const long long slot = a.is_ring ? (j % a.cap) : j;
        kk = *(const u32x4*)(a.ck + (cache_head_base + slot) * kD + ld_col);
        vv = *(const u32x4*)(a.cv + (cache_head_base + slot) * kD + ld_col);
      }
      pk[u] = kk;
      pv[u] = vv;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = ld_row + 16 * u;
      *(u32x4*)(&lds_k[buf][row * kLdsStride + ld_col]) = pk[u];
      *(u32x4*)(&lds_v[buf][row * kLdsStride + ld_col]) = pv[u];
    }
  };

  load_tile(t_begin);
  store_tile(0);
  __syncthreads();  // also publishes theta_rev

  // ---- Q prologue: load, QK-RMSNorm, RoPE, round to bf16 (B operand of S^T)
  bf16x8 qreg[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float x[64];
    if (row_ok[qb]) {
      const uint16_t* src = a.q + (((long long)b * a.S + (row_pos[qb] - p0)) * a.Hq + row_head[qb]) * kD + 8 * h2;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 w = *(const u32x4*)(src + 16 * s);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * s + 2 * e] = bf_lo(w[e]);
          x[8 * s + 2 * e + 1] = bf_hi(w[e]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 64; ++e) x[e] = 0.f;
    }
    if (a.q_gamma) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e) ss += x[e] * x[e];
      ss = xhalf_sum(ss);
      const float rn = rsqrtf(ss * (1.f / kD) + a.eps);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * s + e] *= rn * a.q_gamma[16 * s + 8 * h2 + e];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos(row_pos[qb], theta_rev[16 * s + 8 * h2 + e], sn, cs);
        const float x1 = x[8 * s + e], x2 = x[8 * (s + 4) + e];
        x[8 * s + e] = x1 * cs - x2 * sn;
        x[8 * (s + 4) + e] = x1 * sn + x2 * cs;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = {pack2(x[8 * s], x[8 * s + 1]), pack2(x[8 * s + 2], x[8 * s + 3]),
                 pack2(x[8 * s + 4], x[8 * s + 5]), pack2(x[8 * s + 6], x[8 * s + 7])};
      qreg[qb][s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- main loop over key tiles
  const float sl2 = a.sl2;
  const float NEG_INF = -__builtin_huge_valf();
  float m_run[2] = {NEG_INF, NEG_INF};
  float l_run[2] = {0.f, 0.f};
  f32x16 oacc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][qb][r] = 0.f;

  // transposing-read lane constants (ds_read_b64_tr_b16 groups of 16 lanes)
  const int tr_g = lane >> 4;
  const int tr_w = lane & 15;
  const int tr_key = 4 * (tr_g >> 1) + (tr_w >> 2);       // + 16 t + 8 r
  const int tr_dim = 16 * (tr_g & 1) + 4 * (tr_w & 3);   // + 32 mb

  const int n_t = t_end - t_begin + 1;
  for (int it = 0; it < n_t; ++it) {
    const int t = t_begin + it;
    const int cur = it & 1;
    if (it + 1 < n_t) load_tile(t + 1);
    const int ts = p0 + t * kBN;
    if (ts <= w_hi_max && ts + kBN - 1 >= w_lo_min) {
      const uint16_t* kb_lds = lds_k[cur];
      const uint16_t* vb_lds = lds_v[cur];
      // S^T = K Q^T : [2 key blocks of 32] x [2 query blocks of 32]
      f32x16 sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kop = *(const bf16x8*)(kb_lds + (kb * 32 + ln) * kLdsStride + 16 * s + 8 * h2);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[qb][s], sacc[kb][qb], 0, 0, 0);
        }
      }
      // mask edge tiles: key of (kb, r) = ts + 32 kb + 8 (r/4) + 4 h2 + r%4
      if (!(ts >= w_lo_max && ts + kBN - 1 <= w_hi_min)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = ts + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              if (j < row_lo[qb] || j > row_hi[qb]) sacc[kb][qb][r] = NEG_INF;
          }
      }
      // online softmax, one query per lane (plus its partner lane ^ 32)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = NEG_INF;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        mx = xhalf_max(mx);
        const float m_new = fmaxf(m_run[qb], mx);
        const float mu = (m_new == NEG_INF) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run[qb] - mu) * sl2);
        m_run[qb] = m_new;
        const float msl = mu * sl2;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(__builtin_fmaf(sacc[kb][qb][r], sl2, -msl));
            sacc[kb][qb][r] = p;
            rs += p;
          }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][qb][r] *= alpha;
      }
      // O^T += V^T P^T, 4 steps of 16 keys
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        bf16x8 pb[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const f32x16& sa = sacc[t4 >> 1][qb];
          const int r0 = 8 * (t4 & 1);
          u32x4 w = {pack2(sa[r0], sa[r0 + 1]), pack2(sa[r0 + 2], sa[r0 + 3]), pack2(sa[r0 + 4], sa[r0 + 5]),
                     pack2(sa[r0 + 6], sa[r0 + 7])};
          pb[qb] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint16_t* base = vb_lds + (16 * t4 + tr_key) * kLdsStride + 32 * mb + tr_dim;
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base));
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * kLdsStride));
          const bf16x8 vop = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[mb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[qb], oacc[mb][qb], 0, 0, 0);
        }
      }
    }
    if (it + 1 < n_t) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, bf16, store rows [b][pos][head][dims]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = xhalf_sum(l_run[qb]);
    if (!row_ok[qb]) continue;
    const float inv = 1.f / lt;
    uint16_t* dst = a.o + (((long long)b * a.S + (row_pos[qb] - p0)) * a.Hq + row_head[qb]) * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mb + 8 * q4 + 4 * h2;
        const f32x16& oa = oacc[mb][qb];
        *(u32x2*)(dst + d) = u32x2{pack2(oa[4 * q4] * inv, oa[4 * q4 + 1] * inv),
                                   pack2(oa[4 * q4 + 2] * inv, oa[4 * q4 + 3] * inv)};
      }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt, int G,
                          hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int grid = a.B * a.Hkv * a.n_qtiles;
  if (ev_start) hipEventRecord(ev_start, st);
  switch (G) {
    case 1: hipLaunchKernelGGL(prefill_fwd<1>, dim3(grid), dim3(256), 0, st, a, p0t, spt); break;
    case 2: hipLaunchKernelGGL(prefill_fwd<2>, dim3(grid), dim3(256), 0, st, a, p0t, spt); break;
    case 4: hipLaunchKernelGGL(prefill_fwd<4>, dim3(grid), dim3(256), 0, st, a, p0t, spt); break;
    case 8: hipLaunchKernelGGL(prefill_fwd<8>, dim3(grid), dim3(256), 0, st, a, p0t, spt); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) hipEventRecord(ev_stop, st);
  return e;
}

}  // namespace g3
