// Flash-style prefill for head dimension 256 (Gemma 3 1B: 4 query heads, 1
// kv head; "Gemma explained: What's new in Gemma 3", 1B module print) on
// gfx950.  Same computation as the D = 128 kernel: per query position i and
// query head h (kv head h / G),
//   o_i = sum_j softmax_j(scale * <q_hat_i, k_hat_j>) v_j   over visible j,
// visible = causal j <= i or the same image span, and |i - j| < window on
// local layers (Gemma 3 Technical Report, sections 1-2).
//
// Design (workgroup = 4 waves, one per SIMD, one (sequence, kv head, query
// tile)):
//   * each wave owns 32 query rows = (32/G positions) x (G heads of one kv
//     group); Q^ (QK-RMSNorm, RoPE, scale in log2 units) stays in registers
//     as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, 16 dim
//     steps); P^T goes from the S^T accumulators into the B operand of
//     O^T = V^T P^T (8 blocks of 32 dims), V^T through transposing LDS reads;
//   * K/V tiles of 32 keys x 512 B, double-buffered in LDS and filled by
//     global->LDS loads, chunk c of row r at chunk position c ^ swz(r mod 16)
//     (bank groups repeat every 256 B, so the D = 128 kernel's conflict-free
//     read patterns carry over);
//   * one wave per SIMD with the whole register file: O (128 registers), Q
//     (64) and a whole tile's operands in flight;
//   * softmax without a running maximum (QK-RMSNorm bounds the logits), with
//     the same flagged second pass (ONLINE = true) as the D = 128 kernel.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

constexpr int kDh = 256;             // head dimension
constexpr int kBNh = 32;             // keys per tile
constexpr int kTileH = kBNh * kDh;   // bf16 elements per tile (16 KiB)
constexpr int kNW = kPrefillWavesD256;

__device__ __forceinline__ int swz16(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ float xhalf_sum256(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_max256(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Barrier that waits only for this wave's LDS operations (not for global
// loads still in flight).
__device__ __forceinline__ void barrier_lds256() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_loads256() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte global -> LDS load per lane: lane L writes LDS bytes
// [lds_addr + 16 L, +16) (global_load_lds_dwordx4, address in M0, which is
// saved and restored).
__device__ __forceinline__ void dma16_256(const void* src, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr));
}
__device__ __forceinline__ uint32_t lds_addr256(const uint16_t* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t*)p);
}

// A zero K/V row: the source of tile rows whose key does not exist.
__device__ __attribute__((aligned(256))) uint16_t g_zero_row256[kDh] = {0};

__device__ __forceinline__ int floor_div32(int x) { return x >= 0 ? x / 32 : -((31 - x) / 32); }

struct Range256 {
  int lo, hi;
};
// Visible key range of query position i (inclusive), or lo > hi if none.
__device__ __forceinline__ Range256 row_range256(int i, int b, int kmin_avail, const PrefillArgs& a,
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
  return Range256{lo, hi};
}

}  // namespace

template <int G, bool ONLINE>
__global__ __launch_bounds__(64 * kNW, 1) void prefill_fwd_d256(PrefillArgs a, Pos0Table p0t, SpanTable spt,
                                                                RopeTable rt) {
  constexpr int P = 32 / G;    // positions per wave
  constexpr int WP = kNW * P;  // positions per workgroup
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * kTileH];  // K0 K1 V0 V1
  auto lds_k = [&](int buf) { return lds + buf * kTileH; };
  auto lds_v = [&](int buf) { return lds + (2 + buf) * kTileH; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h2 = lane >> 5;
  const int ln = lane & 31;

  const int li = xcd_remap(blockIdx.x, gridDim.x);
  if (ONLINE && a.flags[li] == 0) return;
  const int bg = li / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (li - bg * a.n_qtiles);  // heaviest tiles first
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int p0 = pos0_of(p0t, b);
  const int chunk_end = p0 + a.S;
  const int kmin_avail = a.has_cache ? (a.is_ring ? max(0, p0 - a.cap) : 0) : p0;
  const int qbase = p0 + qt * WP;
  const int wbase = qbase + wave * P;

  // key tiles of the workgroup (lo(i), hi(i) are non-decreasing in i)
  const int wg_last = min(qbase + WP, chunk_end) - 1;
  const Range256 wf = row_range256(qbase, b, kmin_avail, a, spt);
  const Range256 wl = row_range256(wg_last, b, kmin_avail, a, spt);
  const int t_begin = floor_div32(wf.lo - p0);
  const int n_t = floor_div32(wl.hi - p0) - t_begin + 1;
  int w_lo_min = 0x7fffffff, w_hi_max = -0x7fffffff, w_lo_max = 0x7fffffff, w_hi_min = -0x7fffffff;
  if (wbase < chunk_end) {
    const Range256 f = row_range256(wbase, b, kmin_avail, a, spt);
    const Range256 l = row_range256(min(wbase + P, chunk_end) - 1, b, kmin_avail, a, spt);
    w_lo_min = f.lo;
    w_hi_min = f.hi;
    w_lo_max = l.lo;
    w_hi_max = l.hi;
  }

  // ---- tile loader: wave w fills rows [8w, 8w + 8) of the K and V tiles, 2
  // rows per instruction: lane L lands on row 8w + 2i + L/32, chunk position
  // L % 32, so it fetches logical chunk (L % 32) ^ swz(row mod 16).
  const uint16_t* khat_bg = a.khat + ((long long)b * a.Hkv + g) * a.S * kDh;
  const uint16_t* v_bg = a.v + ((long long)b * a.S * a.Hkv + g) * kDh;
  const int vstride = a.Hkv * kDh;
  const long long cache_bg = ((long long)b * a.Hkv + g) * (long long)a.cap * kDh;
  auto dma_tile = [&](int t, int buf) {
    const int ts = p0 + t * kBNh;
    const int mode = (t >= 0 && ts + kBNh <= chunk_end) ? 0
                     : (a.has_cache && ts >= kmin_avail && ts + kBNh <= p0 && (!a.is_ring || a.cap >= kBNh)) ? 1
                                                                                                      : 2;
    const int slot0 = (mode == 1 && a.is_ring) ? ts % a.cap : ts;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = k & 3;
      const bool is_v = k >= 4;
      const int row = 8 * wave + 2 * i + (lane >> 5);
      const int col = ((lane & 31) ^ swz16(row & 15)) * 8;
      const uint16_t* src;
      if (mode == 0) {
        const int r = t * kBNh + row;
        src = is_v ? v_bg + (long long)r * vstride : khat_bg + (long long)r * kDh;
      } else if (mode == 1) {
        int slot = slot0 + row;
        if (a.is_ring && slot >= a.cap) slot -= a.cap;
        src = (is_v ? a.cv : a.ck) + cache_bg + (long long)slot * kDh;
      } else {
        const int j = ts + row;
        src = g_zero_row256;
        if (j >= p0 && j < chunk_end) {
          src = is_v ? v_bg + (long long)(j - p0) * vstride : khat_bg + (long long)(j - p0) * kDh;
        } else if (a.has_cache && j < p0 && j >= kmin_avail) {
          const long long slot = a.is_ring ? (long long)(j % a.cap) : (long long)j;
          src = (is_v ? a.cv : a.ck) + cache_bg + slot * kDh;
        }
      }
      const uint16_t* dst = (is_v ? lds_v(buf) : lds_k(buf)) + (8 * wave_u + 2 * i) * kDh;
      dma16_256(src + col, lds_addr256(dst));
    }
  };

  // operand read offsets inside a tile (bytes)
  uint32_t adk[16];     // K^T step st: row ln, chunk (2 st + h2)
  uint32_t adv[2][8];   // V^T [row half][dim block]: transposing reads
#pragma unroll
  for (int st = 0; st < 16; ++st) adk[st] = ln * 512 + (((2 * st + h2) ^ swz16(ln & 15)) << 4);
  {
    const int g4 = lane >> 4, w16 = lane & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int row = 8 * hf + 4 * (g4 >> 1) + (w16 >> 2);
        const int c = 4 * mb + 2 * (g4 & 1) + ((w16 & 3) >> 1);
        adv[hf][mb] = row * 512 + ((c ^ swz16(row)) << 4) + 8 * (w16 & 1);
      }
  }

  dma_tile(t_begin, 0);

  // this lane's query row: position offset ln % P, head ln / P of the group
  const int hg = ln / P;
  const int row_pos = wbase + (ln - hg * P);
  const bool row_ok = row_pos < chunk_end;
  int row_lo = 0x7fffffff, row_hi = -0x7fffffff;
  if (row_ok) {
    const Range256 rr = row_range256(row_pos, b, kmin_avail, a, spt);
    row_lo = rr.lo;
    row_hi = rr.hi;
  }

  // ---- Q prologue: QK-RMSNorm, RoPE, scale * log2(e), bf16: lane (ln, h2)
  // holds dims 16 s + 8 h2 + [0, 8) of row ln, s = 0..15; the rotation pairs
  // (d, d + 128) are s and s + 8 of the same lane.
  bf16x8 qreg[16];
  {
    const int r = row_ok ? row_pos - p0 : 0;  // valid address; rows past the end are never stored
    const uint16_t* src = a.q + (((long long)b * a.S + r) * a.Hq + g * G + hg) * kDh + 8 * h2;
    float x[128];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const u32x4 w = *(const u32x4*)(src + 16 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * s + 2 * e] = bf_lo(w[e]);
        x[8 * s + 2 * e + 1] = bf_hi(w[e]);
      }
    }
    float rn = a.sl2;
    if (a.q_gamma) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 128; ++e) ss += x[e] * x[e];
      ss = xhalf_sum256(ss);
      rn *= rsqrtf(ss * (1.f / kDh) + a.eps);
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * s + e] *= a.q_gamma[16 * s + 8 * h2 + e];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos(row_pos, rt.rev[16 * s + 8 * h2 + e], sn, cs);
        const float x1 = x[8 * s + e] * rn, x2 = x[8 * (s + 8) + e] * rn;
        x[8 * s + e] = x1 * cs - x2 * sn;
        x[8 * (s + 8) + e] = x1 * sn + x2 * cs;
      }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      u32x4 w = {pack2(x[8 * s], x[8 * s + 1]), pack2(x[8 * s + 2], x[8 * s + 3]), pack2(x[8 * s + 4], x[8 * s + 5]),
                 pack2(x[8 * s + 6], x[8 * s + 7])};
      qreg[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  wait_loads256();
  barrier_lds256();  // the first tile is in LDS

  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float l_run = 0.f;
  float m_run = -__builtin_huge_valf();
  const float NEG_INF = -__builtin_huge_valf();

  for (int it = 0; it < n_t; ++it) {
    const int t = t_begin + it;
    const int buf = it & 1;
    // Tile t+1 goes to the other buffer: every wave finished reading it
    // (tile t-1) before the previous barrier.
    if (it + 1 < n_t) dma_tile(t + 1, buf ^ 1);
    const int ts = p0 + t * kBNh;
    const bool act = ts <= w_hi_max && ts + kBNh - 1 >= w_lo_min;
    if (act) {
      const bool full = ts >= w_lo_max && ts + kBNh - 1 <= w_hi_min;
      const char* kl = (const char*)lds_k(buf);
      const char* vl = (const char*)lds_v(buf);
      // S^T (32 keys x 32 queries) = K Q^T over 16 dim steps
      bf16x8 kop[16];
#pragma unroll
      for (int st = 0; st < 16; ++st) kop[st] = *(const bf16x8*)(kl + adk[st]);
      f32x16 s = {};
#pragma unroll
      for (int st = 0; st < 16; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[st], qreg[st], s, 0, 0, 0);
      // V^T operands of the whole tile, read while the scores are computed
      bf16x8 vop[2][8];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          const char* base = vl + 8192 * t2;
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + adv[0][mb]));
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + adv[1][mb]));
          vop[t2][mb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      // softmax: key of register r = ts + 8 (r / 4) + 4 h2 + r % 4
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = ts + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (j < row_lo || j > row_hi) s[r] = NEG_INF;
        }
      }
      float off = 0.f;
      if (ONLINE) {
        float mx = NEG_INF;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = xhalf_max256(mx);
        const float m_new = fmaxf(m_run, mx);
        off = (m_new == NEG_INF) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - off);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      }
      bf16x8 pb[2];
      float rs = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(ONLINE ? s[8 * t2 + i] - off : s[8 * t2 + i]);
          rs += e[i];
        }
        u32x4 u = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        pb[t2] = __builtin_bit_cast(bf16x8, u);
      }
      l_run += rs;
      // O^T (256 dims x 32 queries) += V^T P^T
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t2][mb], pb[t2], o[mb], 0, 0, 0);
    }
    wait_loads256();
    barrier_lds256();  // tile t+1 landed; every wave is past tile t's reads
  }

  // Fast pass: a workgroup with a row whose sum leaves [2^-64, 2^64] (extreme
  // gammas, no norm, foreign cache contents) stores nothing and raises its
  // flag; the ONLINE launch redoes it with the running maximum.
  const float lt = xhalf_sum256(l_run);
  if (!ONLINE) {
    const bool bad = row_ok && !(lt >= 0x1p-64f && lt <= 0x1p64f);
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) a.flags[li] = any_bad;
    if (any_bad) return;
  }

  // ---- epilogue: O / l to bf16; one swap between the lane halves per word
  // gives each lane dims [32 mb + 16 j + 8 h2, +8), stored as 16 bytes.
  if (row_ok) {
    const float inv = 1.f / lt;
    uint16_t* dst = a.o + (((long long)b * a.S + (row_pos - p0)) * a.Hq + g * G + hg) * kDh + 8 * h2;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t lo0 = pack2(o[mb][8 * j] * inv, o[mb][8 * j + 1] * inv);
        const uint32_t lo1 = pack2(o[mb][8 * j + 2] * inv, o[mb][8 * j + 3] * inv);
        const uint32_t hi0 = pack2(o[mb][8 * j + 4] * inv, o[mb][8 * j + 5] * inv);
        const uint32_t hi1 = pack2(o[mb][8 * j + 6] * inv, o[mb][8 * j + 7] * inv);
        // lanes 32..63 receive hi of lane - 32; lanes 0..31 receive lo of lane + 32
        const auto r0 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
        const u32x4 ov = h2 ? u32x4{r0[0], r1[0], hi0, hi1} : u32x4{lo0, lo1, r0[1], r1[1]};
        *(u32x4*)(dst + 32 * mb + 16 * j) = ov;
      }
  }
}

hipError_t launch_prefill_d256(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt,
                               const RopeTable& rt, int G, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int n_items = a.B * a.Hkv * a.n_qtiles;
  const dim3 block(64 * kNW);
  if (ev_start) (void)hipEventRecord(ev_start, st);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_fwd_d256<1, false>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 2: hipLaunchKernelGGL((prefill_fwd_d256<2, false>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 4: hipLaunchKernelGGL((prefill_fwd_d256<4, false>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 8: hipLaunchKernelGGL((prefill_fwd_d256<8, false>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) (void)hipEventRecord(ev_stop, st);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_fwd_d256<1, true>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 2: hipLaunchKernelGGL((prefill_fwd_d256<2, true>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 4: hipLaunchKernelGGL((prefill_fwd_d256<4, true>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
    case 8: hipLaunchKernelGGL((prefill_fwd_d256<8, true>), dim3(n_items), block, 0, st, a, p0t, spt, rt); break;
  }
  return hipGetLastError();
}

}  // namespace g3
