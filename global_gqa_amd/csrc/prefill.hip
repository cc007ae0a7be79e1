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
// Design (per workgroup = 8 waves, one (sequence, kv head, query tile)):
//   * GQA packing: each wave owns 32 query rows = (32/G positions) x (G heads
//     of one kv group), so one K/V tile in LDS feeds 256 rows per workgroup.
//   * Q is loaded once (whole rows, through LDS), QK-RMSNorm + RoPE are applied in registers (fp64
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
#include "prefill_common.hpp"

#include <type_traits>

namespace g3 {

namespace {

constexpr int kBN = 64;  // keys per LDS tile (two halves of 32)
// K and V tiles sit in LDS as 64 rows x 256 B with no padding; the 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r).  The swizzle makes
// both operand reads conflict-free on gfx950's 64 x 4-byte banks: the K read
// (32 lanes on 32 rows, one chunk each) and the transposing V read (groups
// of 16 lanes on 4 rows x 32 B).  Tiles are filled by global->LDS loads that
// write 64 consecutive 16-byte chunks per instruction, so the swizzle is
// applied by choosing which chunk each lane fetches.
constexpr int kTileElems = kBN * 128;  // bf16 elements per tile
constexpr int kStageStride = 136;      // Q/O staging rows: 256 + 16 B
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// LDS: four K tile buffers in the first 64 KiB and four V tile buffers in
// the next 64 KiB, so every operand read is one per-lane address register
// plus an immediate offset (buffer, key half or key step) below 64 KiB.
constexpr int kTileBytes = kTileElems * 2;
constexpr uint32_t kVRegion = 4 * kTileBytes;

// Per-lane LDS byte addresses of the operand reads in K buffer 0 / V buffer 0.
struct TileAddr {
  uint32_t k[8];     // K^T operand, dims step st (key half kb adds 32 rows = 8192 B)
  uint32_t v[2][4];  // V^T operand, [row half][dim block] (key step t adds 16 rows = 4096 B)
};

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T* lds_at(uint32_t byte_addr) {
  return (const __attribute__((address_space(3))) T*)(uintptr_t)byte_addr;
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


// Orders this wave's LDS writes before its later LDS reads by other lanes of
// the same wave (LDS instructions of one wave execute in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// All but this wave's `newer` most recent global->LDS tile loads (0 or 4)
// have landed; loads complete in issue order.
__device__ __forceinline__ void wait_tile_loads_but(int newer) {
  if (newer == 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const uint16_t* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t*)p);
}




// Per-wave running state of the flash loop (one query row per lane).
struct WaveState {
  f32x16 o[4];   // O^T accumulators [dim block of 32]
  float l;       // per-lane partial row sum of p
  float m;       // running max (log2 units), online-maximum pass only
};

// One 64-key tile for one wave of 32 query rows, in three steps:
//   qk:      S^T (64 keys x 32 queries) = K Q^T, 16 MFMA 32x32x16, K from LDS
//   softmax: p = exp2(S) (scores are already in log2 units; masked keys -> 0),
//            row sums, p packed to bf16 as the B operand of P V
//   pv:      O^T (128 dims x 32 queries) += V^T P^T, 16 MFMA, V^T through
//            transposing LDS reads
template <bool MASK, bool ONLINE>
__device__ __forceinline__ void softmax(f32x16 (&s)[2], WaveState& w, bf16x8 (&pb)[4], int lo, int hi, int ts,
                                        int h2) {
  const float NEG_INF = -__builtin_huge_valf();
  if (MASK) {
    // key of (kb, r) = ts + 32 kb + 8 (r / 4) + 4 h2 + r % 4
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = ts + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (j < lo || j > hi) s[kb][r] = NEG_INF;
      }
  }
  float off = 0.f;
  if (ONLINE) {
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(w.m, mx);
    off = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = fast_exp2(w.m - off);
    w.m = m_new;
    w.l *= alpha;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.o[mb][r] *= alpha;
  }
  // row sum as a pairwise tree (dependent depth 5 instead of a 32-add chain,
  // which next to the other wave's MFMAs was latency-bound)
  float rs[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = s[t >> 1][8 * (t & 1) + i];
      e[i] = fast_exp2(ONLINE ? x - off : x);
    }
    rs[t] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    u32x4 u = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
    pb[t] = __builtin_bit_cast(bf16x8, u);
  }
  w.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

template <int VB>
__device__ __forceinline__ bf16x8 read_v(const TileAddr& ad, int t, int mb, uint32_t vdyn) {
  const uint32_t off = VB * kTileBytes + 4096 * t + vdyn;
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at<bf16x4>(ad.v[0][mb] + off));
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at<bf16x4>(ad.v[1][mb] + off));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The matrix half of a tile step: QK of this tile (if DO_QK) then PV of the
// previous one (if DO_PV), 16 + 16 MFMAs.  LDS operand reads run four QK
// steps or two PV steps (256 MFMA cycles) ahead of the MFMAs that use them,
// and scheduling fences keep the compiler from pulling them back next to
// their uses, where each MFMA would wait out a full LDS latency.  dma(k), k = 0..7,
// is a hook between the MFMA groups for global->LDS loads; the tile loop
// passes an empty one (its loads go out at the end of the softmax half, which
// measured faster than any placement between the MFMAs).
// VB, KB: the V and K buffers (compile-time); vdyn: a run-time byte offset
// added to the V reads (0 inside the unrolled tile loop).
template <bool DO_PV, bool DO_QK, int VB, int KB, bool PRE = false, typename Dma>
__device__ __forceinline__ void gemm_half(const TileAddr& ad, const bf16x8 (&pb)[4], const bf16x8 (&q)[8],
                                          f32x16 (&s)[2], WaveState& w, Dma&& dma, uint32_t vdyn = 0,
                                          const bf16x8 (&pre)[4] = {}) {
  bf16x8 vop[4][4];  // [16-key step][dim block]
  bf16x8 kop[8][2];  // [16-dim step][key half]
  auto rd_v = [&](int t) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) vop[t][mb] = read_v<VB>(ad, t, mb, vdyn);
  };
  auto rd_k = [&](int st) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kop[st][kb] = *lds_at<bf16x8>(ad.k[st] + KB * kTileBytes + 8192 * kb);
  };
  auto mm_pv = [&](int t) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      w.o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][mb], pb[t], w.o[mb], 0, 0, 0);
  };
  auto mm_qk = [&](int st) {  // step 0 starts the sums from zero
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[st][kb], q[st], st == 0 ? f32x16{} : s[kb], 0, 0, 0);
  };
  auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
  // QK first: its K operands (ds_read_b128) arrive sooner than the
  // transposed V reads, which get the whole QK run as lead time.
  constexpr int KA = 4;  // K steps read ahead of their QK MFMAs (6 measured slower)
  if (DO_QK) {
    if (PRE) {  // K of steps 0 and 1 read before the barrier that opens the half
      kop[0][0] = pre[0];
      kop[0][1] = pre[1];
      kop[1][0] = pre[2];
      kop[1][1] = pre[3];
#pragma unroll
      for (int st = 2; st < KA; ++st) rd_k(st);
    } else {
#pragma unroll
      for (int st = 0; st < KA; ++st) rd_k(st);
    }
    fence();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      mm_qk(st);
      if (st + KA < 8) rd_k(st + KA);
      if (DO_PV && st >= 4 && st < 6) rd_v(st - 4);
      dma(st);
      fence();
    }
  }
  if (DO_PV) {
    if (!DO_QK) {
      rd_v(0);
      rd_v(1);
      fence();
    }
    mm_pv(0);
    rd_v(2);
    fence();
    mm_pv(1);
    rd_v(3);
    fence();
    mm_pv(2);
    fence();
    mm_pv(3);
    fence();
  }
  if (!DO_QK) {
#pragma unroll
    for (int k = 0; k < 8; ++k) dma(k);
  }
}

template <bool DO_PV, int VB, int KB, bool PRE, typename Dma>
__device__ __forceinline__ void gemm_step(bool do_qk, const TileAddr& ad, const bf16x8 (&pb)[4],
                                          const bf16x8 (&q)[8], f32x16 (&s)[2], WaveState& w, Dma&& dma,
                                          const bf16x8 (&pre)[4]) {
  if (do_qk) {
    gemm_half<DO_PV, true, VB, KB, PRE>(ad, pb, q, s, w, dma, 0, pre);
  } else if (DO_PV) {
    gemm_half<DO_PV, false, VB, KB>(ad, pb, q, s, w, dma);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) dma(k);
  }
}

template <bool ONLINE>
__device__ __forceinline__ void softmax_tile(bool full, f32x16 (&s)[2], WaveState& w, bf16x8 (&pb)[4], int lo,
                                             int hi, int ts, int h2) {
  if (full)
    softmax<false, ONLINE>(s, w, pb, lo, hi, ts, h2);
  else
    softmax<true, ONLINE>(s, w, pb, lo, hi, ts, h2);
}

}  // namespace

// Workgroup = NW waves = one (sequence, kv head, query tile).  Each wave owns
// 32 query rows: 32/G positions x the G query heads that share the kv head,
// so one K/V tile in LDS serves all G heads and all NW waves.  With NW = 8
// one workgroup fills a CU (two waves per SIMD): one wave's softmax VALU
// work overlaps the other's MFMAs, and each K/V tile crosses L2 -> LDS once
// per 256 query rows.
// One work item: (sequence, kv head, query tile) li.
template <int G, bool ONLINE, int NW>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt,
                                             const RopeTable& rt, uint16_t* lds, int li) {
  constexpr int P = 32 / G;    // positions per wave
  constexpr int WP = NW * P;   // positions per workgroup
  constexpr int NT = 64 * NW;  // threads per workgroup
  static_assert(NW == 8, "the tile loader gives each wave 8 of the 64 rows");
  // LDS, 16 KiB per tile buffer: K and V in 4 buffers each (tile t is read,
  // tile t+1 has landed or is landing, tile t+2 is being fetched; V of tile
  // t-1 is still read by the PV half), tile t in buffer t & 3 so that, with
  // the loop unrolled by 4, every buffer is a compile-time offset.  Each
  // wave's staging rows for its 32 Q rows (prologue) and O rows (epilogue),
  // through which both move between HBM and registers as whole 256-byte rows,
  // alias K1..K3 (waves 0-4) and V1..V3 (waves 5-7): the first tile (K0, V0)
  // lands while Q is staged, and the second is only fetched once every wave
  // has read its Q rows.
  static_assert(5 * 32 * kStageStride <= 3 * kTileElems, "staging of waves 0-4 must fit in K1..K3");
  static_assert((NW - 5) * 32 * kStageStride <= 3 * kTileElems, "staging of waves 5-7 must fit in V1..V3");
  auto lds_k = [&](int buf) { return lds + buf * kTileElems; };
  auto lds_v = [&](int buf) { return lds + (4 + buf) * kTileElems; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h2 = lane >> 5;
  const int ln = lane & 31;

  // The online-maximum pass only redoes the tiles the fast pass flagged.
  if (ONLINE && a.flags[li] == 0) return;
  int bg, qt;
  prefill_item_coords(li, a.B * a.Hkv, a.n_qtiles, prefill_rank_major(a.local, a.B * a.Hkv), bg, qt);
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  // the per-sequence table is indexed at run time: keep the (uniform) result scalar
  const int p0 = __builtin_amdgcn_readfirstlane(pos0_of(p0t, b));
  const int chunk_end = p0 + a.S;
  const int kmin_avail = a.has_cache ? (a.is_ring ? max(0, p0 - a.cap) : 0) : p0;
  const int qbase = p0 + qt * WP;  // first query position of the workgroup
  const int wbase = qbase + wave * P;  // first query position of this wave

  // ---- Q rows of this wave, loaded row-major: 16 lanes x 16 B per row.
  // Staging row x = (head hg, position offset u) is x = hg * P + u.
  uint16_t* xs = wave < 5 ? lds + kTileElems + wave * 32 * kStageStride
                          : lds + 5 * kTileElems + (wave - 5) * 32 * kStageStride;
  const int x_col = (lane & 15) * 8;
  {
    u32x4 qv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = 4 * k + (lane >> 4);
      const int hg = x / P, u = x - (x / P) * P;
      const int pos = wbase + u;
      const int r = pos < chunk_end ? pos - p0 : 0;  // valid address; rows past the end are never stored
      qv[k] = *(const u32x4*)(a.q + (((long long)b * a.S + r) * a.Hq + g * G + hg) * kD + x_col);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) *(u32x4*)(xs + (4 * k + (lane >> 4)) * kStageStride + x_col) = qv[k];
  }

  // ---- key ranges.  lo(i) and hi(i) are non-decreasing in i, so the union
  // over a run of rows is [lo(first), hi(last)] and the intersection is
  // [lo(last), hi(first)].
  const int wg_last = min(qbase + WP, chunk_end) - 1;
  const RowRange wg_first_r = row_range(qbase, b, kmin_avail, a, spt);
  const RowRange wg_last_r = row_range(wg_last, b, kmin_avail, a, spt);
  const int t_begin = floor_div<64>(wg_first_r.lo - p0);
  const int t_end = floor_div<64>(wg_last_r.hi - p0);  // inclusive
  const int n_t = t_end - t_begin + 1;
  int w_lo_min = 0x7fffffff, w_hi_max = -0x7fffffff, w_lo_max = 0x7fffffff, w_hi_min = -0x7fffffff;
  if (wbase < chunk_end) {
    const RowRange f = row_range(wbase, b, kmin_avail, a, spt);
    const RowRange l = row_range(min(wbase + P, chunk_end) - 1, b, kmin_avail, a, spt);
    w_lo_min = f.lo;
    w_hi_min = f.hi;
    w_lo_max = l.lo;
    w_hi_max = l.hi;
  }

  // ---- tile loader: global -> LDS directly (no registers, no LDS stores).
  // Wave w fills rows [8w, 8w + 8) of the K and V tiles with 4-row
  // instructions: lane L of instruction i lands on row 8w + 4i + L/16, chunk
  // position L % 16, so it fetches logical chunk (L % 16) ^ swz(row).  Keys
  // that do not exist read a zero row, so their p v terms vanish.
  const int dma_r = lane >> 4;
  const uint16_t* khat_bg = a.khat + ((long long)b * a.Hkv + g) * a.S * kD;
  const uint16_t* v_bg = a.v + ((long long)b * a.S * a.Hkv + g) * kD;
  const int vstride = a.Hkv * kD;
  const long long cache_bg = ((long long)b * a.Hkv + g) * (long long)a.cap * kD;
  const uint16_t* ck_bg = a.has_cache ? a.ck + cache_bg : nullptr;
  const uint16_t* cv_bg = a.has_cache ? a.cv + cache_bg : nullptr;
  // Instruction k (0..3) of this wave's share of tile t (k < 2: K rows, else
  // V rows).  Tiles wholly inside the chunk or inside one contiguous stretch
  // of the cache (the long-context case) take a straight path: a wave-uniform
  // base plus a per-lane offset, the mode test hoisted out of the per-load
  // code.  Only tiles at the chunk or cache edges check every row.
  // LDS destination (M0) of this wave's load i (0..1) of a K or V tile
  // buffer.  The wave's base goes through an opaque copy so that the
  // compiler forms each destination where it is used instead of holding all
  // of them in SGPRs across the tile loop.
  const uint32_t wave_lds_base = lds_addr_of(lds) + (uint32_t)(8 * wave_u * kD * 2);
  auto dst_of = [&](bool is_v, int buf, int i) {
    uint32_t wb = wave_lds_base;
    asm volatile("" : "+s"(wb));
    return wb + (uint32_t)((is_v ? 4 + buf : buf) * kTileBytes + 4 * i * kD * 2);
  };
  auto dma_tile = [&](int t, int kbuf, int vbuf) {
    const int ts = p0 + t * kBN;
    const bool in_chunk = t >= 0 && ts + kBN <= chunk_end;
    const bool in_cache = !in_chunk && a.has_cache && ts >= kmin_avail && ts + kBN <= p0;
    const int slot0 = (in_cache && a.is_ring) ? ts % a.cap : ts;
    const bool cache_run = in_cache && (!a.is_ring || slot0 + kBN <= a.cap);
    if (in_chunk || cache_run) {
      const uint16_t* kb = in_chunk ? khat_bg + (long long)t * kBN * kD : ck_bg + (long long)slot0 * kD;
      const uint16_t* vb = in_chunk ? v_bg + (long long)t * kBN * vstride : cv_bg + (long long)slot0 * kD;
      const int vs = in_chunk ? vstride : kD;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = k & 1;
        const bool is_v = k >= 2;
        const int col = ((lane & 15) ^ ((dma_r << 2) | ((2 * wave + i) & 3))) * 8;
        const int row = 8 * wave + 4 * i + dma_r;
        dma16s(is_v ? vb : kb, 2u * (uint32_t)(row * (is_v ? vs : kD) + col), dst_of(is_v, is_v ? vbuf : kbuf, i));
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = k & 1;
      const bool is_v = k >= 2;
      const int col = ((lane & 15) ^ ((dma_r << 2) | ((2 * wave + i) & 3))) * 8;
      const int row = 8 * wave + 4 * i + dma_r;
      const int j = ts + row;
      const uint16_t* src = g_zero_row;
      if (j >= p0 && j < chunk_end) {
        src = is_v ? v_bg + (j - p0) * vstride : khat_bg + (j - p0) * kD;
      } else if (a.has_cache && j < p0 && j >= kmin_avail) {
        const long long slot = a.is_ring ? (long long)(j % a.cap) : (long long)j;
        src = (is_v ? cv_bg : ck_bg) + slot * kD;
      }
      dma16(src + col, dst_of(is_v, is_v ? vbuf : kbuf, i));
    }
  };

  // Items whose every key tile lies inside the chunk (a self-contained prompt
  // of whole tiles) load each tile from two running bases with per-lane
  // offsets fixed for the item: no per-tile choice of source.
  const bool chunk_only = t_begin >= 0 && p0 + (t_begin + n_t) * kBN <= chunk_end;
  // Items over a linear cache (the long-context chunk against its cache)
  // whose tiles are whole cache tiles below the chunk, then whole chunk
  // tiles: the same two running bases, switched once where the chunk starts.
  const bool linear_run = !chunk_only && a.has_cache && !a.is_ring && p0 + t_begin * kBN >= kmin_avail &&
                          p0 + (t_begin + n_t) * kBN <= chunk_end;

  // operand read offsets inside a tile (see TileAddr)
  TileAddr ad;
  const uint32_t lds0 = lds_addr_of(lds);
#pragma unroll
  for (int st = 0; st < 8; ++st) ad.k[st] = lds0 + ln * 256 + ((((2 * st + h2) ^ swz(ln))) << 4);
  {
    const int g4 = lane >> 4, w16 = lane & 15;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 8 * hf + 4 * (g4 >> 1) + (w16 >> 2);
        const int c = 4 * mb + 2 * (g4 & 1) + ((w16 & 3) >> 1);
        ad.v[hf][mb] = lds0 + kVRegion + row * 256 + ((c ^ swz(row)) << 4) + 8 * (w16 & 1);
      }
  }

  dma_tile(t_begin, 0, 0);  // the first tile, in flight while Q is prepared

  // this lane's query row: position offset ln % P, head ln / P of the group
  const int hg = ln / P;
  const int row_pos = wbase + (ln - hg * P);
  const int row_head = g * G + hg;
  const bool row_ok = row_pos < chunk_end;
  int row_lo = 0x7fffffff, row_hi = -0x7fffffff;
  if (row_ok) {
    const RowRange rr = row_range(row_pos, b, kmin_avail, a, spt);
    row_lo = rr.lo;
    row_hi = rr.hi;
  }

  // ---- Q prologue: QK-RMSNorm, RoPE, scale by softmax_scale * log2(e),
  // round to bf16: the B operand of S^T = K Q^T (lane: query ln, dims
  // 16 s + 8 h2 + [0, 8)), so scores come out in log2 units.
  wave_lds_sync();
  bf16x8 qreg[8];
  {
    float x[64];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 wv = *(const u32x4*)(xs + ln * kStageStride + 16 * s + 8 * h2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * s + 2 * e] = bf_lo(wv[e]);
        x[8 * s + 2 * e + 1] = bf_hi(wv[e]);
      }
    }
    float rn = a.sl2;
    if (a.q_gamma) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e) ss += x[e] * x[e];
      ss = xhalf_sum(ss);
      rn *= rsqrtf(ss * (1.f / kD) + a.eps);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * s + e] *= a.q_gamma[16 * s + 8 * h2 + e];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double rev = rt.rev[16 * s + 8 * h2 + e];
        float sn, cs;
        rope_sincos(row_pos, rev, sn, cs);
        const float x1 = x[8 * s + e] * rn, x2 = x[8 * (s + 4) + e] * rn;
        x[8 * s + e] = x1 * cs - x2 * sn;
        x[8 * (s + 4) + e] = x1 * sn + x2 * cs;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 wv = {pack2(x[8 * s], x[8 * s + 1]), pack2(x[8 * s + 2], x[8 * s + 3]),
                  pack2(x[8 * s + 4], x[8 * s + 5]), pack2(x[8 * s + 6], x[8 * s + 7])};
      qreg[s] = __builtin_bit_cast(bf16x8, wv);
    }
  }

  barrier_lds();  // every wave has read its staged Q rows
  if (n_t > 1) dma_tile(t_begin + 1, 1, 1);
  wait_tile_loads_but(n_t > 1 ? 4 : 0);
  barrier_lds();  // the first tile is in LDS

  WaveState ws;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ws.o[mb][r] = 0.f;
  ws.l = 0.f;
  ws.m = -__builtin_huge_valf();
  // Ping-pong between the two waves of each SIMD (waves w and w + NW/2):
  // every tile takes two halves separated by workgroup barriers, and in each
  // half one wave runs its matrix products (PV of the previous tile, then QK
  // of this one: 32 MFMAs) while the other runs its softmax (VALU), so the
  // MFMA pipe and the VALU are busy at the same time instead of in turn.
  //   group A (waves 0..NW/2-1): half 1 PV(t-1) + QK(t), half 2 softmax(t)
  //   group B (waves NW/2..NW-1): half 1 softmax(t-1),   half 2 PV(t-1) + QK(t)
  // Straight chunk tiles: this lane's byte offsets from a tile's first row
  // for the wave's two 4-row loads (K and V rows share the swizzle), held
  // for the item, and per-tile bases advanced by one tile per step.
  uint32_t ck_off[2], cv_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = lane >> 4;
    const int row = 8 * wave_u + 4 * i + r;
    const int col = ((lane & 15) ^ ((r << 2) | ((2 * wave_u + i) & 3))) * 8;
    ck_off[i] = 2u * (uint32_t)(row * kD + col);
    cv_off[i] = 2u * (uint32_t)(row * vstride + col);
  }

  // mode: 0 any tile (per-tile choice of source), 1 chunk tiles only, 2 linear-cache tiles then chunk tiles
  auto run = [&](auto grp_b_tag, auto mode_tag) {
    constexpr bool GB = decltype(grp_b_tag)::value;
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool CHUNK_ONLY = MODE == 1;
    constexpr bool LINEAR_RUN = MODE == 2;
    f32x16 s[2];
    bf16x8 pb[4];
    bool have_p = false;  // pb holds p of the previous tile, PV still to do
    bool have_s = false;  // (group B) s holds scores of the previous tile
    bool s_full = false;
    int s_ts = 0;
    // bases of tile t + 2 (straight chunk tiles)
    const char* kb_next = (const char*)khat_bg + (long long)(t_begin + 2) * (kBN * kD * 2);
    const char* vb_next = (const char*)v_bg + (long long)(t_begin + 2) * kBN * vstride * 2;
    if (LINEAR_RUN && t_begin + 2 < 0) {  // cache tiles: slot = position, rows of kD elements for K and V
      kb_next = (const char*)ck_bg + (long long)(p0 + (t_begin + 2) * kBN) * (kD * 2);
      vb_next = (const char*)cv_bg + (long long)(p0 + (t_begin + 2) * kBN) * (kD * 2);
    }
    // One tile step; tile it sits in K and V buffer U = it & 3.
    auto step = [&](auto u_tag, int it) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int UPREV = (U + 3) & 3;  // V buffer of the previous tile
      constexpr int UNEXT2 = (U + 2) & 3;
      const int t = t_begin + it;
      const int ts = p0 + t * kBN;
      const bool act = ts <= w_hi_max && ts + kBN - 1 >= w_lo_min;
      const bool full = ts >= w_lo_max && ts + kBN - 1 <= w_hi_min;
      // Tile t+2 is fetched during this wave's softmax half (VALU-bound, with
      // slack next to the other wave's matrix half); before the tile's closing
      // barrier only tile t+1's loads must have landed.
      const bool fetch = it + 2 < n_t;
      auto prefetch = [&]() {
        if (fetch) {
          if (CHUNK_ONLY) {
            dma16s(kb_next, ck_off[0], dst_of(false, UNEXT2, 0));
            dma16s(kb_next, ck_off[1], dst_of(false, UNEXT2, 1));
            dma16s(vb_next, cv_off[0], dst_of(true, UNEXT2, 0));
            dma16s(vb_next, cv_off[1], dst_of(true, UNEXT2, 1));
          } else if (LINEAR_RUN) {
            const bool from_cache = t + 2 < 0;  // cache V rows are kD apart, the chunk's vstride
            const uint32_t v0 = from_cache ? ck_off[0] : cv_off[0];
            const uint32_t v1 = from_cache ? ck_off[1] : cv_off[1];
            dma16s(kb_next, ck_off[0], dst_of(false, UNEXT2, 0));
            dma16s(kb_next, ck_off[1], dst_of(false, UNEXT2, 1));
            dma16s(vb_next, v0, dst_of(true, UNEXT2, 0));
            dma16s(vb_next, v1, dst_of(true, UNEXT2, 1));
          } else
            dma_tile(t + 2, UNEXT2, UNEXT2);
        }
      };
      auto no_dma = [](int) {};
      if (!GB) {
        __builtin_amdgcn_s_setprio(1);
        if (have_p)
          gemm_step<true, UPREV, U, false>(act, ad, pb, qreg, s, ws, no_dma, {});
        else
          gemm_step<false, UPREV, U, false>(act, ad, pb, qreg, s, ws, no_dma, {});
        __builtin_amdgcn_s_setprio(0);
        have_p = false;
        barrier_lds();
        if (act) {
          softmax_tile<ONLINE>(full, s, ws, pb, row_lo, row_hi, ts, h2);
          have_p = true;
        }
        prefetch();
        wait_tile_loads_but(fetch ? 4 : 0);
        barrier_lds();
      } else {
        if (have_s) {
          softmax_tile<ONLINE>(s_full, s, ws, pb, row_lo, row_hi, s_ts, h2);
          have_p = true;
        }
        prefetch();
        // Group B reads K of its first two QK steps while it waits at the
        // barrier that opens its matrix half (the tile was published by the
        // previous step's closing barrier), so its MFMAs start without an
        // LDS round trip after the barrier.  (Group A's matrix half opens a
        // step; holding V^T operands across the step boundary for it, with
        // its steps rotated to keep them local, measured slower.)
        bf16x8 kpre[4];
        if (act) {
#pragma unroll
          for (int i = 0; i < 4; ++i) kpre[i] = *lds_at<bf16x8>(ad.k[i >> 1] + U * kTileBytes + 8192 * (i & 1));
        }
        barrier_lds();
        __builtin_amdgcn_s_setprio(1);
        if (have_p)
          gemm_step<true, UPREV, U, true>(act, ad, pb, qreg, s, ws, no_dma, kpre);
        else
          gemm_step<false, UPREV, U, true>(act, ad, pb, qreg, s, ws, no_dma, kpre);
        __builtin_amdgcn_s_setprio(0);
        have_p = false;
        have_s = act;
        s_full = full;
        s_ts = ts;
        wait_tile_loads_but(fetch ? 4 : 0);
        barrier_lds();
      }
      if (CHUNK_ONLY) {
        kb_next += kBN * kD * 2;
        vb_next += (long long)kBN * vstride * 2;
      }
      if (LINEAR_RUN) {  // bases of the next step's tile t + 3
        if (t + 3 == 0) {
          kb_next = (const char*)khat_bg;
          vb_next = (const char*)v_bg;
        } else {
          kb_next += kBN * kD * 2;
          vb_next += t + 3 < 0 ? (long long)kBN * kD * 2 : (long long)kBN * vstride * 2;
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int it = 0; it < n_t; it += 4) {
      step(I0{}, it);
      if (it + 1 >= n_t) break;
      step(I1{}, it + 1);
      if (it + 2 >= n_t) break;
      step(I2{}, it + 2);
      if (it + 3 >= n_t) break;
      step(I3{}, it + 3);
    }
    // drain: the last tile's PV (group A) / softmax then PV (group B)
    if (GB && have_s) {
      softmax_tile<ONLINE>(s_full, s, ws, pb, row_lo, row_hi, s_ts, h2);
      have_p = true;
    }
    barrier_lds();
    if (have_p)  // V of the last tile sits in buffer (n_t - 1) & 3
      gemm_half<true, false, 0, 0>(ad, pb, qreg, s, ws, [](int) {}, (uint32_t)(((n_t - 1) & 3) * kTileBytes));
  };
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  if (wave_u >= NW / 2) {
    if (chunk_only)
      run(std::true_type{}, M1{});
    else if (linear_run)
      run(std::true_type{}, M2{});
    else
      run(std::true_type{}, M0{});
  } else {
    if (chunk_only)
      run(std::false_type{}, M1{});
    else if (linear_run)
      run(std::false_type{}, M2{});
    else
      run(std::false_type{}, M0{});
  }

  // Fast pass (ONLINE = false): QK-RMSNorm bounds every logit by
  // scale * D * max|gamma_q| * max|gamma_k|, so for sane gammas the softmax
  // needs no running maximum: p = exp2(s) directly.  A workgroup with a row
  // whose sum leaves [2^-64, 2^64] (possible only for extreme gammas, no
  // norm, or foreign cache contents) raises its flag, and a second launch
  // with ONLINE = true redoes exactly those tiles with the running maximum.
  const float lt = xhalf_sum(ws.l);
  if (!ONLINE) {
    const bool bad = row_ok && !(lt >= 0x1p-64f && lt <= 0x1p64f);
    const int any_bad = __syncthreads_or(bad);  // also: every wave is past its last V read
    if (tid == 0) a.flags[li] = any_bad;
    if (any_bad) return;
  } else {
    barrier_lds();  // every wave is past its last V read (staging aliases the tiles)
  }

  // ---- epilogue: O / l to bf16 into the wave's staging rows, then whole
  // 256-byte rows out to [b][pos][head][dims]
  {
    const float inv = row_ok ? 1.f / lt : 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mb + 8 * q4 + 4 * h2;
        const f32x16& oa = ws.o[mb];
        *(u32x2*)(xs + ln * kStageStride + d) = u32x2{pack2(oa[4 * q4] * inv, oa[4 * q4 + 1] * inv),
                                                     pack2(oa[4 * q4 + 2] * inv, oa[4 * q4 + 3] * inv)};
      }
  }
  wave_lds_sync();
  // An opaque copy of the lane index keeps the compiler from carrying the Q
  // prologue's row addresses (same offsets) through the tile loop.
  int el = lane;
  asm volatile("" : "+v"(el));
  const int e_col = (el & 15) * 8;
  uint16_t* o_wave = a.o + (((long long)b * a.S + (wbase - p0)) * a.Hq + g * G) * kD;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int x = 4 * k + (el >> 4);
    const int xh = x / P, u = x - (x / P) * P;
    const u32x4 ov = *(const u32x4*)(xs + x * kStageStride + e_col);
    if (wbase + u < chunk_end) *(u32x4*)(o_wave + (u * a.Hq + xh) * kD + e_col) = ov;
  }
}

// With fewer workgroups than items (the local layers, whose items cost
// about the same) each workgroup runs several items back to back on its CU:
// the query tiles prefill_spread_item gives it (one run, tiles nq/K apart,
// the lightest first, so that the workgroups holding a run's short first
// tiles fall out of step and item boundaries, where every workgroup loads
// its Q rows and first tiles at once, spread out: local layers 169 -> 159 us
// at the 27B shape), and the workgroups of one XCD work on neighbouring
// query tiles of the same kv head, which share K/V in that XCD's L2.  Other
// counts take items xcd_remap(g) + k * gridDim.x.  With one workgroup per
// item (the fast pass of a global layer) the item order is that of
// prefill_item_of_workgroup.
template <int G, bool ONLINE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW)
void prefill_fwd(PrefillArgs a, Pos0Table p0t, SpanTable spt, RopeTable rt) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[8 * kTileElems];
  const int n_items = a.B * a.Hkv * a.n_qtiles;
  const int li0 = (!ONLINE && (int)gridDim.x == n_items)
                      ? prefill_item_of_workgroup(blockIdx.x, n_items, prefill_rank_major(a.local, a.B * a.Hkv))
                      : xcd_remap(blockIdx.x, gridDim.x);
  if (ONLINE) {
    // The online-maximum pass usually finds nothing to redo: every wave reads
    // the flags of all of this workgroup's items at once (one per lane) and
    // the workgroup leaves unless one is set.
    int any = 0;
    for (int li = li0 + (int)(threadIdx.x & 63) * (int)gridDim.x; li < n_items; li += 64 * (int)gridDim.x)
      any |= a.flags[li];
    if (__builtin_amdgcn_ballot_w64(any != 0) == 0) return;
  }
  const int per_wg = n_items / (int)gridDim.x;
  if (!ONLINE && a.local && per_wg > 1 && n_items % (int)gridDim.x == 0 && a.n_qtiles % per_wg == 0) {
    for (int kk = 0; kk < per_wg; ++kk)
      prefill_item<G, ONLINE, NW>(a, p0t, spt, rt, lds, prefill_spread_item(li0, kk, per_wg, a.n_qtiles));
    return;
  }
  for (int li = li0; li < n_items; li += gridDim.x) prefill_item<G, ONLINE, NW>(a, p0t, spt, rt, lds, li);
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_prefill(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt, const RopeTable& rt,
                          int G, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int n_items = a.B * a.Hkv * a.n_qtiles;
  const int one_per_cu = n_items < cu_count() ? n_items : cu_count();
  // Local-layer items all cost about the same (window + query tile), so one
  // workgroup per CU runs them back to back; global-layer items range from 1
  // to S/64 key tiles and are left to the hardware's dynamic dispatch.  The
  // online-maximum pass mostly finds nothing to redo: one workgroup per CU.
  const int grid = a.local ? one_per_cu : n_items;
  const int grid_online = one_per_cu;
  constexpr int NW = kPrefillWaves;
  const dim3 block(64 * NW);
  if (ev_start) hipEventRecord(ev_start, st);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_fwd<1, false, NW>), dim3(grid), block, 0, st, a, p0t, spt, rt); break;
    case 2: hipLaunchKernelGGL((prefill_fwd<2, false, NW>), dim3(grid), block, 0, st, a, p0t, spt, rt); break;
    case 4: hipLaunchKernelGGL((prefill_fwd<4, false, NW>), dim3(grid), block, 0, st, a, p0t, spt, rt); break;
    case 8: hipLaunchKernelGGL((prefill_fwd<8, false, NW>), dim3(grid), block, 0, st, a, p0t, spt, rt); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (ev_stop) hipEventRecord(ev_stop, st);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_fwd<1, true, NW>), dim3(grid_online), block, 0, st, a, p0t, spt, rt); break;
    case 2: hipLaunchKernelGGL((prefill_fwd<2, true, NW>), dim3(grid_online), block, 0, st, a, p0t, spt, rt); break;
    case 4: hipLaunchKernelGGL((prefill_fwd<4, true, NW>), dim3(grid_online), block, 0, st, a, p0t, spt, rt); break;
    case 8: hipLaunchKernelGGL((prefill_fwd<8, true, NW>), dim3(grid_online), block, 0, st, a, p0t, spt, rt); break;
  }
  return hipGetLastError();
}

}  // namespace g3
