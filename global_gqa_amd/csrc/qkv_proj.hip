// QKV projection with the key prologue (QK-RMSNorm + RoPE) fused into its
// epilogue, for head dimension 128.
//
// The attention layer's inputs are q = x Wq^T, k = x Wk^T, v = x Wv^T (the
// q_proj / k_proj / v_proj linear maps, no bias; "Gemma explained: What's new
// in Gemma 3", 27B module print), after which k is normalised (k_norm, RMSNorm
// over the head dimension) and rotated at its absolute position (Gemma 3
// Technical Report, section 2).  Here one kernel computes the projections and
// writes k already normed and rotated in the head-major layout the flash
// prefill reads, so the separate key prologue pass (one read and one write of
// every key row) disappears; q and v leave raw (q is normalised inside the
// prefill kernel).
//
// Design (workgroup = 8 waves, two per SIMD; tile = two heads' 256 output
// features x 256 tokens; grid = (token tiles, head pairs)):
//   * C^T = W X^T with v_mfma_f32_32x32x16_bf16: A = 32 weight rows x 16
//     inputs, B = 32 token rows x 16 inputs.  Wave w computes head
//     2 p + (w & 1) for tokens 64 (w >> 1) .. 64 (w >> 1) + 63: 2 x 4
//     accumulator blocks, 6 operand reads per 8 MFMAs.  In the epilogue each lane holds one token's 64 features of the
//     head and the token's other 64 sit in the lane 32 apart: the RMSNorm is
//     an in-lane sum plus one cross-half swap, and the RoPE pairs (d, d + 64)
//     are in the same lane;
//   * both operands are consumed in chunks of 32 inputs (two 16-input
//     steps), staged in LDS by global->LDS loads four chunks deep
//     (4 x 32 KiB).  Each chunk runs as: the 8 MFMAs of step 0 while the
//     operands of step 1 are read; the barrier that publishes chunk c + 1;
//     the 8 MFMAs of step 1 while the operands of step 0 of chunk c + 1 are
//     read and the loads of chunk c + 4 are issued into the stage chunk c
//     leaves.  Operand reads and loads sit between MFMAs, so the matrix
//     pipe keeps running across the barrier;
//   * rows are 64 B (four 16-byte pieces) with the pieces permuted by
//     piece ^ sw(row), sw(r) = (r >> 2) & 3: with lane l reading row l % 32,
//     piece (2 st + l / 32) ^ sw(row), the ds_read_b128 runs in its 4 base
//     cycles with no bank-conflict cycles (measured with the LDS counters on
//     gfx950; the unpermuted layout, and other permutations that spread 16
//     consecutive lanes over the banks, measured 2-4 way conflicts).  sw
//     depends only on the row's low five bits, so operand blocks 32 rows
//     apart read at immediate offsets.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

constexpr int kQD = 128;                      // head dimension
constexpr int kQT = 256;                      // tokens per tile
constexpr int kQF = 256;                      // output features per tile (two heads)
constexpr int kQC = 32;                       // inputs per chunk
constexpr int kQStages = 4;                   // chunks staged in LDS
constexpr int kQTileB = 256 * kQC * 2;        // 16384 bytes: 256 rows x 64 B
constexpr int kQStageB = 2 * kQTileB;         // W tile then X tile
constexpr int kQWaves = 8;
constexpr int kQLoadsPerWave = kQStageB / 1024 / kQWaves;  // 4 global->LDS loads of 1 KiB

typedef __attribute__((address_space(3))) char qlds_char;
typedef __attribute__((address_space(3))) const bf16x8 qlds_bf16x8;

__device__ __forceinline__ void qdma(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds_addr)
      : "m0");
}

// Barrier that waits for this wave's LDS operations only (a full
// __syncthreads would also wait for the loads in flight).
__device__ __forceinline__ void qbarrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int qswz(int r) { return (r >> 2) & 3; }

// q or v rows of one 32-token block: lane (ln, h2) holds token t's features
// n = 32 b + 8 (r / 4) + 4 h2 + r % 4 in acc[b][r], b = 0..3, at offset foff
// of a head of D features.
__device__ __forceinline__ void store_plain_rows(const QkvArgs& a, const f32x16* acc, int head, int t, int h2,
                                                 int foff) {
  uint16_t* dst = (head < a.Hq ? a.q + ((long long)t * a.Hq + head) * a.D
                               : a.v + ((long long)t * a.Hkv + (head - a.Hq - a.Hkv)) * a.D) + foff;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int n = 32 * b + 8 * g4 + 4 * h2;
      *(u32x2*)(dst + n) = u32x2{pack2(acc[b][4 * g4], acc[b][4 * g4 + 1]),
                                 pack2(acc[b][4 * g4 + 2], acc[b][4 * g4 + 3])};
    }
}

// Epilogue of one 32-token block at head dimension 128: lane (ln, h2) holds
// token t's features n = 32 b + 8 (r / 4) + 4 h2 + r % 4 in acc[b][r].
__device__ __forceinline__ void store_head_rows(const QkvArgs& a, const Pos0Table& p0t, const RopeTable& rt,
                                                const f32x16* acc, int head, int t, int h2) {
  if (head < a.Hq || head >= a.Hq + a.Hkv) {
    store_plain_rows(a, acc, head, t, h2, 0);
    return;
  }
  // key head: QK-RMSNorm over the 128 features, then RoPE at the token's
  // absolute position, stored head-major [B][Hkv][S][D]
  const int bt = t / a.S, s = t - bt * a.S;
  float ss = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss += acc[b][r] * acc[b][r];
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
    ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float rn = a.k_gamma ? __frsqrt_rn(ss * (1.f / kQD) + a.eps) : 1.f;
  const int pos = pos0_of(p0t, bt) + s;
  uint16_t* dst = a.khat + (((long long)bt * a.Hkv + (head - a.Hq)) * a.S + s) * kQD;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 32 * b + 8 * g4 + 4 * h2 + e;  // pair (n, n + 64)
        float x1 = acc[b][4 * g4 + e] * rn, x2 = acc[b + 2][4 * g4 + e] * rn;
        if (a.k_gamma) {
          x1 *= a.k_gamma[n];
          x2 *= a.k_gamma[n + 64];
        }
        float sn, cs;
        rope_sincos(pos, rt.rev[n], sn, cs);
        y1[e] = x1 * cs - x2 * sn;
        y2[e] = x1 * sn + x2 * cs;
      }
      const int n = 32 * b + 8 * g4 + 4 * h2;
      *(u32x2*)(dst + n) = u32x2{pack2(y1[0], y1[1]), pack2(y1[2], y1[3])};
      *(u32x2*)(dst + n + 64) = u32x2{pack2(y2[0], y2[1]), pack2(y2[2], y2[3])};
    }
}

// Key head at head dimension 256: the tile is one head; wave w holds
// features 128 (w & 1) .. + 127 for its 64 tokens, so the norm's sum and the
// RoPE pairs (d, d + 128) span the two waves of a token group.  Each 32-token
// block goes through LDS: every wave writes its sum of squares and its fp32
// values (feature-major, 128 x 32 floats), then reads its partner's.  Called
// by every wave of the workgroup (it holds barriers).
__device__ __forceinline__ void store_key_rows_d256(const QkvArgs& a, const Pos0Table& p0t, const RopeTable& rt,
                                                    f32x16 (&acc)[2][4], int head, int t0, int wave, int h2, int ln,
                                                    float* xbuf, float* sbuf) {
  const int wf = wave & 1, wt = wave >> 1, partner = wave ^ 1;
  float* mine = xbuf + wave * (128 * 32);
  const float* theirs = xbuf + partner * (128 * 32);
  __syncthreads();  // every wave is done with the operand stages that xbuf reuses
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 64 * wt + 32 * j + ln;
    float ss = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = 32 * b + 8 * (r / 4) + 4 * h2 + r % 4;
        ss += acc[j][b][r] * acc[j][b][r];
        mine[n * 32 + ln] = acc[j][b][r];
      }
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
      ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (h2 == 0) sbuf[wave * 32 + ln] = ss;
    __syncthreads();
    const float tot = ss + sbuf[partner * 32 + ln];
    const float rn = a.k_gamma ? __frsqrt_rn(tot * (1.f / 256.f) + a.eps) : 1.f;
    if (t < a.T) {
      const int bt = t / a.S, s = t - bt * a.S;
      const int pos = pos0_of(p0t, bt) + s;
      uint16_t* dst = a.khat + (((long long)bt * a.Hkv + (head - a.Hq)) * a.S + s) * 256 + 128 * wf;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = 32 * b + 8 * g4 + 4 * h2 + e;  // pair (n, n + 128); this wave holds n + 128 wf
            float xo = acc[j][b][4 * g4 + e] * rn, xp = theirs[n * 32 + ln] * rn;
            if (a.k_gamma) {
              xo *= a.k_gamma[128 * wf + n];
              xp *= a.k_gamma[128 * (wf ^ 1) + n];
            }
            float sn, cs;
            rope_sincos(pos, rt.rev[n], sn, cs);
            y[e] = wf == 0 ? xo * cs - xp * sn : xp * sn + xo * cs;
          }
          const int n = 32 * b + 8 * g4 + 4 * h2;
          *(u32x2*)(dst + n) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
        }
    }
    __syncthreads();  // the partner has read this block before the next one overwrites it
  }
}

}  // namespace

__global__ __launch_bounds__(512, 1) void qkv_proj(QkvArgs a, Pos0Table p0t, RopeTable rt) {
  __shared__ __attribute__((aligned(1024))) char lds[kQStages * kQStageB];
  qlds_char* const ldsp = (qlds_char*)lds;
  const uint32_t lds0 = (uint32_t)(uintptr_t)ldsp;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, ln = lane & 31;
  const int wf = wave & 1, wt = wave >> 1;
  const int t0 = blockIdx.x * kQT;
  const int f0 = blockIdx.y * kQF;  // first weight row of the tile
  const int K = a.K;
  const int n_chunks = K / kQC;
  const int last = n_chunks - 1;
  const int n_rows = (a.Hq + 2 * a.Hkv) * a.D;

  // loads: load k = wave + 4 j (the W tile for k < 16, else the X tile)
  // fills LDS pieces P = 64 (k mod 16) + lane of its tile: row P / 4, slot
  // P % 4, which holds input piece (P % 4) ^ sw(row).  Rows past the end
  // (tokens, or the missing second head of an odd head count) re-read the
  // last row and are never stored.
  uint32_t off[kQLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kQLoadsPerWave; ++j) {
    const int k = wave + kQWaves * j;
    const bool is_x = k >= 16;
    const int P = 64 * (k & 15) + lane;
    const int r = P >> 2;
    const int g = (P & 3) ^ qswz(r);
    const int row = min(r, is_x ? a.T - 1 - t0 : n_rows - 1 - f0);
    off[j] = 2u * ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)g);
  }
  const uint16_t* wbase = a.w + (long long)f0 * K;
  const uint16_t* xbase = a.x + (long long)t0 * K;
  auto load_one = [&](int c, int stage, int j) __attribute__((always_inline)) {
    const int k = wave + kQWaves * j;
    const bool is_x = k >= 16;
    qdma(is_x ? (const void*)(xbase + c * kQC) : (const void*)(wbase + c * kQC), off[j],
         lds0 + stage * kQStageB + (is_x ? kQTileB : 0) + 1024 * (k & 15));
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][b][r] = 0.f;

  // operand addresses of step st (inputs 16 st .. 16 st + 15, lane half h2
  // = piece 2 st + h2): A = weight row 128 wf + 32 b + ln, B = token row
  // 128 wt + 32 j + ln; sw depends on ln only, blocks add 2048 bytes
  uint32_t aaddr[2], baddr[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int slot = (2 * st + h2) ^ qswz(ln);
    aaddr[st] = lds0 + (128 * wf + ln) * 64 + 16 * slot;
    baddr[st] = lds0 + kQTileB + (64 * wt + ln) * 64 + 16 * slot;
  }
  auto read_ops = [&](int st, int stage, bf16x8 (&ra)[4], bf16x8 (&rb)[2]) __attribute__((always_inline)) {
    const qlds_char* ap = (qlds_char*)(uintptr_t)(aaddr[st] + stage * kQStageB);
    const qlds_char* bp = (qlds_char*)(uintptr_t)(baddr[st] + stage * kQStageB);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *(qlds_bf16x8*)(ap + 2048 * i);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = *(qlds_bf16x8*)(bp + 2048 * i);
  };

  // four chunks in flight before the loop; every chunk issues one more
  // (past the last chunk the loads re-read the last one into a stage nobody
  // reads), so the count of loads in flight is the same on every path
#pragma unroll
  for (int c = 0; c < kQStages; ++c)
#pragma unroll
    for (int j = 0; j < kQLoadsPerWave; ++j) load_one(min(c, last), c, j);
  asm volatile("s_waitcnt vmcnt(12)" ::: "memory");  // this wave's loads of chunk 0
  qbarrier();
  bf16x8 a0[4], b0[2], a1[4], b1[2];
  read_ops(0, 0, a0, b0);
  int stage = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const int nstage = stage == 3 ? 0 : stage + 1;
    // step 0 of chunk c; read step 1 first so the reads land during the MFMAs
    read_ops(1, stage, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[j][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[b], b0[j], acc[j][b], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this wave's loads of chunk c + 1
    qbarrier();  // chunk c + 1 is in LDS for every wave; every read of chunk c has completed
    // step 1 of chunk c; read step 0 of chunk c + 1 and refill chunk c's
    // stage, one load after every other MFMA
    read_ops(0, nstage, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    const int cl = min(c + kQStages, last);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = i >> 2, b = i & 3;
      acc[j][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[b], b1[j], acc[j][b], 0, 0, 0);
      if (i & 1) load_one(cl, stage, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = nstage;
  }
  // no global->LDS load may still be landing when the workgroup's LDS is
  // released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // the input norm's per-token scale, when its gamma is folded into w: the
  // projections of token t are x[t] w^T times x_scale[t]
  if (a.x_scale) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = min(t0 + 64 * wt + 32 * j + ln, a.T - 1);
      const float sc = a.x_scale[t];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][b][r] *= sc;
    }
  }

  if (a.D == 256) {  // one head per tile, wave w holds its features 128 (w & 1) ..
    const int head = blockIdx.y;
    if (head >= a.Hq && head < a.Hq + a.Hkv) {
      __shared__ float sbuf[kQWaves * 32];
      store_key_rows_d256(a, p0t, rt, acc, head, t0, wave, h2, ln, (float*)lds, sbuf);
      return;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = t0 + 64 * wt + 32 * j + ln;
      if (t < a.T) store_plain_rows(a, acc[j], head, t, h2, 128 * wf);
    }
    return;
  }
  const int head = blockIdx.y * 2 + wf;
  if (head >= a.Hq + 2 * a.Hkv) return;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 64 * wt + 32 * j + ln;
    if (t < a.T) store_head_rows(a, p0t, rt, acc[j], head, t, h2);
  }
}

hipError_t launch_qkv_proj(const QkvArgs& a, const Pos0Table& p0t, const RopeTable& rt, hipStream_t st) {
  const int heads = a.Hq + 2 * a.Hkv;
  const dim3 grid((a.T + kQT - 1) / kQT, a.D == 256 ? heads : (heads + 1) / 2);
  hipLaunchKernelGGL(qkv_proj, grid, dim3(64 * kQWaves), 0, st, a, p0t, rt);
  return hipGetLastError();
}

}  // namespace g3
