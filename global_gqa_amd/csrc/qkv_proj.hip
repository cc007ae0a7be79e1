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
// Design (workgroup = 8 waves; tile = two heads' 256 output features x 256
// tokens; grid = (token tiles, head pairs)):
//   * C^T = W X^T with v_mfma_f32_32x32x16_bf16: A = 32 weight rows x 16
//     inputs, B = 32 token rows x 16 inputs, both contiguous along the input
//     dimension.  Wave w computes head 2 p + (w & 1) for tokens
//     64 (w >> 1) .. 64 (w >> 1) + 63: 2 x 4 accumulator blocks, so each
//     16-input step reads 6 operand fragments from LDS for 8 MFMAs.  In the
//     epilogue each lane holds one token's 64 features of the head and the
//     token's other 64 sit in the lane 32 apart: the RMSNorm is an in-lane
//     sum plus one cross-half swap, and the RoPE pairs (d, d + 64) are in
//     the same lane;
//   * 64-input chunks of W and X in LDS, double-buffered (2 x 72 KiB), rows
//     padded to 144 B (conflict-free ds_read_b128, operand reads at immediate
//     offsets), filled by global->LDS loads whose per-lane source offsets are
//     fixed for the whole loop and computed once.
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace g3 {

namespace {

constexpr int kQD = 128;                 // head dimension
constexpr int kQT = 256;                 // tokens per tile
constexpr int kQF = 256;                 // output features per tile (two heads)
constexpr int kQC = 64;                  // inputs per chunk
constexpr int kQRow = 9;                 // row stride in 16-byte pieces (128 B data + 16 B pad)
constexpr int kQLoads = 36;              // 1 KiB loads per 256-row operand tile (256 x 9 pieces)
constexpr int kQTileB = kQLoads * 1024;  // 36864 bytes
constexpr int kQStageB = 2 * kQTileB;    // W tile then X tile
constexpr int kQWaves = 8;
constexpr int kQLoadsPerWave = 2 * kQLoads / kQWaves;  // 9

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
// __syncthreads would also wait for the next chunk's loads in flight).
__device__ __forceinline__ void qbarrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Epilogue of one 32-token block of one head: lane (ln, h2) holds token t's
// features n = 32 b + 8 (r / 4) + 4 h2 + r % 4 in acc[b][r], b = 0..3.
__device__ __forceinline__ void store_head_rows(const QkvArgs& a, const Pos0Table& p0t, const RopeTable& rt,
                                                const f32x16* acc, int head, int t, int h2) {
  if (head < a.Hq || head >= a.Hq + a.Hkv) {
    uint16_t* dst = head < a.Hq ? a.q + ((long long)t * a.Hq + head) * kQD
                                : a.v + ((long long)t * a.Hkv + (head - a.Hq - a.Hkv)) * kQD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = 32 * b + 8 * g4 + 4 * h2;
        *(u32x2*)(dst + n) = u32x2{pack2(acc[b][4 * g4], acc[b][4 * g4 + 1]),
                                   pack2(acc[b][4 * g4 + 2], acc[b][4 * g4 + 3])};
      }
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

}  // namespace

__global__ __launch_bounds__(512, 1) void qkv_proj(QkvArgs a, Pos0Table p0t, RopeTable rt) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kQStageB];
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
  const int n_rows = (a.Hq + 2 * a.Hkv) * kQD;

  // per-lane source offsets of this wave's 9 loads (load k = wave + 8 j: the
  // W tile for k < 36, else the X tile); piece n = 64 (k mod 36) + lane is
  // (row n / 9, 16-byte piece n % 9); the pad piece re-reads piece 0; rows
  // past the end (tokens, or the missing second head of an odd head count)
  // re-read the last row (never stored)
  uint32_t off[kQLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kQLoadsPerWave; ++j) {
    const int k = wave + kQWaves * j;
    const bool is_x = k >= kQLoads;
    const int n = 64 * (is_x ? k - kQLoads : k) + lane;
    int row = n / kQRow;
    int pc = n - row * kQRow;
    if (pc == 8) pc = 0;
    row = min(row, is_x ? a.T - 1 - t0 : n_rows - 1 - f0);
    off[j] = 2u * ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)pc);
  }
  const uint16_t* wbase = a.w + (long long)f0 * K;
  const uint16_t* xbase = a.x + (long long)t0 * K;
  auto load_stage = [&](int c, int buf) __attribute__((always_inline)) {
    const uint32_t dst0 = lds0 + buf * kQStageB;
#pragma unroll
    for (int j = 0; j < kQLoadsPerWave; ++j) {
      const int k = wave + kQWaves * j;
      const bool is_x = k >= kQLoads;
      qdma(is_x ? (const void*)(xbase + c * kQC) : (const void*)(wbase + c * kQC), off[j],
           dst0 + (is_x ? kQTileB + 1024 * (k - kQLoads) : 1024 * k));
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][b][r] = 0.f;

  // operand bases in a stage: A = weight row 128 wf + 32 b + ln, B = token
  // row 64 wt + 32 j + ln, piece 2 st + h2 (+32 rows per block and +2 st
  // pieces as immediates)
  const uint32_t abase = lds0 + (128 * wf + ln) * (16 * kQRow) + 16 * h2;
  const uint32_t bbase = lds0 + kQTileB + (64 * wt + ln) * (16 * kQRow) + 16 * h2;

  load_stage(0, 0);
  if (n_chunks > 1) load_stage(1, 1);
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < n_chunks)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    qbarrier();  // chunk c is in LDS (this wave's loads waited above)
    const qlds_char* ap = (qlds_char*)(uintptr_t)(abase + buf * kQStageB);
    const qlds_char* bp = (qlds_char*)(uintptr_t)(bbase + buf * kQStageB);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 bx[2], aw[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) bx[j] = *(qlds_bf16x8*)(bp + 32 * j * 16 * kQRow + 32 * st);
#pragma unroll
      for (int b = 0; b < 4; ++b) aw[b] = *(qlds_bf16x8*)(ap + 32 * b * 16 * kQRow + 32 * st);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[j][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[b], bx[j], acc[j][b], 0, 0, 0);
    }
    qbarrier();  // every wave is done with this buffer
    if (c + 2 < n_chunks) load_stage(c + 2, buf);
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
  const dim3 grid((a.T + kQT - 1) / kQT, (a.Hq + 2 * a.Hkv + 1) / 2);
  hipLaunchKernelGGL(qkv_proj, grid, dim3(64 * kQWaves), 0, st, a, p0t, rt);
  return hipGetLastError();
}

}  // namespace g3
