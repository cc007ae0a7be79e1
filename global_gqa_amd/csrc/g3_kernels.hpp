// Kernel argument blocks and host launchers shared by the kernels and the
// C-ABI layer.  Pointers are device pointers; all tensors are bf16 (as
// uint16_t) unless noted.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "g3_common.hpp"

namespace g3 {

// Rows of QK-RMSNorm + RoPE: T tokens x H heads, input [T][H][D].
struct RowsArgs {
  const uint16_t* in;
  uint16_t* out;          // [T][H][D], or head-major [T/S][H][S][D]
  const float* gamma;     // fp32 [D] or null (no norm)
  const int32_t* positions;  // device [T] or null: position = pos0[t / S] + t % S
  float eps;
  int T, H, S;            // S: tokens per sequence (for pos0 and head-major)
  int head_major;
  int D;                  // head dimension (128 or 256)
};

// Heads of one token each K1 lane group normalises and rotates (their
// rotation angles are the same, so sin/cos are computed once per group).
constexpr int kRopeHeadsPerGroup = 4;

struct AppendArgs {
  const uint16_t* khat;   // [B][Hkv][S][D]
  const uint16_t* v;      // [B][S][Hkv][D]
  uint16_t* ck;           // [B][Hkv][cap][D]
  uint16_t* cv;
  int B, S, Hkv, cap, is_ring;
  int D;
};

struct PrefillArgs {
  const uint16_t* q;      // [B][S][Hq][D] raw
  const uint16_t* khat;   // [B][Hkv][S][D] normed + rotated chunk keys
  const uint16_t* v;      // [B][S][Hkv][D] raw chunk values
  const uint16_t* ck;     // cache [B][Hkv][cap][D] (null: no cache)
  const uint16_t* cv;
  uint16_t* o;            // [B][S][Hq][D]
  const float* q_gamma;   // fp32 [D] or null
  int* flags;             // [grid] per-workgroup "redo with the online maximum" flags
  float eps;
  int B, S, Hq, Hkv;
  int cap, is_ring, has_cache;
  int local, window;
  float sl2;              // softmax_scale * log2(e)
  int n_qtiles;
};

struct DecodeArgs {
  const uint16_t* q;      // [B][Hq][D] raw
  const uint16_t* k_new;  // [B][Hkv][D] raw
  const uint16_t* v_new;  // [B][Hkv][D] raw
  uint16_t* ck;           // [B][Hkv][cap][D]
  uint16_t* cv;
  const int32_t* positions;  // device [B]
  const float* q_gamma;
  const float* k_gamma;
  float* ws;              // [B][Hq][n_chunks][D + 2] partials (o, m, l)
  int D;                  // head dimension (128 or 256)
  uint16_t* o;            // [B][Hq][D]
  float eps;
  int B, Hq, Hkv, cap, is_ring, local, window;
  int max_pos;            // clamp bound for positions
  int n_slots;            // cache slots scanned
  int split;              // cache slots per split-K workgroup (multiple of 16)
  int n_chunks;           // number of splits
  float sl2;
};

// Fused QKV projection (head dimension 128): W is [Hq + 2 Hkv][128][K]
// (the q, k and v weight matrices stacked, rows = output features), x is
// [T][K] with T = B S tokens.  With Hkv = 0 the kernel is a plain GEMM
// q = x W^T whose [T][Hq][128] output is a row-major [T][128 Hq] (o_proj);
// khat, v, k_gamma and the position/rotation tables are then unused.
struct QkvArgs {
  const uint16_t* x;      // [T][K]
  const uint16_t* w;      // [(Hq + 2 Hkv) * 128][K]
  uint16_t* q;            // [T][Hq][128] raw
  uint16_t* khat;         // [B][Hkv][S][128] normed + rotated
  uint16_t* v;            // [T][Hkv][128] raw
  const float* k_gamma;   // fp32 [D] or null (no norm)
  const float* x_scale;   // fp32 [T] or null: token t's projections are multiplied by x_scale[t]
  float eps;
  int T, S, K, Hq, Hkv;
  int D;                  // head dimension: 128, or 256 (one head per 256-feature tile)
};

// Row RMSNorm over the model width with an optional residual add.
struct NormArgs {
  const uint16_t* x;         // [T][W]
  const uint16_t* residual;  // [T][W] or null
  const float* gamma;        // fp32 [W] or null (gamma = 1)
  uint16_t* out;             // [T][W]; may alias x or residual
  float eps;
  int T, W;                  // W: multiple of 8, at most rmsnorm_max_width()
};

constexpr int kDecodeChunk = 256;  // granularity of split-K decode splits (slots)
// Size of the per-GPU static array behind the decode entry point that
// allocates nothing (G3_DECODE_NOALLOC_MAX_BYTES in the C header).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

hipError_t launch_qknorm_rope(const RowsArgs& a, const Pos0Table& p0t, const RopeTable& rt, hipStream_t st);
hipError_t launch_append_chunk(const AppendArgs& a, const Pos0Table& p0t, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt, const RopeTable& rt,
                          int G, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
// Head dimension 256 (Gemma 3 1B): 8 waves x 32 query rows per workgroup.
hipError_t launch_prefill_d256(const PrefillArgs& a, const Pos0Table& p0t, const SpanTable& spt,
                               const RopeTable& rt, int G, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_qkv_proj(const QkvArgs& a, const Pos0Table& p0t, const RopeTable& rt, hipStream_t st);
hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t st);
int rmsnorm_max_width();
// scale[t] = 1 / sqrt(mean(x[t]^2) + eps) for the rows of a.x (a.out, a.gamma
// and a.residual unused).
hipError_t launch_rms_scale(const NormArgs& a, float* scale, hipStream_t st);
// out[n][k] = w[n][k] * gamma[k], rounded to bf16 ([rows][width]).
hipError_t launch_fold_gamma(const uint16_t* w, const float* gamma, uint16_t* out, long long rows, int width,
                             hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, const RopeTable& rt, int G, hipStream_t st, hipEvent_t ev_start,
                         hipEvent_t ev_stop);
// Address, on the current device, of the static split-K partials array
// (kDecodeScratchBytes); looked up once per device.
hipError_t decode_scratch(void** ptr);

// Flash prefill: waves per workgroup (each wave owns 32 query rows).
#ifndef G3_PREFILL_WAVES
#define G3_PREFILL_WAVES 8
#endif
constexpr int kPrefillWaves = G3_PREFILL_WAVES;
// Tiles: positions per prefill workgroup for a GQA group of size G.
inline int prefill_rows_per_wg(int G) { return kPrefillWaves * (32 / G); }
constexpr int kPrefillWavesD256 = 8;
inline int prefill_rows_per_wg_d256(int G) { return kPrefillWavesD256 * (32 / G); }

}  // namespace g3
