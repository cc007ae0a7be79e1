// C-ABI layer of libg3attn: argument validation, workspace layout and kernel
// launches.  Every check runs before the first launch, so a rejected call has
// no side effects.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/g3attn.h"
#include "g3_common.hpp"
#include "g3_kernels.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int32_t D) { return D == 128 || D == 256; }

int check_heads(int32_t Hq, int32_t Hkv, int32_t D) {
  if (!head_dim_ok(D)) return fail(G3_EUNSUPPORTED, "head dim D=%d not supported (128 or 256)", D);
  if (Hq <= 0 || Hkv <= 0) return fail(G3_EINVAL, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv) return fail(G3_EINVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(G3_EUNSUPPORTED, "GQA group size Hq/Hkv=%d not supported (1, 2, 4 or 8)", G);
  return G3_OK;
}

int check_rope(float rope_base, float interp_scale, float eps) {
  if (!(rope_base > 1.0f) || !std::isfinite(rope_base)) return fail(G3_EINVAL, "rope_base must be > 1 (got %g)", rope_base);
  if (!(interp_scale > 0.0f) || !std::isfinite(interp_scale))
    return fail(G3_EINVAL, "interp_scale must be > 0 (got %g)", interp_scale);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(G3_EINVAL, "eps must be >= 0 (got %g)", eps);
  return G3_OK;
}

int check_scale(float softmax_scale, int32_t D, float* sl2) {
  if (softmax_scale < 0.0f || !std::isfinite(softmax_scale))
    return fail(G3_EINVAL, "softmax_scale must be >= 0 (0 = D^-1/2), got %g", softmax_scale);
  const float s = softmax_scale == 0.0f ? 1.0f / std::sqrt((float)D) : softmax_scale;
  *sl2 = s * 1.4426950408889634f;
  return G3_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// RoPE frequencies base^(-2k/D), in revolutions per (interpolated) position.
g3::RopeTable rope_table(float base, float interp_scale, int D) {
  g3::RopeTable t{};
  const double inv2pi = 0.15915494309189533576888376337251;
  for (int k = 0; k < D / 2; ++k)
    t.rev[k] = std::pow((double)base, -2.0 * k / D) * inv2pi / (double)interp_scale;
  return t;
}

// Prefill workspace: normed+rotated chunk keys [B][Hkv][S][D] bf16, then one
// int32 flag per flash work item, sized for the most items any group size
// can give (G = 8 query heads per kv head).
size_t prefill_ws_keys(int32_t B, int32_t S, int32_t Hkv, int32_t D) {
  return round_up((size_t)B * Hkv * S * D * sizeof(uint16_t), 256);
}
size_t prefill_ws(int32_t B, int32_t S, int32_t Hkv, int32_t D) {
  const int rows1 = D == 256 ? g3::prefill_rows_per_wg_d256(1) : g3::prefill_rows_per_wg(1);
  const size_t tiles = (size_t)B * Hkv * ((S + rows1 - 1) / rows1) * (size_t)8;
  return prefill_ws_keys(B, S, Hkv, D) + round_up(tiles * sizeof(int32_t), 256);
}

int decode_slots(const g3_kv_cache* c, int32_t max_position) {
  if (c->is_ring) return c->capacity;
  const long long n = (long long)max_position + 1;
  return (int)(n < c->capacity ? n : c->capacity);
}

// Split-K shape: splits of 256 * k slots with k chosen so the grid has about
// 2048 workgroups (8 per CU) and each keeps its loads streaming long enough
// (a single 128K-position sequence: 128 splits of 1024 slots per kv head
// measured 10% faster than 256 of 512; 32 sequences of 32K hit the cap of
// 16 units either way).
// Short caches (a local layer's 1024-slot ring) with at least 512 (sequence,
// kv head) pairs take one split each: enough workgroups, and no merge pass.
// With fewer pairs than that a one-unit split can leave most CUs idle (the
// 1B model's 32 sequences x 1 kv head: 128 workgroups on a 1024-slot ring,
// each latency-bound), so the split halves, down to 64 slots, until the grid
// has about one workgroup per CU.  More, shorter splits cost more than they
// give: every workgroup adds to the dispatch and its prologue and merge are
// fixed costs (the 1B ring: 256 workgroups of 128 slots 15.9 us per layer,
// 512 of 64 slots 17.2 us).
int decode_split(int n_slots, int32_t B, int32_t Hkv) {
  const int n_units = (n_slots + g3::kDecodeChunk - 1) / g3::kDecodeChunk;
  const long long pairs = (long long)B * Hkv;
  if (n_units <= 16 && pairs >= 512) return n_units * g3::kDecodeChunk;
  const long long units = (long long)n_units * pairs;
  long long k = units / 2048;
  if (k < 1) k = 1;
  if (k > 16) k = 16;
  int split = (int)k * g3::kDecodeChunk;
  while (split > 64 && (long long)((n_slots + split - 1) / split) * pairs < 256) split /= 2;
  return split;
}
int decode_chunks(int n_slots, int32_t B, int32_t Hkv) {
  const int split = decode_split(n_slots, B, Hkv);
  return (n_slots + split - 1) / split;
}

size_t decode_ws(int32_t B, int32_t Hq, int32_t D, int n_chunks) {
  return round_up((size_t)B * Hq * n_chunks * (D + 2) * sizeof(float), 256);
}

// Per-sequence first positions (NULL: all 0) as the kernels' table.
int make_pos0(const int32_t* pos0, int32_t B, int32_t S, g3::Pos0Table* out) {
  g3::Pos0Table& p0t = *out;
  p0t = g3::Pos0Table{};
  p0t.uniform = 1;
  p0t.v[0] = 0;
  if (pos0) {
    bool uni = true;
    for (int b = 0; b < B; ++b) {
      if (pos0[b] < 0) return fail(G3_EINVAL, "pos0[%d]=%d < 0", b, pos0[b]);
      if ((long long)pos0[b] + S > (1LL << 30)) return fail(G3_EINVAL, "pos0[%d]+S out of range", b);
      if (pos0[b] != pos0[0]) uni = false;
    }
    if (!uni && B > g3::kMaxBatchPos0)
      return fail(G3_EUNSUPPORTED, "per-sequence pos0 supports at most %d sequences", g3::kMaxBatchPos0);
    p0t.uniform = uni ? 1 : 0;
    if (uni)
      p0t.v[0] = pos0[0];
    else
      for (int b = 0; b < B; ++b) p0t.v[b] = pos0[b];
  }
  return G3_OK;
}

}  // namespace

extern "C" {

const char* g3attn_last_error(void) { return g_err; }

int32_t g3attn_version(void) { return 101; }

int g3attn_set_timing_events(void* start, void* stop) {
  g_ev_start = (hipEvent_t)start;
  g_ev_stop = (hipEvent_t)stop;
  if ((start == nullptr) != (stop == nullptr)) {
    g_ev_start = g_ev_stop = nullptr;
    return fail(G3_EINVAL, "timing events must both be set or both be NULL");
  }
  return G3_OK;
}

int g3attn_qknorm_rope(const g3_bf16* q_in, const g3_bf16* k_in, g3_bf16* q_out, g3_bf16* k_out,
                       const float* q_gamma, const float* k_gamma, float eps, const int32_t* positions,
                       int32_t T, int32_t Hq, int32_t Hkv, int32_t D, float rope_base, float interp_scale,
                       void* stream) {
  g_err[0] = 0;
  if (!head_dim_ok(D)) return fail(G3_EUNSUPPORTED, "head dim D=%d not supported (128 or 256)", D);
  if (T < 0) return fail(G3_EINVAL, "T=%d < 0", T);
  if ((q_in == nullptr) != (q_out == nullptr)) return fail(G3_EINVAL, "q_in and q_out must both be set or NULL");
  if ((k_in == nullptr) != (k_out == nullptr)) return fail(G3_EINVAL, "k_in and k_out must both be set or NULL");
  if (q_in && Hq <= 0) return fail(G3_EINVAL, "Hq=%d must be positive", Hq);
  if (k_in && Hkv <= 0) return fail(G3_EINVAL, "Hkv=%d must be positive", Hkv);
  if (int e = check_rope(rope_base, interp_scale, eps)) return e;
  if (T > 0 && positions == nullptr) return fail(G3_EINVAL, "positions is NULL");
  for (const void* p : {(const void*)q_in, (const void*)k_in, (const void*)q_out, (const void*)k_out})
    if (p && !aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  if (T == 0) return G3_OK;
  hipStream_t st = (hipStream_t)stream;
  g3::Pos0Table p0t{};
  p0t.uniform = 1;
  for (int which = 0; which < 2; ++which) {
    const g3_bf16* in = which ? k_in : q_in;
    g3_bf16* out = which ? k_out : q_out;
    if (!in) continue;
    g3::RowsArgs a{};
    a.in = in;
    a.out = out;
    a.gamma = which ? k_gamma : q_gamma;
    a.positions = positions;
    a.eps = eps;
    a.T = T;
    a.H = which ? Hkv : Hq;
    a.S = T;
    a.head_major = 0;
    a.D = D;
    if (hipError_t e = g3::launch_qknorm_rope(a, p0t, rope_table(rope_base, interp_scale, D), st))
      return fail(G3_EHIP, "qknorm_rope launch failed: %s", hipGetErrorString(e));
  }
  return G3_OK;
}

size_t g3attn_prefill_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D) {
  (void)Hq;
  if (B <= 0 || S <= 0 || Hkv <= 0 || D <= 0) return 0;
  return prefill_ws(B, S, Hkv, D);
}

}  // extern "C"

namespace {

// Prefill of one chunk.  With khat_in == NULL the keys k are normed and
// rotated into the workspace first; otherwise khat_in already holds them
// (head-major) and the workspace only carries the flash kernel's flags.
int prefill_impl(const g3_bf16* q, const g3_bf16* k, const g3_bf16* khat_in, const g3_bf16* v, g3_bf16* o,
                 int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t layer_kind, int32_t window,
                 float rope_base, float interp_scale, const float* q_gamma, const float* k_gamma, float eps,
                 float softmax_scale, const g3_span* spans, int32_t n_spans, const int32_t* pos0,
                 const g3_kv_cache* cache, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (int e = check_heads(Hq, Hkv, D)) return e;
  if (B <= 0 || S <= 0) return fail(G3_EINVAL, "B=%d and S=%d must be positive", B, S);
  if (layer_kind != G3_LOCAL && layer_kind != G3_GLOBAL) return fail(G3_EINVAL, "layer_kind=%d", layer_kind);
  if (layer_kind == G3_LOCAL && window < 1) return fail(G3_EINVAL, "window=%d < 1", window);
  if (int e = check_rope(rope_base, interp_scale, eps)) return e;
  float sl2;
  if (int e = check_scale(softmax_scale, D, &sl2)) return e;
  const g3_bf16* kk = khat_in ? khat_in : k;
  if (!q || !kk || !v || !o) return fail(G3_EINVAL, "q, %s, v and o must be non-NULL", khat_in ? "khat" : "k");
  for (const void* p : {(const void*)q, (const void*)kk, (const void*)v, (const void*)o})
    if (!aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  if ((long long)B * S * Hq > (1LL << 31) - 1) return fail(G3_EINVAL, "B*S*Hq too large");
  if ((long long)S * Hkv * D > (1LL << 31) - 1)
    return fail(G3_EUNSUPPORTED, "S*Hkv*D=%lld exceeds the 32-bit row offsets of one sequence",
                (long long)S * Hkv * D);

  g3::Pos0Table p0t;
  if (int e = make_pos0(pos0, B, S, &p0t)) return e;
  auto P0 = [&](int b) { return pos0 ? pos0[b] : 0; };

  g3::SpanTable spt{};
  if (n_spans < 0 || n_spans > g3::kMaxSpans) return fail(G3_EINVAL, "n_spans=%d (0..%d)", n_spans, g3::kMaxSpans);
  if (n_spans > 0 && !spans) return fail(G3_EINVAL, "spans is NULL with n_spans=%d", n_spans);
  spt.n = n_spans;
  for (int i = 0; i < n_spans; ++i) {
    const g3_span s = spans[i];
    if (s.batch < 0 || s.batch >= B) return fail(G3_EINVAL, "span %d: batch %d out of range", i, s.batch);
    if (s.start >= s.end) return fail(G3_EINVAL, "span %d: empty or reversed [%d, %d)", i, s.start, s.end);
    if (s.start < P0(s.batch) || s.end > P0(s.batch) + S)
      return fail(G3_EINVAL, "span %d: [%d, %d) outside the chunk of sequence %d", i, s.start, s.end, s.batch);
    if (i > 0) {
      const g3_span p = spans[i - 1];
      if (p.batch > s.batch || (p.batch == s.batch && p.end > s.start))
        return fail(G3_EINVAL, "spans must be sorted by (batch, start) and non-overlapping (span %d)", i);
    }
    spt.s[i] = g3::Span{s.batch, s.start, s.end};
  }

  if (cache) {
    if (!cache->k || !cache->v) return fail(G3_EINVAL, "cache k/v pointers are NULL");
    if (!aligned16(cache->k) || !aligned16(cache->v)) return fail(G3_EINVAL, "cache pointers must be 16-byte aligned");
    if (cache->capacity <= 0) return fail(G3_EINVAL, "cache capacity %d", cache->capacity);
    if (cache->is_ring) {
      if (layer_kind != G3_LOCAL) return fail(G3_EINVAL, "a ring cache needs a local layer");
      if (window > cache->capacity) return fail(G3_EINVAL, "window %d exceeds ring capacity %d", window, cache->capacity);
    } else {
      for (int b = 0; b < B; ++b)
        if ((long long)P0(b) + S > cache->capacity)
          return fail(G3_EINVAL, "linear cache capacity %d < pos0[%d]+S=%lld", cache->capacity, b, (long long)P0(b) + S);
    }
  }
  const size_t need = prefill_ws(B, S, Hkv, D);
  if (!workspace || workspace_bytes < need)
    return fail(G3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(G3_EINVAL, "workspace must be 256-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  const uint16_t* khat = khat_in ? khat_in : (const uint16_t*)workspace;
  const g3::RopeTable rt = rope_table(rope_base, interp_scale, D);
  if (!khat_in) {
    g3::RowsArgs a{};
    a.in = k;
    a.out = (uint16_t*)workspace;
    a.gamma = k_gamma;
    a.positions = nullptr;
    a.eps = eps;
    a.T = B * S;
    a.H = Hkv;
    a.S = S;
    a.head_major = 1;
    a.D = D;
    if (hipError_t e = g3::launch_qknorm_rope(a, p0t, rt, st))
      return fail(G3_EHIP, "k prologue launch failed: %s", hipGetErrorString(e));
  }
  const int G = Hq / Hkv;
  g3::PrefillArgs a{};
  a.q = q;
  a.khat = khat;
  a.v = v;
  a.ck = cache ? cache->k : nullptr;
  a.cv = cache ? cache->v : nullptr;
  a.o = o;
  a.q_gamma = q_gamma;
  a.flags = (int*)((char*)workspace + (khat_in ? 0 : prefill_ws_keys(B, S, Hkv, D)));
  a.eps = eps;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.cap = cache ? cache->capacity : 0;
  a.is_ring = cache ? cache->is_ring : 0;
  a.has_cache = cache ? 1 : 0;
  a.local = layer_kind == G3_LOCAL;
  // a window past any position reach means no band limit; clamped so the
  // kernels' i + window - 1 cannot overflow
  a.window = layer_kind == G3_LOCAL ? (window < (1 << 30) ? window : (1 << 30)) : (1 << 30);
  a.sl2 = sl2;
  const int rows = D == 256 ? g3::prefill_rows_per_wg_d256(G) : g3::prefill_rows_per_wg(G);
  a.n_qtiles = (S + rows - 1) / rows;
  if ((long long)B * Hkv * a.n_qtiles > (1LL << 31) - 1) return fail(G3_EINVAL, "grid too large");
  const hipError_t le = D == 256 ? g3::launch_prefill_d256(a, p0t, spt, rt, G, st, g_ev_start, g_ev_stop)
                                 : g3::launch_prefill(a, p0t, spt, rt, G, st, g_ev_start, g_ev_stop);
  if (le != hipSuccess) return fail(G3_EHIP, "prefill launch failed: %s", hipGetErrorString(le));
  if (cache) {
    g3::AppendArgs ap{};
    ap.khat = khat;
    ap.v = v;
    ap.ck = cache->k;
    ap.cv = cache->v;
    ap.B = B;
    ap.S = S;
    ap.Hkv = Hkv;
    ap.cap = cache->capacity;
    ap.is_ring = cache->is_ring;
    ap.D = D;
    if (hipError_t e = g3::launch_append_chunk(ap, p0t, st))
      return fail(G3_EHIP, "cache append launch failed: %s", hipGetErrorString(e));
  }
  return G3_OK;
}

}  // namespace

extern "C" {

int g3attn_prefill(const g3_bf16* q, const g3_bf16* k, const g3_bf16* v, g3_bf16* o, int32_t B, int32_t S,
                   int32_t Hq, int32_t Hkv, int32_t D, int32_t layer_kind, int32_t window, float rope_base,
                   float interp_scale, const float* q_gamma, const float* k_gamma, float eps, float softmax_scale,
                   const g3_span* spans, int32_t n_spans, const int32_t* pos0, const g3_kv_cache* cache,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, nullptr, v, o, B, S, Hq, Hkv, D, layer_kind, window, rope_base, interp_scale, q_gamma,
                      k_gamma, eps, softmax_scale, spans, n_spans, pos0, cache, workspace, workspace_bytes, stream);
}

int g3attn_prefill_khat(const g3_bf16* q, const g3_bf16* khat, const g3_bf16* v, g3_bf16* o, int32_t B, int32_t S,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t layer_kind, int32_t window, float rope_base,
                        float interp_scale, const float* q_gamma, float eps, float softmax_scale,
                        const g3_span* spans, int32_t n_spans, const int32_t* pos0, const g3_kv_cache* cache,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!khat) {
    g_err[0] = 0;
    return fail(G3_EINVAL, "khat must be non-NULL");
  }
  return prefill_impl(q, nullptr, khat, v, o, B, S, Hq, Hkv, D, layer_kind, window, rope_base, interp_scale,
                      q_gamma, nullptr, eps, softmax_scale, spans, n_spans, pos0, cache, workspace, workspace_bytes,
                      stream);
}

int g3attn_o_project(const g3_bf16* attn, const g3_bf16* w_o, g3_bf16* y, int32_t T, int32_t in_features,
                     int32_t out_features, void* stream) {
  g_err[0] = 0;
  if (T <= 0) return fail(G3_EINVAL, "T=%d must be positive", T);
  if (in_features <= 0 || in_features % 64)
    return fail(G3_EUNSUPPORTED, "in_features=%d must be a positive multiple of 64", in_features);
  if (out_features <= 0 || out_features % 128)
    return fail(G3_EUNSUPPORTED, "out_features=%d must be a positive multiple of 128", out_features);
  if (out_features / 128 > 2 * 65535) return fail(G3_EINVAL, "out_features=%d too large", out_features);
  if (!attn || !w_o || !y) return fail(G3_EINVAL, "attn, w_o and y must be non-NULL");
  for (const void* p : {(const void*)attn, (const void*)w_o, (const void*)y})
    if (!aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  if ((long long)T > (1LL << 31) - 1 - 256) return fail(G3_EINVAL, "T too large");
  if (256LL * in_features * 2 > (1LL << 32) - 1) return fail(G3_EUNSUPPORTED, "in_features=%d too large", in_features);
  // the projection kernel with no key/value heads is a plain GEMM y = attn W_o^T
  // whose [T][out / 128][128] output is y's [T][out] layout
  g3::QkvArgs a{};
  a.x = attn;
  a.w = w_o;
  a.q = y;
  a.T = T;
  a.S = T;
  a.K = in_features;
  a.Hq = out_features / 128;
  a.Hkv = 0;
  a.D = 128;
  g3::Pos0Table p0t{};
  p0t.uniform = 1;
  g3::RopeTable rt{};
  hipStream_t st = (hipStream_t)stream;
  if (g_ev_start) hipEventRecord(g_ev_start, st);
  const hipError_t le = g3::launch_qkv_proj(a, p0t, rt, st);
  if (le != hipSuccess) return fail(G3_EHIP, "o projection launch failed: %s", hipGetErrorString(le));
  if (g_ev_stop) hipEventRecord(g_ev_stop, st);
  return G3_OK;
}

int g3attn_rmsnorm(const g3_bf16* x, const g3_bf16* residual, const float* gamma, float eps, g3_bf16* out, int32_t T,
                   int32_t width, void* stream) {
  g_err[0] = 0;
  if (T <= 0) return fail(G3_EINVAL, "T=%d must be positive", T);
  if (width <= 0 || width % 8 || width > g3::rmsnorm_max_width())
    return fail(G3_EUNSUPPORTED, "width=%d must be a positive multiple of 8 up to %d", width, g3::rmsnorm_max_width());
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(G3_EINVAL, "eps must be >= 0 (got %g)", eps);
  if (!x || !out) return fail(G3_EINVAL, "x and out must be non-NULL");
  for (const void* p : {(const void*)x, (const void*)residual, (const void*)out})
    if (p && !aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  g3::NormArgs a{};
  a.x = x;
  a.residual = residual;
  a.gamma = gamma;
  a.out = out;
  a.eps = eps;
  a.T = T;
  a.W = width;
  if (hipError_t e = g3::launch_rmsnorm(a, (hipStream_t)stream))
    return fail(G3_EHIP, "rmsnorm launch failed: %s", hipGetErrorString(e));
  return G3_OK;
}

int g3attn_rms_scale(const g3_bf16* x, float eps, float* scale, int32_t T, int32_t width, void* stream) {
  g_err[0] = 0;
  if (T <= 0) return fail(G3_EINVAL, "T=%d must be positive", T);
  if (width <= 0 || width % 8 || width > (1 << 20))
    return fail(G3_EUNSUPPORTED, "width=%d must be a positive multiple of 8 up to %d", width, 1 << 20);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(G3_EINVAL, "eps must be >= 0 (got %g)", eps);
  if (!x || !scale) return fail(G3_EINVAL, "x and scale must be non-NULL");
  if (!aligned16(x)) return fail(G3_EINVAL, "x must be 16-byte aligned");
  g3::NormArgs a{};
  a.x = x;
  a.eps = eps;
  a.T = T;
  a.W = width;
  if (hipError_t e = g3::launch_rms_scale(a, scale, (hipStream_t)stream))
    return fail(G3_EHIP, "rms scale launch failed: %s", hipGetErrorString(e));
  return G3_OK;
}

int g3attn_fold_norm_weight(const g3_bf16* w, const float* gamma, g3_bf16* w_out, int32_t rows, int32_t width,
                            void* stream) {
  g_err[0] = 0;
  if (rows <= 0) return fail(G3_EINVAL, "rows=%d must be positive", rows);
  if (width <= 0 || width % 8) return fail(G3_EUNSUPPORTED, "width=%d must be a positive multiple of 8", width);
  if (!w || !gamma || !w_out) return fail(G3_EINVAL, "w, gamma and w_out must be non-NULL");
  if (!aligned16(w) || !aligned16(w_out)) return fail(G3_EINVAL, "w and w_out must be 16-byte aligned");
  if (hipError_t e = g3::launch_fold_gamma(w, gamma, w_out, rows, width, (hipStream_t)stream))
    return fail(G3_EHIP, "weight fold launch failed: %s", hipGetErrorString(e));
  return G3_OK;
}

int g3attn_qkv_project(const g3_bf16* x, const float* x_scale, const g3_bf16* w, g3_bf16* q, g3_bf16* khat,
                       g3_bf16* v, int32_t B, int32_t S, int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D,
                       float rope_base, float interp_scale, const float* k_gamma, float eps, const int32_t* pos0,
                       void* stream) {
  g_err[0] = 0;
  if (D != 128 && D != 256) return fail(G3_EUNSUPPORTED, "qkv_project supports head dim 128 or 256 (got D=%d)", D);
  if (B <= 0 || S <= 0) return fail(G3_EINVAL, "B=%d and S=%d must be positive", B, S);
  if (Hq <= 0 || Hkv <= 0) return fail(G3_EINVAL, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (d_model <= 0 || d_model % 64)
    return fail(G3_EUNSUPPORTED, "d_model=%d must be a positive multiple of 64", d_model);
  if (int e = check_rope(rope_base, interp_scale, eps)) return e;
  if (!x || !w || !q || !khat || !v) return fail(G3_EINVAL, "x, w, q, khat and v must be non-NULL");
  for (const void* p : {(const void*)x, (const void*)w, (const void*)q, (const void*)khat, (const void*)v})
    if (!aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  const long long T = (long long)B * S;
  if (T * Hq * D > (1LL << 40) || T > (1LL << 31) - 1 - 256) return fail(G3_EINVAL, "B*S too large");
  if ((long long)Hq + 2LL * Hkv > 65535) return fail(G3_EINVAL, "Hq + 2 Hkv = %lld heads too many", (long long)Hq + 2LL * Hkv);
  if (256LL * d_model * 2 > (1LL << 32) - 1) return fail(G3_EUNSUPPORTED, "d_model=%d too large", d_model);
  g3::Pos0Table p0t;
  if (int e = make_pos0(pos0, B, S, &p0t)) return e;
  g3::QkvArgs a{};
  a.x = x;
  a.w = w;
  a.q = q;
  a.khat = khat;
  a.v = v;
  a.k_gamma = k_gamma;
  a.x_scale = x_scale;
  a.eps = eps;
  a.T = (int)T;
  a.S = S;
  a.K = d_model;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  hipStream_t st = (hipStream_t)stream;
  if (g_ev_start) hipEventRecord(g_ev_start, st);
  const hipError_t le = g3::launch_qkv_proj(a, p0t, rope_table(rope_base, interp_scale, D), st);
  if (le != hipSuccess) return fail(G3_EHIP, "qkv projection launch failed: %s", hipGetErrorString(le));
  if (g_ev_stop) hipEventRecord(g_ev_stop, st);
  return G3_OK;
}

size_t g3attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_position,
                                    const g3_kv_cache* cache) {
  if (!cache || B <= 0 || Hq <= 0 || Hkv <= 0 || max_position < 0 || cache->capacity <= 0 || !head_dim_ok(D))
    return 0;
  return decode_ws(B, Hq, D, decode_chunks(decode_slots(cache, max_position), B, Hkv));
}

}  // extern "C"

namespace {

// One decode step.  With noalloc the split-K partials go to the library's
// static per-GPU array instead of the caller's workspace.
int decode_impl(const g3_bf16* q, const g3_bf16* k_new, const g3_bf16* v_new, g3_bf16* o, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t D, const int32_t* positions, int32_t max_position, const g3_kv_cache* cache,
                int32_t layer_kind, int32_t window, float rope_base, float interp_scale, const float* q_gamma,
                const float* k_gamma, float eps, float softmax_scale, void* workspace, size_t workspace_bytes,
                bool noalloc, void* stream) {
  g_err[0] = 0;
  if (int e = check_heads(Hq, Hkv, D)) return e;
  if (B <= 0) return fail(G3_EINVAL, "B=%d must be positive", B);
  if (layer_kind != G3_LOCAL && layer_kind != G3_GLOBAL) return fail(G3_EINVAL, "layer_kind=%d", layer_kind);
  if (layer_kind == G3_LOCAL && window < 1) return fail(G3_EINVAL, "window=%d < 1", window);
  if (int e = check_rope(rope_base, interp_scale, eps)) return e;
  float sl2;
  if (int e = check_scale(softmax_scale, D, &sl2)) return e;
  if (!q || !k_new || !v_new || !o || !positions) return fail(G3_EINVAL, "q, k_new, v_new, o, positions must be non-NULL");
  for (const void* p : {(const void*)q, (const void*)k_new, (const void*)v_new, (const void*)o})
    if (!aligned16(p)) return fail(G3_EINVAL, "tensor pointers must be 16-byte aligned");
  if (!cache || !cache->k || !cache->v) return fail(G3_EINVAL, "decode needs a cache");
  if (!aligned16(cache->k) || !aligned16(cache->v)) return fail(G3_EINVAL, "cache pointers must be 16-byte aligned");
  if (cache->capacity <= 0) return fail(G3_EINVAL, "cache capacity %d", cache->capacity);
  if (max_position < 0) return fail(G3_EINVAL, "max_position %d < 0", max_position);
  if (cache->is_ring) {
    if (layer_kind != G3_LOCAL) return fail(G3_EINVAL, "a ring cache needs a local layer");
    if (window > cache->capacity) return fail(G3_EINVAL, "window %d exceeds ring capacity %d", window, cache->capacity);
  } else if (max_position >= cache->capacity) {
    return fail(G3_EINVAL, "max_position %d does not fit a linear cache of capacity %d", max_position, cache->capacity);
  }
  const int n_slots = decode_slots(cache, max_position);
  const int split = decode_split(n_slots, B, Hkv);
  const int n_chunks = decode_chunks(n_slots, B, Hkv);
  const size_t need = decode_ws(B, Hq, D, n_chunks);
  if (noalloc) {
    if (need > g3::kDecodeScratchBytes)
      return fail(G3_EWORKSPACE,
                  "decode needs %zu bytes of split-K scratch, above the %zu bytes of the static array behind "
                  "g3attn_decode_noalloc; call g3attn_decode with a workspace",
                  need, g3::kDecodeScratchBytes);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(G3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(G3_EINVAL, "workspace must be 256-byte aligned");
  }
  if ((long long)B * Hkv > 65535) return fail(G3_EUNSUPPORTED, "B*Hkv=%lld exceeds 65535", (long long)B * Hkv);
  if (noalloc) {
    if (hipError_t e = g3::decode_scratch(&workspace))
      return fail(G3_EHIP, "static decode scratch unavailable on this device: %s", hipGetErrorString(e));
  }

  g3::DecodeArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.ck = cache->k;
  a.cv = cache->v;
  a.positions = positions;
  a.q_gamma = q_gamma;
  a.k_gamma = k_gamma;
  a.ws = (float*)workspace;
  a.o = o;
  a.eps = eps;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.cap = cache->capacity;
  a.is_ring = cache->is_ring;
  a.local = layer_kind == G3_LOCAL;
  // a window past any position reach means no band limit; clamped so the
  // kernels' i + window - 1 cannot overflow
  a.window = layer_kind == G3_LOCAL ? (window < (1 << 30) ? window : (1 << 30)) : (1 << 30);
  a.max_pos = max_position;
  a.n_slots = n_slots;
  a.split = split;
  a.n_chunks = n_chunks;
  a.sl2 = sl2;
  a.D = D;
  if (hipError_t e = g3::launch_decode(a, rope_table(rope_base, interp_scale, D), Hq / Hkv, (hipStream_t)stream,
                                       g_ev_start, g_ev_stop))
    return fail(G3_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return G3_OK;
}

}  // namespace

extern "C" {

int g3attn_decode(const g3_bf16* q, const g3_bf16* k_new, const g3_bf16* v_new, g3_bf16* o, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, const int32_t* positions, int32_t max_position, const g3_kv_cache* cache,
                  int32_t layer_kind, int32_t window, float rope_base, float interp_scale, const float* q_gamma,
                  const float* k_gamma, float eps, float softmax_scale, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return decode_impl(q, k_new, v_new, o, B, Hq, Hkv, D, positions, max_position, cache, layer_kind, window, rope_base,
                     interp_scale, q_gamma, k_gamma, eps, softmax_scale, workspace, workspace_bytes, false, stream);
}

int g3attn_decode_noalloc(const g3_bf16* q, const g3_bf16* k_new, const g3_bf16* v_new, g3_bf16* o, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t D, const int32_t* positions, int32_t max_position,
                          const g3_kv_cache* cache, int32_t layer_kind, int32_t window, float rope_base,
                          float interp_scale, const float* q_gamma, const float* k_gamma, float eps,
                          float softmax_scale, void* stream) {
  return decode_impl(q, k_new, v_new, o, B, Hq, Hkv, D, positions, max_position, cache, layer_kind, window, rope_base,
                     interp_scale, q_gamma, k_gamma, eps, softmax_scale, nullptr, 0, true, stream);
}

}  // extern "C"
