/*
 * g3attn — Gemma 3 local/global GQA attention stack on AMD Instinct MI355X
 * (gfx950).  C ABI of the shared library libg3attn.so.
 *
 * The stack: five local sliding-window layers (span 1024 tokens, RoPE base
 * 10k) per global layer (full causal span, RoPE base 1M with linear position
 * interpolation), grouped-query attention, and QK-RMSNorm in place of logit
 * soft-capping (Gemma 3 Technical Report, section 1 "Introduction" and
 * section 2 "Model Architecture").  Image-token spans attend bidirectionally
 * ("Gemma explained: What's new in Gemma 3", vision section).
 *
 * Conventions for every call
 *   - Tensors are bf16 (uint16_t bit patterns) or fp32, contiguous row-major,
 *     in DEVICE memory owned by the caller; the head dimension D is innermost.
 *     Device pointers must be 16-byte aligned.  Arrays documented as host
 *     memory (spans, pos0) are read during the call only.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library allocates nothing, keeps no pointer after it
 *     returns, and never synchronises.  Its only mutable state is per calling
 *     thread: the text of the last error, and the two timing events that
 *     g3attn_set_timing_events installs (NULL unless a profiler sets them).
 *   - Return value: G3_OK (0) or a negative G3_E* code.  Argument errors are
 *     detected before any launch and leave every buffer untouched; the text
 *     of the last error on the calling thread is g3attn_last_error().  A
 *     device-side fault surfaces at the caller's next synchronisation.
 *   - GQA: query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 *   - Supported: D = 128 (the 27B print's q/k norms are over 128 values)
 *     and D = 256 (the 1B print: q_proj 1152 -> 1024 = 4 heads x 256,
 *     k_proj/v_proj 1152 -> 256 = 1 KV head, norms over 256 values; both in
 *     "Gemma explained: What's new in Gemma 3", model prints); Hq / Hkv in
 *     {1, 2, 4, 8}.
 */
#ifndef G3ATTN_H
#define G3ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t g3_bf16; /* bfloat16 bit pattern */

enum { G3_LOCAL = 0, G3_GLOBAL = 1 };

enum {
  G3_OK = 0,
  G3_EINVAL = -1,       /* bad argument (shape, pointer, alignment, range) */
  G3_EUNSUPPORTED = -2, /* valid but not implemented (e.g. D not 128 or 256) */
  G3_EHIP = -3,         /* a HIP launch failed */
  G3_EWORKSPACE = -4    /* workspace missing or too small */
};

/* One image span: tokens [start, end) of sequence `batch`, in absolute
 * positions, attend to each other in both directions; text stays causal.
 * (Gemma explained: bidirectional attention on image inputs.) */
typedef struct {
  int32_t batch;
  int32_t start;
  int32_t end;
} g3_span;

/* Per-layer KV cache, caller-owned device memory.
 * k, v: [B][Hkv][capacity][D] bf16.  K holds keys after QK-RMSNorm and RoPE
 * at their absolute position; V holds raw values.
 * is_ring = 0: linear cache, position j lives in slot j (global layers keep
 *              every position; Technical Report, section 1).
 * is_ring = 1: ring of the last `capacity` positions, position j in slot
 *              j mod capacity (local layers only need the last 1024 tokens;
 *              Technical Report, abstract and section 1).  Requires
 *              window <= capacity. */
typedef struct {
  g3_bf16* k;
  g3_bf16* v;
  int32_t capacity;
  int32_t is_ring;
} g3_kv_cache;

/* QK-RMSNorm then RoPE, per token and head (Technical Report, section 2:
 * QK-norm; "Long context": RoPE base, position interpolation; Gemma
 * explained 27B print: RMSNorm over (128,), eps 1e-6).
 *   x_hat = x / sqrt(mean(x^2) + eps) * gamma
 *   pairs (x_k, x_{k+D/2}) rotated by phi = (p / interp_scale) * base^(-2k/D)
 * q_in/q_out: [T][Hq][D]; k_in/k_out: [T][Hkv][D]; either pair may be NULL
 * (both members).  In place (q_out == q_in) is allowed.  gamma: device fp32
 * [D] or NULL for no norm.  positions: device int32 [T], >= 0.
 * interp_scale > 0 (1 = none). */
int g3attn_qknorm_rope(const g3_bf16* q_in, const g3_bf16* k_in, g3_bf16* q_out, g3_bf16* k_out,
                       const float* q_gamma, const float* k_gamma, float eps,
                       const int32_t* positions, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                       float rope_base, float interp_scale, void* stream);

/* Prefill of one attention layer: prologue (QK-RMSNorm + RoPE) and flash
 * attention over the visible keys only.
 * q: [B][S][Hq][D] raw; k, v: [B][S][Hkv][D] raw; o: [B][S][Hq][D].
 * Token r of sequence b is at position pos0[b] + r (pos0: host int32 [B] or
 * NULL for all zero).
 * Visibility of key position j to query position i (same sequence):
 *   global: j <= i, or i and j in one span;   local: that and |i - j| < window.
 * layer_kind: G3_LOCAL or G3_GLOBAL (window is ignored for global; a local
 *   window larger than 2^30 means no band limit).
 * softmax_scale: logit multiplier, 0 means D^-1/2; logits are not capped.
 * spans: host array of n_spans (<= 64) spans sorted by (batch, start),
 *   non-overlapping, each inside [pos0[b], pos0[b] + S); NULL if n_spans = 0.
 * cache: NULL for a self-contained prompt.  Otherwise this is a chunk of a
 *   longer sequence: positions below pos0[b] are read from the cache (a
 *   linear cache must hold 0..pos0[b]-1; a ring the last `capacity` of them)
 *   and, after the attention, the chunk's normed+rotated keys and raw values
 *   are written to their slots (a ring keeps only its last `capacity`).
 *   A linear cache needs capacity >= pos0[b] + S.
 * workspace: device, >= g3attn_prefill_workspace_size(B, S, Hq, Hkv, D)
 *   bytes, 256-byte aligned; its contents on entry do not matter.
 * Limits: B*S*Hq < 2^31 (else G3_EINVAL) and S*Hkv*D < 2^31 (element
 *   offsets inside one sequence are 32-bit; else G3_EUNSUPPORTED). */
int g3attn_prefill(const g3_bf16* q, const g3_bf16* k, const g3_bf16* v, g3_bf16* o,
                   int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t layer_kind, int32_t window, float rope_base, float interp_scale,
                   const float* q_gamma, const float* k_gamma, float eps, float softmax_scale,
                   const g3_span* spans, int32_t n_spans, const int32_t* pos0,
                   const g3_kv_cache* cache, void* workspace, size_t workspace_bytes, void* stream);

size_t g3attn_prefill_workspace_size(int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D);

/* The attention layer's input projections with the key prologue fused in:
 * q = x Wq^T, k = x Wk^T, v = x Wv^T (the layer's q_proj, k_proj and v_proj,
 * linear maps without bias: "Gemma explained: What's new in Gemma 3", 27B
 * module print), then k is QK-RMSNormed with k_gamma and rotated by RoPE at
 * its absolute position (Technical Report, section 2), the same steps as
 * the prologue of g3attn_prefill but applied to the unrounded fp32
 * projection, and written head-major for g3attn_prefill_khat.
 * Accumulation is fp32; outputs are rounded to bf16 once (k after its norm
 * and rotation).
 * x: [B][S][d_model] (the normed hidden states entering the layer, or the
 *   raw ones with x_scale below);
 * x_scale: device fp32 [B*S] or NULL.  When given, token t's projections are
 *   multiplied by x_scale[t] (in fp32, before rounding and before k's norm):
 *   with x the raw hidden states, x_scale from g3attn_rms_scale and w from
 *   g3attn_fold_norm_weight(w, input_layernorm gamma), the call computes the
 *   projections of the normed input without the normed copy of x ever being
 *   written (the input RMSNorm of the Technical Report, section 2, folded
 *   into the projection: (x/rms(x) * gamma) W^T = (1/rms(x)) x (W diag(gamma))^T);
 * w: [(Hq + 2 Hkv) * D][d_model], the rows of Wq, then Wk, then Wv (each
 *   row = one output feature, head h's features at rows h*D .. h*D + D-1);
 * q: [B][S][Hq][D] raw; khat: [B][Hkv][S][D] normed + rotated;
 * v: [B][S][Hkv][D] raw.  All outputs are written in full.
 * k_gamma: device fp32 [D] or NULL (no norm); pos0 as in g3attn_prefill.
 * Supported: D = 128 or 256 and d_model a multiple of 64 (else
 *   G3_EUNSUPPORTED);
 *   Hq + 2 Hkv <= 65535 and B*S < 2^31 - 256 (else G3_EINVAL).
 * The timing hook, when set, brackets the projection kernel. */
int g3attn_qkv_project(const g3_bf16* x, const float* x_scale, const g3_bf16* w, g3_bf16* q,
                       g3_bf16* khat, g3_bf16* v, int32_t B, int32_t S, int32_t d_model, int32_t Hq,
                       int32_t Hkv, int32_t D, float rope_base, float interp_scale,
                       const float* k_gamma, float eps, const int32_t* pos0, void* stream);

/* The per-token scale of the layer's input RMSNorm (Technical Report,
 * section 2: pre-norm with RMSNorm; "Gemma explained" 27B print: RMSNorm over
 * 5376, eps 1e-6) without the normed rows:
 *   scale[t] = 1 / sqrt(mean(x[t]^2) + eps)      (sums in fp32)
 * x: [T][width] bf16; scale: device fp32 [T].  For g3attn_qkv_project's
 * x_scale.  Supported: width a multiple of 8 up to 2^20 (else
 * G3_EUNSUPPORTED). */
int g3attn_rms_scale(const g3_bf16* x, float eps, float* scale, int32_t T, int32_t width, void* stream);

/* The input norm's gamma folded into a projection weight, once per layer at
 * load time: w_out[n][k] = w[n][k] * gamma[k] (fp32 product, rounded to bf16
 * once).  w, w_out: [rows][width] bf16 (w_out may alias w); gamma: device fp32
 * [width].  Supported: width a multiple of 8 (else G3_EUNSUPPORTED). */
int g3attn_fold_norm_weight(const g3_bf16* w, const float* gamma, g3_bf16* w_out, int32_t rows,
                            int32_t width, void* stream);

/* The layer's output projection o_proj: y = attn W_o^T ("Gemma explained:
 * What's new in Gemma 3", 27B module print: Linear 4096 -> 5376, no bias),
 * fp32 accumulation, y rounded to bf16 once.
 * attn: [T][in_features] (the attention output [B][S][Hq][D] seen as rows of
 *   Hq * D); w_o: [out_features][in_features]; y: [T][out_features].
 * Supported: in_features a multiple of 64 and out_features a multiple of 128
 *   (else G3_EUNSUPPORTED).  The timing hook, when set, brackets the kernel. */
int g3attn_o_project(const g3_bf16* attn, const g3_bf16* w_o, g3_bf16* y, int32_t T,
                     int32_t in_features, int32_t out_features, void* stream);

/* Row RMSNorm over the model width with an optional residual add, for the
 * layer's input_layernorm (before q/k/v projection) and
 * post_attention_layernorm (after o_proj, then added to the residual
 * stream): Technical Report, section 2 (pre-norm and post-norm with
 * RMSNorm); "Gemma explained" 27B print (RMSNorm over 5376, eps 1e-6).
 *   out[t] = residual[t] + x[t] / sqrt(mean(x[t]^2) + eps) * gamma
 * x, residual (NULL: no residual), out: [T][width] bf16; out may alias x or
 * residual.  gamma: device fp32 [width] or NULL (gamma = 1).  Sums in fp32,
 * out rounded to bf16 once.  Supported: width a multiple of 8 up to 8192
 * (else G3_EUNSUPPORTED). */
int g3attn_rmsnorm(const g3_bf16* x, const g3_bf16* residual, const float* gamma, float eps,
                   g3_bf16* out, int32_t T, int32_t width, void* stream);

/* g3attn_prefill with the key prologue already done: khat [B][Hkv][S][D]
 * holds the chunk's normed and rotated keys (as g3attn_qkv_project writes
 * them) and is read only.  Every other argument means what it means for
 * g3attn_prefill (q is still normed and rotated inside the flash kernel);
 * the workspace is sized by g3attn_prefill_workspace_size as well. */
int g3attn_prefill_khat(const g3_bf16* q, const g3_bf16* khat, const g3_bf16* v, g3_bf16* o,
                        int32_t B, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                        int32_t layer_kind, int32_t window, float rope_base, float interp_scale,
                        const float* q_gamma, float eps, float softmax_scale,
                        const g3_span* spans, int32_t n_spans, const int32_t* pos0,
                        const g3_kv_cache* cache, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: each sequence b adds one token at position positions[b].
 * Generation attends over the KV cache; local layers keep only the last
 * window of it (span 1024), global layers all of it, which is what keeps the
 * long-context cache small (Technical Report, abstract and section 1; the 5:1
 * local/global interleave, section 2).  The same QK-RMSNorm and RoPE as in
 * g3attn_qknorm_rope apply to q and to the new key.
 * q: [B][Hq][D] raw; k_new, v_new: [B][Hkv][D] raw; o: [B][Hq][D].
 * The new key is normed and rotated, written with v_new to its cache slot,
 * and the token attends to positions [0, p] (global) or
 * [max(0, p - window + 1), p] (local), itself included.  A window larger
 * than 2^30 means no band limit (the local layer then equals a global one).
 * positions: device int32 [B]; every entry must lie in [0, max_position]
 *   (host bound used to size the grid) and, for a linear cache, below
 *   capacity.  Entries outside that range are clamped by the kernels so no
 *   access leaves the cache, but the result for that sequence is undefined.
 * workspace: device, >= g3attn_decode_workspace_size(...) bytes, 256-byte
 *   aligned; contents on entry do not matter.  Split-K partials are merged in
 *   a fixed order, so results are bitwise reproducible. */
int g3attn_decode(const g3_bf16* q, const g3_bf16* k_new, const g3_bf16* v_new, g3_bf16* o,
                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                  const int32_t* positions, int32_t max_position, const g3_kv_cache* cache,
                  int32_t layer_kind, int32_t window, float rope_base, float interp_scale,
                  const float* q_gamma, const float* k_gamma, float eps, float softmax_scale,
                  void* workspace, size_t workspace_bytes, void* stream);

size_t g3attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_position, const g3_kv_cache* cache);

/* Size of the static per-GPU scratch array behind g3attn_decode_noalloc. */
#define G3_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)

/* g3attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Every argument means what it means for g3attn_decode; there is no
 * workspace argument: the split-K partials go to a static device array of
 * G3_DECODE_NOALLOC_MAX_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there).  The call allocates nothing and issues no memset
 * (nothing in the array needs to start at zero).
 * A call whose partials would need more than G3_DECODE_NOALLOC_MAX_BYTES
 * (g3attn_decode_workspace_size tells) returns G3_EWORKSPACE before any
 * launch.  All calls on one GPU share the array: calls that overlap in time
 * on that GPU (different streams, or host threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe. */
int g3attn_decode_noalloc(const g3_bf16* q, const g3_bf16* k_new, const g3_bf16* v_new, g3_bf16* o,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          const int32_t* positions, int32_t max_position, const g3_kv_cache* cache,
                          int32_t layer_kind, int32_t window, float rope_base, float interp_scale,
                          const float* q_gamma, const float* k_gamma, float eps, float softmax_scale,
                          void* stream);

/* Text of the last error on this thread ("" if none); valid until the next
 * call on this thread. */
const char* g3attn_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t g3attn_version(void);

/* Profiling hook for this thread.  When both are non-NULL (hipEvent_t
 * handles), the next g3attn_prefill / g3attn_prefill_khat / g3attn_decode /
 * g3attn_qkv_project / g3attn_o_project calls record `start` immediately
 * before and `stop` immediately after the launch of their main kernel (the
 * flash-attention kernel of a prefill, the split-K kernel of a decode, the
 * projection kernel), on the call's stream.  Pass NULL, NULL to turn it off. */
int g3attn_set_timing_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* G3ATTN_H */
